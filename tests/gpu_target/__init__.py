"""A tiny random causal target model on the GPU (test support).

``GpuTinyTarget`` runs the oracle's ``TinyTarget`` architecture and weights
(cast to fp32) through ``libtinytarget.so`` (tests/gpu_target/tiny_target.hip),
keeping its own KV cache on the device, so that the whole speculative loop --
target passes, drafting, fusion, verification -- runs on the GPU.  Its
per-row path is shape independent: a row's logits and features are bitwise
the same whether it is computed alone or among other rows.
"""

from __future__ import annotations

import ctypes
import os
from typing import List, Tuple

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtinytarget.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m tests.gpu_target.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int
        L.tt_forward.restype = i32
        L.tt_forward.argtypes = [ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_float), ctypes.POINTER(vp),
                                 ctypes.POINTER(vp), ctypes.POINTER(vp), i32, vp, i32, vp, ctypes.POINTER(i32), vp,
                                 vp, vp]
        _lib = L
    return _lib


class GpuTinyTarget:
    def __init__(self, tgt, max_len: int = 256, device="cuda"):
        """tgt: an ``oracle.TinyTarget`` (its weights are copied, as fp32)."""
        self.dev = torch.device(device)
        f32 = lambda a: torch.as_tensor(np.asarray(a, np.float32), device=self.dev).contiguous()  # noqa: E731
        self.V, self.H = tgt.vocab, tgt.hidden
        self.L = tgt.n_layers
        self.feature_layers = tuple(tgt.feature_layers)
        self.max_len = max_len
        ffn = tgt.layers[0]["wg"].shape[0]
        self.dims_i = (ctypes.c_int * 8)(tgt.vocab, tgt.hidden, tgt.n_heads, tgt.n_kv_heads, tgt.head_dim, ffn,
                                         tgt.n_layers, max_len)
        self.dims_f = (ctypes.c_float * 2)(1e-6, tgt.theta)
        self._w = [f32(tgt.embed)]
        for lw in tgt.layers:
            self._w += [f32(lw[k]) for k in ("wq", "wk", "wv", "wo", "wg", "wu", "wd")]
        self._w.append(f32(tgt.w_lm))
        self.w = (ctypes.c_void_p * len(self._w))(*[t.data_ptr() for t in self._w])
        nk = tgt.n_kv_heads * tgt.head_dim
        self.kc = [torch.zeros(max_len, nk, dtype=torch.float32, device=self.dev) for _ in range(self.L)]
        self.vc = [torch.zeros(max_len, nk, dtype=torch.float32, device=self.dev) for _ in range(self.L)]
        self.kcp = (ctypes.c_void_p * self.L)(*[t.data_ptr() for t in self.kc])
        self.vcp = (ctypes.c_void_p * self.L)(*[t.data_ptr() for t in self.vc])
        slot = {l: i for i, l in enumerate(self.feature_layers)}
        self.feat_layer = (ctypes.c_int * self.L)(*[slot.get(l, -1) for l in range(self.L)])
        self.nq = tgt.n_heads * tgt.head_dim
        self.length = 0

    def reset(self) -> None:
        self.length = 0

    def truncate(self, length: int) -> None:
        assert 0 <= length <= self.length
        self.length = length

    def forward(self, tokens) -> Tuple[torch.Tensor, List[torch.Tensor]]:
        """Rows at positions length .. length+n-1, appended to the cache.
        Returns device tensors: logits [n, V] and the fused layers' features,
        a list of [n, H] in the order of ``feature_layers``."""
        tok = torch.as_tensor(tokens, dtype=torch.int32, device=self.dev).reshape(-1).contiguous()
        n = tok.numel()
        if self.length + n > self.max_len:
            raise ValueError("target cache full")
        logits = torch.empty(n, self.V, dtype=torch.float32, device=self.dev)
        feats = torch.empty(len(self.feature_layers), n, self.H, dtype=torch.float32, device=self.dev)
        work = torch.empty(n * (2 * self.H + 2 * self.nq), dtype=torch.float32, device=self.dev)
        rc = lib().tt_forward(self.dims_i, self.dims_f, self.w, self.kcp, self.vcp, self.length, tok.data_ptr(), n,
                              logits.data_ptr(), self.feat_layer, feats.data_ptr(), work.data_ptr(),
                              ctypes.c_void_p(torch.cuda.current_stream(self.dev).cuda_stream))
        if rc != 0:
            raise RuntimeError(f"tt_forward failed: {rc}")
        self.length += n
        return logits, [feats[i] for i in range(len(self.feature_layers))]
