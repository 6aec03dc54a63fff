"""Seeded synthetic inputs shared by the oracle, the GPU parity tests and bench.py.

This module holds none of the method's arithmetic: it only draws random
numbers, rounds stored values to the storage type (torch's own
round-to-nearest-even float32 -> bfloat16 cast) and plants argmax agreement
into synthetic target logits.  It imports neither the oracle nor the
product package.

Workloads (no trained weights exist here; every tensor is random):

* ``tiny-f32-b1``: hidden 256, 4 query / 2 KV heads of 64, 2 layers, FFN 512,
  vocab 1024, block 8, context 64, features from 3 target layers (768 -> 256),
  float32 storage, batch 1; verify logits with planted agreement lengths in
  [0, 8].
* ``qwen3-8b-shape-b1``: hidden 4096, 32/8 heads of 128, 5 layers, FFN 12288,
  vocab 151936, block 16, context 4096, 5 target layers (20480 -> 4096),
  bfloat16 storage, batch 1.
* ``qwen3-8b-shape-b32-ragged``: the same draft at batch 32, context lengths
  uniform in [512, 4096] per sequence, planted agreement uniform in [0, 16].
* ``long-ctx-32k-b4``: the 8-layer variant at batch 4 with 32768 context.
* ``dflash2-27b-shape-conv-b8``: hidden 5120, 40/8 heads of 128, 5 layers,
  FFN 17408, vocab 151936, block 16, context 8192, batch 8, with the width-3
  per-channel block convolution (taps N(0, 0.1)); 5 target layers.
* ``long-ctx-32k-b4-kv8`` / ``qwen3-8b-shape-b1-kv8``: those workloads with
  the 8-bit draft KV cache.

Value recipe: matrices, embedding and LM head N(0, 0.02); RMSNorm gains 1.0;
target hidden states of fused layer j (0-based) N(0, (1 + j)^2) except the
tiny workload (N(0, 1)); pre-filled context K/V entries N(0, (0.02 sqrt(H))^2),
the spread a unit-RMS feature gets through an N(0, 0.02) projection (with the
8-bit cache: integers N(0, 32^2) rounded and clipped to +-127 times a scale
0.02 sqrt(H) / 32 for every run of 32, the same spread); target logits
N(0, 1) with planted agreement.
"""

from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, List, Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_layers: int
    ffn: int
    vocab: int
    block: int
    n_target_layers: int
    batch: int
    ctx_lo: int
    ctx_hi: int
    storage: str  # "f32" | "bf16"
    conv_width: int = 0
    accept_lo: int = 0
    accept_hi: int = 16
    scaled_hidden: bool = True
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    kv: str = "storage"  # draft KV cache: "storage" (the storage dtype) or "int8"

    @property
    def mask_id(self) -> int:
        return self.vocab - 1

    @property
    def n_d(self) -> int:
        """Drafts verified per step in the benchmark layout (all block rows)."""
        return self.block

    @property
    def t_new(self) -> int:
        """Target rows fused per step: the verified positions."""
        return self.block + 1

    @property
    def max_ctx(self) -> int:
        """Cache rows per sequence: the longest context plus two steps of room."""
        room = 2 * (self.block + 1)
        return ((self.ctx_hi + room + 63) // 64) * 64

    @property
    def torch_dtype(self):
        return torch.float32 if self.storage == "f32" else torch.bfloat16

    def with_batch(self, batch: int) -> "Workload":
        return replace(self, batch=batch)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny-f32-b1", 256, 4, 2, 64, 2, 512, 1024, 8, 3, 1, 64, 64, "f32",
                 accept_hi=8, scaled_hidden=False),
        Workload("qwen3-8b-shape-b1", 4096, 32, 8, 128, 5, 12288, 151936, 16, 5, 1, 4096, 4096, "bf16"),
        Workload("qwen3-8b-shape-b32-ragged", 4096, 32, 8, 128, 5, 12288, 151936, 16, 5, 32, 512, 4096,
                 "bf16"),
        Workload("long-ctx-32k-b4", 4096, 32, 8, 128, 8, 12288, 151936, 16, 5, 4, 32768, 32768, "bf16"),
        Workload("dflash2-27b-shape-conv-b8", 5120, 40, 8, 128, 5, 17408, 151936, 16, 5, 8, 8192, 8192,
                 "bf16", conv_width=3),
        Workload("long-ctx-32k-b4-kv8", 4096, 32, 8, 128, 8, 12288, 151936, 16, 5, 4, 32768, 32768, "bf16",
                 kv="int8"),
        Workload("qwen3-8b-shape-b1-kv8", 4096, 32, 8, 128, 5, 12288, 151936, 16, 5, 1, 4096, 4096, "bf16",
                 kv="int8"),
    ]
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, std, gen, device, dtype) -> torch.Tensor:
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def draft_weights(wl: Workload, seed: int, device="cpu") -> dict:
    """Random draft weights in the storage dtype, drawn in a fixed order.

    Layout: matrices [out_features, in_features]; w_fc [H, K*H] whose column
    block j multiplies target layer j; conv [H, 3] taps for rows (i-1, i, i+1).
    """
    g = _gen(seed, device)
    dt = wl.torch_dtype
    h, d = wl.hidden, wl.head_dim
    ones = lambda n: torch.ones(n, device=device, dtype=dt)  # noqa: E731
    w = {
        "embed": _normal((wl.vocab, h), 0.02, g, device, dt),
        "w_fc": _normal((h, wl.n_target_layers * h), 0.02, g, device, dt),
        "g_fc": ones(h),
        "layers": [],
    }
    for _ in range(wl.n_layers):
        lw = {
            "w_q": _normal((wl.n_q_heads * d, h), 0.02, g, device, dt),
            "w_k": _normal((wl.n_kv_heads * d, h), 0.02, g, device, dt),
            "w_v": _normal((wl.n_kv_heads * d, h), 0.02, g, device, dt),
            "w_o": _normal((h, wl.n_q_heads * d), 0.02, g, device, dt),
            "w_gate": _normal((wl.ffn, h), 0.02, g, device, dt),
            "w_up": _normal((wl.ffn, h), 0.02, g, device, dt),
            "w_down": _normal((h, wl.ffn), 0.02, g, device, dt),
            "g_in": ones(h),
            "g_post": ones(h),
            "conv": _normal((h, 3), 0.1, g, device, dt) if wl.conv_width else None,
        }
        w["layers"].append(lw)
    w["g_final"] = ones(h)
    w["w_lm"] = _normal((wl.vocab, h), 0.02, g, device, dt)
    return w


def target_hidden(wl: Workload, batch: int, rows: int, seed: int, device="cpu") -> List[torch.Tensor]:
    """Hidden states of the fused target layers: K tensors [batch, rows, H]."""
    g = _gen(seed, device)
    out = []
    for j in range(wl.n_target_layers):
        s = float(1 + j) if wl.scaled_hidden else 1.0
        out.append(_normal((batch, rows, wl.hidden), s, g, device, wl.torch_dtype))
    return out


def context_lengths(wl: Workload, seed: int, batch: Optional[int] = None) -> np.ndarray:
    b = wl.batch if batch is None else batch
    rng = np.random.default_rng(seed)
    return rng.integers(wl.ctx_lo, wl.ctx_hi + 1, size=b).astype(np.int32)


def context_kv(wl: Workload, ctx_lens: np.ndarray, seed: int, device="cpu", poison: bool = False):
    """Pre-filled draft KV cache: per layer K and V tensors [B, max_ctx, Hkv, D].

    Rows below ctx_lens[b] hold N(0, (0.02 sqrt(H))^2) entries; the rest are
    zero, or NaN with ``poison`` so that any read of them shows.  With the
    8-bit cache every entry is a pair (values int8 [B, max_ctx, Hkv, D],
    run scales float32 [B, max_ctx, Hkv, D/32]); rows past the context have
    zero values and zero (NaN with ``poison``) scales.
    """
    g = _gen(seed, device)
    b = len(ctx_lens)
    shape = (b, wl.max_ctx, wl.n_kv_heads, wl.head_dim)
    std = 0.02 * float(np.sqrt(wl.hidden))
    if wl.kv == "int8":
        return _context_kv8(wl, ctx_lens, g, device, poison, shape, std)
    ks, vs = [], []
    for _ in range(wl.n_layers):
        for lst in (ks, vs):
            t = torch.full(shape, float("nan") if poison else 0.0, device=device, dtype=wl.torch_dtype)
            for i in range(b):
                n = int(ctx_lens[i])
                if n:
                    t[i, :n] = _normal((n,) + shape[2:], std, g, device, wl.torch_dtype)
            lst.append(t)
    return ks, vs


def _context_kv8(wl, ctx_lens, g, device, poison, shape, std):
    b = len(ctx_lens)
    sshape = shape[:-1] + (shape[-1] // 32,)
    ks, vs = [], []
    for _ in range(wl.n_layers):
        for lst in (ks, vs):
            q = torch.zeros(shape, device=device, dtype=torch.int8)
            s = torch.full(sshape, float("nan") if poison else 0.0, device=device, dtype=torch.float32)
            for i in range(b):
                n = int(ctx_lens[i])
                if n:
                    z = torch.randn((n,) + shape[2:], generator=g, device=device, dtype=torch.float32)
                    q[i, :n] = z.mul_(32.0).round_().clamp_(-127, 127).to(torch.int8)
                    s[i, :n] = std / 32.0
            lst.append((q, s))
    return ks, vs


def block_ids(wl: Workload, batch: int, seed: int) -> np.ndarray:
    """Block token ids [B, Bs]: one random token then mask ids."""
    rng = np.random.default_rng(seed)
    ids = np.full((batch, wl.block), wl.mask_id, dtype=np.int32)
    ids[:, 0] = rng.integers(0, wl.vocab - 1, size=batch)
    return ids


def draft_tokens(wl: Workload, batch: int, n: int, seed: int) -> np.ndarray:
    """Random drafted tokens [B, n] (verify inputs independent of any drafter)."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, wl.vocab, size=(batch, n)).astype(np.int32)


def accept_lengths(wl: Workload, batch: int, seed: int, n_d: Optional[int] = None) -> np.ndarray:
    rng = np.random.default_rng(seed)
    hi = min(wl.accept_hi, wl.n_d if n_d is None else n_d)
    return rng.integers(wl.accept_lo, hi + 1, size=batch).astype(np.int32)


def planted_logits(wl: Workload, draft: np.ndarray, accept: np.ndarray, n_d: int, seed: int,
                   device="cpu") -> torch.Tensor:
    """Target logits [B, n_d + 1, V] float32, N(0, 1), with planted agreement.

    For sequence b and row i < accept[b] the drafted token draft[b, i] gets
    the row maximum + 1 (a unique top entry); if accept[b] < n_d, the drafted
    token of row accept[b] gets the row minimum - 1, so it cannot be the top.
    The greedy verify of these logits then accepts exactly accept[b] drafts.
    """
    g = _gen(seed, device)
    b = draft.shape[0]
    lg = torch.randn((b, n_d + 1, wl.vocab), generator=g, device=device, dtype=torch.float32)
    for s in range(b):
        a = int(accept[s])
        for i in range(a):
            lg[s, i, int(draft[s, i])] = lg[s, i].max() + 1.0
        if a < n_d:
            lg[s, a, int(draft[s, a])] = lg[s, a].min() - 1.0
    return lg
