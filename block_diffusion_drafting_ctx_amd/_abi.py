"""Thin ctypes binding of libdflash.so (include/dflash.h).

Argument marshalling only: every function here checks the tensors it is
given (device, dtype, contiguity, shape) on the host and passes raw device
pointers and the current torch stream to the C entry point of the same name.
All compute happens in the library's HIP kernels; there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdflash.so")

DFLASH_OK, DFLASH_EINVAL, DFLASH_EUNSUPPORTED, DFLASH_EHIP, DFLASH_EDEVICE = 0, -1, -2, -3, -4
DTYPE_F32, DTYPE_BF16 = 0, 1
KV_STORAGE, KV_INT8 = 0, 1
ERR_FUSE_OVERFLOW, ERR_TOKEN_RANGE, ERR_VERIFY_OVERFLOW, ERR_DRAFT_OVERFLOW = 1, 2, 4, 8
STAGES = ["fuse_fc", "ctx_kv", "verify", "embed", "qkv", "attn", "oproj", "gateup", "down", "lmhead", "layer_gemm"]
STAGE = {n: i for i, n in enumerate(STAGES)}

EXPORTED = [
    "dflash_workspace_bytes", "dflash_kv_layer_bytes", "dflash_create", "dflash_reload_weights", "dflash_fuse_ctx", "dflash_verify",
    "dflash_verify_sample", "dflash_verify_static", "dflash_draft_block",
    "dflash_check", "dflash_clear_errors", "dflash_stats", "dflash_stage_timing", "dflash_stage_time",
    "dflash_destroy", "dflash_last_error", "dflash_version",
]


class DFlashError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"dflash status {status}: {msg}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "hidden", "n_q_heads", "n_kv_heads", "head_dim", "n_layers", "ffn", "vocab", "block",
        "n_target_layers", "max_batch", "max_ctx", "max_fuse_rows", "conv_width", "dtype")] + [
        ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float), ("kv_dtype", ctypes.c_int32)]


_PP = ctypes.POINTER(ctypes.c_void_p)


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("embed", "w_fc", "g_fc", "g_final", "w_lm")] + [
        (n, _PP) for n in ("w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down", "g_in", "g_post", "conv")]


_lib = None


def lib():
    """Load the library once; raise loudly if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m block_diffusion_drafting_ctx_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64
        sig = {
            "dflash_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Config)]),
            "dflash_kv_layer_bytes": (ctypes.c_size_t, [ctypes.POINTER(Config)]),
            "dflash_create": (i32, [ctypes.POINTER(Config), ctypes.POINTER(Weights), _PP, _PP, vp, vp,
                                    ctypes.c_size_t, ctypes.POINTER(vp)]),
            "dflash_reload_weights": (i32, [vp, vp]),
            "dflash_fuse_ctx": (i32, [vp, i32, _PP, i32, i32, vp, vp]),
            "dflash_verify": (i32, [vp, i32, vp, vp, i32, i32, vp, vp, vp, vp]),
            "dflash_verify_sample": (i32, [vp, i32, vp, vp, i32, i32, ctypes.c_float, vp, vp, vp, vp, vp]),
            "dflash_verify_static": (i32, [i32, i32, vp, vp, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp]),
            "dflash_draft_block": (i32, [vp, i32, vp, vp, vp, vp, vp]),
            "dflash_check": (i32, [vp, ctypes.POINTER(ctypes.c_uint32), vp]),
            "dflash_clear_errors": (i32, [vp, vp]),
            "dflash_stats": (i32, [vp, ctypes.POINTER(u64), vp]),
            "dflash_stage_timing": (i32, [vp, i32, i32]),
            "dflash_stage_time": (i32, [vp, i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64),
                                        vp]),
            "dflash_destroy": (None, [vp]),
            "dflash_last_error": (ctypes.c_char_p, []),
            "dflash_version": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != DFLASH_OK:
        raise DFlashError(status, lib().dflash_last_error().decode())


def _stream(stream: Optional[torch.cuda.Stream]) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t: Optional[torch.Tensor], dtype=None, numel=None, name="tensor") -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    return t.data_ptr()


def make_config(hidden, n_q_heads, n_kv_heads, head_dim, n_layers, ffn, vocab, block, n_target_layers,
                max_batch, max_ctx, max_fuse_rows, conv_width=0, dtype="bf16", rms_eps=1e-6,
                rope_theta=1e6, kv="storage") -> Config:
    """kv: "storage" (the KV cache in the storage dtype) or "int8" (8-bit cache)."""
    if kv not in ("storage", "int8"):
        raise ValueError("kv must be 'storage' or 'int8'")
    return Config(hidden, n_q_heads, n_kv_heads, head_dim, n_layers, ffn, vocab, block, n_target_layers,
                  max_batch, max_ctx, max_fuse_rows, conv_width,
                  DTYPE_BF16 if dtype in ("bf16", torch.bfloat16, DTYPE_BF16) else DTYPE_F32,
                  rms_eps, rope_theta, KV_INT8 if kv == "int8" else KV_STORAGE)


def dflash_workspace_bytes(cfg: Config) -> int:
    return int(lib().dflash_workspace_bytes(ctypes.byref(cfg)))


def dflash_kv_layer_bytes(cfg: Config) -> int:
    return int(lib().dflash_kv_layer_bytes(ctypes.byref(cfg)))


class Context:
    """An opened library context plus the buffers it points at (kept alive here)."""

    def __init__(self, handle, cfg, keep):
        self.handle = handle
        self.cfg = cfg
        self._keep = keep

    def close(self):
        if self.handle:
            lib().dflash_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def dflash_create(cfg: Config, weights: dict, kv_k: Sequence[torch.Tensor], kv_v: Sequence[torch.Tensor],
                  ctx_len: torch.Tensor, workspace: torch.Tensor) -> Context:
    """weights: dict with embed, w_fc, g_fc, g_final, w_lm and ``layers`` (list of
    dicts with w_q, w_k, w_v, w_o, w_gate, w_up, w_down, g_in, g_post, conv)."""
    dt = torch.bfloat16 if cfg.dtype == DTYPE_BF16 else torch.float32
    nl = cfg.n_layers
    if len(weights["layers"]) != nl or len(kv_k) != nl or len(kv_v) != nl:
        raise ValueError("per-layer lists must have n_layers entries")
    h, d = cfg.hidden, cfg.head_dim
    shapes = {"w_q": (cfg.n_q_heads * d, h), "w_k": (cfg.n_kv_heads * d, h), "w_v": (cfg.n_kv_heads * d, h),
              "w_o": (h, cfg.n_q_heads * d), "w_gate": (cfg.ffn, h), "w_up": (cfg.ffn, h),
              "w_down": (h, cfg.ffn), "g_in": (h,), "g_post": (h,), "conv": (h, 3)}
    top = {"embed": (cfg.vocab, h), "w_fc": (h, cfg.n_target_layers * h), "g_fc": (h,), "g_final": (h,),
           "w_lm": (cfg.vocab, h)}
    for k, shp in top.items():
        t = weights[k]
        if tuple(t.shape) != shp:
            raise ValueError(f"{k}: shape {tuple(t.shape)} != {shp}")
        _ptr(t, dt, name=k)
    arrays = {}
    for k, shp in shapes.items():
        ptrs = []
        for lw in weights["layers"]:
            t = lw.get(k)
            if t is None:
                if k == "conv" and not cfg.conv_width:
                    ptrs.append(None)
                    continue
                raise ValueError(f"missing layer weight {k}")
            if tuple(t.shape) != shp:
                raise ValueError(f"{k}: shape {tuple(t.shape)} != {shp}")
            ptrs.append(_ptr(t, dt, name=k))
        arrays[k] = (ctypes.c_void_p * nl)(*ptrs)
    kv_bytes = dflash_kv_layer_bytes(cfg)
    if cfg.kv_dtype == KV_INT8:  # raw buffers of dflash_kv_layer_bytes bytes
        def cache_ptr(t, name):
            p = _ptr(t, None, None, name)
            if t.numel() * t.element_size() < kv_bytes:
                raise ValueError(f"{name} needs {kv_bytes} bytes")
            return p
    else:
        def cache_ptr(t, name):
            return _ptr(t, dt, kv_bytes // (2 if dt == torch.bfloat16 else 4), name)
    kk = (ctypes.c_void_p * nl)(*[cache_ptr(t, "kv_k") for t in kv_k])
    vv = (ctypes.c_void_p * nl)(*[cache_ptr(t, "kv_v") for t in kv_v])
    _ptr(ctx_len, torch.int32, cfg.max_batch, "ctx_len")
    need = dflash_workspace_bytes(cfg)
    if need == 0:
        raise DFlashError(DFLASH_EUNSUPPORTED, "configuration rejected by dflash_workspace_bytes")
    _ptr(workspace, None, None, "workspace")
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    w = Weights(weights["embed"].data_ptr(), weights["w_fc"].data_ptr(), weights["g_fc"].data_ptr(),
                weights["g_final"].data_ptr(), weights["w_lm"].data_ptr(),
                *[ctypes.cast(arrays[k], _PP) for k in ("w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down",
                                                        "g_in", "g_post")],
                ctypes.cast(arrays["conv"], _PP) if cfg.conv_width else None)
    out = ctypes.c_void_p()
    _check(lib().dflash_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.cast(kk, _PP), ctypes.cast(vv, _PP),
                               ctypes.c_void_p(ctx_len.data_ptr()), ctypes.c_void_p(workspace.data_ptr()),
                               workspace.numel() * workspace.element_size(), ctypes.byref(out)))
    keep = dict(weights=weights, kv_k=list(kv_k), kv_v=list(kv_v), ctx_len=ctx_len, workspace=workspace,
                arrays=arrays)
    return Context(out, cfg, keep)


def dflash_fuse_ctx(ctx: Context, hidden: Sequence[torch.Tensor], commit: bool,
                    feat_dbg: Optional[torch.Tensor] = None, stream=None) -> None:
    cfg = ctx.cfg
    if len(hidden) != cfg.n_target_layers:
        raise ValueError("need one hidden-state tensor per fused target layer")
    b, t, h = hidden[0].shape
    dt = torch.bfloat16 if cfg.dtype == DTYPE_BF16 else torch.float32
    for x in hidden:
        if tuple(x.shape) != (b, t, h) or h != cfg.hidden:
            raise ValueError("hidden states must all be [batch, t_new, hidden]")
    arr = (ctypes.c_void_p * len(hidden))(*[_ptr(x, dt, name="hidden") for x in hidden])
    fd = _ptr(feat_dbg, torch.float32, b * t * h, "feat_dbg")
    _check(lib().dflash_fuse_ctx(ctx.handle, b, ctypes.cast(arr, _PP), t, int(bool(commit)), fd, _stream(stream)))


def dflash_verify(ctx: Context, target_logits: torch.Tensor, draft_ids: torch.Tensor, draft_stride: int, n_d: int,
                  n_accept: torch.Tensor, bonus: torch.Tensor, out_tokens: torch.Tensor, stream=None) -> None:
    b = target_logits.shape[0]
    if tuple(target_logits.shape) != (b, n_d + 1, ctx.cfg.vocab):
        raise ValueError("target_logits must be [batch, n_d + 1, vocab]")
    lp = _ptr(target_logits, torch.float32, name="target_logits")
    if n_d > 0:
        if draft_ids.dtype != torch.int32 or not draft_ids.is_cuda:
            raise ValueError("draft_ids must be a device int32 tensor")
        span = (b - 1) * draft_stride + n_d
        base = draft_ids.storage_offset()
        if base + span > draft_ids.untyped_storage().nbytes() // 4:
            raise ValueError("draft_ids too small for batch * draft_stride")
        dp = draft_ids.data_ptr()
    else:
        dp = None
    _check(lib().dflash_verify(ctx.handle, b, lp, dp, draft_stride, n_d,
                               _ptr(n_accept, torch.int32, b, "n_accept"), _ptr(bonus, torch.int32, b, "bonus"),
                               _ptr(out_tokens, torch.int32, b * (n_d + 1), "out_tokens"), _stream(stream)))


def dflash_verify_sample(ctx: Context, target_logits: torch.Tensor, draft_ids: torch.Tensor, draft_stride: int,
                         n_d: int, temperature: float, uniforms: torch.Tensor, n_accept: torch.Tensor,
                         bonus: torch.Tensor, out_tokens: torch.Tensor, stream=None) -> None:
    b = target_logits.shape[0]
    if tuple(target_logits.shape) != (b, n_d + 1, ctx.cfg.vocab):
        raise ValueError("target_logits must be [batch, n_d + 1, vocab]")
    lp = _ptr(target_logits, torch.float32, name="target_logits")
    if n_d > 0:
        if draft_ids.dtype != torch.int32 or not draft_ids.is_cuda:
            raise ValueError("draft_ids must be a device int32 tensor")
        span = (b - 1) * draft_stride + n_d
        if draft_ids.storage_offset() + span > draft_ids.untyped_storage().nbytes() // 4:
            raise ValueError("draft_ids too small for batch * draft_stride")
        dp = draft_ids.data_ptr()
    else:
        dp = None
    _check(lib().dflash_verify_sample(ctx.handle, b, lp, dp, draft_stride, n_d, float(temperature),
                                      _ptr(uniforms, torch.float32, b * (n_d + 1) * 2, "uniforms"),
                                      _ptr(n_accept, torch.int32, b, "n_accept"), _ptr(bonus, torch.int32, b, "bonus"),
                                      _ptr(out_tokens, torch.int32, b * (n_d + 1), "out_tokens"), _stream(stream)))


def dflash_verify_static(target_logits: torch.Tensor, draft_ids: torch.Tensor, draft_stride: int, n_d: int,
                         ctx_len: torch.Tensor, max_ctx: int, n_accept: torch.Tensor, bonus: torch.Tensor,
                         out_tokens: torch.Tensor, stats: Optional[torch.Tensor] = None,
                         error_word: Optional[torch.Tensor] = None, stream=None) -> None:
    """Context-free greedy verify (library-owned static scratch; allocates nothing)."""
    if target_logits.dim() != 3 or target_logits.shape[1] != n_d + 1:
        raise ValueError("target_logits must be [batch, n_d + 1, vocab]")
    b, vocab = target_logits.shape[0], target_logits.shape[2]
    lp = _ptr(target_logits, torch.float32, name="target_logits")
    if n_d > 0:
        if draft_ids.dtype != torch.int32 or not draft_ids.is_cuda:
            raise ValueError("draft_ids must be a device int32 tensor")
        span = (b - 1) * draft_stride + n_d
        if draft_ids.storage_offset() + span > draft_ids.untyped_storage().nbytes() // 4:
            raise ValueError("draft_ids too small for batch * draft_stride")
        dp = draft_ids.data_ptr()
    else:
        dp = None
    sp = None if stats is None else _ptr(stats, torch.int64, 3, "stats")
    ep = None if error_word is None else _ptr(error_word, torch.int32, 1, "error_word")
    _check(lib().dflash_verify_static(b, vocab, lp, dp, draft_stride, n_d, _ptr(ctx_len, torch.int32, b, "ctx_len"),
                                      int(max_ctx), _ptr(n_accept, torch.int32, b, "n_accept"),
                                      _ptr(bonus, torch.int32, b, "bonus"),
                                      _ptr(out_tokens, torch.int32, b * (n_d + 1), "out_tokens"), sp, ep,
                                      _stream(stream)))


def dflash_draft_block(ctx: Context, block_ids: torch.Tensor, draft_ids: torch.Tensor,
                       logits_dbg: Optional[torch.Tensor] = None, hidden_dbg: Optional[torch.Tensor] = None,
                       stream=None) -> None:
    cfg = ctx.cfg
    b = block_ids.shape[0]
    if tuple(block_ids.shape) != (b, cfg.block):
        raise ValueError("block_ids must be [batch, block]")
    m = b * cfg.block
    _check(lib().dflash_draft_block(ctx.handle, b, _ptr(block_ids, torch.int32, m, "block_ids"),
                                    _ptr(draft_ids, torch.int32, m, "draft_ids"),
                                    _ptr(logits_dbg, torch.float32, m * cfg.vocab, "logits_dbg"),
                                    _ptr(hidden_dbg, torch.float32, m * cfg.hidden, "hidden_dbg"),
                                    _stream(stream)))


def dflash_check(ctx: Context, stream=None) -> int:
    bits = ctypes.c_uint32(0)
    st = lib().dflash_check(ctx.handle, ctypes.byref(bits), _stream(stream))
    if st not in (DFLASH_OK, DFLASH_EDEVICE):
        _check(st)
    return int(bits.value)


def dflash_reload_weights(ctx: Context, stream=None) -> None:
    _check(lib().dflash_reload_weights(ctx.handle, _stream(stream)))


def dflash_clear_errors(ctx: Context, stream=None) -> None:
    _check(lib().dflash_clear_errors(ctx.handle, _stream(stream)))


def dflash_stats(ctx: Context, stream=None) -> List[int]:
    out = (ctypes.c_uint64 * 3)()
    _check(lib().dflash_stats(ctx.handle, out, _stream(stream)))
    return [int(v) for v in out]


def dflash_stage_timing(ctx: Context, stage: str, enable: bool) -> None:
    _check(lib().dflash_stage_timing(ctx.handle, STAGE[stage], int(bool(enable))))


def dflash_stage_time(ctx: Context, stage: str, stream=None):
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    _check(lib().dflash_stage_time(ctx.handle, STAGE[stage], ctypes.byref(ms), ctypes.byref(n), _stream(stream)))
    return float(ms.value), int(n.value)


def dflash_version() -> str:
    return lib().dflash_version().decode()
