"""Convenience owner of the caller-side buffers of one library context.

Allocates (with torch, on one device) the persistent draft KV cache, the
context lengths and the workspace, opens a context over given draft weights,
and forwards to the C entry points.  Plumbing only: no arithmetic here.
"""

from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import _abi


class Drafter:
    """kv_k / kv_v: per layer, the cache tensor [max_batch, max_ctx, Hkv, D] of
    the storage dtype, or (8-bit cache) a raw uint8 buffer of
    dflash_kv_layer_bytes bytes (see ``kv8_buffer``)."""

    def __init__(self, cfg: _abi.Config, weights: dict, device="cuda",
                 kv_k: Optional[Sequence[torch.Tensor]] = None, kv_v: Optional[Sequence[torch.Tensor]] = None):
        self.cfg = cfg
        self.device = torch.device(device)
        dt = torch.bfloat16 if cfg.dtype == _abi.DTYPE_BF16 else torch.float32
        shape = (cfg.max_batch, cfg.max_ctx, cfg.n_kv_heads, cfg.head_dim)
        self.kv8 = cfg.kv_dtype == _abi.KV_INT8

        def fresh():
            if self.kv8:
                return torch.zeros(_abi.dflash_kv_layer_bytes(cfg), dtype=torch.uint8, device=self.device)
            return torch.zeros(shape, dtype=dt, device=self.device)

        self.kv_k = list(kv_k) if kv_k is not None else [fresh() for _ in range(cfg.n_layers)]
        self.kv_v = list(kv_v) if kv_v is not None else [fresh() for _ in range(cfg.n_layers)]
        self.ctx_len = torch.zeros(cfg.max_batch, dtype=torch.int32, device=self.device)
        nbytes = _abi.dflash_workspace_bytes(cfg)
        if nbytes == 0:
            raise _abi.DFlashError(_abi.DFLASH_EUNSUPPORTED, "configuration rejected")
        self.workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        off = (-self.workspace.data_ptr()) % 256
        ws = self.workspace[off:off + nbytes]
        self.ctx = _abi.dflash_create(cfg, weights, self.kv_k, self.kv_v, self.ctx_len, ws)

    def kv_values(self, layer: int, kind: str) -> torch.Tensor:
        """The cache values of one layer ("k" or "v") as [max_batch, max_ctx, Hkv, D]
        (int8 for the 8-bit cache)."""
        buf = (self.kv_k if kind == "k" else self.kv_v)[layer]
        if not self.kv8:
            return buf
        c = self.cfg
        n = c.max_batch * c.max_ctx * c.n_kv_heads * c.head_dim
        return buf[:n].view(torch.int8).view(c.max_batch, c.max_ctx, c.n_kv_heads, c.head_dim)

    def kv_scales(self, layer: int, kind: str) -> torch.Tensor:
        """Run scales of the 8-bit cache as float32 [max_batch, max_ctx, Hkv, D/32]."""
        assert self.kv8
        return kv8_scales_view((self.kv_k if kind == "k" else self.kv_v)[layer], self.cfg)

    def reload_weights(self, stream=None):
        _abi.dflash_reload_weights(self.ctx, stream)

    def fuse_ctx(self, hidden, commit: bool, feat_dbg=None, stream=None):
        _abi.dflash_fuse_ctx(self.ctx, hidden, commit, feat_dbg, stream)

    def verify(self, logits, draft_ids, draft_stride, n_d, n_accept, bonus, out_tokens, stream=None):
        _abi.dflash_verify(self.ctx, logits, draft_ids, draft_stride, n_d, n_accept, bonus, out_tokens, stream)

    def verify_sample(self, logits, draft_ids, draft_stride, n_d, temperature, uniforms, n_accept, bonus,
                      out_tokens, stream=None):
        _abi.dflash_verify_sample(self.ctx, logits, draft_ids, draft_stride, n_d, temperature, uniforms, n_accept,
                                  bonus, out_tokens, stream)

    def draft_block(self, block_ids, draft_ids, logits_dbg=None, hidden_dbg=None, stream=None):
        _abi.dflash_draft_block(self.ctx, block_ids, draft_ids, logits_dbg, hidden_dbg, stream)

    def check(self, stream=None) -> int:
        return _abi.dflash_check(self.ctx, stream)

    def clear_errors(self, stream=None):
        _abi.dflash_clear_errors(self.ctx, stream)

    def stats(self, stream=None):
        return _abi.dflash_stats(self.ctx, stream)

    def close(self):
        self.ctx.close()


def kv8_scales_view(buf: torch.Tensor, cfg: _abi.Config) -> torch.Tensor:
    """The float32 scale section [max_batch, max_ctx, Hkv, D/32] of one raw
    8-bit cache buffer (the layout dflash_kv_layer_bytes describes)."""
    n = cfg.max_batch * cfg.max_ctx * cfg.n_kv_heads * cfg.head_dim
    off = (n + 255) // 256 * 256
    return buf[off:off + n // 32 * 4].view(torch.float32).view(cfg.max_batch, cfg.max_ctx, cfg.n_kv_heads,
                                                                cfg.head_dim // 32)


def kv8_buffer(values: torch.Tensor, scales: torch.Tensor, cfg: _abi.Config) -> torch.Tensor:
    """A raw 8-bit cache buffer holding given int8 values [B, max_ctx, Hkv, D]
    and float32 run scales [B, max_ctx, Hkv, D/32] (copied; B <= max_batch)."""
    buf = torch.zeros(_abi.dflash_kv_layer_bytes(cfg), dtype=torch.uint8, device=values.device)
    n = cfg.max_batch * cfg.max_ctx * cfg.n_kv_heads * cfg.head_dim
    vals = buf[:n].view(torch.int8).view(cfg.max_batch, cfg.max_ctx, cfg.n_kv_heads, cfg.head_dim)
    vals[: values.shape[0]].copy_(values)
    kv8_scales_view(buf, cfg)[: scales.shape[0]].copy_(scales)
    return buf
