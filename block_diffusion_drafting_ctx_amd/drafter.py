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
    def __init__(self, cfg: _abi.Config, weights: dict, device="cuda",
                 kv_k: Optional[Sequence[torch.Tensor]] = None, kv_v: Optional[Sequence[torch.Tensor]] = None):
        self.cfg = cfg
        self.device = torch.device(device)
        dt = torch.bfloat16 if cfg.dtype == _abi.DTYPE_BF16 else torch.float32
        shape = (cfg.max_batch, cfg.max_ctx, cfg.n_kv_heads, cfg.head_dim)
        self.kv_k = list(kv_k) if kv_k is not None else [
            torch.zeros(shape, dtype=dt, device=self.device) for _ in range(cfg.n_layers)]
        self.kv_v = list(kv_v) if kv_v is not None else [
            torch.zeros(shape, dtype=dt, device=self.device) for _ in range(cfg.n_layers)]
        self.ctx_len = torch.zeros(cfg.max_batch, dtype=torch.int32, device=self.device)
        nbytes = _abi.dflash_workspace_bytes(cfg)
        if nbytes == 0:
            raise _abi.DFlashError(_abi.DFLASH_EUNSUPPORTED, "configuration rejected")
        self.workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        off = (-self.workspace.data_ptr()) % 256
        ws = self.workspace[off:off + nbytes]
        self.ctx = _abi.dflash_create(cfg, weights, self.kv_k, self.kv_v, self.ctx_len, ws)

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
