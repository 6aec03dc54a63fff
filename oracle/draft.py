"""Oracle for the draft side: context-feature fusion, KV injection, block forward.

Test infrastructure only (see ``oracle/__init__.py``).  float64 numpy.

Readings taken where the pages are silent (each is restated at its function):

* layer form: pre-norm residual transformer layer, RMSNorm before attention
  and before the MLP, final RMSNorm before the shared LM head; no biases, no
  QK-norm; RMSNorm epsilon 1e-6;
* positions: rotary embedding (rotate-half pairing, base 1e6) on queries and
  keys; context row j sits at position j, block row i at position T_b + i;
  context keys are cached after the rotation;
* attention: scale 1/sqrt(D), query head h reads KV head floor(h / G),
  no mask at all (non-causal over context and block);
* the context feature goes through each layer's own K and V projections;
* DFlash-2 local convolution: residual, width 3, centred taps, zero padding
  at the block edges, after the attention residual and before the MLP norm;
* optional 8-bit draft KV cache (the "q8" setting the DFlash-2 page measures
  in its precision-cost section): every K/V entry attention reads, context
  rows and the block's own rows alike, goes through the 8-bit format of
  ``kv8_quantize``.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

F64 = np.float64


@dataclass(frozen=True)
class OracleDims:
    """Shapes and scalar hyper-parameters of one draft model."""

    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_layers: int
    ffn: int
    vocab: int
    block: int
    n_target_layers: int
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    conv_width: int = 0  # 0 (DFlash) or 3 (DFlash-2 local convolution)
    kv_int8: bool = False  # 8-bit draft KV cache (kv8_quantize) instead of the storage type


@dataclass
class LayerWeights:
    """One draft layer.  Matrices are [out_features, in_features]."""

    w_q: np.ndarray  # [Hq*D, H]
    w_k: np.ndarray  # [Hkv*D, H]
    w_v: np.ndarray  # [Hkv*D, H]
    w_o: np.ndarray  # [H, Hq*D]
    w_gate: np.ndarray  # [F, H]
    w_up: np.ndarray  # [F, H]
    w_down: np.ndarray  # [H, F]
    g_in: np.ndarray  # [H]
    g_post: np.ndarray  # [H]
    conv: Optional[np.ndarray] = None  # [H, 3] taps for rows (i-1, i, i+1)


@dataclass
class DraftWeights:
    embed: np.ndarray  # [V, H]   token embedding of the block ids
    w_fc: np.ndarray  # [H, K*H] fusion linear over the concatenated features
    g_fc: np.ndarray  # [H]      gain of the fusion RMSNorm
    g_final: np.ndarray  # [H]
    w_lm: np.ndarray  # [V, H]   shared LM head
    layers: List[LayerWeights] = field(default_factory=list)


# --------------------------------------------------------------------------
# elementary operations
# --------------------------------------------------------------------------


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * g.

    The spec stage list names RMSNorm after the fusion linear; the
    layer norms use the same form.  The pages give no epsilon: 1e-6.
    """
    x = np.asarray(x, dtype=F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, dtype=F64)


def rope(z: np.ndarray, pos: np.ndarray, theta: float = 1e6) -> np.ndarray:
    """Rotary position embedding, rotate-half pairing.

    z: [n, heads, D]; pos: [n] absolute positions.  Pair (j, j + D/2) for
    j < D/2 is rotated by the angle pos * theta^(-2j/D).  The pages do not name
    a position encoding; without one all mask rows of a block would be
    identical under non-causal attention, so rotary embedding (the choice of
    the Qwen-shaped drafts) is taken.  Angles and products in float64.
    """
    z = np.asarray(z, dtype=F64)
    n, _, d = z.shape
    half = d // 2
    j = np.arange(half, dtype=F64)
    inv_freq = theta ** (-2.0 * j / d)
    ang = np.asarray(pos, dtype=F64)[:, None] * inv_freq[None, :]  # [n, half]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    a = z[..., :half]
    b = z[..., half:]
    return np.concatenate([a * cos - b * sin, a * sin + b * cos], axis=-1)


def silu(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=F64)
    return x / (1.0 + np.exp(-x))


def gqa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Non-causal grouped-query softmax attention.

    q: [nq, Hq, D]; k, v: [nk, Hkv, D] -> [nq, Hq, D].  Every query sees every
    key (no mask): the DFlash-2 page describes the drafter as non-causal and
    the block is one parallel pass over masked future positions.  Head h
    reads KV head floor(h / G) with G = Hq / Hkv; scale 1/sqrt(D).
    """
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    nq, hq, d = q.shape
    hkv = k.shape[1]
    assert hq % hkv == 0
    group = hq // hkv
    out = np.empty((nq, hq, d), dtype=F64)
    for h in range(hq):
        kv = h // group
        s = q[:, h, :] @ k[:, kv, :].T / np.sqrt(d)  # [nq, nk]
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, kv, :]
    return out


def depthwise_conv3(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Per-channel width-3 convolution along the block rows (no residual).

    y[i, c] = w[c,0] * x[i-1, c] + w[c,1] * x[i, c] + w[c,2] * x[i+1, c],
    rows outside [0, n) read as zero.  Cross-correlation (taps not flipped),
    no bias, no activation.  The DFlash-2 page places a local convolution
    between attention and MLP that mixes only near neighbours; its width,
    padding and form are not given there.
    """
    x = np.asarray(x, dtype=F64)
    w = np.asarray(w, dtype=F64)
    n = x.shape[0]
    y = np.zeros_like(x)
    for i in range(n):
        for t in range(3):
            src = i + t - 1
            if 0 <= src < n:
                y[i] += w[:, t] * x[src]
    return y


KV8_BLOCK = 32


def kv8_quantize(x: np.ndarray):
    """8-bit KV entries: symmetric integers with one scale per 32 values.

    x: [..., D] with D a multiple of 32 (the last axis is one KV head's row).
    Every run of 32 consecutive values of a row gets the scale
    s = max|x| / 127 and the integers q = round-half-even(x / s), clipped to
    [-127, 127]; a run of zeros gets s = 0 and q = 0.  Returns (q [..., D]
    int64, s [..., D/32] float64); the stored value is q * s.

    The DFlash-2 page's precision-cost section compares an f16 KV cache with
    an 8-bit ("q8") one -- acceptance 78.06% -> 74.88% at its third coding
    stage -- without defining the format.  q8 there is llama.cpp's 8-bit
    block format (32 values, one scale); the scale is kept in float64 here
    (float32 on the GPU) rather than float16.
    """
    x = np.asarray(x, dtype=F64)
    d = x.shape[-1]
    assert d % KV8_BLOCK == 0
    blk = x.reshape(x.shape[:-1] + (d // KV8_BLOCK, KV8_BLOCK))
    s = np.max(np.abs(blk), axis=-1) / 127.0
    safe = np.where(s > 0, s, 1.0)
    q = np.where(s[..., None] > 0, np.rint(blk / safe[..., None]), 0.0)
    q = np.clip(q, -127.0, 127.0)
    return q.reshape(x.shape).astype(np.int64), s


def kv8_dequantize(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Values of 8-bit KV entries: q * s, s repeated over each run of 32."""
    q = np.asarray(q, dtype=F64)
    d = q.shape[-1]
    blk = q.reshape(q.shape[:-1] + (d // KV8_BLOCK, KV8_BLOCK)) * np.asarray(s, dtype=F64)[..., None]
    return blk.reshape(q.shape)


def kv8_roundtrip(x: np.ndarray) -> np.ndarray:
    """What an 8-bit cache entry holds after x is stored in it."""
    return kv8_dequantize(*kv8_quantize(x))


def swiglu_mlp(u: np.ndarray, lw: LayerWeights) -> np.ndarray:
    """SwiGLU feed-forward: (silu(u W_gate^T) * (u W_up^T)) W_down^T."""
    g = u @ np.asarray(lw.w_gate, F64).T
    up = u @ np.asarray(lw.w_up, F64).T
    return (silu(g) * up) @ np.asarray(lw.w_down, F64).T


# --------------------------------------------------------------------------
# stage 1-2: fusion of target hidden states and KV injection
# --------------------------------------------------------------------------


def fuse_features(hidden: Sequence[np.ndarray], w_fc: np.ndarray, g_fc: np.ndarray,
                  eps: float = 1e-6) -> np.ndarray:
    """Context feature c = RMSNorm(concat(h_1..h_K) W_fc^T) * g_fc.

    hidden: K arrays [n, H], in the order the caller lists the target layers;
    the concatenation is along features.  Source: the feature-injection
    bullet of the "Block-diffusion architecture" section (several target
    layers fused into one dense context feature); concat -> linear -> RMSNorm
    is the spec form; no bias.
    """
    x = np.concatenate([np.asarray(h, dtype=F64) for h in hidden], axis=-1)
    y = x @ np.asarray(w_fc, dtype=F64).T
    return rmsnorm(y, g_fc, eps)


def context_kv(c: np.ndarray, lw: LayerWeights, pos: np.ndarray, dims: OracleDims):
    """Project the context feature through one layer's own K and V weights.

    KV-cache-integration bullet of the "Block-diffusion architecture"
    section: the feature goes directly into the Key and Value projections of
    each draft layer.  K is stored after the rotary embedding (and, with the
    8-bit cache, quantised after it).  Returns the stored K, V: [n, Hkv, D].
    """
    n = c.shape[0]
    k = (c @ np.asarray(lw.w_k, F64).T).reshape(n, dims.n_kv_heads, dims.head_dim)
    v = (c @ np.asarray(lw.w_v, F64).T).reshape(n, dims.n_kv_heads, dims.head_dim)
    k = rope(k, pos, dims.rope_theta)
    if dims.kv_int8:
        return kv8_roundtrip(k), kv8_roundtrip(v)
    return k, v


@dataclass
class DraftState:
    """Persistent draft KV cache and committed context lengths.

    The projected context entries stay in the draft KV cache across
    iterations (KV-cache-integration bullet, "Block-diffusion architecture").
    k[l], v[l]: [B, max_ctx, Hkv, D]; ctx_len: [B] committed rows.
    Rows at or beyond ctx_len[b] are not part of the context (speculative or
    rolled back) and are never read.
    """

    k: List[np.ndarray]
    v: List[np.ndarray]
    ctx_len: np.ndarray

    @staticmethod
    def empty(dims: OracleDims, batch: int, max_ctx: int) -> "DraftState":
        shape = (batch, max_ctx, dims.n_kv_heads, dims.head_dim)
        return DraftState(
            k=[np.zeros(shape, F64) for _ in range(dims.n_layers)],
            v=[np.zeros(shape, F64) for _ in range(dims.n_layers)],
            ctx_len=np.zeros(batch, dtype=np.int64),
        )

    @property
    def max_ctx(self) -> int:
        return self.k[0].shape[1]


def fuse_ctx(state: DraftState, w: DraftWeights, dims: OracleDims,
             hidden: Sequence[np.ndarray], commit: bool) -> np.ndarray:
    """Fuse t_new target rows per sequence and write their K/V into the cache.

    hidden: K arrays [B, t_new, H].  Rows go to cache rows ctx_len[b] + i at
    positions ctx_len[b] + i, for every layer.  With commit=False the rows are
    speculative: the verify step decides how many of them enter the context.
    With commit=True ctx_len advances by t_new (prompt pre-fill).
    Returns the context feature c: [B, t_new, H].
    """
    hidden = [np.asarray(h, dtype=F64) for h in hidden]
    batch, t_new, _ = hidden[0].shape
    out = np.empty((batch, t_new, dims.hidden), dtype=F64)
    for b in range(batch):
        t0 = int(state.ctx_len[b])
        if t0 + t_new > state.max_ctx:
            raise ValueError("context overflow")
        c = fuse_features([h[b] for h in hidden], w.w_fc, w.g_fc, dims.rms_eps)
        out[b] = c
        pos = t0 + np.arange(t_new)
        for l, lw in enumerate(w.layers):
            k, v = context_kv(c, lw, pos, dims)
            state.k[l][b, t0:t0 + t_new] = k
            state.v[l][b, t0:t0 + t_new] = v
        if commit:
            state.ctx_len[b] = t0 + t_new
    return out


# --------------------------------------------------------------------------
# stage 3-4: one draft layer and the block forward
# --------------------------------------------------------------------------


def draft_layer(x: np.ndarray, lw: LayerWeights, k_ctx: np.ndarray, v_ctx: np.ndarray,
                pos: np.ndarray, dims: OracleDims) -> np.ndarray:
    """One pre-norm draft layer over the block rows of one sequence.

    x: [Bs, H] residual stream; k_ctx, v_ctx: [T, Hkv, D] this layer's cached
    context entries (T may be 0); pos: [Bs] positions of the block rows.
    Block queries attend to [context keys ; block keys] with no mask.  With
    the 8-bit cache the block's own K/V are read back from it too (the
    attention reads every key from the cache), so they take the 8-bit round
    trip like the context rows.
    """
    n = x.shape[0]
    u = rmsnorm(x, lw.g_in, dims.rms_eps)
    q = (u @ np.asarray(lw.w_q, F64).T).reshape(n, dims.n_q_heads, dims.head_dim)
    k = (u @ np.asarray(lw.w_k, F64).T).reshape(n, dims.n_kv_heads, dims.head_dim)
    v = (u @ np.asarray(lw.w_v, F64).T).reshape(n, dims.n_kv_heads, dims.head_dim)
    q = rope(q, pos, dims.rope_theta)
    k = rope(k, pos, dims.rope_theta)
    if dims.kv_int8:
        k, v = kv8_roundtrip(k), kv8_roundtrip(v)
    keys = np.concatenate([np.asarray(k_ctx, F64), k], axis=0)
    vals = np.concatenate([np.asarray(v_ctx, F64), v], axis=0)
    o = gqa_attention(q, keys, vals).reshape(n, dims.n_q_heads * dims.head_dim)
    x = x + o @ np.asarray(lw.w_o, F64).T
    if dims.conv_width:
        x = x + depthwise_conv3(x, lw.conv)
    u = rmsnorm(x, lw.g_post, dims.rms_eps)
    return x + swiglu_mlp(u, lw)


def lm_head_logits(x: np.ndarray, w: DraftWeights, dims: OracleDims) -> np.ndarray:
    """Final RMSNorm then the shared LM head: [n, H] -> [n, V]."""
    return rmsnorm(x, w.g_final, dims.rms_eps) @ np.asarray(w.w_lm, F64).T


def draft_block(state: DraftState, w: DraftWeights, dims: OracleDims,
                block_ids: np.ndarray):
    """Draft a whole block for every sequence in one forward pass.

    block_ids: [B, Bs] token ids of the block rows (mask id on masked rows).
    Block row i of sequence b sits at position ctx_len[b] + i and attends to
    the committed context rows [0, ctx_len[b]) of every layer's cache plus
    all block rows.  Returns (draft_ids [B, Bs] int64, logits [B, Bs, V],
    final hidden [B, Bs, H] before the final norm).
    """
    # imported here to keep the module import graph acyclic
    from .verify import argmax_lowest

    block_ids = np.asarray(block_ids)
    batch, bs = block_ids.shape
    logits = np.empty((batch, bs, dims.vocab), dtype=F64)
    hidden = np.empty((batch, bs, dims.hidden), dtype=F64)
    ids = np.empty((batch, bs), dtype=np.int64)
    for b in range(batch):
        t = int(state.ctx_len[b])
        x = np.asarray(w.embed, F64)[block_ids[b]]
        pos = t + np.arange(bs)
        for l, lw in enumerate(w.layers):
            x = draft_layer(x, lw, state.k[l][b, :t], state.v[l][b, :t], pos, dims)
        hidden[b] = x
        logits[b] = lm_head_logits(x, w, dims)
        ids[b] = [argmax_lowest(row) for row in logits[b]]
    return ids, logits, hidden
