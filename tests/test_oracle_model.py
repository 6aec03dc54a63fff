"""Pins of the oracle's composed draft model: layer wiring against torch
building blocks, and the invariants the pages imply (non-causal block,
positions, KV injection into every layer, speculative fuse + rollback)."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from harness import gen
from oracle import (DraftState, draft_block, draft_layer, fuse_ctx, lm_head_logits, rope,
                    verify_step)
from oracle.draft import context_kv
from tests.oracle_adapt import dims_of, np64, weights_of

WL = gen.WORKLOADS["tiny-f32-b1"]
CONV = gen.Workload("tiny-conv", 64, 4, 2, 16, 2, 96, 128, 8, 2, 2, 10, 12, "f32", conv_width=3,
                    scaled_hidden=False)


def _torch_layer(x, lw, k_ctx, v_ctx, pos, dims):
    """The same layer from torch.nn.functional building blocks (float64)."""
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))  # noqa: E731
    n = x.shape[0]
    hq, hkv, d = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    xt = t(x)
    u = F.rms_norm(xt, (dims.hidden,), weight=t(lw.g_in), eps=dims.rms_eps)
    q = F.linear(u, t(lw.w_q)).reshape(n, hq, d)
    k = F.linear(u, t(lw.w_k)).reshape(n, hkv, d)
    v = F.linear(u, t(lw.w_v)).reshape(n, hkv, d)
    q = t(rope(q.numpy(), pos, dims.rope_theta))  # rope itself is pinned in test_oracle_ops
    k = t(rope(k.numpy(), pos, dims.rope_theta))
    keys = torch.cat([t(k_ctx), k]).transpose(0, 1)
    vals = torch.cat([t(v_ctx), v]).transpose(0, 1)
    o = F.scaled_dot_product_attention(q.transpose(0, 1), keys, vals, is_causal=False, enable_gqa=True)
    xt = xt + F.linear(o.transpose(0, 1).reshape(n, hq * d), t(lw.w_o))
    if dims.conv_width:
        w = t(lw.conv)[:, None, :]
        xt = xt + F.conv1d(xt.T[None], w, padding=1, groups=dims.hidden)[0].T
    u = F.rms_norm(xt, (dims.hidden,), weight=t(lw.g_post), eps=dims.rms_eps)
    mlp = F.linear(F.silu(F.linear(u, t(lw.w_gate))) * F.linear(u, t(lw.w_up)), t(lw.w_down))
    return (xt + mlp).numpy()


@pytest.mark.parametrize("wl", [WL, CONV], ids=["tiny", "tiny-conv"])
@pytest.mark.parametrize("ctx", [0, 11])
def test_layer_matches_torch_building_blocks(wl, ctx):
    dims = dims_of(wl)
    w = weights_of(gen.draft_weights(wl, seed=3))
    rng = np.random.default_rng(5)
    x = rng.standard_normal((wl.block, wl.hidden))
    kc = rng.standard_normal((ctx, wl.n_kv_heads, wl.head_dim))
    vc = rng.standard_normal((ctx, wl.n_kv_heads, wl.head_dim))
    pos = ctx + np.arange(wl.block)
    for lw in w.layers:
        np.testing.assert_allclose(draft_layer(x, lw, kc, vc, pos, dims),
                                   _torch_layer(x, lw, kc, vc, pos, dims), rtol=1e-10, atol=1e-12)


def test_lm_head_matches_torch():
    dims = dims_of(WL)
    w = weights_of(gen.draft_weights(WL, seed=3))
    x = np.random.default_rng(2).standard_normal((4, WL.hidden))
    ref = F.linear(F.rms_norm(torch.from_numpy(x), (WL.hidden,), weight=torch.from_numpy(w.g_final),
                              eps=1e-6), torch.from_numpy(w.w_lm)).numpy()
    np.testing.assert_allclose(lm_head_logits(x, w, dims), ref, rtol=1e-10, atol=1e-12)


def test_block_is_non_causal():
    """Changing the last block row changes the first row's output."""
    dims = dims_of(WL)
    w = weights_of(gen.draft_weights(WL, seed=3))
    rng = np.random.default_rng(9)
    x = rng.standard_normal((WL.block, WL.hidden))
    kc = rng.standard_normal((5, WL.n_kv_heads, WL.head_dim))
    vc = rng.standard_normal((5, WL.n_kv_heads, WL.head_dim))
    pos = 5 + np.arange(WL.block)
    a = draft_layer(x, w.layers[0], kc, vc, pos, dims)
    x2 = x.copy()
    x2[-1] += 1.0
    b = draft_layer(x2, w.layers[0], kc, vc, pos, dims)
    assert np.max(np.abs(a[0] - b[0])) > 1e-6


def test_positions_break_symmetry_of_mask_rows():
    """Identical mask rows give identical outputs without positions, distinct with them."""
    dims = dims_of(WL)
    w = weights_of(gen.draft_weights(WL, seed=3))
    rng = np.random.default_rng(4)
    x = np.tile(rng.standard_normal(WL.hidden), (WL.block, 1))
    kc = rng.standard_normal((7, WL.n_kv_heads, WL.head_dim))
    vc = rng.standard_normal((7, WL.n_kv_heads, WL.head_dim))
    same = draft_layer(x, w.layers[0], kc, vc, np.zeros(WL.block, dtype=int), dims)
    np.testing.assert_allclose(same - same[0], 0.0, atol=1e-12)
    diff = draft_layer(x, w.layers[0], kc, vc, 7 + np.arange(WL.block), dims)
    assert np.min(np.abs(diff[1:] - diff[0]).max(axis=1)) > 1e-6


def test_fuse_injects_into_every_layer_kv():
    dims = dims_of(WL)
    w = weights_of(gen.draft_weights(WL, seed=3))
    st = DraftState.empty(dims, 1, 64)
    hid = [np64(h) for h in gen.target_hidden(WL, 1, 5, seed=8)]
    c = fuse_ctx(st, w, dims, hid, commit=True)
    assert st.ctx_len[0] == 5
    for l, lw in enumerate(w.layers):
        k_exp = rope((c[0] @ lw.w_k.T).reshape(5, WL.n_kv_heads, WL.head_dim), np.arange(5), WL.rope_theta)
        v_exp = (c[0] @ lw.w_v.T).reshape(5, WL.n_kv_heads, WL.head_dim)
        np.testing.assert_allclose(st.k[l][0, :5], k_exp, rtol=1e-12)
        np.testing.assert_allclose(st.v[l][0, :5], v_exp, rtol=1e-12)
    # each layer uses its own projections
    assert np.max(np.abs(st.k[0][0, :5] - st.k[1][0, :5])) > 1e-3
    # the next fuse appends at ctx_len with positions continuing
    fuse_ctx(st, w, dims, hid, commit=False)
    k2, _ = context_kv(c[0], w.layers[1], 5 + np.arange(5), dims)
    np.testing.assert_allclose(st.k[1][0, 5:10], k2, rtol=1e-12)
    assert st.ctx_len[0] == 5


def test_speculative_fuse_then_commit_equals_fusing_committed_rows():
    """Rolled-back rows are never read: fuse(t rows) + commit(n+1) == fuse(n+1 rows)."""
    dims = dims_of(WL)
    w = weights_of(gen.draft_weights(WL, seed=3))
    pre = [np64(h) for h in gen.target_hidden(WL, 1, 20, seed=10)]
    new = [np64(h) for h in gen.target_hidden(WL, 1, WL.block + 1, seed=11)]
    ids = gen.block_ids(WL, 1, seed=12)
    for n_keep in (1, 4, WL.block + 1):
        a = DraftState.empty(dims, 1, 64)
        fuse_ctx(a, w, dims, pre, commit=True)
        fuse_ctx(a, w, dims, new, commit=False)
        # verify with logits that accept exactly n_keep - 1 drafts
        drafts = np.arange(WL.block)
        logits = np.zeros((1, WL.block + 1, WL.vocab))
        for i in range(n_keep - 1):
            logits[0, i, drafts[i]] = 1.0
        if n_keep - 1 < WL.block:
            logits[0, n_keep - 1, drafts[n_keep - 1] + 1] = 1.0
        n, _, _ = verify_step(a, logits, drafts, WL.block, WL.block)
        assert n[0] == n_keep - 1 and a.ctx_len[0] == 20 + n_keep
        # poison the rolled-back rows
        for l in range(dims.n_layers):
            a.k[l][0, 20 + n_keep:] = np.nan
            a.v[l][0, 20 + n_keep:] = np.nan
        b = DraftState.empty(dims, 1, 64)
        fuse_ctx(b, w, dims, pre, commit=True)
        fuse_ctx(b, w, dims, [h[:, :n_keep] for h in new], commit=True)
        da, la, _ = draft_block(a, w, dims, ids)
        db, lb, _ = draft_block(b, w, dims, ids)
        # equal up to BLAS rounding of different row counts; a read of a
        # poisoned (rolled-back) row would turn everything NaN
        np.testing.assert_array_equal(da, db)
        assert np.all(np.isfinite(la))
        np.testing.assert_allclose(la, lb, rtol=1e-12, atol=1e-13)


def test_empty_context_draft_is_plain_bidirectional_block():
    dims = dims_of(WL)
    w = weights_of(gen.draft_weights(WL, seed=3))
    st = DraftState.empty(dims, 1, 64)
    ids = gen.block_ids(WL, 1, seed=2)
    d, lg, hid = draft_block(st, w, dims, ids)
    x = w.embed[ids[0]]
    empty = np.zeros((0, WL.n_kv_heads, WL.head_dim))
    for lw in w.layers:
        x = _torch_layer(x, lw, empty, empty, np.arange(WL.block), dims)
    np.testing.assert_allclose(hid[0], x, rtol=1e-10, atol=1e-12)
