"""Pins of the 8-bit draft KV cache format (oracle.kv8_quantize) and its use.

The DFlash-2 page ("DFlash-2: z-lab boosts speculative-decoding throughput",
Precision cost) measures an 8-bit KV cache against f16 without defining it;
the reading is symmetric integers with one scale per 32 values of a row
(s = max|x| / 127, round half to even, clip to +-127).  The pins check it by
other means than retyping it: a brute-force nearest-integer search, the
error bound, exactly representable runs, and where the round trip sits in
the draft's cache path.
"""

import numpy as np
import pytest

from oracle import (DraftState, DraftWeights, LayerWeights, OracleDims, draft_block, fuse_ctx, kv8_dequantize,
                    kv8_quantize, kv8_roundtrip, rmsnorm)


def brute_force(x):
    """For every run of 32: scale max|x|/127, then for every value the integer
    k in [-127, 127] nearest to x / s found by trying them all (ties: even k)."""
    x = np.asarray(x, np.float64).reshape(-1, 32)
    q = np.zeros(x.shape, np.int64)
    ks = np.arange(-127, 128)
    for r, run in enumerate(x):
        s = np.max(np.abs(run)) / 127.0
        if s == 0:
            continue
        for c, v in enumerate(run):
            dist = np.abs(v - ks * s)
            best = np.flatnonzero(dist == dist.min())
            q[r, c] = ks[best[0]] if len(best) == 1 else [k for k in ks[best] if k % 2 == 0][0]
    return q


def test_matches_brute_force_nearest_integer_search():
    rng = np.random.default_rng(1)
    x = rng.normal(size=(3, 2, 64)) * np.array([0.01, 1.0, 30.0])[:, None, None]
    q, s = kv8_quantize(x)
    np.testing.assert_array_equal(q.reshape(-1, 32), brute_force(x))
    np.testing.assert_allclose(s.reshape(-1), np.max(np.abs(x.reshape(-1, 32)), axis=1) / 127.0, rtol=0, atol=0)


def test_ties_round_to_even():
    # values at exact half steps: x / s = k + 1/2 (s = 1 with the 127 anchor)
    x = np.zeros(32)
    x[0] = 127.0
    x[1:6] = [0.5, 1.5, 2.5, -0.5, -2.5]
    q, s = kv8_quantize(x)
    assert s[0] == 1.0
    assert list(q[1:6]) == [0, 2, 2, 0, -2]


def test_error_bound_and_extremes():
    rng = np.random.default_rng(2)
    x = rng.standard_t(3, size=(50, 128))
    q, s = kv8_quantize(x)
    err = np.abs(kv8_dequantize(q, s) - x).reshape(-1, 4, 32)
    assert np.all(err <= s[..., None] / 2 * (1 + 1e-12))
    assert np.all(np.abs(q) <= 127)
    # the largest magnitude of every run lands on +-127
    run = x.reshape(-1, 32)
    qr = q.reshape(-1, 32)
    top = np.argmax(np.abs(run), axis=1)
    assert np.all(np.abs(qr[np.arange(len(run)), top]) == 127)


def test_representable_runs_round_trip_exactly_and_zero_runs():
    rng = np.random.default_rng(3)
    k = rng.integers(-127, 128, size=(4, 32))
    k[:, 5] = 127 * np.where(rng.random(4) < 0.5, 1, -1)
    x = k * 2.0 ** -5
    np.testing.assert_array_equal(kv8_roundtrip(x), x)
    z = np.zeros((2, 64))
    q, s = kv8_quantize(z)
    assert np.all(q == 0) and np.all(s == 0) and np.all(kv8_roundtrip(z) == 0)


def test_runs_are_independent_32_value_blocks_of_a_row():
    rng = np.random.default_rng(4)
    x = rng.normal(size=(2, 128))
    y = x.copy()
    y[0, 32:64] *= 1000.0  # only the second run of row 0 changes
    a, b = kv8_roundtrip(x), kv8_roundtrip(y)
    np.testing.assert_array_equal(a[1], b[1])
    np.testing.assert_array_equal(a[0, :32], b[0, :32])
    np.testing.assert_array_equal(a[0, 64:], b[0, 64:])


def _tiny(kv_int8, H=128, hq=2, hkv=1, D=64, conv=0):
    return OracleDims(hidden=H, n_q_heads=hq, n_kv_heads=hkv, head_dim=D, n_layers=1, ffn=64, vocab=96,
                      block=1, n_target_layers=2, kv_int8=kv_int8, conv_width=conv)


def _weights(dims, rng, eye_o=False, zero_mlp=False):
    H, D = dims.hidden, dims.head_dim
    n = lambda *s: rng.normal(size=s) * 0.1  # noqa: E731
    lw = LayerWeights(w_q=n(dims.n_q_heads * D, H), w_k=n(dims.n_kv_heads * D, H), w_v=n(dims.n_kv_heads * D, H),
                      w_o=np.eye(H) if eye_o else n(H, dims.n_q_heads * D),
                      w_gate=np.zeros((dims.ffn, H)) if zero_mlp else n(dims.ffn, H),
                      w_up=np.zeros((dims.ffn, H)) if zero_mlp else n(dims.ffn, H),
                      w_down=np.zeros((H, dims.ffn)) if zero_mlp else n(H, dims.ffn),
                      g_in=np.ones(H), g_post=np.ones(H))
    return DraftWeights(embed=n(dims.vocab, H), w_fc=n(H, 2 * H), g_fc=np.ones(H), g_final=np.ones(H),
                        w_lm=n(dims.vocab, H), layers=[lw])


def test_context_rows_hold_the_round_trip_of_the_rotated_keys():
    # the 8-bit cache stores what the 16-bit path stores (K after rotation),
    # round-tripped: quantising before the rotation would not match
    rng = np.random.default_rng(5)
    d16, d8 = _tiny(False), _tiny(True)
    w = _weights(d16, rng)
    hid = [rng.normal(size=(1, 5, d16.hidden)) for _ in range(2)]
    s16, s8 = DraftState.empty(d16, 1, 16), DraftState.empty(d8, 1, 16)
    s16.ctx_len[:] = s8.ctx_len[:] = 3
    fuse_ctx(s16, w, d16, hid, commit=True)
    fuse_ctx(s8, w, d8, hid, commit=True)
    np.testing.assert_array_equal(s8.k[0][0, 3:8], kv8_roundtrip(s16.k[0][0, 3:8]))
    np.testing.assert_array_equal(s8.v[0][0, 3:8], kv8_roundtrip(s16.v[0][0, 3:8]))
    # every stored K run is on its own 8-bit grid (a rotation after the
    # quantisation would leave it off the grid)
    q, sc = kv8_quantize(s8.k[0][0, 3:8])
    np.testing.assert_allclose(kv8_dequantize(q, sc), s8.k[0][0, 3:8], rtol=1e-15, atol=0)


def test_single_block_key_attends_to_its_own_round_tripped_value():
    # empty context, one block row: attention over the one key returns its V
    # exactly; with W_o = I and no MLP the final hidden is x + that V, so the
    # block's own V must have gone through the 8-bit format
    rng = np.random.default_rng(6)
    dims = _tiny(True, H=128, hq=2, hkv=1, D=64)
    w = _weights(dims, rng, eye_o=True, zero_mlp=True)
    st = DraftState.empty(dims, 1, 8)
    ids = np.array([[7]])
    _, _, hid = draft_block(st, w, dims, ids)
    x = w.embed[7][None]
    v = rmsnorm(x, w.layers[0].g_in) @ w.layers[0].w_v.T  # [1, D] of the one KV head
    want = x + np.concatenate([kv8_roundtrip(v)] * 2, axis=-1)  # both query heads read KV head 0
    np.testing.assert_allclose(hid[0], want, rtol=1e-12, atol=1e-14)
    assert not np.allclose(hid[0], x + np.concatenate([v] * 2, axis=-1), rtol=1e-9, atol=0)


@pytest.mark.parametrize("kv_int8", [False, True])
def test_kv8_changes_the_draft_little(kv_int8):
    # sanity: the 8-bit path stays close to the 16-bit one (the format's
    # relative error is about 0.5% per entry)
    rng = np.random.default_rng(7)
    d16, d = _tiny(False), _tiny(kv_int8)
    w = _weights(d16, rng)
    hid = [rng.normal(size=(1, 9, d16.hidden)) for _ in range(2)]
    out = []
    for dims in (d16, d):
        st = DraftState.empty(dims, 1, 32)
        fuse_ctx(st, w, dims, hid, commit=True)
        out.append(draft_block(st, w, dims, np.array([[3]]))[2])
    rel = np.linalg.norm(out[1] - out[0]) / np.linalg.norm(out[0])
    assert (rel == 0) == (not kv_int8) and rel < 2e-2
