"""Pins of greedy verification, its statistics and the lossless invariant."""

import os

import numpy as np
import pytest

from harness import gen
from oracle import (AcceptanceStats, DraftState, TinyTarget, argmax_lowest, greedy_generate,
                    greedy_verify, speculative_generate, verify_step)
from oracle.spec_loop import ForcedDrafter, OracleDrafter
from tests.oracle_adapt import dims_of, weights_of

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "acceptance_stats.txt")


def test_argmax_matches_numpy_on_finite_rows_and_ties():
    rng = np.random.default_rng(0)
    for _ in range(50):
        v = rng.standard_normal(300)
        v[rng.integers(0, 300, 5)] = v.max()  # planted exact ties
        assert argmax_lowest(v) == int(np.argmax(v))
    v = rng.integers(0, 3, 64).astype(float)  # many ties
    assert argmax_lowest(v) == int(np.argmax(v))
    assert argmax_lowest(np.array([-0.0, 0.0])) == 0
    assert argmax_lowest(np.array([0.0, -0.0])) == 0


def test_argmax_nan_rules():
    assert argmax_lowest(np.array([np.nan, 1.0, 2.0])) == 2
    assert argmax_lowest(np.array([1.0, np.nan, 1.0])) == 0
    assert argmax_lowest(np.array([np.nan, -np.inf])) == 1
    assert argmax_lowest(np.full(7, np.nan)) == 0


def test_full_acceptance():
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((9, 50))
    g = lg.argmax(axis=1)
    n, bonus, out = greedy_verify(lg, g[:8], 8)
    assert n == 8 and bonus == g[8] and out == list(g)


def test_zero_acceptance():
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((9, 50))
    g = lg.argmax(axis=1)
    d = g[:8].copy()
    d[0] = (d[0] + 1) % 50
    n, bonus, out = greedy_verify(lg, d, 8)
    assert n == 0 and bonus == g[0] and out == [g[0]]


def test_partial_acceptance_and_commit():
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((2, 5, 30))
    g = lg.argmax(axis=2)
    d = g[:, :4].copy()
    d[0, 2] = (d[0, 2] + 1) % 30  # sequence 0 accepts 2, sequence 1 accepts all 4
    st = DraftState(k=[np.zeros((2, 40, 1, 2))], v=[np.zeros((2, 40, 1, 2))], ctx_len=np.array([10, 20]))
    stats = AcceptanceStats()
    n, bonus, out = verify_step(st, lg, d.reshape(-1), 4, 4, stats)
    assert list(n) == [2, 4]
    assert list(bonus) == [g[0, 2], g[1, 4]]
    assert list(out[0]) == [g[0, 0], g[0, 1], g[0, 2], -1, -1]
    assert list(st.ctx_len) == [13, 25]
    assert (stats.steps, stats.accepted, stats.drafted) == (2, 6, 8)


def test_planted_logits_accept_exactly_the_planted_length():
    wl = gen.WORKLOADS["tiny-f32-b1"]
    d = gen.draft_tokens(wl, 6, wl.n_d, seed=4)
    a = np.array([0, 1, 3, 7, 8, 8])
    lg = gen.planted_logits(wl, d, a, wl.n_d, seed=5).double().numpy()
    for b in range(6):
        n, _, _ = greedy_verify(lg[b], d[b], wl.n_d)
        assert n == a[b]


def _golden_rows():
    rows = []
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            rate, n_max, mean, dec = line.split()
            rows.append((float(rate) / 100.0, int(n_max), float(mean), int(dec)))
    return rows


@pytest.mark.parametrize("rate,n_max,mean,dec", _golden_rows())
def test_stats_semantics_reproduce_printed_pairs(rate, n_max, mean, dec):
    """Counting the bonus token and rate = accepted / drafted gives the pages' pairs."""
    steps = 10000
    accepted = round(rate * n_max * steps)
    st = AcceptanceStats()
    per = [accepted // steps + (1 if i < accepted % steps else 0) for i in range(steps)]
    for n in per:
        assert 0 <= n <= n_max
        st.add(n, n_max)
    assert abs(st.acceptance_rate - rate) < 1e-9
    assert round(st.mean_length, dec) == pytest.approx(mean)
    assert 1.0 <= st.mean_length <= n_max + 1


def test_mean_length_above_n_max_needs_bonus():
    # 4.12 at a draft maximum of 4: without counting the bonus it could not exceed 4
    st = AcceptanceStats()
    for _ in range(100):
        st.add(4, 4)
    assert st.mean_length == 5.0
    assert st.accepted / st.steps <= 4


# ------------------------------------------------------------ lossless loop
WL = gen.WORKLOADS["tiny-f32-b1"]
N_TOK = 64
PROMPT = [5, 17, 901, 33, 250, 7, 64, 1000, 3, 12]


@pytest.fixture(scope="module")
def target_and_greedy():
    tgt = TinyTarget(vocab=WL.vocab, hidden=WL.hidden, n_heads=WL.n_q_heads, n_kv_heads=WL.n_kv_heads,
                     head_dim=WL.head_dim, ffn=WL.ffn, n_layers=4, feature_layers=(1, 2, 3), seed=7,
                     max_len=256)
    return tgt, greedy_generate(tgt, PROMPT, N_TOK)


def test_tiny_target_rows_are_shape_independent(target_and_greedy):
    tgt, _ = target_and_greedy
    tgt.reset()
    a, fa = tgt.forward(PROMPT + [1, 2, 3])
    tgt.reset()
    tgt.forward(PROMPT)
    b = [tgt.forward([t]) for t in (1, 2, 3)]
    np.testing.assert_array_equal(a[-3:], np.concatenate([x[0] for x in b]))
    np.testing.assert_array_equal(fa[2][-1], b[-1][1][2][0])


@pytest.mark.parametrize("layout", ["anchor", "shifted"])
@pytest.mark.parametrize("kind", ["random", "nan", "forced"])
def test_speculative_output_equals_greedy(target_and_greedy, layout, kind):
    tgt, greedy = target_and_greedy
    dims = dims_of(WL)
    w = weights_of(gen.draft_weights(WL, seed=21))
    if kind == "nan":
        for lw in w.layers:
            lw.w_o[:] = np.nan
    if kind == "forced":
        dr = ForcedDrafter(w, dims, 256, greedy, layout)
    else:
        dr = OracleDrafter(w, dims, 256)
    out, acc = speculative_generate(tgt, dr, PROMPT, N_TOK, WL.block, WL.mask_id, layout)
    assert out == greedy
    n_d = WL.block - 1 if layout == "anchor" else WL.block
    assert all(0 <= n <= n_d for n in acc)
    if kind == "forced":
        assert all(n == n_d for n in acc[:-1])
    st = dr.stats
    assert st.steps == len(acc) and st.accepted == sum(acc)
    assert st.mean_length == pytest.approx(1 + st.acceptance_rate * n_d)
