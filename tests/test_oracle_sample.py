"""Pins of the sampling-mode verification rule (oracle.sample_verify).

Reading: the standard lossless speculative-sampling rule for a drafter that
proposes single tokens.  The pins check what that rule must guarantee rather
than retyping it: the emitted token's distribution is the target's softmax
whatever the draft; the low-temperature limit is greedy verification.
"""

import numpy as np
import pytest

from oracle import greedy_verify, inverse_cdf, sample_verify


def softmax(x, T):
    z = np.asarray(x, dtype=np.float64) / T
    e = np.exp(z - z.max())
    return e / e.sum()


@pytest.mark.parametrize("T", [0.5, 1.0, 2.0])
@pytest.mark.parametrize("draft_tok", [0, 2, 4])
def test_first_emitted_token_has_the_target_distribution(T, draft_tok):
    # integrate the rule over a midpoint grid of (accept, sample) uniforms:
    # P(first emitted token = v) must be softmax(x_0 / T)[v] for any draft
    rng = np.random.default_rng(3)
    logits = rng.normal(size=(2, 5)) * 1.5
    G = 250
    grid = (np.arange(G) + 0.5) / G
    counts = np.zeros(5)
    for ua in grid:
        for us in grid:
            u = np.array([[ua, us], [0.5, 0.5]])
            _, _, out = sample_verify(logits, np.array([draft_tok]), 1, T, u)
            counts[out[0]] += 1
    np.testing.assert_allclose(counts / G**2, softmax(logits[0], T), atol=4.0 / G)


def test_low_temperature_is_greedy_verification():
    rng = np.random.default_rng(4)
    logits = rng.normal(size=(5, 64)) * 3.0
    g = [int(np.argmax(r)) for r in logits]
    for draft in (np.array(g[:4]), np.array([g[0], g[1], (g[2] + 1) % 64, g[3]]), np.array([(g[0] + 7) % 64] * 4)):
        u = rng.uniform(size=(5, 2)) * 0.98 + 0.01
        assert sample_verify(logits, draft, 4, 1e-4, u) == greedy_verify(logits, draft, 4)


def test_full_acceptance_draws_the_bonus_by_inverse_cdf():
    rng = np.random.default_rng(5)
    logits = rng.normal(size=(4, 32))
    draft = np.array([3, 9, 17])
    u = np.zeros((4, 2))
    u[3, 1] = 0.637
    n, tok, out = sample_verify(logits, draft, 3, 0.8, u)
    p = softmax(logits[3], 0.8)
    assert n == 3 and out == [3, 9, 17, tok]
    assert tok == int(np.searchsorted(np.cumsum(p), 0.637))
    assert inverse_cdf(p, 0.0) == int(np.flatnonzero(p > 0)[0])


def test_draft_outside_the_vocabulary_is_rejected_and_removes_nothing():
    # (p - delta_d)+ = p when d has no target mass: rejected even at a tiny
    # uniform, and the draw is the plain inverse CDF of p (the last token
    # carries most of the mass, so an id read modulo the vocabulary, -1 or
    # -40, would be accepted or would move this draw)
    rng = np.random.default_rng(6)
    logits = rng.normal(size=(3, 40))
    logits[0, 39] = 6.0
    logits[0, 0] = 5.0
    p = softmax(logits[0], 1.3)
    for bad in (-1, -40, 40, 1000):
        draft = np.array([bad, 5])
        u = np.array([[0.001, 0.99], [0.0, 0.0], [0.0, 0.0]])
        n, tok, out = sample_verify(logits, draft, 2, 1.3, u)
        assert n == 0 and out == [tok]
        assert tok == int(np.searchsorted(np.cumsum(p), 0.99)) == 39


@pytest.mark.parametrize("draft_tok", [1, 3])
def test_nan_entries_carry_no_mass(draft_tok):
    # entries 1 and 4 are NaN: over a grid of uniforms the emitted token has
    # the softmax distribution of the finite entries alone, a draft on a NaN
    # entry is never accepted, and no draw lands on a NaN entry
    rng = np.random.default_rng(8)
    logits = rng.normal(size=(2, 6)) * 1.2
    logits[0, [1, 4]] = np.nan
    finite = [0, 2, 3, 5]
    want = np.zeros(6)
    want[finite] = softmax(logits[0, finite], 0.9)
    G = 200
    grid = (np.arange(G) + 0.5) / G
    counts = np.zeros(6)
    for ua in grid:
        for us in grid:
            u = np.array([[ua, us], [0.5, 0.5]])
            n, _, out = sample_verify(logits, np.array([draft_tok]), 1, 0.9, u)
            if draft_tok == 1:
                assert n == 0
            counts[out[0]] += 1
    assert counts[1] == 0 and counts[4] == 0
    np.testing.assert_allclose(counts / G**2, want, atol=4.0 / G)
