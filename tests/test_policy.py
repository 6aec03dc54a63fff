"""Draft-length tuning rule (host logic), pinned to the pages' own figures.

[P2] "DFlash-2: z-lab boosts speculative-decoding throughput", section
Optimising for maximum speed: a mean length of 7.5 moves the maximum to 8;
4.12 at a maximum of 4 keeps it; a mean below 2 drops the drafter.
"""

import pytest

from block_diffusion_drafting_ctx_amd.policy import DraftLengthPolicy


def feed(policy, windows):
    """windows: (steps, accepted) per window; returns the decisions."""
    steps = acc = 0
    out = []
    for s, a in windows:
        steps += s
        acc += a
        out.append(policy.update([steps, acc, 0]))
    return out


def test_pages_example_mean_7_5_raises_to_8():
    p = DraftLengthPolicy(n_max=6, patience=3)
    assert feed(p, [(10, 65)] * 3) == [6, 6, 8]  # mean 1 + 6.5 = 7.5 >= 6 + 1


def test_mean_4_12_at_maximum_4_keeps_it():
    p = DraftLengthPolicy(n_max=4, patience=2)
    assert feed(p, [(100, 312)] * 5) == [4] * 5  # mean 4.12 < 5


def test_low_mean_drops_the_drafter_and_it_stays_dropped():
    p = DraftLengthPolicy(n_max=4, patience=3)
    assert feed(p, [(10, 5)] * 3 + [(10, 40)]) == [4, 4, 0, 0]  # mean 1.5 three times
    assert not p.enabled


def test_only_consistent_windows_count():
    p = DraftLengthPolicy(n_max=4, patience=2)
    # full acceptance (mean 5) interrupted by a poor window: no raise yet
    assert feed(p, [(10, 40), (10, 10), (10, 40), (10, 40)]) == [4, 4, 4, 6]  # floor(5) + 1


def test_raise_is_capped_by_the_layout():
    p = DraftLengthPolicy(n_max=6, cap=7, patience=1)
    assert feed(p, [(4, 28)]) == [7]  # mean 8 -> 9, capped at 7


def test_empty_window_keeps_and_bad_counters_raise():
    p = DraftLengthPolicy(n_max=4)
    assert p.update([0, 0, 0]) == 4
    p.update([10, 20, 40])
    with pytest.raises(ValueError):
        p.update([5, 20, 40])
    with pytest.raises(ValueError):
        DraftLengthPolicy(n_max=0)
