"""Oracle for lossless greedy verification, commit / rollback and its statistics.

Test infrastructure only (see ``oracle/__init__.py``).

Source: "NVIDIA tests DFlash to cut LLM inference bottlenecks"
(stechtimes.com), section "DFlash moves token drafting to parallel compute":
the draft proposes a block, the target keeps the verification pass, so what
the target emits is unchanged.  At temperature 0 that is: the target's own
greedy token at each verified position decides; the longest prefix of draft
tokens that equals those greedy tokens is accepted and the target's token
right after it (the bonus token) is emitted too.

The statistics follow what "DFlash-2: z-lab boosts speculative-decoding
throughput" prints in "Performance results" and "Optimising for maximum
speed": a mean acceptance length above the configured draft maximum (4.12
at a maximum of 4) shows the bonus token is counted, and every printed
(rate, mean length) pair satisfies mean = 1 + rate * n_max.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Tuple

import numpy as np


def argmax_lowest(v: np.ndarray) -> int:
    """Index of the largest value; exact ties go to the lowest index.

    NaN never wins; an all-NaN row gives 0.  -0.0 and +0.0 compare equal.
    (The pages say nothing about ties or NaN; this matches numpy.argmax on
    finite data.)
    """
    v = np.asarray(v)
    valid = ~np.isnan(v)
    if not valid.any():
        return 0
    top = np.max(v[valid])
    # first index holding the top value (NaN compares unequal, -0.0 == +0.0)
    return int(np.flatnonzero(v == top)[0])


def greedy_verify(logits: np.ndarray, draft: np.ndarray, n_d: int) -> Tuple[int, int, List[int]]:
    """Greedy verification of one sequence.

    logits: [n_d + 1, V] target logits at the n_d + 1 verified positions;
    draft: [>= n_d] drafted tokens, draft[i] proposed for the position that
    logits[i] predicts.  Returns (n, bonus, out): n = number of leading
    drafts equal to the target's greedy tokens g_i, bonus = g_n, and
    out = [g_0, ..., g_n] (n + 1 committed tokens).
    """
    g = [argmax_lowest(logits[i]) for i in range(n_d + 1)]
    n = 0
    while n < n_d and int(draft[n]) == g[n]:
        n += 1
    return n, g[n], g[: n + 1]


@dataclass
class AcceptanceStats:
    """Counters over verify steps, one step per sequence per verify call.

    steps: sequence-steps; accepted: sum of n; drafted: sum of n_d.
    """

    steps: int = 0
    accepted: int = 0
    drafted: int = 0

    def add(self, n: int, n_d: int) -> None:
        self.steps += 1
        self.accepted += n
        self.drafted += n_d

    @property
    def acceptance_rate(self) -> float:
        return self.accepted / self.drafted

    @property
    def mean_length(self) -> float:
        """Committed tokens per step, counting the bonus token."""
        return (self.accepted + self.steps) / self.steps


def verify_step(state, logits: np.ndarray, draft: np.ndarray, draft_stride: int, n_d: int,
                stats: AcceptanceStats | None = None):
    """Verify every sequence and commit its accepted rows.

    state: an ``oracle.draft.DraftState`` whose rows ctx_len[b] .. +n_d were
    written speculatively by ``fuse_ctx(commit=False)``; logits [B, n_d+1, V];
    draft: flat int array, sequence b's drafts at draft[b*draft_stride + i].
    Commit advances ctx_len[b] by n + 1; the other speculative rows are rolled
    back by not advancing over them (their data stays and is overwritten by
    a later fuse).  Returns (n [B], bonus [B], out [B, n_d+1] padded with -1).
    """
    logits = np.asarray(logits)
    draft = np.asarray(draft).reshape(-1)
    batch = logits.shape[0]
    n_acc = np.zeros(batch, dtype=np.int64)
    bonus = np.zeros(batch, dtype=np.int64)
    out = np.full((batch, n_d + 1), -1, dtype=np.int64)
    for b in range(batch):
        d = draft[b * draft_stride: b * draft_stride + n_d]
        n, bon, toks = greedy_verify(logits[b], d, n_d)
        n_acc[b] = n
        bonus[b] = bon
        out[b, : n + 1] = toks
        if int(state.ctx_len[b]) + n_d + 1 > state.max_ctx:
            raise ValueError("context overflow")
        state.ctx_len[b] += n + 1
        if stats is not None:
            stats.add(n, n_d)
    return n_acc, bonus, out
