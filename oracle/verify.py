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


def inverse_cdf(p: np.ndarray, u: float) -> int:
    """Smallest index v with p[0] + ... + p[v] > u * sum(p) (u in [0, 1));
    the last index holding mass when rounding leaves u * sum(p) at the top."""
    c = np.cumsum(np.asarray(p, dtype=np.float64))
    v = int(np.searchsorted(c, u * c[-1], side="right"))
    if v >= len(c):
        v = int(np.flatnonzero(np.asarray(p) > 0)[-1])
    return v


def sample_verify(logits: np.ndarray, draft: np.ndarray, n_d: int, temperature: float,
                  uniforms: np.ndarray) -> Tuple[int, int, List[int]]:
    """Verification when the target samples at temperature T > 0.

    The pages measure this mode ([P1] Real-world integration: a "thinking" setting that samples) but state
    no rule; the reading here is the standard lossless speculative-sampling
    rule for a drafter whose proposal is a single token (its distribution is
    all on the drafted token): with p_i = softmax(logits[i] / T), draft d_i
    is accepted when uniforms[i, 0] < p_i(d_i); at the first rejected row i
    the emitted token is drawn from p_i with d_i removed (renormalised) by
    the inverse CDF at uniforms[i, 1]; when every draft is accepted, the
    bonus token is drawn from p_{n_d} at uniforms[n_d, 1].  Each emitted
    token then has exactly the target's sampling distribution.  A draft id
    outside the vocabulary has p = 0: it is rejected, and since the target
    has no mass there, the draw is from p_i unchanged.  A NaN logit is read
    as carrying no mass (as -inf would): a draft there is rejected and the
    draws never land on it (the pages say nothing about NaN; this keeps one
    bad entry from voiding the whole row).  A row needs one non-NaN, finite
    logit; +inf entries are outside this definition.

    Returns (n, token, out): n accepted drafts, the drawn token, and the n + 1
    committed tokens [d_0 .. d_{n-1}, token].
    """
    x = np.asarray(logits, dtype=np.float64) / float(temperature)
    x = np.where(np.isnan(x), -np.inf, x)  # no mass on NaN entries
    u = np.asarray(uniforms, dtype=np.float64)
    for i in range(n_d):
        p = np.exp(x[i] - np.max(x[i]))
        p /= p.sum()
        d = int(draft[i])
        inside = 0 <= d < len(p)  # an id outside the vocabulary has no target mass
        if u[i, 0] < (p[d] if inside else 0.0):
            continue
        r = p.copy()
        if inside:
            r[d] = 0.0
        tok = inverse_cdf(r, u[i, 1])
        return i, tok, [int(t) for t in draft[:i]] + [tok]
    p = np.exp(x[n_d] - np.max(x[n_d]))
    tok = inverse_cdf(p, u[n_d, 1])
    return n_d, tok, [int(t) for t in draft[:n_d]] + [tok]


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
