"""Draft-length tuning over the library's verify counters (host logic only).

[P2] "DFlash-2: z-lab boosts speculative-decoding throughput", section
Optimising for maximum speed (the tuning strategy): start with a draft
maximum of 4 or 6; when the mean length stays below 2, stop using the
drafter for that model; when the mean length stays high against the current
maximum, raise the maximum to the smallest integer above the observed mean
(the page's example: a mean of 7.5 gives 8); otherwise keep it.

Readings (the pages leave these open):
- The mean length is the tokens committed per verify step, 1 + accepted /
  steps, the bonus token included: the pages report 4.12 at a maximum of 4,
  which only that count allows.  It therefore never exceeds maximum + 1.
- The raise trigger.  Taken literally ("at least 1 above the maximum") it
  could fire only at 100% acceptance and would always raise by exactly 2, so
  the page's own 7.5 -> 8 example could never occur.  The reading here is
  that the mean has reached the maximum (mean >= n_max: the drafts alone
  average at least n_max - 1 accepted, the bonus token being the "1"); then
  the 7.5 -> 8 example is the case n_max = 7 at 93% acceptance, and the
  page's 4.12 at a maximum of 4 raises the maximum to 5.
- "Stays" means over `patience` consecutive evaluation windows, a window
  being the verify steps between two calls of `update`.
- The raised maximum is capped by what the block layout can verify (block - 1
  drafts in the anchor layout, block in the shifted one).
"""

from __future__ import annotations

import math
from typing import Sequence


class DraftLengthPolicy:
    """Feed it the cumulative (steps, accepted, drafted) counters, e.g. from
    ``Drafter.stats()``; `update` returns the draft maximum to verify next
    (n_d), or 0 once the drafter has been dropped."""

    def __init__(self, n_max: int = 4, cap: int = 64, patience: int = 3, min_mean: float = 2.0):
        if not 1 <= n_max <= cap:
            raise ValueError("need 1 <= n_max <= cap")
        if patience < 1:
            raise ValueError("patience must be >= 1")
        self.n_max = n_max
        self.cap = cap
        self.patience = patience
        self.min_mean = min_mean
        self.enabled = True
        self._prev = (0, 0, 0)
        self._low = 0
        self._high = 0
        self._target = 0

    @staticmethod
    def window_mean(steps: int, accepted: int) -> float:
        return 1.0 + accepted / steps

    def update(self, counters: Sequence[int]) -> int:
        steps, accepted, drafted = int(counters[0]), int(counters[1]), int(counters[2])
        d_steps, d_acc, d_dr = steps - self._prev[0], accepted - self._prev[1], drafted - self._prev[2]
        if d_steps < 0 or d_acc < 0 or d_dr < 0:
            raise ValueError("counters went backwards (cleared context?)")
        if d_acc > d_dr:
            raise ValueError("more drafts accepted than drafted: not verify counters")
        self._prev = (steps, accepted, drafted)
        if not self.enabled or d_steps == 0:
            return self.n_max if self.enabled else 0
        mean = self.window_mean(d_steps, d_acc)
        self._low = self._low + 1 if mean < self.min_mean else 0
        if mean >= self.n_max:
            self._high += 1
            self._target = max(self._target, math.floor(mean) + 1)
        else:
            self._high = 0
            self._target = 0
        if self._low >= self.patience:
            self.enabled = False
            return 0
        if self._high >= self.patience:
            self.n_max = min(self.cap, self._target)
            self._high = 0
            self._target = 0
        return self.n_max
