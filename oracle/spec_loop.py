"""Block-autoregressive speculative loop and the greedy autoregressive baseline.

Test infrastructure only (see ``oracle/__init__.py``).

"DFlash: how block diffusion boosts NVIDIA Blackwell throughput"
(dothoosh.com), section "Block-diffusion architecture": DFlash combines
parallel generation with a block-autoregressive structure -- blocks are
drafted one after another, each in a single pass, and the target verifies
each block.  "NVIDIA tests DFlash to cut LLM inference bottlenecks"
(stechtimes.com), section "DFlash moves token drafting to parallel compute":
the target keeps the verification pass, so its output is unchanged.

Block layouts (the pages do not fix which block row carries what):

* ``"anchor"``: block ids = [bonus, mask x (Bs-1)]; block row i sits at
  position T + i where T is the committed context length, so row 0 is the
  last emitted token and rows 1..Bs-1 are drafts (n_d = Bs - 1).
* ``"shifted"``: same block ids, but all Bs outputs are used as drafts for
  the Bs positions after the bonus token (n_d = Bs).

The drafter is any object with ``prefill(feats)``, ``draft(ids)``,
``fuse(feats)`` and ``verify(logits, draft, n_d)``; ``OracleDrafter`` wraps the
oracle draft model, and GPU tests plug in the library instead.
"""

from __future__ import annotations

from typing import List, Sequence

import numpy as np

from .draft import DraftState, DraftWeights, OracleDims, draft_block, fuse_ctx
from .verify import AcceptanceStats, argmax_lowest, verify_step


class OracleDrafter:
    """Single-sequence drafter built from the oracle functions."""

    def __init__(self, weights: DraftWeights, dims: OracleDims, max_ctx: int):
        self.w, self.dims = weights, dims
        self.state = DraftState.empty(dims, 1, max_ctx)
        self.stats = AcceptanceStats()

    def prefill(self, feats: Sequence[np.ndarray]) -> None:
        fuse_ctx(self.state, self.w, self.dims, [f[None] for f in feats], commit=True)

    def draft(self, ids: Sequence[int]) -> np.ndarray:
        out, _, _ = draft_block(self.state, self.w, self.dims, np.asarray(ids)[None])
        return out[0]

    def fuse(self, feats: Sequence[np.ndarray]) -> None:
        fuse_ctx(self.state, self.w, self.dims, [f[None] for f in feats], commit=False)

    def verify(self, logits: np.ndarray, draft: np.ndarray, n_d: int):
        n, bonus, out = verify_step(self.state, logits[None], np.asarray(draft), n_d, n_d, self.stats)
        return int(n[0]), int(bonus[0]), [int(t) for t in out[0, : n[0] + 1]]


class ForcedDrafter(OracleDrafter):
    """Oracle drafter whose drafts are overwritten with given future tokens.

    Used to drive the loop through full acceptance: ``future`` is the target's
    greedy stream; the block drafted at output index j proposes future[j+1..].
    """

    def __init__(self, weights, dims, max_ctx, future: Sequence[int], layout: str):
        super().__init__(weights, dims, max_ctx)
        self.future = list(future)
        self.layout = layout
        self.emitted = 1  # the bonus of the prompt pass is the first output

    def draft(self, ids):
        d = np.array(super().draft(ids))
        first = 1 if self.layout == "anchor" else 0
        for i in range(first, len(d)):
            j = self.emitted + (i - first)
            d[i] = self.future[j] if j < len(self.future) else 0
        return d

    def verify(self, logits, draft, n_d):
        n, bonus, out = super().verify(logits, draft, n_d)
        self.emitted += len(out)
        return n, bonus, out


def greedy_generate(target, prompt: Sequence[int], n_tokens: int) -> List[int]:
    """The target's own greedy stream: one token per forward pass."""
    target.reset()
    logits, _ = target.forward(list(prompt))
    out = [argmax_lowest(logits[-1])]
    while len(out) < n_tokens:
        logits, _ = target.forward([out[-1]])
        out.append(argmax_lowest(logits[-1]))
    return out


def speculative_generate(target, drafter, prompt: Sequence[int], n_tokens: int, block: int,
                         mask_id: int, layout: str = "anchor"):
    """Greedy speculative decoding with a block drafter; returns (tokens, per-step n)."""
    assert layout in ("anchor", "shifted")
    target.reset()
    logits, feats = target.forward(list(prompt))
    drafter.prefill(feats)
    bonus = argmax_lowest(logits[-1])
    out = [bonus]
    accepted = []
    while len(out) < n_tokens:
        ids = [bonus] + [mask_id] * (block - 1)
        d_all = np.asarray(drafter.draft(ids))
        if layout == "anchor":
            d, n_d = d_all[1:block], block - 1
        else:
            d, n_d = d_all[:block], block
        base = target.length
        logits, feats = target.forward([bonus] + [int(t) for t in d])
        drafter.fuse(feats)
        n, bonus, toks = drafter.verify(logits, d, n_d)
        target.truncate(base + n + 1)
        out.extend(toks)
        accepted.append(n)
    return out[:n_tokens], accepted
