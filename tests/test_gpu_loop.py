"""GPU: the library drafter inside a whole greedy speculative loop.

The oracle's loop (prefill, draft a block, target forward over [bonus, drafts],
speculative fusion, verify, roll back) runs with the library as the drafter
and the oracle's float64 tiny causal target as the target.  Verification is
lossless whatever the drafts are, so the emitted tokens must equal the
target's own greedy stream exactly -- with the library's random-weight drafts,
with a broken drafter whose output projections are all NaN (every draft is
garbage: NaN logits draft token 0 by the argmax rule), and with drafts forced
to the target's future tokens (full acceptance).  The
library's counters must match the loop's accepted lengths, and the draft-length
policy reads them.
"""

from typing import List, Sequence

import numpy as np
import pytest
import torch

from block_diffusion_drafting_ctx_amd.policy import DraftLengthPolicy
from harness import gen
from oracle import TinyTarget, greedy_generate, speculative_generate
from tests.gpu_cases import _to, config_for, log

pytestmark = pytest.mark.gpu

WL = gen.WORKLOADS["tiny-f32-b1"]
N_TOK = 64
PROMPT = [5, 17, 901, 33, 250, 7, 64, 1000, 3, 12]


class LibraryDrafter:
    """One sequence through the C-ABI library (fp32 storage)."""

    def __init__(self, wl, seed: int, future: Sequence[int] = (), layout: str = "anchor", nan_weights=False):
        from block_diffusion_drafting_ctx_amd import Drafter

        w = gen.draft_weights(wl, seed=seed)
        if nan_weights:
            for lw in w["layers"]:
                lw["w_o"].fill_(float("nan"))
        self.w = _to(w, "cuda")
        self.dr = Drafter(config_for(wl, 1, max_fuse_rows=64), self.w, "cuda")
        self.wl = wl
        self.future = list(future)
        self.layout = layout
        self.emitted = 1
        self.accepted: List[int] = []
        self.drafts_seen: List[np.ndarray] = []

    def _rows(self, feats):
        return [torch.as_tensor(np.asarray(f), dtype=torch.float32, device="cuda")[None].contiguous() for f in feats]

    def prefill(self, feats):
        self.dr.fuse_ctx(self._rows(feats), commit=True)

    def draft(self, ids):
        bid = torch.tensor([list(ids)], dtype=torch.int32, device="cuda")
        out = torch.zeros(1, self.wl.block, dtype=torch.int32, device="cuda")
        self.dr.draft_block(bid, out)
        d = out[0].cpu().numpy()
        self.drafts_seen.append(d.copy())
        if self.future:
            first = 1 if self.layout == "anchor" else 0
            for i in range(first, len(d)):
                j = self.emitted + (i - first)
                d[i] = self.future[j] if j < len(self.future) else 0
        return d

    def fuse(self, feats):
        self.dr.fuse_ctx(self._rows(feats), commit=False)

    def verify(self, logits, draft, n_d):
        lg = torch.as_tensor(np.asarray(logits), dtype=torch.float32, device="cuda")[None].contiguous()
        d = torch.as_tensor(np.asarray(draft, dtype=np.int32), device="cuda")[None].contiguous()
        n_acc = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        bonus = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        toks = torch.full((1, n_d + 1), -7, dtype=torch.int32, device="cuda")
        self.dr.verify(lg, d, n_d, n_d, n_acc, bonus, toks)
        torch.cuda.synchronize()
        assert self.dr.check() == 0
        n = int(n_acc[0])
        out = [int(t) for t in toks[0, : n + 1].cpu()]
        assert all(int(t) == -1 for t in toks[0, n + 1:].cpu())
        self.emitted += len(out)
        self.accepted.append(n)
        return n, int(bonus[0]), out


@pytest.fixture(scope="module")
def target_and_greedy():
    tgt = TinyTarget(vocab=WL.vocab, hidden=WL.hidden, n_heads=WL.n_q_heads, n_kv_heads=WL.n_kv_heads,
                     head_dim=WL.head_dim, ffn=WL.ffn, n_layers=4, feature_layers=(1, 2, 3), seed=7,
                     max_len=256)
    return tgt, greedy_generate(tgt, PROMPT, N_TOK)


@pytest.mark.parametrize("layout", ["anchor", "shifted"])
@pytest.mark.parametrize("kind", ["random", "nan", "forced"])
def test_library_loop_output_equals_greedy(target_and_greedy, layout, kind):
    tgt, greedy = target_and_greedy
    log(f"[case] loop layout={layout} drafts={kind}")
    dr = LibraryDrafter(WL, seed=21, future=greedy if kind == "forced" else (), layout=layout,
                        nan_weights=kind == "nan")
    out, acc = speculative_generate(tgt, dr, PROMPT, N_TOK, WL.block, WL.mask_id, layout)
    assert out == greedy
    n_d = WL.block - 1 if layout == "anchor" else WL.block
    assert acc == dr.accepted and all(0 <= n <= n_d for n in acc)
    if kind == "forced":
        assert all(n == n_d for n in acc[:-1])
    if kind == "nan":  # all-NaN logits: the argmax rule drafts index 0 everywhere
        assert all(np.all(d == 0) for d in dr.drafts_seen)
    steps, accepted, drafted = dr.dr.stats()
    assert (steps, accepted, drafted) == (len(acc), sum(acc), len(acc) * n_d)
    # the tuning rule over the same counters: random drafts are rarely
    # accepted (mean below 2: drop the drafter); forced ones keep the mean near
    # n_d + 1, where any raise is capped by the layout
    mean = DraftLengthPolicy.window_mean(steps, accepted)
    pol = DraftLengthPolicy(n_max=n_d, cap=n_d, patience=1)
    assert pol.update([steps, accepted, drafted]) == (0 if mean < 2.0 else n_d)
    log(f"[case] loop layout={layout} drafts={kind}: {steps} steps, mean length {mean:.2f}")
    dr.dr.close()
