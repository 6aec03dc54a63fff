"""GPU parity at the method's edges: the argmax rule and stale attention pieces.

* Greedy verification must be bit-exact, so the tie / NaN rule of the argmax
  (lowest index wins exact ties, NaN never wins, an all-NaN row gives 0,
  -0 equals +0) is driven through the verify kernels with target logits that
  hold exactly those cases, at a small vocabulary (one 8192-entry chunk) and
  at 151936 entries (ties across chunks), and compared with the oracle.
* The LM-head argmax follows the same rule: with duplicated LM-head rows every
  logit appears twice, bit for bit, and the lower index must be drafted; with
  NaN LM-head rows those columns are never drafted.
* A split attention segment merges only the pieces of the current context:
  slots left by an earlier, longer context (here holding NaN) must not reach
  the output.
"""

import numpy as np
import pytest
import torch

from harness import gen
from oracle import DraftState, draft_block, greedy_verify
from tests.gpu_cases import _to, config_for, log, rel_l2, run_step, REL_L2
from tests.oracle_adapt import dims_of, np64, weights_of

pytestmark = pytest.mark.gpu

KINDS = ["unique", "tie_near", "tie_far", "nan_mixed", "all_nan", "zero_pm", "zero_mp",
         "all_neginf", "neginf_in_nan", "posinf_tie", "all_equal", "nan_first"]


def edge_row(kind: str, V: int, rng) -> tuple:
    """One target-logit row of the given kind and the index that a *wrong*
    tie-break would pick (-1 if none): the drafted token at the first
    rejected row is set to it, so a kernel picking it would accept a draft."""
    x = rng.normal(size=V).astype(np.float32)
    alt = -1
    if kind == "unique":
        pass
    elif kind in ("tie_near", "tie_far"):
        i = int(rng.integers(0, V // 2))
        j = i + 1 + int(rng.integers(0, 40)) if kind == "tie_near" else V - 1 - int(rng.integers(0, 40))
        x[i] = x[j] = x.max() + 1.0
        alt = j
    elif kind == "nan_mixed":
        x[rng.choice(V, size=V // 8, replace=False)] = np.nan
        x[0] = np.nan  # NaN below the winner's index must not win
    elif kind == "all_nan":
        x[:] = np.nan
        alt = V - 1
    elif kind in ("zero_pm", "zero_mp"):
        x = -np.abs(x) - 1.0
        i = int(rng.integers(0, V // 2))
        j = int(rng.integers(V // 2, V))
        x[i], x[j] = (np.float32(-0.0), np.float32(0.0)) if kind == "zero_mp" else (np.float32(0.0), np.float32(-0.0))
        alt = j
    elif kind == "all_neginf":
        x[:] = -np.inf
        alt = V - 1
    elif kind == "neginf_in_nan":
        x[:] = np.nan
        k = int(rng.integers(1, V))
        x[k] = -np.inf
        alt = 0
    elif kind == "posinf_tie":
        i = int(rng.integers(0, V // 2))
        j = int(rng.integers(V // 2, V))
        x[i] = x[j] = np.inf
        alt = j
    elif kind == "all_equal":
        x[:] = np.float32(0.25)
        alt = V - 1
    elif kind == "nan_first":
        x[: V // 2] = np.nan
    return x, alt


@pytest.mark.parametrize("vocab", [1024, 151936])
def test_verify_tie_nan_signed_zero_inf_rows_bit_exact(vocab):
    from block_diffusion_drafting_ctx_amd import Drafter

    n_d, B = 8, 12
    wl = gen.Workload("verify-edges", 256, 4, 2, 64, 2, 512, vocab, n_d, 3, B, 10, 60, "bf16")
    log(f"[case] verify edge rows V={vocab} B={B}")
    rng = np.random.default_rng(61)
    logits = np.empty((B, n_d + 1, vocab), np.float32)
    drafts = np.zeros((B, n_d), np.int32)
    plan = []
    for b in range(B):
        a = int(rng.integers(0, n_d + 1))  # rows before a are accepted
        for i in range(n_d + 1):
            kind = KINDS[(b * (n_d + 1) + i) % len(KINDS)]
            x, alt = edge_row(kind, vocab, rng)
            logits[b, i] = x
            if i < n_d:
                from oracle import argmax_lowest

                g = argmax_lowest(x)
                # accepted rows draft the greedy token; the first rejected row
                # drafts what a wrong tie-break would pick, else a wrong token
                drafts[b, i] = g if i < a else (alt if alt >= 0 and alt != g else (g + 1) % vocab)
        plan.append(a)
    dr = Drafter(config_for(wl, B), _to(gen.draft_weights(wl, 62, "cpu"), "cuda"), "cuda")
    ctx = gen.context_lengths(wl, 63, B)
    dr.ctx_len.copy_(torch.from_numpy(ctx))
    n_acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    bonus = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    out = torch.full((B, n_d + 1), -7, dtype=torch.int32, device="cuda")
    dr.verify(torch.from_numpy(logits).cuda(), torch.from_numpy(drafts).cuda(), n_d, n_d, n_acc, bonus, out)
    torch.cuda.synchronize()
    assert dr.check() == 0
    n_acc, bonus, out, cl = n_acc.cpu().numpy(), bonus.cpu().numpy(), out.cpu().numpy(), dr.ctx_len.cpu().numpy()
    for b in range(B):
        n, bon, toks = greedy_verify(logits[b], drafts[b], n_d)
        assert n == plan[b]
        assert int(n_acc[b]) == n, f"seq {b}: accepted {n_acc[b]} != {n}"
        assert int(bonus[b]) == bon, f"seq {b}: bonus {bonus[b]} != {bon}"
        assert list(out[b, : n + 1]) == toks and np.all(out[b, n + 1:] == -1), f"seq {b}: committed tokens"
        assert int(cl[b]) == int(ctx[b]) + n + 1
    assert dr.stats() == [B, int(sum(plan)), B * n_d]
    dr.close()


def _dup_lm_rows(w):
    V = w["w_lm"].shape[0]
    w["w_lm"][V // 2:] = w["w_lm"][: V // 2]


@pytest.mark.parametrize("storage,batch", [("bf16", 1), ("f32", 1), ("bf16", 8)])
def test_lm_head_exact_ties_draft_the_lower_index(storage, batch):
    # every logit v and v + V/2 is bitwise equal: the lower index must win on
    # every row (batch 8 x block 8 = 64 rows takes the tiled matrix-core product)
    wl = gen.Workload("lm-ties", 256, 4, 2, 64, 2, 512, 1024, 8, 3, batch, 20, 200, storage)
    res = run_step(wl, seed=64, mutate=_dup_lm_rows)
    log(f"[case] lm-head ties {storage} B={batch}: {res.worst}")


def test_lm_head_ties_all_rows_low_half():
    # the same tie directly on the drafted ids of every row (no margin filter)
    from block_diffusion_drafting_ctx_amd import Drafter

    wl = gen.Workload("lm-ties-ids", 256, 4, 2, 64, 2, 512, 1024, 8, 3, 4, 20, 200, "bf16")
    w = gen.draft_weights(wl, 65, "cpu")
    _dup_lm_rows(w)
    ctx = gen.context_lengths(wl, 66, 4)
    ks, vs = gen.context_kv(wl, ctx, 66, "cpu")
    dr = Drafter(config_for(wl, 4), _to(w, "cuda"), "cuda", [k.cuda() for k in ks], [v.cuda() for v in vs])
    dr.ctx_len.copy_(torch.from_numpy(ctx))
    ids = torch.from_numpy(gen.block_ids(wl, 4, 67)).cuda()
    out = torch.full((4, wl.block), -7, dtype=torch.int32, device="cuda")
    lg = torch.empty(4, wl.block, wl.vocab, dtype=torch.float32, device="cuda")
    dr.draft_block(ids, out, lg)
    torch.cuda.synchronize()
    assert dr.check() == 0
    out, lg = out.cpu().numpy(), lg.cpu().numpy()
    half = wl.vocab // 2
    assert np.array_equal(lg[..., :half], lg[..., half:]), "duplicated LM-head rows gave different logits"
    assert np.all((out >= 0) & (out < half)), "a tie went to the higher index"
    # and it is the first maximum of the kernel's own logits
    assert np.array_equal(out, np.argmax(lg, axis=-1))
    dr.close()


def test_lm_head_nan_rows_are_never_drafted():
    # NaN LM-head rows give NaN logit columns: never drafted.  The rows chosen
    # are those the clean draft picks, so the rule is exercised on every row.
    wl = gen.Workload("lm-nan", 256, 4, 2, 64, 2, 512, 1024, 8, 3, 1, 20, 200, "bf16")
    w0 = gen.draft_weights(wl, 68, "cpu")
    ctx = gen.context_lengths(wl, 69, 1)
    ks, vs = gen.context_kv(wl, ctx, 69, "cpu")
    st = DraftState(k=[np64(t) for t in ks], v=[np64(t) for t in vs], ctx_len=ctx.astype(np.int64).copy())
    ids = gen.block_ids(wl, 1, 70)
    d_clean, _, _ = draft_block(st, weights_of(w0), dims_of(wl), ids)
    bad = sorted(set(int(t) for t in d_clean.reshape(-1)) | {0, 1, 2, 511})

    def poison(w):
        w["w_lm"][bad] = float("nan")

    res = run_step(wl, seed=68, mutate=poison)
    log(f"[case] lm-head NaN rows {bad}: {res.worst}")


def test_combine_skips_stale_pieces_of_a_longer_context():
    # First a 700-row context whose cache rows are all NaN (every piece of the
    # split segment NaN), then a 150-row clean context in the same workspace:
    # the merge takes the 3 pieces the new segment has and none of the 12 slots
    # the first call wrote.
    from block_diffusion_drafting_ctx_amd import Drafter

    wl = gen.Workload("stale-pieces", 256, 4, 2, 64, 2, 512, 1024, 8, 3, 1, 150, 700, "bf16")
    w = gen.draft_weights(wl, 71, "cpu")
    short = np.array([150], np.int32)
    ks, vs = gen.context_kv(wl, short, 72, "cpu", poison=True)
    dr = Drafter(config_for(wl, 1), _to(w, "cuda"), "cuda", [k.cuda() for k in ks], [v.cuda() for v in vs])
    saved = [(k[:, :150].clone(), v[:, :150].clone()) for k, v in zip(dr.kv_k, dr.kv_v)]
    for k, v in zip(dr.kv_k, dr.kv_v):
        k.fill_(float("nan"))
        v.fill_(float("nan"))
    ids = torch.from_numpy(gen.block_ids(wl, 1, 73)).cuda()
    out = torch.zeros(1, wl.block, dtype=torch.int32, device="cuda")
    dr.ctx_len.fill_(700)
    log("[case] stale pieces: NaN context of 700 rows")
    dr.draft_block(ids, out)
    torch.cuda.synchronize()
    for (k0, v0), k, v in zip(saved, dr.kv_k, dr.kv_v):
        k[:, :150] = k0
        v[:, :150] = v0
    dr.ctx_len.fill_(150)
    hid = torch.empty(1, wl.block, wl.hidden, dtype=torch.float32, device="cuda")
    log("[case] stale pieces: clean context of 150 rows")
    dr.draft_block(ids, out, None, hid)
    torch.cuda.synchronize()
    assert dr.check() == 0
    st = DraftState(k=[np64(t) for t in ks], v=[np64(t) for t in vs], ctx_len=short.astype(np.int64).copy())
    _, _, h_or = draft_block(st, weights_of(w), dims_of(wl), ids.cpu().numpy())
    h = hid.cpu().numpy()
    assert np.all(np.isfinite(h)), "a stale NaN piece reached the output"
    e = rel_l2(h[0], h_or[0])
    assert e <= REL_L2, f"hidden rel L2 {e}"
    dr.close()
