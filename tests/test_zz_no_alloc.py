"""GPU: the context-free greedy verify (dflash_verify_static) against dflash_verify.

dflash_verify_static keeps its argmax keys in a library-owned static device
array instead of a context workspace, for callers that cannot allocate.  Two
calls in a row, the second smaller (fewer sequences, fewer drafts, a smaller
vocabulary), must give bit-for-bit the outputs of dflash_verify on the same
inputs (accepted counts, bonus tokens, committed tokens, context lengths,
counters), and those of the oracle.  The overflow bit, the null counters and
the size limit are checked too.
"""

import numpy as np
import pytest
import torch

from harness import gen
from oracle import greedy_verify
from tests.gpu_cases import _to, config_for, log

pytestmark = pytest.mark.gpu


def _inputs(vocab, batch, n_d, seed):
    wl = gen.Workload("static-verify", 256, 4, 2, 64, 2, 512, vocab, max(n_d, 1), 3, batch, 10, 300, "bf16",
                      accept_hi=max(n_d, 1))
    drafts = gen.draft_tokens(wl, batch, max(n_d, 1), seed)
    accept = gen.accept_lengths(wl, batch, seed + 1, n_d)
    logits = gen.planted_logits(wl, drafts, accept, n_d, seed + 2, "cpu")
    ctx = gen.context_lengths(wl, seed + 3, batch)
    return wl, drafts, accept, logits, ctx


def _run_ctx(wl, drafts, logits, ctx, n_d):
    """The existing entry point (a context with its workspace)."""
    from block_diffusion_drafting_ctx_amd import Drafter

    B = len(ctx)
    dr = Drafter(config_for(wl, B), _to(gen.draft_weights(wl, 5, "cpu"), "cuda"), "cuda")
    dr.ctx_len.copy_(torch.from_numpy(ctx))
    n_acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    bonus = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    out = torch.full((B, n_d + 1), -7, dtype=torch.int32, device="cuda")
    dr.verify(logits.cuda(), torch.from_numpy(drafts).cuda(), drafts.shape[1], n_d, n_acc, bonus, out)
    torch.cuda.synchronize()
    assert dr.check() == 0
    res = (n_acc.cpu().numpy(), bonus.cpu().numpy(), out.cpu().numpy(), dr.ctx_len[:B].cpu().numpy(),
           list(dr.stats()))
    dr.close()
    return res


def _run_static(wl, drafts, logits, ctx, n_d, stats, err):
    from block_diffusion_drafting_ctx_amd import _abi

    B = len(ctx)
    cl = torch.from_numpy(ctx.copy()).cuda()
    n_acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    bonus = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    out = torch.full((B, n_d + 1), -7, dtype=torch.int32, device="cuda")
    _abi.dflash_verify_static(logits.cuda(), torch.from_numpy(drafts).cuda(), drafts.shape[1], n_d, cl, wl.max_ctx,
                              n_acc, bonus, out, stats, err)
    torch.cuda.synchronize()
    return n_acc.cpu().numpy(), bonus.cpu().numpy(), out.cpu().numpy(), cl.cpu().numpy()


def test_static_verify_matches_context_verify_twice_second_smaller():
    stats = torch.zeros(3, dtype=torch.int64, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    total = np.zeros(3, np.int64)
    for call, (vocab, batch, n_d, seed) in enumerate([(151936, 24, 16, 81), (1024, 5, 7, 91)]):
        log(f"[case] static verify call {call}: V={vocab} B={batch} n_d={n_d}")
        wl, drafts, accept, logits, ctx = _inputs(vocab, batch, n_d, seed)
        want = _run_ctx(wl, drafts, logits, ctx, n_d)
        got = _run_static(wl, drafts, logits, ctx, n_d, stats, err)
        for name, g, w in zip(("n_accept", "bonus", "out_tokens", "ctx_len"), got, want[:4]):
            assert np.array_equal(g, w), f"call {call}: {name} differs from dflash_verify"
        lg = logits.numpy()
        for b in range(batch):
            n, bon, toks = greedy_verify(lg[b], drafts[b], n_d)
            assert n == int(accept[b]) == int(got[0][b]) and bon == int(got[1][b])
            assert list(got[2][b, : n + 1]) == toks and np.all(got[2][b, n + 1:] == -1)
        total += np.array(want[4], np.int64)
        assert np.array_equal(stats.cpu().numpy(), total), "counters differ from dflash_verify's"
    assert int(err.item()) == 0


def test_static_verify_overflow_bit_and_null_counters():
    from block_diffusion_drafting_ctx_amd import _abi

    wl, drafts, accept, logits, ctx = _inputs(1024, 4, 8, 101)
    ctx = ctx.copy()
    ctx[2] = wl.max_ctx - 8  # ctx + n_d + 1 passes max_ctx: not committed, bit set
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    n_acc, bonus, out, cl = _run_static(wl, drafts, logits, ctx, 8, None, err)
    assert int(err.item()) == _abi.ERR_VERIFY_OVERFLOW
    assert int(cl[2]) == int(ctx[2])
    for b in (0, 1, 3):
        assert int(cl[b]) == int(ctx[b]) + int(accept[b]) + 1 and int(n_acc[b]) == int(accept[b])


def test_static_verify_rejects_sizes_beyond_the_scratch():
    from block_diffusion_drafting_ctx_amd import _abi

    # 129 sequences x 17 rows x 19 chunks = 41667 keys fits; 200 x 17 x 19 = 64600 fits;
    # 204 x 17 x 19 = 65892 does not
    i32 = lambda *s: torch.zeros(*s, dtype=torch.int32, device="cuda")  # noqa: E731
    lg = torch.zeros(204, 17, 151936, dtype=torch.float32, device="cuda")
    with pytest.raises(_abi.DFlashError):
        _abi.dflash_verify_static(lg, i32(204, 16), 16, 16, i32(204), 10000, i32(204), i32(204), i32(204, 17))
    with pytest.raises(_abi.DFlashError):  # vocabulary not a multiple of 64
        _abi.dflash_verify_static(torch.zeros(1, 2, 1000, device="cuda"), i32(1, 1), 1, 1, i32(1), 100, i32(1),
                                  i32(1), i32(1, 2))
    del lg
    torch.cuda.empty_cache()
