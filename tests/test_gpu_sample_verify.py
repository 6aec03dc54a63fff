"""GPU parity of sampling-mode verification (dflash_verify_sample) with the oracle.

The library decides in fp32 and the oracle in float64, so a decision can only
differ where a uniform lies within rounding of its boundary: the accept test
u < p(d) or a step of the inverse CDF.  Sequences with a margin below 1e-5 are
reported as ambiguous and not compared; the seeded inputs keep them rare, and
every other sequence must match exactly (accepted count, drawn token,
committed tokens, context length).
"""

import numpy as np
import pytest
import torch

from harness import gen
from oracle import sample_verify
from tests.gpu_cases import _to, config_for, log

pytestmark = pytest.mark.gpu

MARGIN = 1e-5


def margins(logits, draft, n_d, T, u):
    """Smallest distance of a deciding uniform to its boundary (float64)."""
    x = np.asarray(logits, np.float64) / T
    x = np.where(np.isnan(x), -np.inf, x)
    worst = np.inf
    for i in range(n_d + 1):
        p = np.exp(x[i] - x[i].max())
        p /= p.sum()
        if i < n_d:
            d = int(draft[i])
            inside = 0 <= d < p.size
            pd = p[d] if inside else 0.0
            worst = min(worst, abs(u[i, 0] - pd))
            if u[i, 0] < pd:
                continue
            if inside:
                p[d] = 0.0
            p /= p.sum()
        c = np.cumsum(p)
        worst = min(worst, float(np.min(np.abs(c - u[i, 1]))))
        break
    return worst


def check_against_oracle(vocab, batch, n_d, T, sigma, plant="prefix", bad_ids=False, seed=33, nan_entries=False):
    """Seeded logits [batch, n_d+1, vocab] ~ N(0, sigma^2), drafts and uniforms;
    plant: 'prefix' makes a random-length prefix of drafts likely (row max + 3),
    'all' makes every draft near-certain (row max + 30, accept uniforms < 0.9);
    bad_ids puts ids outside the vocabulary (negative and >= vocab) into the
    drafts; nan_entries puts NaN logits at random entries of every row and
    under some drafts (no mass there: such a draft is rejected).  Every
    sequence off a rounding boundary must match the oracle."""
    stride = max(1, n_d)
    block = max(16, n_d)
    wl = gen.Workload("sv", 256, 4, 2, 64, 2, 512, vocab, block, 3, batch, 10, 60, "bf16")
    log(f"[case] sample verify V={vocab} B={batch} n_d={n_d} T={T} plant={plant} bad_ids={bad_ids} "
        f"nan={nan_entries}")
    from block_diffusion_drafting_ctx_amd import Drafter

    dr = Drafter(config_for(wl, batch), _to(gen.draft_weights(wl, 41, "cpu"), "cuda"), "cuda")
    rng = np.random.default_rng(seed)
    logits = (rng.normal(size=(batch, n_d + 1, vocab)) * sigma).astype(np.float32)
    drafts = rng.integers(0, vocab, size=(batch, stride)).astype(np.int32)
    u = rng.uniform(size=(batch, n_d + 1, 2)).astype(np.float32)
    for b in range(batch):
        if plant == "all":
            for i in range(n_d):
                logits[b, i, drafts[b, i]] = logits[b, i].max() + 30.0
            u[b, :n_d, 0] *= 0.9
        else:
            for i in range(int(rng.integers(0, n_d + 1))):
                logits[b, i, drafts[b, i]] = logits[b, i].max() + 3.0
        if nan_entries:
            for i in range(n_d + 1):
                logits[b, i, rng.choice(vocab, size=vocab // 16, replace=False)] = np.nan
            for i in range(0, n_d, 3):
                logits[b, i, drafts[b, i]] = np.nan
        if bad_ids and n_d:
            for i in rng.choice(n_d, size=min(n_d, 3), replace=False):
                drafts[b, i] = int(rng.choice([-1, -7, vocab, vocab + 12345]))
    ctx = gen.context_lengths(wl, 34, batch)
    dr.ctx_len.copy_(torch.from_numpy(ctx))
    n_acc = torch.full((batch,), -7, dtype=torch.int32, device="cuda")
    tok = torch.full((batch,), -7, dtype=torch.int32, device="cuda")
    out = torch.full((batch, n_d + 1), -7, dtype=torch.int32, device="cuda")
    dr.verify_sample(torch.from_numpy(logits).cuda(), torch.from_numpy(drafts).cuda(), stride, n_d, T,
                     torch.from_numpy(u).cuda(), n_acc, tok, out)
    torch.cuda.synchronize()
    assert dr.check() == 0
    n_acc, tok, out, cl = n_acc.cpu().numpy(), tok.cpu().numpy(), out.cpu().numpy(), dr.ctx_len.cpu().numpy()
    compared = ambiguous = 0
    total_acc = 0
    for b in range(batch):
        ub = u[b].astype(np.float64)
        if margins(logits[b], drafts[b], n_d, T, ub) < MARGIN:
            ambiguous += 1
            continue
        n, t, toks = sample_verify(logits[b], drafts[b], n_d, T, ub)
        assert int(n_acc[b]) == n, f"seq {b}: accepted {n_acc[b]} != {n}"
        assert int(tok[b]) == t, f"seq {b}: drawn {tok[b]} != {t}"
        assert list(out[b, : n + 1]) == toks and np.all(out[b, n + 1:] == -1), f"seq {b}: out tokens"
        assert int(cl[b]) == int(ctx[b]) + n + 1
        compared += 1
        total_acc += n
    log(f"[case] sample verify: {compared} compared, {ambiguous} ambiguous, accepted {total_acc}")
    assert compared >= batch - 1 and compared >= min(batch, 2)
    steps, accepted, drafted = dr.stats()
    assert (steps, drafted) == (batch, batch * n_d) and accepted == int(n_acc.sum())
    dr.close()
    return int(n_acc.sum())  # over every sequence, ambiguous draws included


# (the full vocabulary takes peaky logits, sigma 6: with sigma 2 a draw over
# 151936 tokens falls within 1e-5 of a CDF step most of the time, where the
# fp32 and float64 sums may pick neighbouring tokens)
@pytest.mark.parametrize("vocab,batch,n_d,T,sigma", [(1024, 8, 8, 0.7, 2.0), (151936, 10, 16, 1.0, 6.0)])
def test_sample_verify_matches_oracle(vocab, batch, n_d, T, sigma):
    check_against_oracle(vocab, batch, n_d, T, sigma)


def test_sample_verify_no_drafts_draws_the_bonus():
    assert check_against_oracle(1024, 6, 0, 1.0, 2.0) == 0


def test_sample_verify_all_64_accepted():
    assert check_against_oracle(4096, 3, 64, 0.9, 2.0, plant="all") == 3 * 64


def test_sample_verify_drafts_outside_the_vocabulary():
    check_against_oracle(1024, 8, 8, 1.0, 2.0, bad_ids=True)


@pytest.mark.parametrize("vocab", [1024, 151936])
def test_sample_verify_nan_entries_carry_no_mass(vocab):
    check_against_oracle(vocab, 8, 8, 1.0, 2.0 if vocab == 1024 else 6.0, nan_entries=True)


def test_sample_verify_partials_beyond_lds():
    # 65 rows x 40 vocabulary chunks of partials exceed the LDS staging: the
    # per-sequence pass reads them from global memory
    check_against_oracle(327680, 3, 64, 1.0, 8.0)


def test_sample_verify_rejects_bad_temperature():
    from block_diffusion_drafting_ctx_amd import Drafter, _abi

    wl = gen.Workload("sv-bad", 256, 4, 2, 64, 2, 512, 1024, 8, 3, 1, 10, 20, "bf16")
    dr = Drafter(config_for(wl, 1), _to(gen.draft_weights(wl, 42, "cpu"), "cuda"), "cuda")
    z = lambda *s: torch.zeros(*s, dtype=torch.int32, device="cuda")  # noqa: E731
    lg = torch.zeros(1, 9, 1024, dtype=torch.float32, device="cuda")
    uu = torch.zeros(1, 9, 2, dtype=torch.float32, device="cuda")
    # (1e-39 and 1e-45 are fp32 subnormals whose reciprocal overflows)
    for T in (0.0, -1.0, float("inf"), float("nan"), 1e-39, 1e-45):
        with pytest.raises(_abi.DFlashError):
            dr.verify_sample(lg, z(1, 8), 8, 8, T, uu, z(1), z(1), z(1, 9))
    dr.close()
