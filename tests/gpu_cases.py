"""One fuse -> verify -> draft step on the GPU library, checked against the oracle.

Used by the GPU parity tests and by ``__graft_entry__.smoke()``.  Inputs come
from ``harness.gen`` only; the oracle's starting state is copied from the
generator's tensors before the library touches them, so no oracle input and
no expected value comes from the HIP path.

Bars (floating point: bf16 operands, fp32 accumulation on the GPU):
  context feature, cache rows: relative L2 <= 1e-2;
  final hidden state: relative L2 <= 1e-2 over the block and for every row;
  logits: NaN in the same entries as the oracle, max |diff| <= 5e-2 *
  std(oracle logits) over the others;
  draft ids: equal wherever the oracle's top-1 minus top-2 margin > 0.1
  (the margin to the next smaller distinct value, NaN ignored, so an exact
  tie of the top value is decided by the lowest-index rule); on the other
  rows the drafted id must be a non-NaN entry whose oracle logit is within
  2 * 5e-2 * std of the row maximum (a near-top token); optionally a floor on
  the share of rows compared exactly;
  verify (accepted length, bonus, committed tokens, context lengths,
  counters): bit-exact.
"""

from __future__ import annotations

import sys
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

from harness import gen
from oracle import DraftState, draft_block, fuse_ctx, kv8_dequantize, verify_step, AcceptanceStats
from tests.oracle_adapt import dims_of, np64, weights_of

REL_L2 = 1e-2
LOGIT_TOL = 5e-2
MARGIN = 0.1


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def top2_margin(logits: np.ndarray) -> np.ndarray:
    """Per row: largest value minus the largest value below it (NaN ignored;
    inf when the row holds a single distinct value)."""
    x = np.asarray(logits, dtype=np.float64)
    flat = x.reshape(-1, x.shape[-1])
    out = np.empty(flat.shape[0])
    for r, row in enumerate(flat):
        v = row[~np.isnan(row)]
        if v.size == 0:
            out[r] = np.inf
            continue
        m1 = v.max()
        below = v[v < m1]
        out[r] = m1 - below.max() if below.size else np.inf
    return out.reshape(x.shape[:-1])


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def config_for(wl: gen.Workload, batch: int, max_fuse_rows: Optional[int] = None):
    from block_diffusion_drafting_ctx_amd import make_config

    return make_config(wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.n_layers, wl.ffn, wl.vocab,
                       wl.block, wl.n_target_layers, batch, wl.max_ctx,
                       max_fuse_rows or wl.t_new, wl.conv_width, wl.storage, wl.rms_eps, wl.rope_theta, wl.kv)


def oracle_cache(t, seqs):
    """The oracle's float64 view of generated cache entries for sequences `seqs`
    (an 8-bit entry is a (values, scales) pair: its value is values * scale)."""
    if isinstance(t, tuple):
        return kv8_dequantize(np64(t[0][seqs]), np64(t[1][seqs]))
    return np64(t[seqs])


def device_cache(t, cfg, device, batch):
    """One generated cache entry as the library's buffer for a context of
    cfg.max_batch sequences (the first `batch` filled)."""
    from block_diffusion_drafting_ctx_amd import kv8_buffer

    if isinstance(t, tuple):
        return kv8_buffer(t[0].to(device), t[1].to(device), cfg)
    t = t.to(device)
    if cfg.max_batch == batch:
        return t
    full = torch.zeros((cfg.max_batch,) + tuple(t.shape[1:]), dtype=t.dtype, device=device)
    full[:batch] = t
    return full


def cache_rows(dr, layer, kind, b, lo, hi):
    """Rows [lo, hi) of sequence b of one layer's cache as the library left
    them: a tensor, or (values, scales) for the 8-bit cache."""
    if not dr.kv8:
        return (dr.kv_k if kind == "K" else dr.kv_v)[layer][b, lo:hi].clone()
    k = kind.lower()
    return dr.kv_values(layer, k)[b, lo:hi].clone(), dr.kv_scales(layer, k)[b, lo:hi].clone()


def cache_rows_f64(rows):
    if isinstance(rows, tuple):
        q, sc = np64(rows[0]), np64(rows[1])
        # the format itself: integers in [-127, 127], and every non-zero run
        # reaches +-127 (its scale is max|x| / 127)
        assert np.all(np.abs(q) <= 127)
        runs = np.abs(q).reshape(q.shape[:-1] + (-1, 32)).max(axis=-1)
        assert np.all((runs == 127) | ((runs == 0) & (sc == 0))), "8-bit runs off their scale"
        return kv8_dequantize(q, sc)
    return np64(rows)


@dataclass
class StepResult:
    checks: List[str] = field(default_factory=list)
    worst: dict = field(default_factory=dict)

    def note(self, key: str, value: float) -> None:
        self.worst[key] = max(self.worst.get(key, 0.0), value)


def run_step(wl: gen.Workload, seed: int, device="cuda", seqs: Optional[Sequence[int]] = None,
             prefill: bool = False, poison: bool = False, n_d: Optional[int] = None,
             check_oracle: bool = True, accept: Optional[Sequence[int]] = None,
             max_batch: Optional[int] = None, mutate=None, min_sure: float = 0.0) -> StepResult:
    """Run one step on the library and compare with the oracle on `seqs`.

    `accept` overrides the planted acceptance lengths (one per sequence);
    `max_batch` sizes the context for more sequences than the call passes;
    `mutate(w)` edits the generated weights in place before either side
    sees them; `min_sure` is the least share of the compared draft rows whose
    oracle margin must exceed the bar (so that the exact comparison is not
    vacuous)."""
    from block_diffusion_drafting_ctx_amd import Drafter

    res = StepResult()
    B = wl.batch
    n_d = wl.n_d if n_d is None else n_d
    t_new = n_d + 1
    seqs = list(range(B)) if seqs is None else list(seqs)
    log(f"[case] {wl.name} B={B} seed={seed} prefill={prefill} poison={poison} n_d={n_d} seqs={seqs}")
    gdev = device if wl.hidden >= 1024 else "cpu"  # big inputs are drawn on the GPU
    w = gen.draft_weights(wl, seed, gdev)
    if mutate is not None:
        mutate(w)
    w_dev = _to(w, device)
    if prefill:
        ctx_lens = np.zeros(B, dtype=np.int32)
        ks = vs = None
        pre = gen.target_hidden(wl, B, wl.ctx_hi, seed + 1, gdev)
    else:
        ctx_lens = gen.context_lengths(wl, seed + 1, B)
        ks, vs = gen.context_kv(wl, ctx_lens, seed + 1, gdev, poison=poison)
    hid = gen.target_hidden(wl, B, t_new, seed + 2, gdev)
    drafts = gen.draft_tokens(wl, B, n_d, seed + 3)
    accept = (gen.accept_lengths(wl, B, seed + 4, n_d) if accept is None
              else np.asarray(accept, dtype=np.int32))
    logits = gen.planted_logits(wl, drafts, accept, n_d, seed + 5, gdev)
    ids = gen.block_ids(wl, B, seed + 6)

    # oracle copies taken before the library runs
    W = weights_of(w) if check_oracle else None
    dims = dims_of(wl)
    if check_oracle:
        if prefill:
            st = DraftState.empty(dims, len(seqs), wl.max_ctx)
        else:
            st = DraftState(k=[oracle_cache(t, seqs) for t in ks], v=[oracle_cache(t, seqs) for t in vs],
                            ctx_len=ctx_lens[seqs].astype(np.int64).copy())

    cfg = config_for(wl, max_batch or B, max(t_new, wl.ctx_hi if prefill else 0))
    kv_dev = None if ks is None else ([device_cache(t, cfg, device, B) for t in ks],
                                      [device_cache(t, cfg, device, B) for t in vs])
    dr = Drafter(cfg, w_dev, device, *(kv_dev or (None, None)))
    dr.ctx_len[:B].copy_(torch.from_numpy(ctx_lens))
    M_f = B * t_new
    H = wl.hidden
    if prefill:
        pre_feat = torch.empty(B, wl.ctx_hi, H, dtype=torch.float32, device=device)
        dr.fuse_ctx([h.to(device) for h in pre], commit=True, feat_dbg=pre_feat)
    feat = torch.empty(B, t_new, H, dtype=torch.float32, device=device)
    dr.fuse_ctx([h.to(device) for h in hid], commit=False, feat_dbg=feat)
    ctx_after_fuse = dr.ctx_len.clone()
    # the fused rows of the sampled sequences as the fusion left them (the
    # draft later stages its block's keys in the rows past the committed ones)
    fused_rows = {}
    if check_oracle:
        for b in seqs:
            t0 = int(ctx_after_fuse[b])
            lo = 0 if prefill else t0
            for l in range(wl.n_layers):
                for kind in ("K", "V"):
                    fused_rows[(b, l, kind)] = cache_rows(dr, l, kind, b, lo, t0 + t_new)
    d_dev = torch.from_numpy(drafts).to(device)
    n_acc = torch.full((B,), -7, dtype=torch.int32, device=device)
    bonus = torch.full((B,), -7, dtype=torch.int32, device=device)
    out_tok = torch.full((B, t_new), -7, dtype=torch.int32, device=device)
    dr.verify(logits.to(device), d_dev, n_d, n_d, n_acc, bonus, out_tok)
    ctx_after_verify = dr.ctx_len.clone()
    ids_dev = torch.from_numpy(ids).to(device)
    draft_ids = torch.full((B, wl.block), -7, dtype=torch.int32, device=device)
    lg_dbg = torch.empty(B, wl.block, wl.vocab, dtype=torch.float32, device=device)
    hid_dbg = torch.empty(B, wl.block, H, dtype=torch.float32, device=device)
    dr.draft_block(ids_dev, draft_ids, lg_dbg, hid_dbg)
    torch.cuda.synchronize()
    err = dr.check()
    assert err == 0, f"device error word {err:#x}"
    stats = dr.stats()
    log(f"[case] {wl.name}: library step done, stats={stats}")

    # ---------------- verify: bit-exact against the oracle on all sequences
    lg_np = logits.cpu().numpy()
    exp_n = np.zeros(B, np.int64)
    for b in range(B):
        from oracle import greedy_verify

        n, bon, toks = greedy_verify(lg_np[b], drafts[b], n_d)
        exp_n[b] = n
        assert int(n_acc[b]) == n, f"seq {b}: accepted {int(n_acc[b])} != {n}"
        assert int(bonus[b]) == bon, f"seq {b}: bonus {int(bonus[b])} != {bon}"
        got = out_tok[b].cpu().numpy()
        assert list(got[: n + 1]) == toks and np.all(got[n + 1:] == -1), f"seq {b}: out tokens"
        base = int(ctx_lens[b]) + (wl.ctx_hi if prefill else 0)
        assert int(ctx_after_fuse[b]) == base
        assert int(ctx_after_verify[b]) == base + n + 1
    np.testing.assert_array_equal(exp_n, accept)  # the planted lengths
    assert stats == [B, int(exp_n.sum()), B * n_d]
    res.checks.append("verify bit-exact")
    if not check_oracle:
        return res

    # ---------------- oracle: same call sequence on the sampled sequences
    if prefill:
        c_pre = fuse_ctx(st, W, dims, [np64(h[seqs]) for h in pre], commit=True)
        e = rel_l2(pre_feat.cpu().numpy()[seqs], c_pre)
        res.note("prefill_feature_rel_l2", e)
        assert e <= REL_L2, f"prefill feature rel L2 {e}"
    c = fuse_ctx(st, W, dims, [np64(h[seqs]) for h in hid], commit=False)
    e = rel_l2(feat.cpu().numpy()[seqs], c)
    res.note("feature_rel_l2", e)
    assert e <= REL_L2, f"feature rel L2 {e}"
    for j, b in enumerate(seqs):
        t0 = int(st.ctx_len[j])
        lo = 0 if prefill else t0
        for l in range(wl.n_layers):
            for name, ref in (("K", st.k[l]), ("V", st.v[l])):
                got = cache_rows_f64(fused_rows[(b, l, name)])
                e = rel_l2(got, ref[j, lo:t0 + t_new])
                res.note(f"cache_{name}_rel_l2", e)
                assert e <= REL_L2, f"seq {b} layer {l} cache {name} rel L2 {e}"
    lg_sel = lg_np[seqs]
    verify_step(st, lg_sel, drafts[seqs].reshape(-1), n_d, n_d, AcceptanceStats())
    for j, b in enumerate(seqs):
        assert int(st.ctx_len[j]) == int(ctx_after_verify[b])
    d_or, l_or, h_or = draft_block(st, W, dims, ids[seqs])
    h_gpu = hid_dbg.cpu().numpy()[seqs]
    l_gpu = lg_dbg.cpu().numpy()[seqs]
    i_gpu = draft_ids.cpu().numpy()[seqs]
    n_sure = n_rows = 0
    for j, b in enumerate(seqs):
        e = rel_l2(h_gpu[j], h_or[j])
        res.note("hidden_rel_l2", e)
        assert e <= REL_L2, f"seq {b} final hidden rel L2 {e}"
        for i in range(wl.block):
            e = rel_l2(h_gpu[j][i], h_or[j][i])
            res.note("hidden_row_rel_l2", e)
            assert e <= REL_L2, f"seq {b} row {i} final hidden rel L2 {e}"
        nan_or = np.isnan(l_or[j])
        assert np.array_equal(np.isnan(l_gpu[j]), nan_or), f"seq {b}: NaN logits differ from the oracle's"
        std = float(np.std(l_or[j][~nan_or]))
        tol = LOGIT_TOL * std
        dmax = float(np.max(np.abs(l_gpu[j][~nan_or] - l_or[j][~nan_or])))
        res.note("logit_maxdiff_over_std", dmax / std)
        assert dmax <= tol, f"seq {b} logits max diff {dmax} > {tol}"
        marg = top2_margin(l_or[j])
        sure = marg > MARGIN
        assert np.all(i_gpu[j][sure] == d_or[j][sure]), f"seq {b} draft ids differ where margin > {MARGIN}"
        for i in np.flatnonzero(~sure):  # low margin: a near-top, non-NaN token
            g = int(i_gpu[j][i])
            assert 0 <= g < wl.vocab and not nan_or[i, g], f"seq {b} row {i}: drafted id {g} invalid or NaN"
            top = float(np.nanmax(l_or[j][i]))
            assert l_or[j][i, g] >= top - 2 * tol, \
                f"seq {b} row {i}: drafted id {g} at {l_or[j][i, g]:.4f}, row max {top:.4f}"
        res.note("rows_with_margin", float(sure.sum()))
        n_sure += int(sure.sum())
        n_rows += wl.block
    assert n_sure >= min_sure * n_rows, f"only {n_sure} of {n_rows} draft rows have margin > {MARGIN}"
    res.checks.append("oracle parity")
    log(f"[case] {wl.name}: parity ok {res.worst}")
    dr.close()
    return res


def _to(w: dict, device) -> dict:
    out = {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in w.items() if k != "layers"}
    out["layers"] = [{k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in lw.items()}
                     for lw in w["layers"]]
    return out


def run_error_paths(wl: gen.Workload, seed: int, device="cuda", draft_overflow: bool = False) -> None:
    """Device-detected faults, forced from the host: a context that would pass
    max_ctx (fuse and verify skip that sequence's writes and commit; with
    draft_overflow the drafted block would pass it too, and the draft stages
    nothing for it) and a block token outside the vocabulary (embedded as
    zeros).  The other sequences must still match the oracle bit for bit /
    within the bars, and the sticky error word must name exactly the faults."""
    from block_diffusion_drafting_ctx_amd import Drafter, _abi

    B = wl.batch
    assert B >= 3
    n_d, t_new = wl.n_d, wl.t_new
    log(f"[case] {wl.name} error paths B={B} seed={seed}")
    w = gen.draft_weights(wl, seed, "cpu")
    w_dev = _to(w, device)
    ctx_lens = gen.context_lengths(wl, seed + 1, B)
    # fuse (t_new rows) and verify would pass max_ctx; with draft_overflow the block (Bs rows) too
    ctx_lens[1] = wl.max_ctx - (wl.block if draft_overflow else t_new) + 1
    ks, vs = gen.context_kv(wl, np.minimum(ctx_lens, wl.max_ctx), seed + 1, "cpu")
    hid = gen.target_hidden(wl, B, t_new, seed + 2, "cpu")
    drafts = gen.draft_tokens(wl, B, n_d, seed + 3)
    accept = gen.accept_lengths(wl, B, seed + 4, n_d)
    logits = gen.planted_logits(wl, drafts, accept, n_d, seed + 5, "cpu")
    ids = gen.block_ids(wl, B, seed + 6)
    ids[2, 1] = wl.vocab  # out of range

    W = weights_of(w)
    dims = dims_of(wl)
    good = [0]
    st = DraftState(k=[np64(t[good]) for t in ks], v=[np64(t[good]) for t in vs],
                    ctx_len=ctx_lens[good].astype(np.int64).copy())
    cfg = config_for(wl, B)
    dr = Drafter(cfg, w_dev, device, [t.to(device) for t in ks], [t.to(device) for t in vs])
    dr.ctx_len.copy_(torch.from_numpy(ctx_lens))
    k1_before = [dr.kv_k[l][1].clone() for l in range(wl.n_layers)]
    feat = torch.empty(B, t_new, wl.hidden, dtype=torch.float32, device=device)
    dr.fuse_ctx([h.to(device) for h in hid], commit=False, feat_dbg=feat)
    n_acc = torch.full((B,), -7, dtype=torch.int32, device=device)
    bonus = torch.full((B,), -7, dtype=torch.int32, device=device)
    out_tok = torch.full((B, t_new), -7, dtype=torch.int32, device=device)
    dr.verify(logits.to(device), torch.from_numpy(drafts).to(device), n_d, n_d, n_acc, bonus, out_tok)
    ctx_after = dr.ctx_len.cpu().numpy()
    draft_ids = torch.full((B, wl.block), -7, dtype=torch.int32, device=device)
    hid_dbg = torch.empty(B, wl.block, wl.hidden, dtype=torch.float32, device=device)
    dr.draft_block(torch.from_numpy(ids).to(device), draft_ids, None, hid_dbg)
    torch.cuda.synchronize()
    err = dr.check()
    want = _abi.ERR_FUSE_OVERFLOW | _abi.ERR_VERIFY_OVERFLOW | _abi.ERR_TOKEN_RANGE
    if draft_overflow:
        want |= _abi.ERR_DRAFT_OVERFLOW
    assert err == want, f"error word {err:#x}, expected {want:#x}"
    # the overflowing sequence: committed rows untouched (rows past ctx_len only
    # stage the drafted block's keys), length not advanced
    t1 = int(ctx_lens[1])
    for l in range(wl.n_layers):
        assert torch.equal(dr.kv_k[l][1][:t1], k1_before[l][:t1]), \
            f"layer {l}: committed cache rows of the overflowing sequence written"
    assert int(ctx_after[1]) == int(ctx_lens[1])
    # the healthy sequences: verify bit-exact, sequence 0 matches the oracle
    from oracle import greedy_verify

    lg_np = logits.numpy()
    for b in (0, 2):
        n, bon, toks = greedy_verify(lg_np[b], drafts[b], n_d)
        assert int(n_acc[b]) == n and int(bonus[b]) == bon
        assert int(ctx_after[b]) == int(ctx_lens[b]) + n + 1
    c = fuse_ctx(st, W, dims, [np64(h[good]) for h in hid], commit=False)
    assert rel_l2(feat.cpu().numpy()[good], c) <= REL_L2
    verify_step(st, lg_np[good], drafts[good].reshape(-1), n_d, n_d, AcceptanceStats())
    _, _, h_or = draft_block(st, W, dims, ids[good])
    e = rel_l2(hid_dbg.cpu().numpy()[good][0], h_or[0])
    assert e <= REL_L2, f"healthy sequence hidden rel L2 {e}"
    dr.clear_errors()
    torch.cuda.synchronize()
    assert dr.check() == 0
    log(f"[case] {wl.name}: error paths ok (error word {err:#x})")
    dr.close()
