"""GPU parity of prompt-scale context fusion: whole prompts through dflash_fuse_ctx in chunks.

The prompt rows of every sequence are fused with commit in chunks of
max_fuse_rows (the last chunk ragged), the way a caller pre-fills the draft
cache from the target's prompt pass.  Fusion is row-independent, so sampled
rows of the fused feature and of every layer's cache K/V are compared with the
oracle's fusion and K/V projection of those rows alone at their positions.
"""

import types
from dataclasses import replace

import numpy as np
import pytest
import torch

from harness import gen
from oracle import fuse_features
from oracle.draft import context_kv
from tests.gpu_cases import REL_L2, _to, cache_rows, cache_rows_f64, config_for, log, rel_l2
from tests.oracle_adapt import dims_of, np64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,batch,rows,chunk,sample", [
    # full-size fusion: 2 x 3000 prompt rows in chunks of 1024 (1024 + 1024 + 952)
    ("qwen3-8b-shape-b1", 2, 3000, 1024, [0, 1, 517, 1023, 1024, 2047, 2048, 2500, 2999]),
    # fp32 storage, 3 sequences, every row compared (256 + 256 + 188)
    ("tiny-f32-b1", 3, 700, 256, None),
    # the 8-bit cache: every fused row quantised on the way in
    ("qwen3-8b-shape-b1-kv8", 2, 3000, 1024, [0, 1, 517, 1023, 1024, 2047, 2048, 2500, 2999]),
])
def test_prompt_fusion_in_chunks(name, batch, rows, chunk, sample):
    from block_diffusion_drafting_ctx_amd import Drafter

    wl = replace(gen.WORKLOADS[name], batch=batch, ctx_lo=rows, ctx_hi=rows)
    log(f"[case] prefill {name} B={batch} rows={rows} chunk={chunk}")
    dev = "cuda"
    gdev = dev if wl.hidden >= 1024 else "cpu"
    w = gen.draft_weights(wl, 31, gdev)
    w_dev = _to(w, dev)
    hidden = [h.to(dev) for h in gen.target_hidden(wl, batch, rows, 32, gdev)]
    dr = Drafter(config_for(wl, batch, chunk), w_dev, dev)
    H = wl.hidden
    feat = torch.empty(batch, rows, H, dtype=torch.float32, device=dev)
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        part = [h[:, r0:r1].contiguous() for h in hidden]
        fd = torch.empty(batch, r1 - r0, H, dtype=torch.float32, device=dev)
        dr.fuse_ctx(part, commit=True, feat_dbg=fd)
        feat[:, r0:r1] = fd
    torch.cuda.synchronize()
    assert dr.check() == 0
    assert dr.ctx_len.cpu().tolist() == [rows] * batch

    dims = dims_of(wl)
    rows_sel = np.arange(rows) if sample is None else np.asarray(sample)
    w_fc, g_fc = np64(w["w_fc"]), np64(w["g_fc"])
    proj = [types.SimpleNamespace(w_k=np64(lw["w_k"]), w_v=np64(lw["w_v"])) for lw in w["layers"]]
    worst = {}
    for b in range(batch):
        c = fuse_features([np64(h[b, rows_sel]) for h in hidden], w_fc, g_fc, wl.rms_eps)
        e = rel_l2(np64(feat[b, rows_sel]), c)
        worst["feature"] = max(worst.get("feature", 0.0), e)
        assert e <= REL_L2, f"seq {b} feature rel L2 {e}"
        for l, lw in enumerate(proj):
            k, v = context_kv(c, lw, rows_sel, dims)
            for nm, ref in (("K", k), ("V", v)):
                got = cache_rows_f64(cache_rows(dr, l, nm, b, 0, rows))[rows_sel]
                e = rel_l2(got, ref)
                worst[nm] = max(worst.get(nm, 0.0), e)
                assert e <= REL_L2, f"seq {b} layer {l} cache {nm} rel L2 {e}"
    log(f"[case] prefill {name}: worst rel L2 {worst}")
    dr.close()
    del dr, hidden, feat
    torch.cuda.empty_cache()
