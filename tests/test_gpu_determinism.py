"""GPU determinism: one fuse -> verify -> draft step run twice from the same
state gives bitwise equal outputs.

Every split-K sum, attention piece merge, row norm and argmax in the library
runs in a fixed order (no atomics on values), so a rerun reproduces every
bit: the fused feature, every cache entry (the appended rows, the block rows
staged past them and the untouched context), the verify outputs and
counters, the final hidden states, the logits and the draft ids.  The cases
cover each kernel family: fp32 storage (register-staged attention), the
batch-1 weight-streaming products with fixed-chunk attention, the batch-32
LDS-DMA products with planned attention pieces, 32k contexts with bf16 and
8-bit caches, and the 27B shape with the block conv.  Inputs come from
``harness.gen`` only (the same recipe as the parity tests).
"""

import pytest
import torch

from harness import gen
from tests.gpu_cases import _to, config_for, device_cache, log

pytestmark = pytest.mark.gpu


def _step_outputs(wl: gen.Workload, seed: int, device="cuda") -> dict:
    from block_diffusion_drafting_ctx_amd import Drafter

    B, n_d = wl.batch, wl.n_d
    t_new = n_d + 1
    gdev = device if wl.hidden >= 1024 else "cpu"
    w = _to(gen.draft_weights(wl, seed, gdev), device)
    ctx_lens = gen.context_lengths(wl, seed + 1, B)
    ks, vs = gen.context_kv(wl, ctx_lens, seed + 1, gdev, poison=True)
    hid = gen.target_hidden(wl, B, t_new, seed + 2, gdev)
    drafts = gen.draft_tokens(wl, B, n_d, seed + 3)
    accept = gen.accept_lengths(wl, B, seed + 4, n_d)
    logits = gen.planted_logits(wl, drafts, accept, n_d, seed + 5, gdev)
    ids = gen.block_ids(wl, B, seed + 6)

    cfg = config_for(wl, B, t_new)
    dr = Drafter(cfg, w, device, [device_cache(t, cfg, device, B) for t in ks],
                 [device_cache(t, cfg, device, B) for t in vs])
    dr.ctx_len[:B].copy_(torch.from_numpy(ctx_lens))
    feat = torch.empty(B, t_new, wl.hidden, dtype=torch.float32, device=device)
    dr.fuse_ctx([h.to(device) for h in hid], commit=False, feat_dbg=feat)
    n_acc = torch.full((B,), -7, dtype=torch.int32, device=device)
    bonus = torch.full((B,), -7, dtype=torch.int32, device=device)
    out_tok = torch.full((B, t_new), -7, dtype=torch.int32, device=device)
    dr.verify(logits.to(device), torch.from_numpy(drafts).to(device), n_d, n_d, n_acc, bonus, out_tok)
    draft_ids = torch.full((B, wl.block), -7, dtype=torch.int32, device=device)
    lg = torch.empty(B, wl.block, wl.vocab, dtype=torch.float32, device=device)
    hd = torch.empty(B, wl.block, wl.hidden, dtype=torch.float32, device=device)
    dr.draft_block(torch.from_numpy(ids).to(device), draft_ids, lg, hd)
    torch.cuda.synchronize()
    assert dr.check() == 0
    out = {"feature": feat, "n_accept": n_acc, "bonus": bonus, "tokens": out_tok, "ctx_len": dr.ctx_len.clone(),
           "stats": torch.tensor(dr.stats()), "draft_ids": draft_ids, "logits": lg, "hidden": hd}
    for l in range(wl.n_layers):
        out[f"cache K{l}"] = dr.kv_k[l].clone()
        out[f"cache V{l}"] = dr.kv_v[l].clone()
    dr.close()
    return out


def _bits(t: torch.Tensor) -> torch.Tensor:
    """The tensor's bit pattern (so NaN entries compare equal to themselves)."""
    t = t.contiguous()
    if t.is_floating_point():
        return t.view(torch.int32) if t.element_size() == 4 else t.view(torch.int16)
    return t


@pytest.mark.parametrize("name", ["tiny-f32-b1", "qwen3-8b-shape-b1", "qwen3-8b-shape-b32-ragged",
                                  "long-ctx-32k-b4", "long-ctx-32k-b4-kv8", "dflash2-27b-shape-conv-b8"])
def test_step_twice_is_bitwise_equal(name):
    wl = gen.WORKLOADS[name]
    log(f"[case] determinism {name}")
    a = _step_outputs(wl, seed=41)
    torch.cuda.empty_cache()
    b = _step_outputs(wl, seed=41)
    assert a.keys() == b.keys()
    for k in a:
        assert torch.equal(_bits(a[k]), _bits(b[k])), f"{name}: {k} differs between two runs"
    # the comparison is not vacuous: the step drafted real ids and moved the contexts
    assert int((a["draft_ids"] >= 0).sum()) == a["draft_ids"].numel()
    assert int((a["n_accept"] >= 0).sum()) == wl.batch


@pytest.mark.parametrize("name", ["tiny-f32-b1", "qwen3-8b-shape-b1"])
def test_the_comparison_sees_another_seed(name):
    # control: the same comparison tells two different inputs apart
    wl = gen.WORKLOADS[name]
    a = _step_outputs(wl, seed=41)
    b = _step_outputs(wl, seed=42)
    for k in ("feature", "logits", "hidden", "cache K0"):
        assert not torch.equal(_bits(a[k]), _bits(b[k])), f"{name}: {k} equal for two seeds"
