"""GPU parity: the library's fuse -> verify -> draft step against the oracle.

Small cases span several tiles and ragged tails; the full-size workloads run in
the launch configuration the benchmark times and compare the sequences the
oracle computes one by one (bars in tests/gpu_cases.py).
"""

from dataclasses import replace

import pytest
import torch

from harness import gen
from tests.gpu_cases import run_error_paths, run_step

pytestmark = pytest.mark.gpu

TINY = gen.WORKLOADS["tiny-f32-b1"]


def test_tiny_with_prefill_through_fusion():
    run_step(TINY, seed=11, prefill=True)


def test_tiny_random_context():
    run_step(TINY, seed=12)


def test_tiny_ragged_batch_bf16_multi_split():
    # 5 sequences, contexts 0..700 (several attention splits), bf16 storage
    wl = gen.Workload("tiny-ragged", 256, 4, 2, 64, 2, 512, 1024, 8, 3, 5, 0, 700, "bf16", accept_hi=8)
    run_step(wl, seed=13, poison=True)


def test_context_sized_for_more_sequences_than_the_call():
    # a context created for 12 sequences driven with 5: workspace, partial
    # buffers and the attention plan are laid out for the larger batch
    wl = gen.Workload("tiny-ragged-under", 256, 4, 2, 64, 2, 512, 1024, 8, 3, 5, 0, 700, "bf16", accept_hi=8)
    run_step(wl, seed=27, poison=True, max_batch=12)


def test_tiny_conv_block16():
    wl = gen.Workload("tiny-conv", 256, 8, 2, 64, 2, 384, 2048, 16, 2, 3, 40, 300, "bf16", conv_width=3)
    run_step(wl, seed=14, poison=True)


def test_tiny_head128_gqa5():
    # query group 5 (80 query rows per KV head), head_dim 128, fp32 storage
    wl = gen.Workload("tiny-g5", 384, 10, 2, 128, 1, 256, 640, 16, 2, 2, 100, 600, "f32", conv_width=3)
    run_step(wl, seed=15)


def test_anchor_layout_fewer_drafts():
    # n_d = block - 1 (anchor layout): logits rows = block, fused rows = block
    run_step(TINY, seed=16, n_d=TINY.block - 1)


def test_empty_contexts():
    # no committed context at all: attention runs over the block alone
    wl = gen.Workload("tiny-empty", 256, 4, 2, 64, 2, 512, 1024, 8, 3, 3, 0, 0, "bf16", accept_hi=8)
    run_step(wl, seed=17, poison=True)


def test_full_and_zero_acceptance():
    wl = gen.Workload("tiny-accept", 256, 4, 2, 64, 2, 512, 1024, 8, 3, 4, 10, 90, "bf16", accept_hi=8)
    run_step(wl, seed=18, accept=[8, 0, 8, 0])


def test_zero_drafts_verifies_the_bonus_row_only():
    run_step(TINY, seed=19, n_d=0)


def test_device_faults_set_error_bits_and_spare_other_sequences():
    wl = gen.Workload("tiny-faults", 256, 4, 2, 64, 2, 512, 1024, 8, 3, 3, 10, 60, "bf16", accept_hi=8)
    run_error_paths(wl, seed=21)


def test_block_past_the_cache_is_flagged_and_spares_other_sequences():
    # ctx_len = max_ctx - Bs + 1: the fusion, the verify commit and the drafted block all pass max_ctx
    wl = gen.Workload("tiny-faults-draft", 256, 4, 2, 64, 2, 512, 1024, 8, 3, 3, 10, 60, "bf16", accept_hi=8)
    run_error_paths(wl, seed=22, draft_overflow=True)


def test_many_equal_sequences_one_attention_piece_each():
    # 128 sequences x 2 KV heads: attention planned on the device, one balanced
    # piece per segment
    wl = gen.Workload("tiny-b128-equal", 256, 4, 2, 64, 2, 512, 1024, 8, 3, 128, 100, 100, "bf16", accept_hi=8)
    run_step(wl, seed=23, seqs=[0, 77, 127], poison=True)


def test_many_ragged_sequences_flattened_attention():
    # 160 ragged sequences: the key axis of the batch cut into equal ranges,
    # workgroups crossing segment ends
    wl = gen.Workload("tiny-b160-ragged", 256, 4, 2, 64, 2, 512, 1024, 8, 3, 160, 0, 300, "bf16", accept_hi=8)
    run_step(wl, seed=24, seqs=[0, 51, 159], poison=True)


def test_half_filled_last_row_group_in_fragment_blocks():
    # 17 sequences x block 8 = 136 draft rows: the products run on 256-row
    # LDS-DMA blocks and the normalised residual is stored in 16-row fragment
    # blocks, the last of them half filled (rows past the batch never stored)
    wl = gen.Workload("tiny-b17-block8", 256, 4, 2, 64, 2, 512, 1024, 8, 3, 17, 0, 300, "bf16", accept_hi=8)
    run_step(wl, seed=28, poison=True)


def test_full_size_silu_epilogue_with_a_partial_row_block():
    # 17 sequences at the Qwen3-8B shape (272 draft rows): gate/up computes the
    # SiLU product in its epilogue over two 256-row blocks, the second holding
    # 16 rows; the row scales come from the sums of squares inside that kernel
    wl = gen.WORKLOADS["qwen3-8b-shape-b32-ragged"].with_batch(17)
    run_step(wl, seed=30, seqs=[0, 16], poison=True, min_sure=0.25)
    torch.cuda.empty_cache()


def test_full_size_block8_odd_rows_on_every_dma_path():
    # 35 sequences x block 8 = 280 draft rows at the Qwen3-8B shape: gate/up
    # with the SiLU epilogue over two 256-row blocks (24 rows in the second),
    # the other products on 192-row blocks, and the normalised residual in
    # fragment blocks whose last 16-row group holds 8 rows
    wl = replace(gen.WORKLOADS["qwen3-8b-shape-b32-ragged"], name="qwen3-8b-shape-b35-block8", block=8, batch=35)
    run_step(wl, seed=31, seqs=[0, 34], poison=True, min_sure=0.25)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("storage", ["bf16", "f32"])
def test_batch1_finishes_split_k_slices_over_lanes(storage):
    # one sequence, hidden 1024: every product runs 4 or 8 k-slices over a grid
    # smaller than the chip, so the finishes share each output quad among 4 lanes
    # (the residual finish with the block conv included)
    wl = gen.Workload("tiny-b1-split", 1024, 8, 2, 128, 2, 2048, 1024, 16, 2, 1, 40, 300, storage, conv_width=3)
    run_step(wl, seed=25, poison=True)


def test_reload_weights_after_in_place_change():
    # The products stream the tiled copy made at create.  After the caller
    # changes matrices in place the old copy stays in use until
    # dflash_reload_weights; then the draft equals that of a context created
    # on the changed weights, bit for bit.
    from block_diffusion_drafting_ctx_amd import Drafter
    from tests.gpu_cases import config_for

    wl = gen.Workload("tiny-reload", 256, 4, 2, 64, 2, 512, 1024, 8, 3, 2, 10, 20, "bf16")
    w = gen.draft_weights(wl, 41, "cuda")
    ctx_lens = gen.context_lengths(wl, 42, 2)
    ks, vs = gen.context_kv(wl, ctx_lens, 42, "cuda")
    ids = torch.from_numpy(gen.block_ids(wl, 2, 43)).cuda()
    cfg = config_for(wl, 2)

    def draft(dr):
        dr.ctx_len.copy_(torch.from_numpy(ctx_lens).cuda())
        out = torch.zeros(2, wl.block, dtype=torch.int32, device="cuda")
        lg = torch.empty(2, wl.block, wl.vocab, dtype=torch.float32, device="cuda")
        dr.draft_block(ids, out, lg)
        torch.cuda.synchronize()
        assert dr.check() == 0
        return out.clone(), lg.clone()

    dr = Drafter(cfg, w, "cuda", [k.clone() for k in ks], [v.clone() for v in vs])
    before = draft(dr)
    w["w_lm"].mul_(-1.0)
    w["layers"][1]["w_up"].mul_(0.5)
    stale = draft(dr)
    dr.reload_weights()
    after = draft(dr)
    fresh = Drafter(cfg, w, "cuda", [k.clone() for k in ks], [v.clone() for v in vs])
    ref = draft(fresh)
    assert torch.equal(stale[1], before[1])
    assert torch.equal(after[1], ref[1]) and torch.equal(after[0], ref[0])
    assert not torch.equal(after[1], before[1])
    dr.close()
    fresh.close()


def test_host_checks_reject_bad_sizes():
    from block_diffusion_drafting_ctx_amd import Drafter, _abi
    from tests.gpu_cases import config_for

    wl = gen.Workload("tiny-host", 256, 4, 2, 64, 2, 512, 1024, 8, 3, 2, 10, 20, "bf16")
    w = {k: v for k, v in gen.draft_weights(wl, 3, "cuda").items()}
    dr = Drafter(config_for(wl, 2), w, "cuda")
    H, V = wl.hidden, wl.vocab
    too_many = [torch.zeros(3, wl.t_new, H, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    too_long = [torch.zeros(2, wl.t_new + 1, H, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    for hid in (too_many, too_long):
        with pytest.raises(_abi.DFlashError):
            dr.fuse_ctx(hid, commit=False)
    i32 = lambda *s: torch.zeros(*s, dtype=torch.int32, device="cuda")  # noqa: E731
    lg = torch.zeros(2, 66, V, dtype=torch.float32, device="cuda")
    with pytest.raises(_abi.DFlashError):  # n_d above 64
        dr.verify(lg, i32(2, 65), 65, 65, i32(2), i32(2), i32(2, 66))
    with pytest.raises(_abi.DFlashError):  # batch above max_batch
        dr.draft_block(i32(3, wl.block), i32(3, wl.block))
    # batch 0 is a no-op
    dr.draft_block(i32(0, wl.block), i32(0, wl.block))
    torch.cuda.synchronize()
    assert dr.check() == 0
    dr.close()


@pytest.mark.parametrize("storage,kv_conv", [("bf16", 0), ("f32", 0), ("bf16", 3)])
def test_int8_kv_cache_ragged(storage, kv_conv):
    # the 8-bit cache: pre-filled rows as (values, scales), NaN scales past
    # the contexts; fused and staged rows quantised by the library; attention
    # dequantises.  Several attention splits, ragged contexts, every sequence.
    wl = gen.Workload("tiny-kv8", 256, 4, 2, 64, 2, 512, 1024, 8, 3, 5, 0, 700, storage, conv_width=kv_conv,
                      accept_hi=8, kv="int8")
    run_step(wl, seed=26, poison=True)


def test_int8_kv_cache_head128_planned_attention():
    # head_dim 128 (4 runs of 32 per row), 72 sequences x 2 KV heads: attention planned on the device
    wl = gen.Workload("tiny-kv8-h128", 512, 8, 2, 128, 1, 512, 1024, 16, 2, 72, 0, 400, "bf16", kv="int8")
    run_step(wl, seed=28, seqs=[0, 35, 71], poison=True)


def test_int8_kv_cache_through_prefill():
    wl = gen.Workload("tiny-kv8-pre", 256, 4, 2, 64, 2, 512, 1024, 8, 3, 1, 64, 64, "f32", accept_hi=8,
                      scaled_hidden=False, kv="int8")
    run_step(wl, seed=29, prefill=True)


@pytest.mark.parametrize("name,seqs", [
    ("qwen3-8b-shape-b1", [0]),
    ("qwen3-8b-shape-b32-ragged", [0, 13, 31]),
    ("long-ctx-32k-b4", [3]),
    ("dflash2-27b-shape-conv-b8", [0, 7]),
    ("qwen3-8b-shape-b1-kv8", [0]),
    ("long-ctx-32k-b4-kv8", [1]),
])
def test_full_size(name, seqs):
    # at these widths about 70% of the draft rows clear the 0.1 margin; a
    # quarter is the floor below which the exact comparison would say little
    wl = gen.WORKLOADS[name]
    run_step(wl, seed=20, seqs=seqs, poison=True, min_sure=0.25)
    torch.cuda.empty_cache()
