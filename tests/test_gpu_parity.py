"""GPU parity: the library's fuse -> verify -> draft step against the oracle.

Small cases span several tiles and ragged tails; the full-size workloads run in
the launch configuration the benchmark times and compare the sequences the
oracle computes one by one (bars in tests/gpu_cases.py).
"""

import pytest
import torch

from harness import gen
from tests.gpu_cases import run_step

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


@pytest.mark.parametrize("name,seqs", [
    ("qwen3-8b-shape-b1", [0]),
    ("qwen3-8b-shape-b32-ragged", [0, 13, 31]),
    ("long-ctx-32k-b4", [3]),
    ("dflash2-27b-shape-conv-b8", [0, 7]),
])
def test_full_size(name, seqs):
    wl = gen.WORKLOADS[name]
    run_step(wl, seed=20, seqs=seqs, poison=True)
    torch.cuda.empty_cache()
