"""Benchmark: draft+verify block-tokens/s of one fuse -> verify -> draft step.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step = reset of the context lengths (so every step sees the same
workload), dflash_fuse_ctx of the n_d+1 verified target rows (speculative),
dflash_verify against planted target logits, and dflash_draft_block of one
block per sequence -- every stage of the hot path, on inputs already resident
in HBM.  value = batch * block / step time.

Also reported: the achieved HBM bandwidth of the kernel that takes most of
the batch-1 step -- the weight-streaming main kernel of the layer products
(Q/K/V, O, gate/up, down; their algorithmic bytes over their launch times
from HIP events recorded around every such launch inside the timed region)
-- against the MI355X peak; a per-stage table from a separate pass with
events around every stage; and the float64 numpy oracle timed on the host
cores on a bounded sample of the same step.  Secondary lines of the same JSON
object cover the batch-32 ragged, 32k-context and 27B-shaped workloads.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "draft+verify block-tokens/sec at batch 1/32; % HBM / MFMA roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3-8b-shape-b1")
    ap.add_argument("--secondary", default="qwen3-8b-shape-b32-ragged,long-ctx-32k-b4,long-ctx-32k-b4-kv8,"
                                           "dflash2-27b-shape-conv-b8",
                    help="comma-separated extra workloads reported under 'secondary' ('' for none)")
    ap.add_argument("--prefill", default="qwen3-8b-shape-b1:4096:4096",
                    help="WORKLOAD:ROWS:CHUNK -- also time prompt-scale fusion of ROWS prompt rows per sequence "
                         "in chunks of CHUNK, reported under 'prefill' ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-verify-modes", dest="verify_modes", action="store_false",
                    help="skip timing greedy vs sampling-mode verification (reported under 'verify_modes')")
    ap.add_argument("--stage", default="layer_gemm", help="kernel stage timed with HIP events for the roofline")
    ap.add_argument("--no-stage-table", dest="stage_table", action="store_false",
                    help="skip the separate pass that times every stage with HIP events")
    ap.add_argument("--eager", action="store_true",
                    help="eager launches only (skip the timed HIP-graph replay pass)")
    ap.add_argument("--graph", action="store_true",
                    help="report the HIP-graph replays of the captured step as the headline instead of the "
                         "eager launches")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run one device-to-device copy of this many MiB (the known-size kernel "
                         "that scales rocprofv3 FETCH_SIZE / WRITE_SIZE counts)")
    return ap.parse_args()


def stage_bytes(wl, batch, ctx_lens):
    """Algorithmic HBM bytes per launch of each stage (weights once, inputs and outputs once)."""
    S = 2 if wl.storage == "bf16" else 4
    KV = 1 + 4 / 32 if wl.kv == "int8" else S  # bytes per cache entry (8-bit: value + its share of a run scale)
    H, D, F, V = wl.hidden, wl.head_dim, wl.ffn, wl.vocab
    Nq, Nk = wl.n_q_heads * D, wl.n_kv_heads * D
    Md, Mf = batch * wl.block, batch * wl.t_new
    act = 4  # activations move as hi/lo bf16 pairs (or fp32)
    ctx = float(np.sum(ctx_lens))
    b = {
        "fuse_fc": H * wl.n_target_layers * H * S + Mf * wl.n_target_layers * H * S + Mf * H * (4 + act),
        "ctx_kv": wl.n_layers * 2 * Nk * H * S + Mf * H * act + wl.n_layers * 2 * Mf * Nk * KV,
        "verify": Mf * V * 4,
        "embed": Md * H * S + Md * H * (4 + act),
        "qkv": (Nq + 2 * Nk) * H * S + Md * H * act + Md * (Nq * act + 2 * Nk * KV),
        "attn": (ctx + Md) * 2 * Nk * KV + Md * Nq * 2 * act,
        "oproj": H * Nq * S + Md * Nq * act + Md * H * (8 + act),
        "gateup": 2 * F * H * S + Md * H * act + Md * F * act,
        "down": H * F * S + Md * F * act + Md * H * (8 + act),
        "lmhead": V * H * S + Md * H * act,
    }
    return b


def layer_gemm_bytes(wl, batch):
    """Algorithmic bytes of one step's layer-product main kernels: weights once,
    the activation rows read once, the fp32 product written once."""
    S = 2 if wl.storage == "bf16" else 4
    H, F = wl.hidden, wl.ffn
    Nq, Nk = wl.n_q_heads * wl.head_dim, wl.n_kv_heads * wl.head_dim
    Md = batch * wl.block
    act = 4
    per_layer = ((Nq + 2 * Nk) * H + H * Nq + 2 * F * H + H * F) * S \
        + Md * (H + Nq + H + F) * act + Md * ((Nq + 2 * Nk) + H + 2 * F + H) * 4
    return wl.n_layers * per_layer, 4 * wl.n_layers


def stage_flops(wl, batch, ctx_lens):
    H, D, F, V = wl.hidden, wl.head_dim, wl.ffn, wl.vocab
    Nq, Nk = wl.n_q_heads * D, wl.n_kv_heads * D
    Md, Mf = batch * wl.block, batch * wl.t_new
    ctx = float(np.sum(ctx_lens))
    return {
        "fuse_fc": 2.0 * Mf * wl.n_target_layers * H * H,
        "ctx_kv": 2.0 * Mf * H * wl.n_layers * 2 * Nk,
        "qkv": 2.0 * Md * H * (Nq + 2 * Nk),
        "attn": 4.0 * wl.block * wl.n_q_heads * D * (ctx + batch * wl.block),
        "oproj": 2.0 * Md * Nq * H,
        "gateup": 4.0 * Md * H * F,
        "down": 2.0 * Md * F * H,
        "lmhead": 2.0 * Md * H * V,
        "layer_gemm": 2.0 * Md * H * (Nq + 2 * Nk + 3 * F) + 2.0 * Md * Nq * H,
    }


PER_LAYER = ("qkv", "attn", "oproj", "gateup", "down", "layer_gemm")
STEP_STAGES = ("fuse_fc", "ctx_kv", "verify", "embed", "qkv", "attn", "oproj", "gateup", "down", "lmhead")


def step_totals(wl, batch, ctx_lens):
    sb, sf = stage_bytes(wl, batch, ctx_lens), stage_flops(wl, batch, ctx_lens)
    tb = sum(v * (wl.n_layers if k in PER_LAYER else 1) for k, v in sb.items() if k in STEP_STAGES)
    tf = sum(v * (wl.n_layers if k in PER_LAYER else 1) for k, v in sf.items() if k in STEP_STAGES)
    return tb, tf


def stage_launch_bytes(wl, batch, ctx_lens, stage):
    """Algorithmic bytes of one launch of a timed stage (the layer products:
    their mean over the four products of a layer)."""
    if stage == "layer_gemm":
        tot, launches = layer_gemm_bytes(wl, batch)
        return tot / launches
    return stage_bytes(wl, batch, ctx_lens)[stage]


def stage_table(wb, steps):
    """Every stage timed with HIP events around its launches over `steps` more
    steps (a separate pass: the events perturb the step).  Per stage: mean
    launch ms, launches per step, algorithmic GB/s and TFLOP/s, and the
    fractions of the HBM and bf16 peaks."""
    import torch
    from block_diffusion_drafting_ctx_amd import _abi

    wl = wb.wl
    for s in _abi.STAGES:
        _abi.dflash_stage_timing(wb.dr.ctx, s, True)
    for _ in range(steps):
        wb.step()
    torch.cuda.synchronize()
    sf = stage_flops(wl, wl.batch, wb.ctx_lens)
    out = {}
    for s in _abi.STAGES:
        mean_ms, n = _abi.dflash_stage_time(wb.dr.ctx, s)
        _abi.dflash_stage_timing(wb.dr.ctx, s, False)
        if n == 0:
            continue
        nb = stage_launch_bytes(wl, wl.batch, wb.ctx_lens, s)
        fl = sf.get(s, 0.0) / (4 if s == "layer_gemm" else 1)  # (its flops are per layer: 4 launches)
        gbs = nb / (mean_ms * 1e-3) / 1e9
        tfs = fl / (mean_ms * 1e-3) / 1e12
        out[s] = {"mean_ms": round(mean_ms, 5), "per_step": round(n / steps, 2), "gb_s": round(gbs, 1),
                  "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "tflop_s": round(tfs, 1),
                  "mfma_frac": round(tfs / BF16_PEAK_TFLOPS, 4)}
    assert wb.dr.check() == 0
    return out


def source_hash() -> str:
    h = hashlib.sha256()
    for f in ("gemm.hip", "common.h", "kernels.h"):
        with open(os.path.join(ROOT, "block_diffusion_drafting_ctx_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(stage, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match the current source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{stage}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_hash") != source_hash():
        return None
    return rec.get("bytes_per_launch")


class Workbench:
    """Resident inputs and a library context for one workload."""

    def __init__(self, wl, seed=1):
        import torch
        from harness import gen
        from block_diffusion_drafting_ctx_amd import Drafter, make_config

        self.wl = wl
        dev = "cuda"
        B = wl.batch
        self.ctx_lens = gen.context_lengths(wl, seed + 1, B)
        self.w = gen.draft_weights(wl, seed, dev)
        ks, vs = gen.context_kv(wl, self.ctx_lens, seed + 1, dev)
        cfg = make_config(wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.n_layers, wl.ffn, wl.vocab,
                          wl.block, wl.n_target_layers, B, wl.max_ctx, wl.t_new, wl.conv_width, wl.storage,
                          wl.rms_eps, wl.rope_theta, wl.kv)
        if wl.kv == "int8":  # (values, run scales) pairs -> the library's raw 8-bit cache buffers
            from block_diffusion_drafting_ctx_amd import kv8_buffer

            ks = [kv8_buffer(q, sc, cfg) for q, sc in ks]
            vs = [kv8_buffer(q, sc, cfg) for q, sc in vs]
        self.dr = Drafter(cfg, self.w, dev, ks, vs)
        self.ctx0 = torch.from_numpy(self.ctx_lens).to(dev)
        self.dr.ctx_len.copy_(self.ctx0)
        self.hidden = gen.target_hidden(wl, B, wl.t_new, seed + 2, dev)
        self.block_ids = torch.from_numpy(gen.block_ids(wl, B, seed + 6)).to(dev)
        self.draft_ids = torch.zeros(B, wl.block, dtype=torch.int32, device=dev)  # draft output
        self.n_acc = torch.zeros(B, dtype=torch.int32, device=dev)
        self.bonus = torch.zeros(B, dtype=torch.int32, device=dev)
        self.out_tok = torch.zeros(B, wl.t_new, dtype=torch.int32, device=dev)
        # The block verified each step is the one drafted by an untimed first
        # pass; the target logits plant the chosen acceptance lengths against it.
        # Each step therefore commits the same rows and drafts from the same
        # context, so every step does identical work.
        self.verify_ids = torch.zeros(B, wl.block, dtype=torch.int32, device=dev)
        self.dr.draft_block(self.block_ids, self.verify_ids)
        torch.cuda.synchronize()
        self.accept = gen.accept_lengths(wl, B, seed + 4)
        self.logits = gen.planted_logits(wl, self.verify_ids.cpu().numpy(), self.accept, wl.n_d, seed + 5, dev)

    def step(self):
        wl = self.wl
        self.dr.ctx_len.copy_(self.ctx0)
        self.dr.fuse_ctx(self.hidden, commit=False)
        self.dr.verify(self.logits, self.verify_ids, wl.block, wl.n_d, self.n_acc, self.bonus, self.out_tok)
        self.dr.draft_block(self.block_ids, self.draft_ids)


def time_workload(wl, steps, warmup, stage, graph_pass=True, graph_headline=False):
    """Time `steps` steps; returns (workbench, ms per step, {stage: (mean launch ms, launches)}).

    The headline pass enqueues the step's kernels one by one on the stream
    (no host synchronisation inside the timed region); a second timed pass of
    the same steps records HIP events around every launch of the roofline's
    stage (wb.ms_events).  With graph_pass the step is then captured once into a
    HIP graph and `steps` replays are timed as well (wb.ms_graph);
    graph_headline reports those instead.  (Measured here, the replays are
    2-3% slower: the weight-streaming products run 3-6% longer inside a graph
    while every other kernel takes the same time.)"""
    import torch
    from block_diffusion_drafting_ctx_amd import _abi

    wb = Workbench(wl)
    for _ in range(warmup):
        wb.step()
    torch.cuda.synchronize()
    err = wb.dr.check()
    if err:
        raise RuntimeError(f"device error word {err:#x}")
    stages = [stage]

    def timed(run):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms_eager = timed(wb.step)
    # The roofline kernel's launches are bracketed by HIP events in a second
    # timed pass of the same steps: each recorded event costs a few
    # microseconds of queue time, which would otherwise inflate the headline
    # (20 bracketed launches per batch-1 step add ~0.12 ms).
    for s in stages:
        _abi.dflash_stage_timing(wb.dr.ctx, s, True)
    wb.ms_events = timed(wb.step)
    per_stage = {}
    for s in stages:
        mean_ms, n = _abi.dflash_stage_time(wb.dr.ctx, s)
        _abi.dflash_stage_timing(wb.dr.ctx, s, False)
        per_stage[s] = (mean_ms, n)
    wb.ms_graph = None
    if graph_pass or graph_headline:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                wb.step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for _ in range(max(2, warmup)):
            g.replay()
        wb.ms_graph = timed(g.replay)
        wb.graph = g
    assert wb.dr.check() == 0
    n_acc = wb.n_acc.cpu().numpy()
    if not np.array_equal(n_acc, wb.accept):
        raise RuntimeError(f"planted acceptance not reproduced: {n_acc} vs {wb.accept}")
    wb.ms_eager = ms_eager
    ms = wb.ms_graph if graph_headline else ms_eager
    return wb, ms, per_stage


def time_prefill(wl, rows, chunk, steps, warmup):
    """Prompt-scale fusion: `rows` prompt rows of every sequence fused with
    commit in chunks of `chunk` rows (how a caller fills the draft cache from
    the target's prompt pass).  Returns ms per prompt and its algorithmic flops."""
    import torch
    from block_diffusion_drafting_ctx_amd import Drafter, make_config
    from harness import gen

    B = wl.batch
    w = gen.draft_weights(wl, 1, "cuda")
    max_ctx = ((rows + 2 * (wl.block + 1) + 63) // 64) * 64
    cfg = make_config(wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.n_layers, wl.ffn, wl.vocab,
                      wl.block, wl.n_target_layers, B, max_ctx, chunk, wl.conv_width, wl.storage,
                      wl.rms_eps, wl.rope_theta)
    dr = Drafter(cfg, w, "cuda")
    hidden = gen.target_hidden(wl, B, rows, 3, "cuda")
    parts = [[h[:, r0:min(rows, r0 + chunk)].contiguous() for h in hidden] for r0 in range(0, rows, chunk)]
    del hidden

    def prompt():
        dr.ctx_len.zero_()
        for p in parts:
            dr.fuse_ctx(p, commit=True)

    for _ in range(warmup):
        prompt()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        prompt()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    assert dr.check() == 0 and dr.ctx_len.cpu().tolist() == [rows] * B
    H, Nk = wl.hidden, wl.n_kv_heads * wl.head_dim
    flops = 2.0 * B * rows * H * (wl.n_target_layers * H + wl.n_layers * 2 * Nk)
    dr.close()
    return ms, flops


def time_verify_modes(wb, calls, temperature=1.0):
    """Greedy and sampling-mode verification of the workbench's resident target
    logits, `calls` launches of each (each after the same context-length reset),
    timed by the library's HIP events around the verify stage.  Returns
    {mode: mean ms per launch} and the logits bytes one launch reads."""
    import torch
    from block_diffusion_drafting_ctx_amd import _abi

    wl, dr = wb.wl, wb.dr
    g = torch.Generator(device="cuda").manual_seed(11)
    u = torch.rand(wl.batch, wl.n_d + 1, 2, generator=g, device="cuda")
    runs = {
        "greedy": lambda: dr.verify(wb.logits, wb.verify_ids, wl.block, wl.n_d, wb.n_acc, wb.bonus, wb.out_tok),
        "sample": lambda: dr.verify_sample(wb.logits, wb.verify_ids, wl.block, wl.n_d, temperature, u, wb.n_acc,
                                           wb.bonus, wb.out_tok),
    }
    out = {}
    for mode, run in runs.items():
        for _ in range(3):
            dr.ctx_len.copy_(wb.ctx0)
            run()
        torch.cuda.synchronize()
        _abi.dflash_stage_timing(dr.ctx, "verify", True)
        for _ in range(calls):
            dr.ctx_len.copy_(wb.ctx0)
            run()
        torch.cuda.synchronize()
        out[mode] = _abi.dflash_stage_time(dr.ctx, "verify")[0]
        _abi.dflash_stage_timing(dr.ctx, "verify", False)
    assert dr.check() == 0
    return out, wl.batch * (wl.n_d + 1) * wl.vocab * 4


def cpu_baseline(wb, min_seconds=10.0, max_steps=60):
    """The oracle, as it stands, on full steps of the workload's first sequence.

    The step (fuse the verified rows, verify, draft one block) is repeated
    from copies of the same state (copies untimed) until about `min_seconds`
    of timed CPU work have run."""
    import threadpoolctl
    from oracle import DraftState, draft_block, fuse_ctx, verify_step
    from tests.oracle_adapt import dims_of, np64, weights_of

    wl = wb.wl
    W = weights_of(wb.w)
    dims = dims_of(wl)
    b = 0
    T = int(wb.ctx_lens[b])
    base = DraftState(k=[np64(t[b:b + 1, :T + wl.t_new]) for t in wb.dr.kv_k],
                      v=[np64(t[b:b + 1, :T + wl.t_new]) for t in wb.dr.kv_v],
                      ctx_len=np.array([T], dtype=np.int64))
    hid = [np64(h[b:b + 1]) for h in wb.hidden]
    logits = wb.logits[b:b + 1].cpu().numpy()
    drafts = wb.verify_ids[b:b + 1].cpu().numpy().reshape(-1)
    ids = wb.block_ids[b:b + 1].cpu().numpy()
    info = threadpoolctl.threadpool_info()
    blas = [i for i in info if i.get("user_api") == "blas"]
    threads = max([i.get("num_threads", 1) for i in blas] or [1])
    blas_desc = ", ".join(f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)"
                          for i in blas) or "none found"
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    total, steps = 0.0, 0
    while total < min_seconds and steps < max_steps:
        st = DraftState(k=[x.copy() for x in base.k], v=[x.copy() for x in base.v], ctx_len=base.ctx_len.copy())
        t0 = time.perf_counter()
        fuse_ctx(st, W, dims, hid, commit=False)
        verify_step(st, logits, drafts, wl.block, wl.n_d)
        draft_block(st, W, dims, ids)
        total += time.perf_counter() - t0
        steps += 1
    return {"value": round(steps * wl.block / total, 3), "unit": "block-tokens/s", "cores": int(threads),
            "kind": "oracle", "precision": "float64 (the oracle's own arithmetic, not tuned)",
            "cpu_model": cpu_model, "blas": blas_desc, "host_cpus": os.cpu_count(),
            "sample": f"{steps} full steps of sequence 0 of {wl.name}, each from the same state (fuse {wl.t_new} "
                      f"rows, verify, draft of one {wl.block}-row block through {wl.n_layers} layers and the full "
                      f"vocabulary), float64 numpy",
            "seconds": round(total, 3)}


def secondary_line(wl, args):
    """One secondary workload: its step time, the step's roofline fractions,
    the LM head's and attention's rates, and its stage table."""
    import torch

    wb, ms, ps = time_workload(wl, max(5, args.steps // 2), args.warmup, "lmhead",
                               graph_pass=not args.eager, graph_headline=args.graph)
    tb, tf = step_totals(wl, wl.batch, wb.ctx_lens)
    sf = stage_flops(wl, wl.batch, wb.ctx_lens)
    line = {"workload": wl.name, "batch": wl.batch, "context": int(np.max(wb.ctx_lens)),
            "value": round(wl.batch * wl.block / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
            "ms_per_step_graph": None if wb.ms_graph is None else round(wb.ms_graph, 4),
            "step_mfma_frac": round(tf / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4),
            "step_hbm_frac": round(tb / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
            "lmhead_tflops": round(sf["lmhead"] / (ps["lmhead"][0] * 1e-3) / 1e12, 1)}
    if args.stage_table:
        tab = stage_table(wb, max(5, args.steps // 4))
        line["attn_hbm_frac"] = tab["attn"]["hbm_frac"]
        line["stages"] = tab
    return wb, line


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; pass --gpus 1 "
                                   "(the sharded design is described, not built)"}))
        sys.exit(2)
    import torch
    from harness import gen

    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    wl = gen.WORKLOADS[args.workload]
    wb, ms, per_stage = time_workload(wl, args.steps, args.warmup, args.stage,
                                      graph_pass=not args.eager, graph_headline=args.graph)
    B = wl.batch
    value = B * wl.block / (ms * 1e-3)
    tb, tf = step_totals(wl, B, wb.ctx_lens)
    mean_ms, n = per_stage[args.stage]
    nb = stage_launch_bytes(wl, B, wb.ctx_lens, args.stage)
    achieved = nb / (mean_ms * 1e-3) / 1e9
    kernel_desc = {"layer_gemm": "weight-streaming main kernel of the layer products (Q/K/V, O, gate/up, down; "
                                 "finish kernels excluded)",
                   "lmhead": "LM head with per-tile argmax"}.get(args.stage, args.stage)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "block-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.storage,
        "data": "synthetic (seeded random-init draft weights and inputs)",
        "config": {"workload": wl.name, "batch": B, "block": wl.block, "context": int(np.max(wb.ctx_lens)),
                   "layers": wl.n_layers, "hidden": wl.hidden, "vocab": wl.vocab,
                   "launch": "hip-graph replay of the whole step" if args.graph else
                   "eager (the step's kernels enqueued one by one, no host sync inside the timed region)"},
        "roofline": {"bound": "hbm", "kernel": args.stage, "kernel_desc": kernel_desc, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profiles(args.stage, wl.name),
                     "algorithmic_bytes_per_launch": int(nb), "mean_launch_ms": round(mean_ms, 5),
                     "launches": n, "timed_pass_ms_per_step": round(wb.ms_events, 4)},
        "step_roofline": {"algorithmic_bytes": int(tb), "algorithmic_flops": int(tf),
                          "hbm_frac": round(tb / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
                          "mfma_frac": round(tf / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4)},
    }
    if wb.ms_graph is not None:
        out["ms_per_step_graph"] = round(wb.ms_graph, 4)
    if args.stage_table:
        out["stages"] = stage_table(wb, max(10, args.steps // 2))
    vm = {}
    if args.verify_modes:
        vm[wl.name] = time_verify_modes(wb, max(20, args.steps))
    sec = []
    for name in [s for s in args.secondary.split(",") if s]:
        wl2 = gen.WORKLOADS[name]
        del wb
        torch.cuda.empty_cache()
        print(f"[bench] secondary {name}", file=sys.stderr, flush=True)
        wb, line = secondary_line(wl2, args)
        sec.append(line)
        if args.verify_modes and wl2.batch > 1 and name.startswith("qwen3"):
            vm[name] = time_verify_modes(wb, max(20, args.steps))
    if sec:
        out["secondary"] = sec
    if vm:
        out["verify_modes"] = [
            {"workload": name, "temperature": 1.0,
             **{f"{m}_ms": round(t, 5) for m, t in times.items()},
             **{f"{m}_hbm_frac": round(nb_ / (t * 1e-3) / (HBM_PEAK_GBS * 1e9), 4) for m, t in times.items()}}
            for name, (times, nb_) in vm.items()]
    if args.prefill:
        pname, prows, pchunk = args.prefill.split(":")
        wl3 = gen.WORKLOADS[pname]
        del wb
        torch.cuda.empty_cache()
        print("[bench] prompt fusion", file=sys.stderr, flush=True)
        pms, pfl = time_prefill(wl3, int(prows), int(pchunk), max(3, args.steps // 10), 2)
        out["prefill"] = {"workload": f"{pname}: {wl3.batch} x {int(prows)} prompt rows fused in chunks of {pchunk}",
                          "prompt_rows_per_s": round(wl3.batch * int(prows) / (pms * 1e-3), 1),
                          "ms_per_prompt": round(pms, 4),
                          "mfma_frac": round(pfl / (pms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4)}
        torch.cuda.empty_cache()
        wb = None
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = n
        del src, dst
    if not args.no_cpu_baseline:
        wb_c = wb if wb is not None and wb.wl.name == wl.name else None
        if wb_c is None:
            del wb
            torch.cuda.empty_cache()
            wb_c = Workbench(wl)
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wb_c)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
