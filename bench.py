#!/usr/bin/env python3
"""Benchmark of the quantized-resident projection GEMM on one MI355X.

A step is one pass of the whole path over every projection of the 12 RT-J
blocks (rtq_block_project with n_blocks = 12), with the packed weights and the
activations already resident in HBM.

Workloads (synthetic, seeded; shapes of the "Backends" page, section "Meta"):
  m80    M = 80 (the golden batch B=5, S=16 of the int4 card, "Accuracy"):
         12 blocks x 16 independently seeded weight sets (630 MB of packed
         weights, more than the 256 MB MALL); step c uses set c mod 16; each
         block reads its own four fp32 activations.
  m65536 M = 65536 (256 contexts x 256 cells), one weight set, four fp32
         activations shared by the blocks, distinct outputs per block.

Prints one JSON line. `value` is dequant-GEMM TFLOP/s (2*M*N*K per
projection) on the m80 workload; the m65536 figures ride along under
"m65536". The lower-precision bf16-activation mode (x rounded to bf16) is
timed on both workloads and reported apart, under "bf16_activation_path".
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_FP32_MFMA_TFLOPS = 157.3      # MI355X dense fp32 matrix
PEAK_BF16_MFMA_TFLOPS = 2516.6     # MI355X dense bf16 matrix
WEIGHT_SETS = 16
KERNELS = {  # main GEMM kernel of each (math, workload), as rocprofv3 names it
    ("split16", "m80"): "split_grouped_kernel<5, 2>",
    ("split16", "m65536"): "split_gemm_kernel<1|2, 2>",
    ("split", "m80"): "split_grouped_kernel<5, 3>",
    ("split", "m65536"): "split_gemm_kernel<1|2, 3>",
    ("bf16", "m80"): "split_grouped_kernel<5, 1>",
    ("bf16", "m65536"): "split_gemm_kernel<1|2, 1>",
    ("fp32", "m80"): "grouped_stream_kernel<5>",
    ("fp32", "m65536"): "gemm_kernel<1|2,2,2,4,4>",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000, help="timed steps of the m80 workload")
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--steps-large", type=int, default=10, help="timed steps of the m65536 workload")
    ap.add_argument("--warmup-large", type=int, default=2)
    ap.add_argument("--workload", choices=["m80", "m65536", "both"], default="both")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--recipe", choices=["mixed", "all_q8", "all_f8"], default="mixed",
                    help="weight formats: the int4 card's mixed int4/int8 recipe (default), the int8 card's "
                         "all-int8 recipe, or the FP8 card's all-E4M3 weights")
    ap.add_argument("--math", choices=["split16", "split", "fp32", "bf16"], default="split16",
                    help="GEMM arithmetic: row-scaled activations in two fp16 limbs on the fp16 MFMA (default), "
                         "the exact bf16x3 split on the bf16 MFMA, fp32 MFMA, or activations rounded to bf16 "
                         "(lower precision)")
    ap.add_argument("--no-bf16-path", action="store_true",
                    help="skip the separately reported bf16-activation timing")
    ap.add_argument("--no-exact-path", action="store_true",
                    help="skip the separately reported exact bf16x3 timing (with --math split16)")
    ap.add_argument("--compare-fp32", action="store_true",
                    help="also time the fp32-MFMA path (few steps) and report it alongside")
    ap.add_argument("--m-sweep", default=None,
                    help="M values of the diagnostic sweep on the m80 weight sets (default with --workload both: "
                         "1,2,4,8,16,32,48,80; '' to skip; given explicitly it runs with any workload)")
    ap.add_argument("--bias", action="store_true",
                    help="give every projection an fp32 bias (y = x.W^T + b) to time the bias epilogue")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-attainable", action="store_true",
                    help="skip the measured ceilings (streaming read, matrix-instruction loop)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the single-GEMM and one-block configurations (config_cases)")
    return ap.parse_args()


RECIPES = ("mixed", "all_q8", "all_f8")


def recipe_map(name):
    import weight_only_quantized_rtq_amd as rtq
    return {"mixed": rtq.RECIPE_MIXED, "all_q8": rtq.RECIPE_ALL_Q8, "all_f8": rtq.RECIPE_ALL_F8}[name]


def block_bytes_flops(M, recipe="mixed"):
    """Packed weight bytes and GEMM flops of one RT-J block: int4 0.5 B codes +
    4 B (scale, min) per 32; int8 1 B codes + 4 B scale per row; FP8 1 B codes."""
    import synth
    rec = recipe_map(recipe)
    wbytes = 0
    flops = 0
    for name in synth.PROJ_ORDER:
        N, K, _ = synth.BLOCK_SHAPES[name]
        if rec[name] == "q4":
            wbytes += N * K // 2 + N * (K // 32) * 4
        elif rec[name] == "q8":
            wbytes += N * K + N * 4
        else:
            wbytes += N * K
        flops += 2 * M * N * K
    return wbytes, flops


BIAS = False


def build_sets(torch, rtq, synth, cfg, M, n_sets, xs_per_block, heavy=None, recipe="mixed"):
    """Packed weights (quantized on the GPU) for n_sets x 12 blocks, plus inputs
    and outputs, and the host descriptor arrays of each set."""
    dev = "cuda:0"
    nb = synth.NUM_BLOCKS
    if xs_per_block:
        xs = [{n: torch.from_numpy(synth.activation(cfg, b, n, M)).to(dev) for n in synth.INPUT_WIDTH}
              for b in range(nb)]
    else:
        shared = {n: torch.from_numpy(synth.activation(cfg, synth.SHARED_BLOCK, n, M)).to(dev)
                  for n in synth.INPUT_WIDTH}
        xs = [shared] * nb
    ys = [{n: torch.empty((M, synth.BLOCK_SHAPES[n][0]), dtype=torch.float32, device=dev)
           for n in synth.PROJ_ORDER} for _ in range(nb)]
    bs = [{n: (torch.from_numpy(synth.activation(cfg, b, "h", 1, synth.BLOCK_SHAPES[n][0])[0]).to(dev)
               if BIAS else None) for n in synth.PROJ_ORDER} for b in range(nb)]
    sets = []
    for s in range(n_sets):
        blocks = []
        for b in range(nb):
            blk = {}
            for name in synth.PROJ_ORDER:
                W = torch.from_numpy(synth.weight(cfg, s, b, name, heavy=heavy)).to(dev)
                w = rtq.quantize(W, recipe_map(recipe)[name])
                del W
                blk[name] = rtq.Projection(w, xs[b][synth.BLOCK_SHAPES[name][2]], ys[b][name], bs[b][name])
            blocks.append(blk)
        sets.append((blocks, rtq.pack_blocks(blocks, M)))
    torch.cuda.synchronize()
    return sets


def workspace_for(torch, rtq, sets, M, math):
    """One caller workspace for every weight set of a workload (the largest
    any call needs), allocated once before timing: the calls then go through
    rtq_block_project_ws and allocate nothing."""
    need = max(rtq.block_workspace_bytes(blocks, M, math, packed=packed) for blocks, packed in sets)
    return torch.empty(max(need, 256), dtype=torch.uint8, device="cuda:0")


def time_workload(torch, rtq, sets, M, steps, warmup, math, ws=None):
    """Times exactly `steps` steps twice. First with nothing else in the
    stream (wall clock between synchronizations): the step time. Then the same
    steps again with the library's event timing on, which brackets every main
    GEMM kernel launch with HIP events on its stream: the kernel time (the
    events themselves add a few us to each step, so that pass does not give
    the step time)."""
    def step(i):
        blocks, packed = sets[i % len(sets)]
        rtq.block_project(blocks, M, packed=packed, math=math, workspace=ws)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    rtq.timing_enable(True)
    t1 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall_events = time.perf_counter() - t1
    kernel_ms, launches = rtq.timing_read()
    rtq.timing_enable(False)
    return wall, kernel_ms, launches, wall_events


def measure(torch, rtq, synth, workload, steps, warmup, math, recipe="mixed"):
    nb = synth.NUM_BLOCKS
    if workload == "m80":
        M = synth.M_GOLDEN
        sets = build_sets(torch, rtq, synth, 4, M, WEIGHT_SETS, xs_per_block=True, recipe=recipe)
    else:
        M = synth.M_LARGE
        sets = build_sets(torch, rtq, synth, 5, M, 1, xs_per_block=False, recipe=recipe)
    wb, fl = block_bytes_flops(M, recipe)
    ws = workspace_for(torch, rtq, sets, M, math)
    wall, kernel_ms, launches, wall_events = time_workload(torch, rtq, sets, M, steps, warmup, math, ws)
    pool_ms = None
    if workload == "m80":
        # the same steps with the library's own per-call workspace (stream-ordered pool allocation)
        pool_wall, _, _, _ = time_workload(torch, rtq, sets, M, steps, warmup, math, None)
        pool_ms = pool_wall / steps * 1e3
    ws_bytes = ws.numel()
    del sets, ws
    torch.cuda.empty_cache()
    flops_step, bytes_step = fl * nb, wb * nb
    act_bytes = sum(M * k * 4 for k in synth.INPUT_WIDTH.values())    # the four inputs of a block
    out_bytes = sum(M * synth.BLOCK_SHAPES[n][0] * 4 for n in synth.PROJ_ORDER)
    alg_step = bytes_step + nb * (out_bytes + (act_bytes if workload == "m80" else 0)) + \
        (act_bytes if workload != "m80" else 0)
    ms_step = wall / steps * 1e3
    per_step = launches / steps
    launch_ms = kernel_ms / launches
    return {
        "M": M, "ms_per_step": ms_step, "tflops": flops_step / (ms_step * 1e-3) / 1e12,
        "weight_gbs": bytes_step / (ms_step * 1e-3) / 1e9,
        "kernel_launches_per_step": per_step, "kernel_ms_per_launch": launch_ms,
        "kernel_tflops": flops_step / per_step / (launch_ms * 1e-3) / 1e12,
        "kernel_weight_gbs": bytes_step / per_step / (launch_ms * 1e-3) / 1e9,
        "flops_per_step": flops_step, "weight_bytes_per_step": bytes_step, "steps": steps,
        "algorithmic_bytes_per_step": alg_step,
        "ms_per_step_with_kernel_events": wall_events / steps * 1e3,
        "ms_per_step_pool_workspace": pool_ms, "workspace_bytes": ws_bytes,
    }


def m_sweep(torch, rtq, synth, Ms, math, steps=200, warmup=20, recipe="mixed"):
    """Diagnostic: the m80 weight sets (12 blocks x 16 sets) at other M, to show
    where the weight stream stops being the only cost. Same timing as the main
    workload; the weights are quantized once and shared across M."""
    dev = "cuda:0"
    nb = synth.NUM_BLOCKS
    weights = [[{name: rtq.quantize(torch.from_numpy(synth.weight(4, s, b, name)).to(dev), recipe_map(recipe)[name])
                 for name in synth.PROJ_ORDER} for b in range(nb)] for s in range(WEIGHT_SETS)]
    wb, _ = block_bytes_flops(1, recipe)
    out = []
    for M in Ms:
        xs = [{n: torch.from_numpy(synth.activation(4, b, n, M)).to(dev) for n in synth.INPUT_WIDTH} for b in range(nb)]
        ys = [{n: torch.empty((M, synth.BLOCK_SHAPES[n][0]), dtype=torch.float32, device=dev)
               for n in synth.PROJ_ORDER} for _ in range(nb)]
        sets = []
        for s in range(WEIGHT_SETS):
            blocks = [{name: rtq.Projection(weights[s][b][name], xs[b][synth.BLOCK_SHAPES[name][2]], ys[b][name])
                       for name in synth.PROJ_ORDER} for b in range(nb)]
            sets.append((blocks, rtq.pack_blocks(blocks, M)))
        ws = workspace_for(torch, rtq, sets, M, math)
        wall, kernel_ms, launches, _ = time_workload(torch, rtq, sets, M, steps, warmup, math, ws)
        _, fl = block_bytes_flops(M, recipe)
        ms = wall / steps * 1e3
        per_launch = kernel_ms / launches
        out.append({"M": M, "ms_per_step": round(ms, 5), "tflops": round(fl * nb / (ms * 1e-3) / 1e12, 3),
                    "weight_gbs": round(wb * nb / (ms * 1e-3) / 1e9, 1),
                    "kernel_ms_per_launch": round(per_launch, 5),
                    "weight_gbs_in_kernel": round(wb * nb / (launches / steps) / (per_launch * 1e-3) / 1e9, 1)})
        del sets, xs, ys, ws
    del weights
    torch.cuda.empty_cache()
    return out


def measured_ceilings(torch, rtq, gib=4, reps=5):
    """The chip's measured ceilings beside the published peaks: the library's
    streaming-read kernel (rtq_diag_stream_read) over a `gib` GiB buffer, best
    of a small sweep of loads in flight and grid sizes, and its back-to-back
    matrix-instruction loop (rtq_diag_mfma_loop) for fp16, bf16 and fp32.
    Timed with events on the stream the kernels run on."""
    dev = "cuda:0"
    buf = torch.ones(gib * (1 << 28), dtype=torch.float32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = None
    sweep = []
    for unroll in (4, 8, 16):
        for blocks in (2048, 4096, 8192):
            rtq.diag_stream_read(buf, unroll, blocks, sink)
            ev0.record()
            for _ in range(reps):
                rtq.diag_stream_read(buf, unroll, blocks, sink)
            ev1.record()
            ev1.synchronize()
            gbs = buf.numel() * 4 * reps / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
            sweep.append({"unroll": unroll, "blocks": blocks, "gbs": round(gbs, 1)})
            if best is None or gbs > best["gbs"]:
                best = sweep[-1]
    del buf
    torch.cuda.empty_cache()
    # A read of the 12-block weight size (39.4 MB) from 16 buffers cycled like
    # the weight sets: the ceiling a kernel that streams those weights once
    # can reach, launch ramp included (64 launches back to back per shape).
    wsize = block_bytes_flops(1)[0] * 12 // 16 * 16
    wbufs = [torch.ones(wsize // 4, dtype=torch.float32, device=dev) for _ in range(WEIGHT_SETS)]
    wbest = None
    wsweep = []
    for unroll, blocks in ((4, 512), (8, 2048), (16, 512), (16, 2048), (16, 4096)):
        for b in wbufs:
            rtq.diag_stream_read(b, unroll, blocks, sink)
        ev0.record()
        for r in range(64):
            rtq.diag_stream_read(wbufs[r % len(wbufs)], unroll, blocks, sink)
        ev1.record()
        ev1.synchronize()
        us = ev0.elapsed_time(ev1) * 1e3 / 64
        wsweep.append({"unroll": unroll, "blocks": blocks, "us_per_launch": round(us, 3),
                       "gbs": round(wsize / us / 1e3, 1)})
        if wbest is None or wsweep[-1]["gbs"] > wbest["gbs"]:
            wbest = wsweep[-1]
    del wbufs
    torch.cuda.empty_cache()
    fsink = torch.zeros(1, dtype=torch.float32, device=dev)
    mfma = {}
    for kind, name, peak in ((0, "fp16", PEAK_BF16_MFMA_TFLOPS), (1, "bf16", PEAK_BF16_MFMA_TFLOPS),
                             (2, "fp32", PEAK_FP32_MFMA_TFLOPS)):
        iters = 20000 if kind < 2 else 5000
        rtq.diag_mfma_loop(kind, 100, 2048, fsink)
        ev0.record()
        flops = rtq.diag_mfma_loop(kind, iters, 2048, fsink)
        ev1.record()
        ev1.synchronize()
        tf = flops / (ev0.elapsed_time(ev1) * 1e-3) / 1e12
        mfma[name] = {"tflops": round(tf, 1), "frac_of_peak": round(tf / peak, 4),
                      "instruction": ["v_mfma_f32_16x16x32_f16", "v_mfma_f32_16x16x32_bf16",
                                      "v_mfma_f32_16x16x4_f32"][kind]}
    return {"hbm_read_gbs": best["gbs"], "hbm_frac_of_peak": round(best["gbs"] / PEAK_HBM_GBS, 4),
            "weight_size_read_gbs": wbest["gbs"], "weight_size_read_us": wbest["us_per_launch"],
            "weight_size_read_how": f"rtq_diag_stream_read of {wsize} B (the 12-block weight size) from "
                                    f"{WEIGHT_SETS} buffers cycled, 64 launches back to back between HIP events, "
                                    "best of 5 shapes",
            "weight_size_read_sweep": wsweep,
            "hbm_how": f"rtq_diag_stream_read over a {gib} GiB buffer (16-byte loads, best of the sweep), "
                       f"{reps} passes timed with HIP events",
            "hbm_sweep": sweep, "mfma": mfma,
            "mfma_how": "rtq_diag_mfma_loop: 2048 workgroups x 4 waves, 8 independent accumulators per wave"}


def config_cases(torch, rtq, synth, math, reps=2000, warmup=100):
    """The small single-GEMM and one-block configurations at M = 80 (weights
    resident, one seeded weight set): time per call, TFLOP/s, weight GB/s."""
    dev = "cuda:0"
    M = synth.M_GOLDEN
    out = {}
    cases = [("cfg1_q4_wq_512x512", "q4", "wq", 512, 512, "x_attn"),
             ("cfg2_q8_wo_512x512", "q8", "wo", 512, 512, "x_o"),
             ("cfg2_q8_w2_512x2048", "q8", "w2", 512, 2048, "h")]
    for name, fmt, proj, N, K, xin in cases:
        w = rtq.quantize(torch.from_numpy(synth.weight(1, 0, 0, proj, N, K)).to(dev), fmt)
        x = torch.from_numpy(synth.activation(1, 0, xin, M, K)).to(dev)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        for _ in range(warmup):
            rtq.gemm(x, w, y=y, math=math)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            rtq.gemm(x, w, y=y, math=math)
        torch.cuda.synchronize()
        t = (time.perf_counter() - t0) / reps
        wb = N * K // 2 + N * (K // 32) * 4 if fmt == "q4" else N * K + N * 4
        out[name] = {"us_per_call": round(t * 1e6, 3), "tflops": round(2 * M * N * K / t / 1e12, 3),
                     "weight_gbs": round(wb / t / 1e9, 2), "M": M, "N": N, "K": K, "fmt": fmt}
    # one RT-J block (8 projections, 4 inputs)
    xs = {n: torch.from_numpy(synth.activation(3, 0, n, M)).to(dev) for n in synth.INPUT_WIDTH}
    blk = {}
    for name in synth.PROJ_ORDER:
        N, K, xin = synth.BLOCK_SHAPES[name]
        w = rtq.quantize(torch.from_numpy(synth.weight(3, 0, 0, name)).to(dev), rtq.RECIPE_MIXED[name])
        blk[name] = rtq.Projection(w, xs[xin], torch.empty((M, N), dtype=torch.float32, device=dev))
    packed = rtq.pack_blocks([blk], M)
    for _ in range(warmup):
        rtq.block_project([blk], M, packed=packed, math=math)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        rtq.block_project([blk], M, packed=packed, math=math)
    torch.cuda.synchronize()
    t = (time.perf_counter() - t0) / reps
    wb, fl = block_bytes_flops(M)
    out["cfg3_one_block"] = {"us_per_call": round(t * 1e6, 3), "tflops": round(fl / t / 1e12, 3),
                             "weight_gbs": round(wb / t / 1e9, 2), "M": M}
    return out


def load_traffic(workload, math, recipe="mixed"):
    """HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE /
    WRITE_SIZE, copy-kernel calibrated), if recorded for the current sources."""
    import weight_only_quantized_rtq_amd.traffic as tr
    return tr.lookup(workload, math) if recipe == "mixed" else None


def roofline(res, math, workload, recipe="mixed"):
    """Roofline of the main GEMM kernel from its average launch time (HIP
    events on the launch stream). At M = 80 the binding roof is HBM: the
    achieved figure is the packed weight bytes one launch streams over the
    launch time, against 8 TB/s (the matrix-unit figures ride along under
    "mfma"). At M = 65536 it is the matrix unit: algorithmic flops over the
    launch time, against the peak of the unit the arithmetic runs on (split:
    bf16 MFMA, three limb products per multiply-add; split16: fp16 MFMA, two;
    bf16: one; fp32: the fp32 matrix peak)."""
    ach = res["kernel_tflops"]
    if math == "split":
        peak, issued = PEAK_BF16_MFMA_TFLOPS, 3
    elif math == "split16":
        peak, issued = PEAK_BF16_MFMA_TFLOPS, 2            # the dense fp16 matrix peak equals the bf16 one
    elif math == "bf16":
        peak, issued = PEAK_BF16_MFMA_TFLOPS, 1
    else:
        peak, issued = PEAK_FP32_MFMA_TFLOPS, 1
    tr = load_traffic(workload, math, recipe)
    mfma = {"achieved": round(ach, 3), "peak": peak, "unit": "TFLOP/s", "frac": round(ach / peak, 5),
            "mfma_flops_per_algorithmic_flop": issued, "matrix_unit_frac": round(ach * issued / peak, 5)}
    out = {"kernel": KERNELS[(math, workload)], "kernel_ms_per_launch": round(res["kernel_ms_per_launch"], 6),
           "launches_per_step": res["kernel_launches_per_step"],
           "traffic": tr["bytes_per_launch"] if tr else None, "traffic_detail": tr}
    if workload == "m80":
        gbs = res["kernel_weight_gbs"]
        per_launch_s = res["kernel_ms_per_launch"] * 1e-3
        all_bytes = res["algorithmic_bytes_per_step"] / res["kernel_launches_per_step"]
        return {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 5), **out,
                "basis": "packed weight bytes per launch / average launch time",
                "all_algorithmic_bytes_gbs": round(all_bytes / per_launch_s / 1e9, 2),
                "all_algorithmic_bytes_frac": round(all_bytes / per_launch_s / 1e9 / PEAK_HBM_GBS, 5),
                "mfma": mfma}
    return {"bound": "mfma", **mfma, **out,
            "weight_gbs_in_kernel": round(res["kernel_weight_gbs"], 2),
            "weight_hbm_frac_in_kernel": round(res["kernel_weight_gbs"] / PEAK_HBM_GBS, 5)}


def cpu_baseline(cfg, M, seconds, rows=None, recipe="mixed"):
    """The oracle (numpy dequant + fp64 GEMM) on a bounded sample: whole
    blocks of this workload, quantized by the oracle's own quantizer."""
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:                                                   # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    Ms = M if rows is None else rows
    blocks = []
    for b in range(2):
        projs = []
        for name in synth.PROJ_ORDER:
            fmt = {"mixed": oracle.RECIPE_MIXED, "all_q8": oracle.RECIPE_ALL_Q8,
                   "all_f8": oracle.RECIPE_ALL_F8}[recipe][name]
            N, K, xin = synth.BLOCK_SHAPES[name]
            W = synth.weight(cfg, 0, b, name)
            x = synth.activation(cfg, b, xin, Ms)
            projs.append((fmt, x, oracle.quantize(W, fmt)))
        blocks.append(projs)
    _, flops_block = block_bytes_flops(Ms, recipe)
    done = 0
    t0 = time.perf_counter()
    while True:
        for projs in blocks:
            for fmt, x, packed in projs:
                oracle.project(fmt, x, *packed)
            done += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(done * flops_block / el / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} RT-J block passes (8 projections, M={Ms}, numpy dequant + fp64 matmul) "
                      f"in {el:.1f} s, cycling 2 oracle-quantized blocks"}


def cpu_baseline_extra(seconds):
    """Beside the all-thread baseline: the same oracle on one thread (bounded
    sample at M = 80), and one whole RT-J block at M = 65536 timed once and
    reported x 12 as the 12-block pass (an explicit extrapolation)."""
    import oracle
    import synth
    out = {}
    try:
        from threadpoolctl import threadpool_limits
    except Exception:                                                   # noqa: BLE001
        threadpool_limits = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            r = cpu_baseline(4, synth.M_GOLDEN, seconds)
        r["cores"] = 1
        out["single_core_m80"] = r
    blk = []
    for name in synth.PROJ_ORDER:
        fmt = oracle.RECIPE_MIXED[name]
        N, K, xin = synth.BLOCK_SHAPES[name]
        blk.append((fmt, oracle.quantize(synth.weight(5, 0, 0, name), fmt), xin))
    xs = {n: synth.activation(5, synth.SHARED_BLOCK, n, synth.M_LARGE) for n in synth.INPUT_WIDTH}
    _, fl = block_bytes_flops(synth.M_LARGE)
    t0 = time.perf_counter()
    for fmt, packed, xin in blk:
        oracle.project(fmt, xs[xin], *packed)
    el = time.perf_counter() - t0
    out["m65536_one_block_x12"] = {
        "value": round(fl / el / 1e12, 6), "unit": "TFLOP/s", "s_per_block": round(el, 3),
        "s_per_12_block_pass_extrapolated": round(12 * el, 3),
        "sample": "one RT-J block (8 projections) at M=65536 in full, timed once; the 12-block pass is 12x that "
                  "(extrapolated, not run)"}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (the path needs no "
              f"collectives; see the sharding notes in the design document)", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import weight_only_quantized_rtq_amd as rtq
    global BIAS
    BIAS = args.bias
    rtq.load_library()
    torch.cuda.init()
    modes = rtq.MATHS
    main_math = modes[args.math]
    fp32_modes = ("split16", "split")
    out = {}
    if args.workload in ("m80", "both"):
        out["m80"] = measure(torch, rtq, synth, "m80", args.steps, args.warmup, main_math, args.recipe)
    if args.workload in ("m65536", "both"):
        out["m65536"] = measure(torch, rtq, synth, "m65536", args.steps_large, args.warmup_large, main_math,
                                args.recipe)
    fp32 = {}
    if args.compare_fp32 and args.math in fp32_modes:
        for wl in out:
            r = measure(torch, rtq, synth, wl, 300 if wl == "m80" else 3, 10 if wl == "m80" else 1,
                        rtq.MATH_FP32_MFMA, args.recipe)
            fp32[wl] = {"ms_per_step": round(r["ms_per_step"], 5), "tflops": round(r["tflops"], 3),
                        "roofline": roofline(r, "fp32", wl, args.recipe)}
    exact = {}
    if not args.no_exact_path and args.math == "split16":
        for wl in out:
            st, wu = (args.steps, args.warmup) if wl == "m80" else (args.steps_large, args.warmup_large)
            r = measure(torch, rtq, synth, wl, st, wu, rtq.MATH_SPLIT_BF16, args.recipe)
            exact[wl] = {"ms_per_step": round(r["ms_per_step"], 5), "tflops": round(r["tflops"], 3),
                         "weight_gbs": round(r["weight_gbs"], 2), "steps": r["steps"],
                         "roofline": roofline(r, "split", wl, args.recipe)}
    bf16 = {}
    if not args.no_bf16_path and args.math in fp32_modes:
        for wl in out:
            st, wu = (args.steps, args.warmup) if wl == "m80" else (args.steps_large, args.warmup_large)
            r = measure(torch, rtq, synth, wl, st, wu, rtq.MATH_BF16, args.recipe)
            bf16[wl] = {"ms_per_step": round(r["ms_per_step"], 5), "tflops": round(r["tflops"], 3),
                        "weight_gbs": round(r["weight_gbs"], 2),
                        "weight_hbm_frac": round(r["weight_gbs"] / PEAK_HBM_GBS, 5), "steps": r["steps"],
                        "roofline": roofline(r, "bf16", wl, args.recipe)}

    prim_name = "m80" if "m80" in out else "m65536"
    prim = out[prim_name]
    wdesc = {"mixed": "wq/wk/wv/wg/w1/w3 int4 g32, wo/w2 int8", "all_q8": "every projection int8",
             "all_f8": "every projection FP8 E4M3"}[args.recipe]
    set_mb = WEIGHT_SETS * synth.NUM_BLOCKS * block_bytes_flops(1, args.recipe)[0] / 1e6
    cfg = {"m80": f"m80: 12 RT-J blocks ({wdesc}), M=80, {WEIGHT_SETS} weight sets cycled "
                  f"({set_mb:.0f} MB packed), per-block fp32 activations",
           "m65536": f"m65536: 12 RT-J blocks ({wdesc}), M=65536, one weight set, fp32 "
                     "activations shared by the blocks"}[prim_name]
    line = {
        "metric": "dequant-GEMM TFLOP/s + weight-payload HBM GB/s (frac. of peak), M=80 and M=65536",
        "value": round(prim["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": prim["steps"],
        "warmup": args.warmup if prim_name == "m80" else args.warmup_large,
        "ms_per_step": round(prim["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"split16": "f16x2/f32", "split": "bf16x3/f32", "fp32": "f32", "bf16": "bf16/f32"}[args.math],
        "data": "synthetic",
        "config": {"workload": cfg, "M": prim["M"], "n_blocks": synth.NUM_BLOCKS,
                   "weight_sets": WEIGHT_SETS if prim_name == "m80" else 1, "recipe": {"mixed": "mixed int4/int8", "all_q8": "all int8",
                                                                               "all_f8": "all FP8 E4M3"}[args.recipe],
                   "d_model": synth.D_MODEL, "d_ff": synth.D_FF, "bias": bool(args.bias),
                   "math": {"split16": "each activation row scaled by a power of two and split into 2 fp16 limbs "
                                       "(22 significant bits), exact code products, fp32 accumulation; rows of "
                                       "M <= 32 calls take the exact 3-limb direct kernel",
                            "split": "activations split exactly into 3 bf16 limbs, exact products, fp32 accumulation",
                            "fp32": "fp32 MFMA on dequantized weights",
                            "bf16": "activations rounded to bf16 (lower precision), exact weight products, "
                                    "fp32 accumulation"}[args.math]},
        "weight_gbs": round(prim["weight_gbs"], 2),
        "weight_hbm_frac": round(prim["weight_gbs"] / PEAK_HBM_GBS, 5),
        "roofline": roofline(prim, args.math, prim_name, args.recipe),
        "timing": {
            "step": "wall clock over the timed steps between synchronizations, nothing else in the stream; "
                    "every call through rtq_block_project_ws with one device workspace allocated before timing",
            "kernel": "a second pass over the same steps with HIP events recorded around every main GEMM "
                      "launch on its stream (rtq_timing_enable); the events add to that pass's step time",
            "ms_per_step_with_kernel_events": round(prim["ms_per_step_with_kernel_events"], 5),
            "ms_per_step_pool_workspace": (round(prim["ms_per_step_pool_workspace"], 5)
                                           if prim["ms_per_step_pool_workspace"] else None),
            "workspace_bytes": prim["workspace_bytes"],
        },
    }
    for wl, r in out.items():
        if wl == prim_name:
            continue
        line[wl] = {"ms_per_step": round(r["ms_per_step"], 5), "tflops": round(r["tflops"], 3),
                    "weight_gbs": round(r["weight_gbs"], 3), "steps": r["steps"],
                    "frac_of_fp32_mfma_peak": round(r["tflops"] / PEAK_FP32_MFMA_TFLOPS, 4),
                    "roofline": roofline(r, args.math, wl, args.recipe)}
    if fp32:
        line["fp32_mfma_path"] = fp32
    if exact:
        line["exact_bf16x3_path"] = {
            "note": "activations split exactly into 3 bf16 limbs (the library's default arithmetic), same "
                    "workloads; reported next to the headline two-limb fp16 figures",
            **exact}
    if bf16:
        line["bf16_activation_path"] = {
            "note": "x rounded to the nearest bf16 (lower precision: 3e-3 bar, not 1e-5), one bf16 MFMA per "
                    "product; reported apart from the fp32-activation figures above",
            **bf16}
    if not args.no_attainable:
        ceil = measured_ceilings(torch, rtq)
        line["measured_ceilings"] = ceil
        hbm = ceil["hbm_read_gbs"]
        rl = line["roofline"]
        if rl["bound"] == "hbm":
            rl["frac_of_measured_ceiling"] = round(rl["achieved"] / hbm, 5)
            rl["frac_of_weight_size_read"] = round(rl["achieved"] / ceil["weight_size_read_gbs"], 5)
        unit = {"split16": "fp16", "split": "bf16", "bf16": "bf16", "fp32": "fp32"}[args.math]
        line["weight_frac_of_measured_hbm"] = round(prim["weight_gbs"] / hbm, 5)
        for wl in out:
            tgt = rl if wl == prim_name else line[wl]["roofline"]
            if tgt["bound"] == "mfma":
                tgt["frac_of_measured_ceiling"] = round(tgt["achieved"] / ceil["mfma"][unit]["tflops"], 5)
            else:
                tgt["mfma"]["frac_of_measured_ceiling"] = round(
                    tgt["mfma"]["achieved"] / ceil["mfma"][unit]["tflops"], 5)
    if not args.no_configs and args.workload in ("m80", "both"):
        line["config_cases"] = {
            "note": "single GEMMs and one block at M = 80, one resident weight set, per call (dispatch included)",
            **config_cases(torch, rtq, synth, main_math)}
    if args.m_sweep is None:
        args.m_sweep = "1,2,4,8,16,32,48,80" if args.workload == "both" else ""
    if args.m_sweep:
        line["m_sweep"] = {
            "note": f"diagnostic: the m80 weight sets at other M ({args.math} arithmetic); per-step and "
                    "in-kernel weight GB/s against the 8000 GB/s HBM peak",
            "points": m_sweep(torch, rtq, synth, [int(v) for v in args.m_sweep.split(",")], main_math,
                              recipe=args.recipe)}
        if "measured_ceilings" in line:
            for pt in line["m_sweep"]["points"]:
                pt["weight_frac_of_measured_hbm_in_kernel"] = round(
                    pt["weight_gbs_in_kernel"] / line["measured_ceilings"]["hbm_read_gbs"], 4)
                pt["weight_frac_of_weight_size_read_in_kernel"] = round(
                    pt["weight_gbs_in_kernel"] / line["measured_ceilings"]["weight_size_read_gbs"], 4)
    if not args.no_cpu_baseline and prim_name == "m80":
        line["cpu_baseline"] = cpu_baseline(4, synth.M_GOLDEN, args.cpu_seconds, recipe=args.recipe)
        if args.recipe == "mixed":
            line["cpu_baseline"].update(cpu_baseline_extra(args.cpu_seconds / 2))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
