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
                    help="skip the measured streaming-read ceiling (hbm_attainable)")
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


def time_workload(torch, rtq, sets, M, steps, warmup, math):
    """Times exactly `steps` steps (wall clock between synchronizations) and,
    through the library's event timing, the main GEMM kernel launches inside
    them (HIP events recorded on the launch stream)."""
    for i in range(warmup):
        blocks, packed = sets[i % len(sets)]
        rtq.block_project(blocks, M, packed=packed, math=math)
    torch.cuda.synchronize()
    rtq.timing_enable(True)
    t0 = time.perf_counter()
    for i in range(steps):
        blocks, packed = sets[i % len(sets)]
        rtq.block_project(blocks, M, packed=packed, math=math)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms, launches = rtq.timing_read()
    rtq.timing_enable(False)
    return wall, kernel_ms, launches


def measure(torch, rtq, synth, workload, steps, warmup, math, recipe="mixed"):
    nb = synth.NUM_BLOCKS
    if workload == "m80":
        M = synth.M_GOLDEN
        sets = build_sets(torch, rtq, synth, 4, M, WEIGHT_SETS, xs_per_block=True, recipe=recipe)
    else:
        M = synth.M_LARGE
        sets = build_sets(torch, rtq, synth, 5, M, 1, xs_per_block=False, recipe=recipe)
    wb, fl = block_bytes_flops(M, recipe)
    wall, kernel_ms, launches = time_workload(torch, rtq, sets, M, steps, warmup, math)
    del sets
    torch.cuda.empty_cache()
    flops_step, bytes_step = fl * nb, wb * nb
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
        wall, kernel_ms, launches = time_workload(torch, rtq, sets, M, steps, warmup, math)
        _, fl = block_bytes_flops(M, recipe)
        ms = wall / steps * 1e3
        per_launch = kernel_ms / launches
        out.append({"M": M, "ms_per_step": round(ms, 5), "tflops": round(fl * nb / (ms * 1e-3) / 1e12, 3),
                    "weight_gbs": round(wb * nb / (ms * 1e-3) / 1e9, 1),
                    "kernel_ms_per_launch": round(per_launch, 5),
                    "weight_gbs_in_kernel": round(wb * nb / (launches / steps) / (per_launch * 1e-3) / 1e9, 1)})
        del sets, xs, ys
    del weights
    torch.cuda.empty_cache()
    return out


def attainable_hbm_gbs(torch, gib=4, reps=10):
    """Read bandwidth a plain device-wide streaming reduction (torch.sum over a
    `gib` GiB fp32 buffer) attains on this GPU: the measured ceiling the weight
    stream is compared with, beside the 8 TB/s published peak."""
    buf = torch.ones(gib * (1 << 28), dtype=torch.float32, device="cuda:0")
    for _ in range(2):
        buf.sum()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        buf.sum()
    t1.record()
    t1.synchronize()
    gbs = buf.numel() * 4 * reps / (t0.elapsed_time(t1) * 1e-3) / 1e9
    del buf
    torch.cuda.empty_cache()
    return gbs


def load_traffic(workload, math, recipe="mixed"):
    """HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE /
    WRITE_SIZE, copy-kernel calibrated), if recorded for the current sources."""
    import weight_only_quantized_rtq_amd.traffic as tr
    return tr.lookup(workload, math) if recipe == "mixed" else None


def roofline(res, math, workload, recipe="mixed"):
    """Roofline of the main GEMM kernel: algorithmic flops per launch over the
    kernel's average launch duration, against the peak of the matrix unit it
    runs on (split: bf16 MFMA, three limb products per algorithmic multiply-add;
    split16: fp16 MFMA, two)."""
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
    out = {"bound": "mfma", "achieved": round(ach, 3), "peak": peak, "unit": "TFLOP/s",
           "frac": round(ach / peak, 5), "traffic": tr["bytes_per_launch"] if tr else None,
           "traffic_detail": tr,
           "kernel": KERNELS[(math, workload)],
           "kernel_ms_per_launch": round(res["kernel_ms_per_launch"], 6),
           "launches_per_step": res["kernel_launches_per_step"],
           "mfma_flops_per_algorithmic_flop": issued,
           "matrix_unit_frac": round(ach * issued / peak, 5),
           "weight_gbs_in_kernel": round(res["kernel_weight_gbs"], 2),
           "weight_hbm_frac_in_kernel": round(res["kernel_weight_gbs"] / PEAK_HBM_GBS, 5)}
    return out


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
        hbm = attainable_hbm_gbs(torch)
        line["hbm_attainable"] = {"gbs": round(hbm, 1), "frac_of_peak": round(hbm / PEAK_HBM_GBS, 4),
                                  "how": "torch.sum over a 4 GiB fp32 buffer, 10 passes (HIP events)",
                                  "weight_frac_of_attainable": round(prim["weight_gbs"] / hbm, 5)}
    if args.m_sweep is None:
        args.m_sweep = "1,2,4,8,16,32,48,80" if args.workload == "both" else ""
    if args.m_sweep:
        line["m_sweep"] = {
            "note": f"diagnostic: the m80 weight sets at other M ({args.math} arithmetic); per-step and "
                    "in-kernel weight GB/s against the 8000 GB/s HBM peak",
            "points": m_sweep(torch, rtq, synth, [int(v) for v in args.m_sweep.split(",")], main_math,
                              recipe=args.recipe)}
        if "hbm_attainable" in line:
            for pt in line["m_sweep"]["points"]:
                pt["weight_frac_of_attainable_in_kernel"] = round(
                    pt["weight_gbs_in_kernel"] / line["hbm_attainable"]["gbs"], 4)
    if not args.no_cpu_baseline and prim_name == "m80":
        line["cpu_baseline"] = cpu_baseline(4, synth.M_GOLDEN, args.cpu_seconds, recipe=args.recipe)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
