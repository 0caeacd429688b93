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
"m65536".
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
PEAK_FP32_MFMA_TFLOPS = 157.3
WEIGHT_SETS = 16


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000, help="timed steps of the m80 workload")
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--steps-large", type=int, default=10, help="timed steps of the m65536 workload")
    ap.add_argument("--warmup-large", type=int, default=2)
    ap.add_argument("--workload", choices=["m80", "m65536", "both"], default="both")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    return ap.parse_args()


def block_bytes_flops(M):
    import synth
    import weight_only_quantized_rtq_amd as rtq
    wbytes = 0
    flops = 0
    for name in synth.PROJ_ORDER:
        N, K, _ = synth.BLOCK_SHAPES[name]
        if rtq.RECIPE_MIXED[name] == "q4":
            wbytes += N * K // 2 + N * (K // 32) * 4
        else:
            wbytes += N * K + N * 4
        flops += 2 * M * N * K
    return wbytes, flops


def build_sets(torch, rtq, synth, cfg, M, n_sets, xs_per_block, heavy=None):
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
    sets = []
    for s in range(n_sets):
        blocks = []
        for b in range(nb):
            blk = {}
            for name in synth.PROJ_ORDER:
                W = torch.from_numpy(synth.weight(cfg, s, b, name, heavy=heavy)).to(dev)
                w = rtq.quantize(W, rtq.RECIPE_MIXED[name])
                del W
                blk[name] = rtq.Projection(w, xs[b][synth.BLOCK_SHAPES[name][2]], ys[b][name])
            blocks.append(blk)
        sets.append((blocks, rtq.pack_blocks(blocks, M)))
    torch.cuda.synchronize()
    return sets


def time_workload(torch, rtq, sets, M, steps, warmup):
    """Times exactly `steps` steps; also brackets every launch with events on
    the launch stream to get the per-launch kernel duration."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        blocks, packed = sets[i % len(sets)]
        rtq.block_project(blocks, M, packed=packed)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        blocks, packed = sets[i % len(sets)]
        ev[i][0].record(stream)
        rtq.block_project(blocks, M, packed=packed)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([a.elapsed_time(b) for a, b in ev])      # ms
    return wall, per


def cpu_baseline(cfg, M, seconds, rows=None):
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
            fmt = oracle.RECIPE_MIXED[name]
            N, K, xin = synth.BLOCK_SHAPES[name]
            W = synth.weight(cfg, 0, b, name)
            x = synth.activation(cfg, b, xin, Ms)
            projs.append((fmt, x, oracle.quantize(W, fmt)))
        blocks.append(projs)
    _, flops_block = block_bytes_flops(Ms)
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
    rtq.load_library()
    torch.cuda.init()
    out = {}

    wb, fl80 = block_bytes_flops(synth.M_GOLDEN)
    nb = synth.NUM_BLOCKS
    if args.workload in ("m80", "both"):
        sets = build_sets(torch, rtq, synth, 4, synth.M_GOLDEN, WEIGHT_SETS, xs_per_block=True)
        wall, per = time_workload(torch, rtq, sets, synth.M_GOLDEN, args.steps, args.warmup)
        ms_step = wall / args.steps * 1e3
        flops_step = fl80 * nb
        bytes_step = wb * nb
        launch_ms = float(per.mean())
        achieved_tf = flops_step / (launch_ms * 1e-3) / 1e12
        out["m80"] = {
            "ms_per_step": ms_step, "tflops": flops_step / (ms_step * 1e-3) / 1e12,
            "weight_gbs": bytes_step / (ms_step * 1e-3) / 1e9,
            "launch_ms": launch_ms, "launch_ms_min": float(per.min()),
            "kernel_tflops": achieved_tf, "kernel_weight_gbs": bytes_step / (launch_ms * 1e-3) / 1e9,
            "flops_per_step": flops_step, "weight_bytes_per_step": bytes_step,
        }
        del sets
        torch.cuda.empty_cache()

    if args.workload in ("m65536", "both"):
        M = synth.M_LARGE
        _, flL = block_bytes_flops(M)
        sets = build_sets(torch, rtq, synth, 5, M, 1, xs_per_block=False)
        wall, per = time_workload(torch, rtq, sets, M, args.steps_large, args.warmup_large)
        ms_step = wall / args.steps_large * 1e3
        flops_step = flL * nb
        out["m65536"] = {
            "ms_per_step": ms_step, "tflops": flops_step / (ms_step * 1e-3) / 1e12,
            "weight_gbs": wb * nb / (ms_step * 1e-3) / 1e9,
            "step_event_ms": float(per.mean()), "flops_per_step": flops_step,
            "fp32_mfma_frac": flops_step / (ms_step * 1e-3) / 1e12 / PEAK_FP32_MFMA_TFLOPS,
        }
        del sets
        torch.cuda.empty_cache()

    prim = out.get("m80")
    line = {
        "metric": "dequant-GEMM TFLOP/s + weight-payload HBM GB/s (frac. of peak), M=80 and M=65536",
        "value": round(prim["tflops"], 3) if prim else None,
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(prim["ms_per_step"], 5) if prim else None,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "m80: 12 RT-J blocks (wq/wk/wv/wg/w1/w3 int4 g32, wo/w2 int8), "
                               "M=80, 16 weight sets cycled (630 MB packed)",
                   "M": synth.M_GOLDEN, "n_blocks": nb, "weight_sets": WEIGHT_SETS, "recipe": "mixed int4/int8",
                   "d_model": synth.D_MODEL, "d_ff": synth.D_FF},
    }
    if prim:
        line["weight_gbs"] = round(prim["weight_gbs"], 2)
        line["weight_hbm_frac"] = round(prim["weight_gbs"] / PEAK_HBM_GBS, 5)
        line["roofline"] = {
            "bound": "mfma", "achieved": round(prim["kernel_tflops"], 3), "peak": PEAK_FP32_MFMA_TFLOPS,
            "unit": "TFLOP/s", "frac": round(prim["kernel_tflops"] / PEAK_FP32_MFMA_TFLOPS, 4),
            "traffic": None,
            "kernel": "grouped_stream_kernel (one launch per step)",
            "launch_ms": round(prim["launch_ms"], 5),
            "weight_gbs_in_kernel": round(prim["kernel_weight_gbs"], 2),
        }
    if "m65536" in out:
        line["m65536"] = {k: (round(v, 5) if isinstance(v, float) else v) for k, v in out["m65536"].items()}
        line["m65536"]["steps"] = args.steps_large
    if not args.no_cpu_baseline and prim:
        line["cpu_baseline"] = cpu_baseline(4, synth.M_GOLDEN, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
