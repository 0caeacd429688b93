"""GPU test of the allocation-free entry point rtq_block_project_noalloc,
called through the C ABI: its outputs equal rtq_block_project_ex's bit for
bit (and meet the oracle's bar) on two calls in a row, the second with a
smaller input, on the grouped small-M route (workspace in the scratch
array), the tiled large-M route and the direct route (no workspace); a call
whose workspace exceeds the scratch is rejected before anything runs.
"""
from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import synth  # noqa: E402
import weight_only_quantized_rtq_amd as rtq  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SHAPE = 2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def make_blocks(seed, n_blocks, M, names=synth.PROJ_ORDER):
    """Quantized weights, inputs and two sets of outputs (for the two entry points)."""
    blocks, blocks2, refs = [], [], []
    for b in range(n_blocks):
        xs = {n: synth.activation(seed, b, n, M) for n in synth.INPUT_WIDTH}
        dx = {n: torch.from_numpy(v).to(DEV) for n, v in xs.items()}
        blk, blk2, ref = {}, {}, {}
        for name in names:
            N, K, xin = synth.BLOCK_SHAPES[name]
            W = synth.weight(seed, 0, b, name)
            fmt = rtq.RECIPE_MIXED[name]
            w = rtq.quantize(torch.from_numpy(W).to(DEV), fmt)
            blk[name] = rtq.Projection(w, dx[xin], torch.full((M, N), np.nan, dtype=torch.float32, device=DEV))
            blk2[name] = rtq.Projection(w, dx[xin], torch.full((M, N), np.nan, dtype=torch.float32, device=DEV))
            ref[name] = (fmt, oracle.quantize(W, fmt), xs[xin])
        blocks.append(blk)
        blocks2.append(blk2)
        refs.append(ref)
    return blocks, blocks2, refs


def run_both(blocks, blocks2, M, math):
    lib = rtq.load_library()
    st = torch.cuda.current_stream().cuda_stream
    arr, _k = rtq.pack_blocks(blocks, M)
    arr2, _k2 = rtq.pack_blocks(blocks2, M)
    assert lib.rtq_block_project_ex(arr, len(arr), M, math, st) == 0, lib.rtq_last_error()
    assert lib.rtq_block_project_noalloc(arr2, len(arr2), M, math, st) == 0, lib.rtq_last_error()
    torch.cuda.synchronize()


@pytest.mark.parametrize("math", [rtq.MATH_SPLIT_BF16, rtq.MATH_SPLIT_F16, rtq.MATH_BF16, rtq.MATH_FP32_MFMA])
def test_noalloc_equals_block_project_on_two_calls(math):
    # call 1: the 12-block projection set at M = 80 (grouped route, workspace
    # in the scratch); call 2: a smaller input, 3 blocks at M = 40
    for seed, n_blocks, M in ((81, 12, 80), (82, 3, 40)):
        say(f"noalloc math={math} blocks={n_blocks} M={M}")
        blocks, blocks2, refs = make_blocks(seed, n_blocks, M)
        run_both(blocks, blocks2, M, math)
        for b in range(n_blocks):
            for name in synth.PROJ_ORDER:
                y = blocks[b][name].y.cpu().numpy()
                y2 = blocks2[b][name].y.cpu().numpy()
                assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), (b, name)
                if b in (0, n_blocks - 1):
                    fmt, r, x = refs[b][name]
                    want = oracle.project_bf16(fmt, x, *r) if math == rtq.MATH_BF16 else oracle.project(fmt, x, *r)
                    assert oracle.rel_fro(y2, want) <= 1e-5, (b, name)


@pytest.mark.parametrize("M", [300, 16])
def test_noalloc_tiled_and_direct_routes(M):
    # M = 300: the tiled route (images in the scratch); M = 16: the direct
    # kernel (no workspace); then a smaller call of each route
    for seed, Mc in ((83, M), (84, M // 2)):
        say(f"noalloc routes M={Mc}")
        blocks, blocks2, refs = make_blocks(seed, 1, Mc, names=("wq", "wo", "w1", "w2"))
        run_both(blocks, blocks2, Mc, rtq.MATH_SPLIT_F16)
        for name in ("wq", "wo", "w1", "w2"):
            y = blocks[0][name].y.cpu().numpy()
            y2 = blocks2[0][name].y.cpu().numpy()
            assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), name
            fmt, r, x = refs[0][name]
            assert oracle.rel_fro(y2, oracle.project(fmt, x, *r)) <= 1e-5, name


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    # 4 blocks at M = 2000 need well over 32 MiB of limb images: rejected,
    # nothing launched (the outputs keep their NaN fill)
    M = 2000
    blocks, blocks2, _ = make_blocks(85, 4, M, names=("wq", "w2"))
    lib = rtq.load_library()
    arr2, _k = rtq.pack_blocks(blocks2, M)
    st = torch.cuda.current_stream().cuda_stream
    assert lib.rtq_block_project_noalloc(arr2, len(arr2), M, rtq.MATH_SPLIT_BF16, st) == SHAPE
    assert b"scratch" in lib.rtq_last_error()
    torch.cuda.synchronize()
    for blk in blocks2:
        for p in blk.values():
            assert torch.isnan(p.y).all().item()
    # the same call in an arithmetic that needs no workspace runs
    assert lib.rtq_block_project_noalloc(arr2, len(arr2), M, rtq.MATH_FP32_MFMA, st) == 0
    torch.cuda.synchronize()
    assert torch.isfinite(blocks2[0]["wq"].y).all().item()
