"""GPU tests of the caller-workspace entry point rtq_block_project_ws (and the
size query rtq_block_workspace_bytes), through the C ABI.

The call must equal rtq_block_project_ex bit for bit in every arithmetic and
on every route: the grouped launch with K-chunked w2 (12 blocks at M = 80),
the same workspace reused by a second, smaller call (3 blocks at M = 40), the
tiled large-M route (M = 300) and the direct kernel (M = 16, no workspace).
Outputs of the first and last block also meet the oracle's bar, and a call
given too small a workspace launches nothing (its outputs keep their fill).
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import synth  # noqa: E402
import weight_only_quantized_rtq_amd as rtq  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MATHS = [rtq.MATH_SPLIT_F16, rtq.MATH_SPLIT_BF16, rtq.MATH_BF16, rtq.MATH_FP32_MFMA]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def make_blocks(seed, n_blocks, M):
    """Two projection sets over the same weights and inputs with separate
    NaN-filled outputs, and the oracle's inputs."""
    blocks, blocks2, refs = [], [], []
    for b in range(n_blocks):
        xs = {n: synth.activation(seed, b, n, M) for n in synth.INPUT_WIDTH}
        dx = {n: torch.from_numpy(v).to(DEV) for n, v in xs.items()}
        blk, blk2, ref = {}, {}, {}
        for name in synth.PROJ_ORDER:
            N, K, xin = synth.BLOCK_SHAPES[name]
            W = synth.weight(seed, 0, b, name)
            fmt = rtq.RECIPE_MIXED[name]
            w = rtq.quantize(torch.from_numpy(W).to(DEV), fmt)
            blk[name] = rtq.Projection(w, dx[xin], torch.full((M, N), np.nan, dtype=torch.float32, device=DEV))
            blk2[name] = rtq.Projection(w, dx[xin], torch.full((M, N), np.nan, dtype=torch.float32, device=DEV))
            ref[name] = (fmt, W, xs[xin])
        blocks.append(blk)
        blocks2.append(blk2)
        refs.append(ref)
    return blocks, blocks2, refs


def check(blocks, blocks2, refs, math, sampled=(0, -1)):
    n = len(blocks)
    for b in range(n):
        for name in synth.PROJ_ORDER:
            y = blocks[b][name].y.cpu().numpy()
            y2 = blocks2[b][name].y.cpu().numpy()
            assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), (b, name)
    for b in sampled:
        for name in synth.PROJ_ORDER:
            fmt, W, x = refs[b][name]
            packed = oracle.quantize(W, fmt)
            want = oracle.project_bf16(fmt, x, *packed) if math == rtq.MATH_BF16 else oracle.project(fmt, x, *packed)
            err = oracle.rel_fro(blocks2[b][name].y.cpu().numpy(), want)
            assert err <= 1e-5, (b, name, err)


@pytest.mark.parametrize("math", MATHS)
def test_workspace_call_equals_pool_call_on_two_calls(math):
    """One workspace, sized for both calls, serves a 12-block call at M = 80
    and then a 3-block call at M = 40 (whose shorter K chunks need more
    partials per projection)."""
    calls = [(n_blocks, M, make_blocks(seed, n_blocks, M)) for seed, n_blocks, M in ((91, 12, 80), (92, 3, 40))]
    needs = [rtq.block_workspace_bytes(c[2][1], c[1], math) for c in calls]
    if math == rtq.MATH_FP32_MFMA:
        assert needs == [0, 0]
    ws = torch.empty(max(max(needs), 1), dtype=torch.uint8, device=DEV)
    for n_blocks, M, (blocks, blocks2, refs) in calls:
        say(f"workspace math={math} blocks={n_blocks} M={M}")
        rtq.block_project(blocks, M, math=math)
        rtq.block_project(blocks2, M, math=math, workspace=ws)
        torch.cuda.synchronize()
        check(blocks, blocks2, refs, math)


@pytest.mark.parametrize("math", [rtq.MATH_SPLIT_F16, rtq.MATH_BF16])
@pytest.mark.parametrize("M", [300, 16])
def test_workspace_call_on_the_tiled_and_direct_routes(M, math):
    say(f"workspace route M={M} math={math}")
    blocks, blocks2, refs = make_blocks(93, 2, M)
    need = rtq.block_workspace_bytes(blocks2, M, math)
    if M <= 32:
        assert need == 0                                   # the direct kernel splits x itself
        ws = torch.empty(0, dtype=torch.uint8, device=DEV)
    else:
        assert need > 0
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    rtq.block_project(blocks, M, math=math)
    rtq.block_project(blocks2, M, math=math, workspace=ws)
    torch.cuda.synchronize()
    check(blocks, blocks2, refs, math)


def test_too_small_a_workspace_launches_nothing():
    M, math = 80, rtq.MATH_SPLIT_F16
    blocks, _, _ = make_blocks(94, 2, M)
    need = rtq.block_workspace_bytes(blocks, M, math)
    ws = torch.empty(need - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(rtq.RtqError):
        rtq.block_project(blocks, M, math=math, workspace=ws)
    torch.cuda.synchronize()
    for blk in blocks:
        for p in blk.values():
            assert torch.isnan(p.y).all()
