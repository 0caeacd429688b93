"""GPU parity of the bf16-activation mode (RTQ_MATH_BF16, passed to every call).

In this mode x is rounded once to the nearest bf16 and the kernels compute
y = bf16(x) . W^T with exact weight-side products and fp32 accumulation. Two
bars, both against the CPU oracle on the same seeded inputs:
  * rel. Frobenius <= 1e-5 against oracle.project_bf16 (the same rounded x,
    fp64 GEMM): pins the rounding and everything after it;
  * rel. Frobenius <= 3e-3 against oracle.project (fp32 x): the accuracy bar of
    a bf16-activation path.
Shapes the split kernels do not take run on the fp32 kernels in every mode;
they meet the fp32 bar (1e-5 against oracle.project).
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import synth  # noqa: E402
import weight_only_quantized_rtq_amd as rtq  # noqa: E402

pytestmark = pytest.mark.gpu
MATH = rtq.MATH_BF16          # the arithmetic every call below passes

TIGHT = 1e-5
BAR = 3e-3
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()




def check(y, fmt, x, ref):
    tight = oracle.rel_fro(y, oracle.project_bf16(fmt, x, *ref))
    loose = oracle.rel_fro(y, oracle.project(fmt, x, *ref))
    assert tight <= TIGHT, ("against bf16(x)", tight)
    assert loose <= BAR, ("against fp32 x", loose)
    return tight, loose


SHAPES = {
    "q4": [(80, 512, 512), (1, 64, 32), (17, 40, 96), (77, 130, 544), (81, 200, 256), (300, 129, 64),
           (129, 128, 1024), (256, 256, 2048)],
    "q8": [(80, 512, 512), (80, 512, 2048), (5, 3, 32), (200, 130, 96), (257, 129, 2048)],
    "f8": [(80, 512, 512), (80, 512, 2048), (33, 70, 64), (300, 129, 64), (257, 129, 2048)],
}
CASES = [(fmt, *s) for fmt, shapes in SHAPES.items() for s in shapes]


@pytest.mark.parametrize("fmt,M,N,K", CASES)
def test_gemm_bf16_parity(fmt, M, N, K):
    say(f"bf16 gemm {fmt} M={M} N={N} K={K}")
    W = synth.weight(31, 0, 0, "w1", N, K, heavy="rows")
    x = synth.activation(31, 0, "x_ffn", M, K)
    ref = oracle.quantize(W, fmt)
    w = rtq.quantize(dev(W), fmt)
    y = host(rtq.gemm(dev(x), w, math=MATH))
    tight, loose = check(y, fmt, x, ref)
    say(f"  rel err vs bf16(x) {tight:.2e}, vs fp32 x {loose:.2e}")


def test_bf16_mode_rounds_the_activations():
    """x chosen off the bf16 grid: the result follows bf16(x), not x."""
    M, N, K = 80, 256, 512
    W = synth.weight(32, 0, 0, "wq", N, K)
    x = synth.activation(32, 0, "x_attn", M, K)
    x_off = (x.view(np.uint32) | np.uint32(0x5555)).view(np.float32)      # low bits set everywhere
    ref = oracle.quantize(W, "q4")
    y = host(rtq.gemm(dev(x_off), rtq.quantize(dev(W), "q4"), math=MATH))
    assert oracle.rel_fro(y, oracle.project_bf16("q4", x_off, *ref)) <= TIGHT
    assert oracle.rel_fro(y, oracle.project("q4", x_off, *ref)) > 1e-4


@pytest.mark.parametrize("fmt,K", [("q4", 64), ("q4", 512), ("q8", 160), ("f8", 64)])
def test_bf16_identity_is_bit_exact(fmt, K):
    """x = I is exact in bf16, so y = W^T bit for bit (zeros by value)."""
    N = 72
    W = synth.weight(33, 0, 0, "wv", N, K, heavy="rows")
    ref = oracle.quantize(W, fmt)
    y = host(rtq.gemm(dev(np.eye(K, dtype=np.float32)), rtq.quantize(dev(W), fmt), math=MATH))
    want = np.ascontiguousarray(oracle.dequant(fmt, *ref).T)
    assert np.array_equal(y, want)
    nz = want != 0
    assert np.array_equal(y[nz].view(np.uint32), want[nz].view(np.uint32))


def test_bf16_exact_integer_arithmetic():
    """Small integer x is exact in bf16 and every partial sum is exact in fp32."""
    M, N, K = 80, 512, 512
    x = synth.uniform_ints(M, (M, K), -4, 4).astype(np.float32)
    payload = synth.uniform_bytes(N, (N, K // 2))
    pairs = np.zeros((N, K // 32, 2), dtype=np.float16)
    pairs[..., 0] = 0.25
    pairs[..., 1] = -2.0
    y = host(rtq.gemm_q4(dev(x), rtq.Q4Weight(dev(payload), dev(pairs)), math=MATH))
    assert np.array_equal(y.astype(np.float64), oracle.project_q4(x, payload, pairs))


@pytest.mark.parametrize("fmt,M,N,K", [("q8", 33, 70, 33), ("f8", 5, 3, 7), ("q8", 100, 50, 100)])
def test_bf16_mode_fallback_shapes_stay_fp32(fmt, M, N, K):
    """K not a multiple of 32: the fp32 kernels run, at the fp32 bar."""
    W = synth.weight(34, 0, 0, "wo", N, K)
    x = synth.activation(34, 0, "h", M, K)
    ref = oracle.quantize(W, fmt)
    y = host(rtq.gemm(dev(x), rtq.quantize(dev(W), fmt), math=MATH))
    assert oracle.rel_fro(y, oracle.project(fmt, x, *ref)) <= TIGHT


@pytest.mark.parametrize("recipe_name", ["mixed", "all_q8", "all_f8"])
def test_bf16_block_project_one_block(recipe_name):
    recipe = {"mixed": rtq.RECIPE_MIXED, "all_q8": rtq.RECIPE_ALL_Q8, "all_f8": rtq.RECIPE_ALL_F8}[recipe_name]
    M = 80
    xs = {n: synth.activation(35, 0, n, M) for n in synth.INPUT_WIDTH}
    dxs = {n: dev(v) for n, v in xs.items()}
    blk, refs = {}, {}
    for name in synth.PROJ_ORDER:
        N, K, xin = synth.BLOCK_SHAPES[name]
        W = synth.weight(35, 0, 0, name)
        fmt = recipe[name]
        refs[name] = (fmt, oracle.quantize(W, fmt), xin)
        blk[name] = rtq.Projection(rtq.quantize(dev(W), fmt), dxs[xin],
                                   torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV))
    rtq.block_project([blk], M, math=MATH)
    for name, (fmt, ref, xin) in refs.items():
        check(host(blk[name].y), fmt, xs[xin], ref)


@pytest.mark.parametrize("M", [synth.M_GOLDEN, synth.M_LARGE])
def test_bf16_full_size_twelve_blocks_sampled(M):
    """The benchmark's launch configuration (12 blocks, mixed recipe), outputs
    sampled and computed one by one by the oracle."""
    say(f"bf16 full-size 12 blocks M={M}")
    per_block = M == synth.M_GOLDEN
    shared = None if per_block else {n: synth.activation(36, synth.SHARED_BLOCK, n, M) for n in synth.INPUT_WIDTH}
    blocks, refs_w, xs_all = [], [], []
    for b in range(synth.NUM_BLOCKS):
        xs_host = {n: synth.activation(36, b, n, M) for n in synth.INPUT_WIDTH} if per_block else shared
        xs_dev = {n: dev(v) for n, v in xs_host.items()} if (per_block or b == 0) else xs_dev
        xs_all.append(xs_host)
        blk, rw = {}, {}
        for name in synth.PROJ_ORDER:
            N, K, xin = synth.BLOCK_SHAPES[name]
            W = synth.weight(36, 0, b, name, heavy="rows" if not per_block else None)
            fmt = rtq.RECIPE_MIXED[name]
            blk[name] = rtq.Projection(rtq.quantize(dev(W), fmt), xs_dev[xin],
                                       torch.empty((M, N), dtype=torch.float32, device=DEV))
            rw[name] = (fmt, W)
        blocks.append(blk)
        refs_w.append(rw)
    rtq.block_project(blocks, M, math=MATH)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M + 1)
    worst = [0.0, 0.0]
    for b, blk in enumerate(blocks):
        for name, p in blk.items():
            N, K, xin = synth.BLOCK_SHAPES[name]
            fmt, W = refs_w[b][name]
            rows = np.sort(rng.choice(M, size=min(24, M), replace=False))
            cols = np.sort(rng.choice(N, size=24, replace=False))
            ref_w = oracle.quantize(W[cols], fmt)
            y = host(p.y[torch.as_tensor(rows, device=DEV)][:, torch.as_tensor(cols, device=DEV)])
            t, l = check(y, fmt, xs_all[b][xin][rows], ref_w)
            worst = [max(worst[0], t), max(worst[1], l)]
    say(f"  worst sampled rel err vs bf16(x) {worst[0]:.2e}, vs fp32 x {worst[1]:.2e}")
    del blocks
    torch.cuda.empty_cache()
