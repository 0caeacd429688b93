"""GPU parity of the direct small-M path (M <= 32 and K in {256, 512, 1024,
2048}): one launch, whole K per workgroup, x stages built in the kernel, one
or two row tiles. Checked against the oracle in every arithmetic mode (the
bf16 mode against its own bf16(x) reference at 1e-5 and fp32 x at 3e-3), at
ragged N, every K the path takes, M from 1 to 32 on both sides of the row tile
boundary, with and without biases, and through the block projection at the
benchmark's shapes. The cases with M above 32 check the hand-off to the
grouped kernel (pre-pass, K chunks) at the same shapes."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import synth  # noqa: E402
import weight_only_quantized_rtq_amd as rtq  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MODES = {"split_bf16": rtq.MATH_SPLIT_BF16, "fp32_mfma": rtq.MATH_FP32_MFMA, "bf16": rtq.MATH_BF16,
         "split_f16": rtq.MATH_SPLIT_F16}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.fixture(params=list(MODES), ids=list(MODES))
def mode(request):
    """Arithmetic of the calls (its name; MODES gives the value passed to each call)."""
    return request.param


def check(y, mode, fmt, x, ref, b=None):
    bias = 0.0 if b is None else b.astype(np.float64)[None, :]
    if mode == "bf16":
        tight = oracle.rel_fro(y, oracle.project_bf16(fmt, x, *ref) + bias)
        assert tight <= 1e-5, ("against bf16(x)", tight)
        loose = oracle.rel_fro(y, oracle.project(fmt, x, *ref) + bias)
        assert loose <= 3e-3, ("against fp32 x", loose)
    else:
        err = oracle.rel_fro(y, oracle.project(fmt, x, *ref) + bias)
        assert err <= 1e-5, err


CASES = [(fmt, M, N, K) for fmt in ("q4", "q8", "f8")
         for (M, N, K) in [(1, 512, 512), (3, 100, 256), (5, 300, 1024), (16, 520, 2048), (8, 64, 2048),
                           (16, 257, 512), (2, 17, 1024),
                           (17, 300, 512), (32, 257, 1024), (33, 100, 2048), (48, 520, 256),
                           (49, 64, 512), (64, 130, 2048), (80, 512, 512), (80, 96, 1024), (79, 33, 256)]]


@pytest.mark.parametrize("fmt,M,N,K", CASES)
def test_direct_gemm_parity(fmt, M, N, K, mode):
    say(f"direct {fmt} M={M} N={N} K={K} mode={mode}")
    W = synth.weight(61, 0, 0, "w1", N, K, heavy="rows")
    x = synth.activation(61, 0, "x_ffn", M, K)
    ref = oracle.quantize(W, fmt)
    y = host(rtq.gemm(dev(x), rtq.quantize(dev(W), fmt), math=MODES[mode]))
    check(y, mode, fmt, x, ref)


@pytest.mark.parametrize("M", [1, 16, 40, 80])
def test_direct_block_project_twelve_blocks_with_biases(M, mode):
    """The benchmark's 12 blocks (mixed recipe) at small M, biases on half the
    projections, every output checked."""
    say(f"direct 12 blocks M={M} mode={mode}")
    blocks, refs = [], []
    for b in range(synth.NUM_BLOCKS):
        xs = {n: synth.activation(62, b, n, M) for n in synth.INPUT_WIDTH}
        dxs = {n: dev(v) for n, v in xs.items()}
        blk, ref = {}, {}
        for j, name in enumerate(synth.PROJ_ORDER):
            N, K, xin = synth.BLOCK_SHAPES[name]
            W = synth.weight(62, 0, b, name)
            fmt = rtq.RECIPE_MIXED[name]
            bias = synth.activation(63, b, "h", 1, N)[0] if (b + j) % 2 == 0 else None
            blk[name] = rtq.Projection(rtq.quantize(dev(W), fmt), dxs[xin],
                                       torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV),
                                       None if bias is None else dev(bias))
            ref[name] = (fmt, oracle.quantize(W, fmt), xs[xin], bias)
        blocks.append(blk)
        refs.append(ref)
    rtq.block_project(blocks, M, math=MODES[mode])
    for b in range(synth.NUM_BLOCKS):
        for name, (fmt, r, x, bias) in refs[b].items():
            check(host(blocks[b][name].y), mode, fmt, x, r, bias)


@pytest.mark.parametrize("M", [16, 80])
def test_direct_exact_integer_and_identity(M):
    """Integer x and dyadic (scale, min): bit-exact; x = rows of I: y = W^T rows, bit for bit."""
    N, K = 256, 512
    x = synth.uniform_ints(M, (M, K), -4, 4).astype(np.float32)
    payload = synth.uniform_bytes(N, (N, K // 2))
    pairs = np.zeros((N, K // 32, 2), dtype=np.float16)
    pairs[..., 0] = 0.25
    pairs[..., 1] = -2.0
    y = host(rtq.gemm_q4(dev(x), rtq.Q4Weight(dev(payload), dev(pairs))))
    assert np.array_equal(y.astype(np.float64), oracle.project_q4(x, payload, pairs))
    W = synth.weight(64, 0, 0, "wq", 96, 256, heavy="rows")
    for fmt in ("q4", "q8", "f8"):
        ref = oracle.quantize(W, fmt)
        eye = np.eye(256, dtype=np.float32)
        for r0 in (0, 256 - M):                           # two M-row windows of the identity
            yi = host(rtq.gemm(dev(eye[r0:r0 + M]), rtq.quantize(dev(W), fmt)))
            want = np.ascontiguousarray(oracle.dequant(fmt, *ref).T[r0:r0 + M])
            assert np.array_equal(yi, want), fmt


@pytest.mark.parametrize("M", [8, 80])
def test_direct_full_size_weight_sets_sampled(M):
    """The benchmark's weight-set shapes (12 blocks, two of the 16 sets) at M = 8
    and at M = 80, the benchmark's own launch configuration, sampled outputs
    against the oracle."""
    rng = np.random.default_rng(65)
    for s in (0, 15):
        blocks, refs = [], []
        for b in range(synth.NUM_BLOCKS):
            xs = {n: synth.activation(4, b, n, M) for n in synth.INPUT_WIDTH}
            dxs = {n: dev(v) for n, v in xs.items()}
            blk, ref = {}, {}
            for name in synth.PROJ_ORDER:
                N, K, xin = synth.BLOCK_SHAPES[name]
                W = synth.weight(4, s, b, name)
                fmt = rtq.RECIPE_MIXED[name]
                blk[name] = rtq.Projection(rtq.quantize(dev(W), fmt), dxs[xin],
                                           torch.empty((M, N), dtype=torch.float32, device=DEV))
                ref[name] = (fmt, W, xs[xin])
            blocks.append(blk)
            refs.append(ref)
        rtq.block_project(blocks, M)
        torch.cuda.synchronize()
        for b in range(synth.NUM_BLOCKS):
            for name, (fmt, W, x) in refs[b].items():
                cols = np.sort(rng.choice(W.shape[0], 32, replace=False))
                ref_w = oracle.quantize(W[cols], fmt)
                y = host(blocks[b][name].y[:, torch.as_tensor(cols, device=DEV)])
                assert oracle.rel_fro(y, oracle.project(fmt, x, *ref_w)) <= 1e-5, (s, b, name)


def test_direct_call_with_a_k_it_does_not_take_runs_grouped():
    """A call is routed as a whole: with one K outside {256, 512, 1024, 2048}
    (here 96) every projection takes the pre-pass + grouped path, at M <= 32."""
    M = 8
    shapes = {"wq": (100, 512), "wk": (64, 96), "w2": (70, 2048)}
    blk, ref = {}, {}
    for j, (name, (N, K)) in enumerate(shapes.items()):
        fmt = ("q4", "q8", "f8")[j]
        W = synth.weight(66, 0, j, "w1", N, K, heavy="rows")
        x = synth.activation(66, j, "x_ffn", M, K)
        blk[name] = rtq.Projection(rtq.quantize(dev(W), fmt), dev(x),
                                   torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV))
        ref[name] = (fmt, oracle.quantize(W, fmt), x)
    rtq.block_project([blk], M)
    for name, (fmt, r, x) in ref.items():
        assert oracle.rel_fro(host(blk[name].y), oracle.project(fmt, x, *r)) <= 1e-5, name


@pytest.mark.parametrize("M", [3, 20])
def test_direct_call_split_over_launches(M):
    """13 blocks of small projections: 104 projections reading 52 distinct
    inputs, more than one launch's argument block holds (96 and 48), so the
    call runs as several direct launches; every output checked."""
    nb = 13
    blocks, refs = [], []
    for b in range(nb):
        xs = {i: synth.activation(67, 4 * b + i, "x_ffn", M, 256 if i % 2 else 512) for i in range(4)}
        dxs = {i: dev(v) for i, v in xs.items()}
        blk, ref = {}, {}
        for j, name in enumerate(("wq", "wk", "wv", "wg", "wo", "w1", "w3", "w2")):
            N, K = 64 + 16 * (j % 3), (256 if j % 2 else 512)
            fmt = ("q4", "q8", "f8")[(b + j) % 3]
            W = synth.weight(67, b, j, "w1", N, K, heavy="rows")
            blk[name] = rtq.Projection(rtq.quantize(dev(W), fmt), dxs[j % 4],
                                       torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV))
            ref[name] = (fmt, oracle.quantize(W, fmt), xs[j % 4])
        blocks.append(blk)
        refs.append(ref)
    rtq.block_project(blocks, M)
    for b in range(nb):
        for name, (fmt, r, x) in refs[b].items():
            assert oracle.rel_fro(host(blocks[b][name].y), oracle.project(fmt, x, *r)) <= 1e-5, (b, name)


@pytest.mark.parametrize("fmt,K", [("q4", 512), ("q8", 2048), ("f8", 1024), ("q4", 256)])
@pytest.mark.parametrize("M", [1, 30])
def test_direct_guard_bands_and_determinism(fmt, K, M, mode):
    """Outputs land only inside y (canaries around it survive, also past the
    ragged last column block) and a rerun is bitwise identical: the direct
    kernel has no atomics and a fixed summation order."""
    N = 130
    W = synth.weight(68, 0, 0, "w1", N, K, heavy="rows")
    x = dev(synth.activation(68, 0, "x_ffn", M, K))
    w = rtq.quantize(dev(W), fmt)
    guard = 4096
    buf = torch.full((guard + M * N + guard,), 1234.5, dtype=torch.float32, device=DEV)
    y = buf[guard:guard + M * N].view(M, N)
    rtq.gemm(x, w, y=y, math=MODES[mode])
    y1 = host(y).copy()
    b = host(buf)
    assert np.all(b[:guard] == 1234.5) and np.all(b[guard + M * N:] == 1234.5)
    rtq.gemm(x, w, y=y, math=MODES[mode])
    assert np.array_equal(host(y).view(np.uint32), y1.view(np.uint32))


@pytest.mark.parametrize("M", [1, 20])
def test_direct_int4_pairs_not_16_byte_aligned(M, mode):
    """The direct kernel reads int4 (scale, min) words 16 bytes at a time, so a
    pair array that is only 4-byte aligned (the ABI's minimum) sends the call
    to the grouped path; the result is the same."""
    N, K = 512, 512          # the bf16 mode's fp32-x bar is statistical: full-width outputs
    W = synth.weight(69, 0, 0, "w1", N, K)
    x = synth.activation(69, 0, "x_ffn", M, K)
    ref = oracle.quantize(W, "q4")
    payload = dev(ref[0])
    buf = torch.empty(N * (K // 32) * 2 + 2, dtype=torch.float16, device=DEV)
    pairs = buf[2:].view(N, K // 32, 2)                           # 4 bytes past a 16-byte boundary
    pairs.copy_(dev(ref[1]))
    assert pairs.data_ptr() % 16 == 4
    y = host(rtq.gemm(dev(x), rtq.Q4Weight(payload, pairs), math=MODES[mode]))
    check(y, mode, "q4", x, ref)
