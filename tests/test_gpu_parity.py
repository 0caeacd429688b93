"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bars: bit-exact for the quantizers' codes/pairs/scales, for unpacking and for
dequantized weights; relative Frobenius error <= 1e-5 for the fp32-activation
GEMM output against the fp64 oracle.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import synth  # noqa: E402
import weight_only_quantized_rtq_amd as rtq  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = 1e-5
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.fixture(params=[rtq.MATH_SPLIT_BF16, rtq.MATH_FP32_MFMA, rtq.MATH_SPLIT_F16],
                ids=["split_bf16", "fp32_mfma", "split_f16"])
def math(request):
    """Runs a test under each fp32-activation arithmetic of the GEMM entry points
    (passed to every call; the library keeps no arithmetic state)."""
    return request.param


def gpu_quantize(W: np.ndarray, fmt: str):
    return rtq.quantize(dev(W), fmt)


def assert_same_quant(wg, ref, fmt):
    if fmt == "q4":
        p, s = ref
        assert np.array_equal(host(wg.payload), p), "int4 codes differ"
        assert np.array_equal(host(wg.pairs).view(np.uint16), s.view(np.uint16)), "int4 pairs differ"
    elif fmt == "q8":
        q, s = ref
        assert np.array_equal(host(wg.payload), q), "int8 codes differ"
        assert np.array_equal(host(wg.scale).view(np.uint32), s.view(np.uint32)), "int8 scales differ"
    else:
        codes, _ = ref
        assert np.array_equal(host(wg.payload), codes), "FP8 codes differ"


# ----------------------------------------------------------------------------
# Quantizers: bit-exact.
# ----------------------------------------------------------------------------
def _edge_weights(N, K, seed):
    W = synth.weight(7, seed, 0, "wq", N, K)
    W[0, :] = 0.0                                  # all-zero row / groups
    W[1, :32] = 0.125                              # constant group
    W[2, :] *= 1e-6                                # tiny: fp16 subnormal scales
    W[3, :] = np.float32(2.0 ** -30)               # below fp16 range
    W[4, ::2] *= 500.0                             # large dynamic range
    if K >= 64:
        W[5, 32:64] = np.linspace(-1, 1, 32, dtype=np.float32)   # exact grid-ish
    return W


@pytest.mark.parametrize("N,K,heavy", [(512, 512, None), (64, 2048, "rows"), (96, 512, "cols"), (7, 32, None)])
def test_quantize_q4_bit_exact(N, K, heavy):
    say(f"quantize_q4 N={N} K={K} heavy={heavy}")
    W = synth.weight(1, 0, 0, "w1", N, K, heavy=heavy)
    assert_same_quant(gpu_quantize(W, "q4"), oracle.quantize_q4(W), "q4")


def test_quantize_q4_edge_cases():
    W = _edge_weights(16, 128, 3)
    assert_same_quant(gpu_quantize(W, "q4"), oracle.quantize_q4(W), "q4")


@pytest.mark.parametrize("N,K,heavy", [(512, 512, None), (512, 2048, "rows"), (33, 100, None), (5, 7, None)])
def test_quantize_q8_bit_exact(N, K, heavy):
    say(f"quantize_q8 N={N} K={K} heavy={heavy}")
    W = synth.weight(2, 0, 0, "wo", N, K, heavy=heavy)
    assert_same_quant(gpu_quantize(W, "q8"), oracle.quantize_q8(W), "q8")


def test_quantize_q8_edge_cases():
    W = _edge_weights(16, 96, 4)
    W[6, :] = np.float32(1e-39)                    # subnormal fp32 row
    W[7, :4] = [127, -63.5, 1, 0.25]               # halves round to even
    assert_same_quant(gpu_quantize(W, "q8"), oracle.quantize_q8(W), "q8")


@pytest.mark.parametrize("N,K,heavy", [(512, 512, None), (512, 2048, "rows"), (33, 100, "cols"), (5, 7, None)])
def test_quantize_f8_bit_exact(N, K, heavy):
    say(f"quantize_f8 N={N} K={K} heavy={heavy}")
    W = synth.weight(16, 0, 0, "wq", N, K, heavy=heavy)
    assert_same_quant(gpu_quantize(W, "f8"), (oracle.quantize_f8(W), None), "f8")


def test_quantize_f8_edge_cases():
    """Ties, the subnormal range, the 448/464/480 overflow boundary, signed
    zeros, infinities and NaN (PyTorch's float8_e4m3fn cast semantics)."""
    specials = np.array([0.0, -0.0, 448, 449, 463.99997, 464, 464.00003, 480, 1e9, np.inf, -np.inf, np.nan,
                         -448, -465, 2 ** -9, 2 ** -10, 3 * 2 ** -11, 7.5 * 2 ** -9, 2 ** -6, 1.0625, 1.1875,
                         17, 19, -19, 1e-39, -1e-39, 2 ** -149, 0.0146484375], dtype=np.float32)
    W = np.resize(specials, (8, 64)).astype(np.float32)
    W[4:] = synth.weight(16, 1, 0, "wk", 4, 64) * np.float32(10.0) ** np.arange(-3, 1, dtype=np.float32)[:, None]
    assert_same_quant(gpu_quantize(W, "f8"), (oracle.quantize_f8(W), None), "f8")


# ----------------------------------------------------------------------------
# Unpacking and dequantization: bit-exact.
# ----------------------------------------------------------------------------
def _random_pairs(seed, shape):
    bits = synth.uniform_ints(seed, shape, 0, 0xFFFF).astype(np.uint16)
    exp = (bits >> 10) & 0x1F
    bits = np.where(exp == 0x1F, bits & ~np.uint16(0x4000), bits)    # no inf/nan
    return bits.view(np.float16)


@pytest.mark.parametrize("N,K", [(512, 512), (3, 32), (130, 2048)])
def test_dequant_q4_bit_exact(N, K):
    payload = synth.uniform_bytes(N + K, (N, K // 2))
    pairs = _random_pairs(N * K, (N, K // 32, 2))
    got = host(rtq.dequant(rtq.Q4Weight(dev(payload), dev(pairs))))
    want = oracle.dequant_q4(payload, pairs)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_unpack_probe_bit_exact():
    """(scale, min) = (1, 0) makes the dequantized weight the raw nibble."""
    payload = np.arange(256, dtype=np.uint8).reshape(16, 16).repeat(2, axis=0)   # [32, 16], K = 32
    pairs = np.zeros((32, 1, 2), dtype=np.float16)
    pairs[..., 0] = 1.0
    got = host(rtq.dequant(rtq.Q4Weight(dev(payload), dev(pairs))))
    assert np.array_equal(got, oracle.unpack_q4(payload).astype(np.float32))


@pytest.mark.parametrize("N,K", [(512, 512), (5, 7), (64, 2048)])
def test_dequant_q8_bit_exact(N, K):
    q = synth.uniform_ints(N, (N, K), -127, 127).astype(np.int8)
    scale = (synth.activation(5, 0, "x_o", 1, N)[0] * 0.01).astype(np.float32)
    scale[0] = np.float32(1e-40)                    # subnormal scale
    got = host(rtq.dequant(rtq.Q8Weight(dev(q), dev(scale))))
    want = oracle.dequant_q8(q, scale)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("N,K", [(16, 16), (512, 512), (7, 33)])
def test_dequant_f8_bit_exact(N, K):
    """Every E4M3 code decodes to its exact value (NaN codes to NaN)."""
    codes = np.resize(np.arange(256, dtype=np.uint8), (N, K)) if N * K <= 256 else \
        synth.uniform_bytes(N * K, (N, K))
    got = host(rtq.dequant(rtq.F8Weight(dev(codes))))
    want = oracle.dequant_f8(codes)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


# ----------------------------------------------------------------------------
# GEMM parity.
# ----------------------------------------------------------------------------
# The grouped small-M workgroup covers 256 columns with eight waves of two
# 16-column tiles: N = 16 leaves all but one wave without a live column,
# N = 272 is one workgroup plus a single tile.
Q4_SHAPES = [(80, 512, 512), (1, 64, 32), (17, 40, 96), (77, 130, 544), (81, 200, 256),
             (300, 129, 64), (129, 128, 1024), (256, 256, 2048), (40, 16, 512), (48, 272, 1024)]
Q8_SHAPES = [(80, 512, 512), (80, 512, 2048), (33, 70, 33), (100, 50, 100), (5, 3, 7),
             (200, 130, 96), (257, 129, 2048), (40, 16, 2048), (64, 272, 512)]


@pytest.mark.parametrize("M,N,K", Q4_SHAPES)
def test_gemm_q4_parity(M, N, K, math):
    say(f"gemm_q4 M={M} N={N} K={K} math={math}")
    W = synth.weight(11, 0, 0, "wq", N, K)
    x = synth.activation(11, 0, "x_attn", M, K)
    ref = oracle.quantize_q4(W)
    w = gpu_quantize(W, "q4")
    assert_same_quant(w, ref, "q4")
    y = host(rtq.gemm_q4(dev(x), w, math=math))
    err = oracle.rel_fro(y, oracle.project_q4(x, *ref))
    assert err <= TOL, err


@pytest.mark.parametrize("M,N,K", Q8_SHAPES)
def test_gemm_q8_parity(M, N, K, math):
    say(f"gemm_q8 M={M} N={N} K={K} math={math}")
    W = synth.weight(12, 0, 0, "w2", N, K, heavy="rows")
    x = synth.activation(12, 0, "h", M, K)
    ref = oracle.quantize_q8(W)
    w = gpu_quantize(W, "q8")
    assert_same_quant(w, ref, "q8")
    y = host(rtq.gemm_q8(dev(x), w, math=math))
    err = oracle.rel_fro(y, oracle.project_q8(x, *ref))
    assert err <= TOL, err


@pytest.mark.parametrize("fmt,K", [("q4", 64), ("q4", 96), ("q4", 512), ("q8", 64), ("q8", 160), ("q8", 40),
                                   ("f8", 64), ("f8", 40)])
def test_gemm_identity_is_bit_exact(fmt, K, math):
    """x = I_K gives y = W^T exactly: checks the in-GEMM unpack/dequant bit for
    bit. Zeros compare by value: a -0 weight (FP8 code 0x80) sums to +0 in any
    IEEE dot product, the oracle's included; the signed zero itself is checked
    by the dequant tests."""
    say(f"identity {fmt} K={K} math={math}")
    N = 72
    W = synth.weight(13, 0, 0, "wv", N, K, heavy="rows")
    ref = oracle.quantize(W, fmt)
    w = gpu_quantize(W, fmt)
    assert_same_quant(w, ref, fmt)
    y = host(rtq.gemm(dev(np.eye(K, dtype=np.float32)), w, math=math))
    want = np.ascontiguousarray(oracle.dequant(fmt, *ref).T)
    assert np.array_equal(y, want)
    nz = want != 0
    assert np.array_equal(y[nz].view(np.uint32), want[nz].view(np.uint32))


F8_SHAPES = [(80, 512, 512), (80, 512, 2048), (33, 70, 33), (5, 3, 7), (257, 129, 2048), (300, 129, 64),
             (40, 16, 512), (80, 272, 1024)]


@pytest.mark.parametrize("M,N,K", F8_SHAPES)
def test_gemm_f8_parity(M, N, K, math):
    say(f"gemm_f8 M={M} N={N} K={K} math={math}")
    W = synth.weight(17, 0, 0, "w1", N, K, heavy="rows")
    x = synth.activation(17, 0, "x_ffn", M, K)
    codes = oracle.quantize_f8(W)
    w = gpu_quantize(W, "f8")
    assert_same_quant(w, (codes, None), "f8")
    y = host(rtq.gemm_f8(dev(x), w, math=math))
    err = oracle.rel_fro(y, oracle.project_f8(x, codes))
    assert err <= TOL, err


@pytest.mark.parametrize("M,N,K", [(80, 512, 512), (200, 96, 2048)])
def test_gemm_exact_integer_arithmetic(M, N, K, math):
    """Integer x and dyadic (scale, min): every partial sum is exact in fp32, so
    any summation order must reproduce the oracle bit for bit."""
    x = synth.uniform_ints(M, (M, K), -4, 4).astype(np.float32)
    payload = synth.uniform_bytes(N, (N, K // 2))
    pairs = np.zeros((N, K // 32, 2), dtype=np.float16)
    pairs[..., 0] = 0.25
    pairs[..., 1] = -2.0
    y = host(rtq.gemm_q4(dev(x), rtq.Q4Weight(dev(payload), dev(pairs)), math=math))
    want = oracle.project_q4(x, payload, pairs)
    assert np.array_equal(y.astype(np.float64), want)
    q = synth.uniform_ints(N + 1, (N, K), -127, 127).astype(np.int8)
    scale = np.full(N, 0.5, dtype=np.float32)
    y8 = host(rtq.gemm_q8(dev(x), rtq.Q8Weight(dev(q), dev(scale)), math=math))
    assert np.array_equal(y8.astype(np.float64), oracle.project_q8(x, q, scale))


def test_gemm_guard_bands_and_determinism(math):
    """Outputs land only inside y (canaries around it survive) and a rerun is
    bitwise identical (no atomics, fixed reduction order)."""
    M, N, K = 77, 130, 512
    W = synth.weight(14, 0, 0, "w3", N, K)
    x = dev(synth.activation(14, 0, "x_ffn", M, K))
    w = gpu_quantize(W, "q4")
    guard = 4096
    buf = torch.full((guard + M * N + guard,), 1234.5, dtype=torch.float32, device=DEV)
    y = buf[guard:guard + M * N].view(M, N)
    rtq.gemm_q4(x, w, y=y, math=math)
    y1 = host(y).copy()
    b = host(buf)
    assert np.all(b[:guard] == 1234.5) and np.all(b[guard + M * N:] == 1234.5)
    rtq.gemm_q4(x, w, y=y, math=math)
    assert np.array_equal(host(y).view(np.uint32), y1.view(np.uint32))


def test_gemm_m_zero_and_errors():
    w = gpu_quantize(synth.weight(15, 0, 0, "wq", 64, 64), "q4")
    y = rtq.gemm_q4(dev(np.zeros((0, 64), np.float32)), w)
    assert tuple(y.shape) == (0, 64)
    with pytest.raises(rtq.RtqError, match="ALIGN"):
        xbig = torch.zeros(4 * 64 + 1, device=DEV)
        rtq.load_library()
        rtq._check(rtq.load_library().rtq_gemm_q4(xbig.data_ptr() + 4, w.payload.data_ptr(),
                                                  w.pairs.data_ptr(), torch.empty(4, 64, device=DEV).data_ptr(),
                                                  4, 64, 64, rtq._stream(None)))


# ----------------------------------------------------------------------------
# Block projection.
# ----------------------------------------------------------------------------
def make_block(cfg, set_, b, M, recipe, xs=None, heavy=None, skip=()):
    """GPU-quantized weights of one block plus the oracle's own quantization."""
    blk, refs = {}, {}
    if xs is None:
        xs = {n: synth.activation(cfg, b, n, M) for n in synth.INPUT_WIDTH}
    dxs = {n: dev(v) for n, v in xs.items()}
    for name in synth.PROJ_ORDER:
        if name in skip:
            continue
        N, K, xin = synth.BLOCK_SHAPES[name]
        W = synth.weight(cfg, set_, b, name, heavy=heavy)
        fmt = recipe[name]
        w = gpu_quantize(W, fmt)
        refs[name] = (fmt, oracle.quantize(W, fmt), xin)
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        blk[name] = rtq.Projection(w, dxs[xin], y)
    return blk, refs, xs


@pytest.mark.parametrize("recipe_name", ["mixed", "all_q8", "all_f8"])
def test_block_project_one_block(recipe_name, math):
    say(f"block_project one block recipe={recipe_name}")
    recipe = {"mixed": rtq.RECIPE_MIXED, "all_q8": rtq.RECIPE_ALL_Q8, "all_f8": rtq.RECIPE_ALL_F8}[recipe_name]
    assert recipe == {"mixed": oracle.RECIPE_MIXED, "all_q8": oracle.RECIPE_ALL_Q8,
                      "all_f8": oracle.RECIPE_ALL_F8}[recipe_name]
    M = 80
    blk, refs, xs = make_block(3, 0, 0, M, recipe)
    rtq.block_project([blk], M, math=math)
    for name, (fmt, ref, xin) in refs.items():
        assert_same_quant(blk[name].weight, ref, fmt)
        err = oracle.rel_fro(host(blk[name].y), oracle.project(fmt, xs[xin], *ref))
        assert err <= TOL, (name, err)


def test_block_project_skips_missing_gate_and_runs_multi_tile(math):
    """A block without wg (ungated attention) leaves nothing behind for it, and
    M above one row tile goes through the per-projection launches."""
    for M in (80, 333):
        say(f"block_project two blocks M={M}")
        blocks, refss, xss = [], [], []
        for b in range(2):
            blk, refs, xs = make_block(4, 0, b, M, rtq.RECIPE_MIXED, skip=("wg",) if b == 1 else ())
            blocks.append(blk)
            refss.append(refs)
            xss.append(xs)
        rtq.block_project(blocks, M, math=math)
        for b in range(2):
            assert ("wg" in blocks[b]) == (b == 0)
            for name, (fmt, ref, xin) in refss[b].items():
                err = oracle.rel_fro(host(blocks[b][name].y), oracle.project(fmt, xss[b][xin], *ref))
                assert err <= TOL, (M, b, name, err)


# ----------------------------------------------------------------------------
# Full-size configurations, in the benchmark's launch configuration, checked on
# sampled outputs the oracle computes one by one.
# ----------------------------------------------------------------------------
def _sampled_check(blocks, refs_w, xs_all, M, rng, n_rows=24, n_cols=24):
    worst = 0.0
    for b, blk in enumerate(blocks):
        for name, p in blk.items():
            N, K, xin = synth.BLOCK_SHAPES[name]
            fmt, W = refs_w[b][name]
            rows = np.sort(rng.choice(M, size=min(n_rows, M), replace=False))
            cols = np.sort(rng.choice(N, size=min(n_cols, N), replace=False))
            ref_w = oracle.quantize(W[cols], fmt)          # per-row quantization: rows are independent
            got = host(p.weight.payload[torch.as_tensor(cols, device=DEV)])
            assert np.array_equal(got, ref_w[0]), (b, name, "codes")
            y_ref = oracle.project(fmt, xs_all[b][xin][rows], *ref_w)
            y = host(p.y[torch.as_tensor(rows, device=DEV)][:, torch.as_tensor(cols, device=DEV)])
            err = oracle.rel_fro(y, y_ref)
            worst = max(worst, err)
            assert err <= TOL, (b, name, err)
    return worst


@pytest.mark.parametrize("M,heavy", [(synth.M_GOLDEN, None), (synth.M_LARGE, "rows")])
def test_full_size_twelve_blocks_sampled(M, heavy, math):
    say(f"full-size 12 blocks M={M} heavy={heavy} math={math}")
    cfg = 4 if M == synth.M_GOLDEN else 5
    per_block = M == synth.M_GOLDEN          # as in the benchmark: own inputs per block at M=80
    shared = None if per_block else {n: synth.activation(cfg, synth.SHARED_BLOCK, n, M) for n in synth.INPUT_WIDTH}
    blocks, refs_w, xs_all = [], [], []
    for b in range(synth.NUM_BLOCKS):
        xs_host = {n: synth.activation(cfg, b, n, M) for n in synth.INPUT_WIDTH} if per_block else shared
        xs_dev = {n: dev(v) for n, v in xs_host.items()} if (per_block or b == 0) else xs_dev
        xs_all.append(xs_host)
        blk, rw = {}, {}
        for name in synth.PROJ_ORDER:
            N, K, xin = synth.BLOCK_SHAPES[name]
            W = synth.weight(cfg, 0, b, name, heavy=heavy)
            fmt = rtq.RECIPE_MIXED[name]
            blk[name] = rtq.Projection(rtq.quantize(dev(W), fmt), xs_dev[xin],
                                       torch.empty((M, N), dtype=torch.float32, device=DEV))
            rw[name] = (fmt, W)
        blocks.append(blk)
        refs_w.append(rw)
    rtq.block_project(blocks, M, math=math)
    torch.cuda.synchronize()
    worst = _sampled_check(blocks, refs_w, xs_all, M, np.random.default_rng(M))
    say(f"  worst sampled rel err {worst:.3e}")
    del blocks
    torch.cuda.empty_cache()


def test_calls_run_on_the_callers_streams():
    """Two 12-projection calls issued back to back on two non-default streams
    (each with its own workspace), then a third on the first stream that reuses
    the outputs of the first as inputs only after an event: every result equals
    the oracle's, so each call ran in its own stream's order."""
    M = 80
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()     # default priority
    torch.cuda.synchronize()
    calls = []
    for cfg, st in ((6, s1), (7, s2)):
        blk, refs, xs = make_block(cfg, 0, 0, M, rtq.RECIPE_MIXED)
        torch.cuda.synchronize()
        with torch.cuda.stream(st):
            rtq.block_project([blk], M, stream=st)
        calls.append((blk, refs, xs, st))
    # chain on s1: the wq output of call 1 feeds a second int8 projection
    blk1, refs1, xs1, _ = calls[0]
    W = synth.weight(8, 0, 0, "wo")
    w = gpu_quantize(W, "q8")
    ref_w = oracle.quantize(W, "q8")
    torch.cuda.synchronize()
    with torch.cuda.stream(s1):
        y2 = torch.empty((M, 512), dtype=torch.float32, device=DEV)
        rtq.block_project([{"wo": rtq.Projection(w, blk1["wq"].y, y2)}], M, stream=s1)
    s1.synchronize()
    s2.synchronize()
    for blk, refs, xs, _ in calls:
        for name, (fmt, ref, xin) in refs.items():
            err = oracle.rel_fro(host(blk[name].y), oracle.project(fmt, xs[xin], *ref))
            assert err <= TOL, (name, err)
    x2 = host(blk1["wq"].y)
    assert oracle.rel_fro(host(y2), oracle.project("q8", x2, *ref_w)) <= TOL


@pytest.mark.parametrize("M,K", [(80, 512), (200, 96), (17, 40)])
def test_f8_nan_code_makes_its_column_nan(M, K, math):
    """An E4M3 NaN code (S.1111.111) in row o of W makes column o of y NaN in
    every row; every other column still matches the oracle."""
    N = 48
    W = synth.weight(18, 0, 0, "wq", N, K)
    codes = oracle.quantize_f8(W)
    codes[5, K // 3] = 0x7F
    codes[31, K - 1] = 0xFF
    x = synth.activation(18, 0, "x_attn", M, K)
    y = host(rtq.gemm_f8(dev(x), rtq.F8Weight(dev(codes)), math=math))
    nan_cols = np.zeros(N, dtype=bool)
    nan_cols[[5, 31]] = True
    assert np.isnan(y[:, nan_cols]).all()
    assert np.isfinite(y[:, ~nan_cols]).all()
    ref = oracle.project_f8(x, codes)
    assert oracle.rel_fro(y[:, ~nan_cols], ref[:, ~nan_cols]) <= TOL
