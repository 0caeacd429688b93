"""The host quantizers (rtq_quantize_q4_host / _q8_host / _f8_host): the int4,
int8 and FP8 formats written without a GPU, bit for bit what the oracle's
quantizers give (and so what the GPU quantizers give, which their own GPU test
checks against the same oracle). Seeded RT-J-like weights, heavy-tailed rows
and columns, and the edge cases of each format: zero rows, constant groups,
fp16-subnormal and out-of-range scales, half-way roundings, the E4M3 overflow
boundary, signed zeros, infinities and NaN. Runs on the CPU."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import synth  # noqa: E402
import weight_only_quantized_rtq_amd as rtq  # noqa: E402


def same(w, ref, fmt):
    if fmt == "q4":
        assert np.array_equal(w.payload.numpy(), ref[0]), "int4 codes differ"
        assert np.array_equal(w.pairs.numpy().view(np.uint16), ref[1].view(np.uint16)), "int4 pairs differ"
    elif fmt == "q8":
        assert np.array_equal(w.payload.numpy(), ref[0]), "int8 codes differ"
        assert np.array_equal(w.scale.numpy().view(np.uint32), ref[1].view(np.uint32)), "int8 scales differ"
    else:
        assert np.array_equal(w.payload.numpy(), ref), "FP8 codes differ"


def ref_of(W, fmt):
    return {"q4": oracle.quantize_q4, "q8": oracle.quantize_q8, "f8": oracle.quantize_f8}[fmt](W)


def edge_weights(N, K, seed):
    W = synth.weight(7, seed, 0, "wq", N, K)
    W[0, :] = 0.0                                  # all-zero row / groups
    W[1, :32] = 0.125                              # constant group
    W[2, :] *= 1e-6                                # tiny: fp16 subnormal scales
    W[3, :] = np.float32(2.0 ** -30)               # below fp16 range
    W[4, ::2] *= 500.0                             # large dynamic range
    W[5, 32:64] = np.linspace(-1, 1, 32, dtype=np.float32)
    W[6, :] = -0.0                                 # negative zeros
    return W


@pytest.mark.parametrize("fmt", ["q4", "q8", "f8"])
@pytest.mark.parametrize("N,K,heavy", [(512, 512, None), (64, 2048, "rows"), (96, 512, "cols"), (7, 32, None)])
def test_host_quantizer_matches_oracle(fmt, N, K, heavy):
    W = synth.weight(31, 0, 0, "w1", N, K, heavy=heavy)
    same(rtq.quantize_host(torch.from_numpy(W), fmt), ref_of(W, fmt), fmt)


@pytest.mark.parametrize("fmt", ["q4", "q8", "f8"])
def test_host_quantizer_edge_cases(fmt):
    W = edge_weights(16, 128, 5)
    if fmt == "q8":
        W[7, :] = np.float32(1e-39)                # subnormal fp32 row
        W[8, :4] = [127, -63.5, 1, 0.25]           # halves round to even
    same(rtq.quantize_host(torch.from_numpy(W), fmt), ref_of(W, fmt), fmt)


def test_host_f8_special_values():
    specials = np.array([0.0, -0.0, 448, 449, 463.99997, 464, 464.00003, 480, 1e9, np.inf, -np.inf, np.nan,
                         -448, -465, 2 ** -9, 2 ** -10, 3 * 2 ** -11, 7.5 * 2 ** -9, 2 ** -6, 1.0625, 1.1875,
                         17, 19, -19, 1e-39, -1e-39, 2 ** -149, 0.0146484375], dtype=np.float32)
    W = np.resize(specials, (8, 64)).astype(np.float32)
    same(rtq.quantize_host(torch.from_numpy(W), "f8"), oracle.quantize_f8(W), "f8")


@pytest.mark.parametrize("threads", [1, 3, 0])
def test_host_quantizer_thread_count_does_not_change_the_result(threads):
    W = synth.weight(32, 0, 0, "w2", 37, 256, heavy="cols")
    for fmt in ("q4", "q8", "f8"):
        same(rtq.quantize_host(torch.from_numpy(W), fmt, threads=threads), ref_of(W, fmt), fmt)


def test_host_quantizer_validation():
    W = torch.zeros(4, 48)
    with pytest.raises(rtq.RtqError, match="SHAPE"):
        rtq.quantize_host(W, "q4")                 # K not a multiple of 32
    with pytest.raises(ValueError):
        rtq.quantize_host(torch.zeros(4, 64, dtype=torch.float64), "q8")
    lib = rtq.load_library()
    w = torch.zeros(4, 64)
    q = torch.empty(4, 64, dtype=torch.int8)
    with pytest.raises(rtq.RtqError, match="NULL"):
        rtq._check(lib.rtq_quantize_q8_host(w.data_ptr(), q.data_ptr(), None, 4, 64, 1))
    with pytest.raises(rtq.RtqError, match="OVERLAP"):
        rtq._check(lib.rtq_quantize_f8_host(w.data_ptr(), w.data_ptr() + 8, 4, 64, 1))
    empty = rtq.quantize_host(torch.zeros(0, 64), "q4")
    assert tuple(empty.payload.shape) == (0, 32)


@pytest.mark.gpu
@pytest.mark.parametrize("fmt", ["q4", "q8", "f8"])
def test_host_and_gpu_quantizers_agree(fmt):
    """The host and GPU quantizers share their arithmetic: the same bytes on
    RT-J-shaped weights with heavy columns and the edge rows."""
    W = synth.weight(33, 0, 0, "w1", 2048, 512, heavy="cols")
    W[:16] = edge_weights(16, 512, 6)
    h = rtq.quantize_host(torch.from_numpy(W), fmt)
    g = rtq.quantize(torch.from_numpy(W).to("cuda:0"), fmt)
    torch.cuda.synchronize()
    assert np.array_equal(h.payload.numpy(), g.payload.cpu().numpy())
    if fmt != "f8":
        assert np.array_equal(h.scale_tensor.numpy().view(np.uint8), g.scale_tensor.cpu().numpy().view(np.uint8))
