"""Python binding of librtq.so, the quantized-resident projection GEMM for MI355X.

Argument marshalling only: every step of the path (unpacking, dequantization,
the contraction, the quantizers) runs in the library's HIP kernels. PyTorch
supplies device memory and the current stream. There is no fallback: if the
library is missing or fails to load, every call raises.

Formats (RT-J int4 / int8 model cards, section "Quantization format"; FP8
model card, section "FP8 Format"):
  Q4Weight(payload uint8 [N, K/2], pairs float16 [N, K/32, 2])   (scale, min)
  Q8Weight(payload int8 [N, K],    scale float32 [N])
  F8Weight(payload uint8 [N, K])   E4M3 ("float8_e4m3fn") codes, no scale
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librtq.so")

FMT_NONE, FMT_Q4, FMT_Q8, FMT_F8 = 0, 1, 2, 3
Q4_GROUP = 32
MAX_BLOCKS = 64
PROJ_NAMES = ("wq", "wk", "wv", "wg", "wo", "w1", "w3", "w2")

# Format routing. Mixed: the int4 card's recipe (int4 for wq/wk/wv/wg and
# ffn.w1/w3, int8 for the residual-writing wo and ffn.w2). All-int8: the int8
# card's recipe (every block projection int8).
RECIPE_MIXED = {"wq": "q4", "wk": "q4", "wv": "q4", "wg": "q4",
                "wo": "q8", "w1": "q4", "w3": "q4", "w2": "q8"}
RECIPE_ALL_Q8 = {n: "q8" for n in PROJ_NAMES}
RECIPE_ALL_F8 = {n: "f8" for n in PROJ_NAMES}   # FP8 card: every matrix weight E4M3

STATUS = {0: "RTQ_OK", 1: "RTQ_ERR_NULL", 2: "RTQ_ERR_SHAPE", 3: "RTQ_ERR_ALIGN",
          4: "RTQ_ERR_FORMAT", 5: "RTQ_ERR_HIP", 6: "RTQ_ERR_OVERLAP"}

# Every symbol include/rtq.h declares.
EXPORTS = ("rtq_gemm_q4", "rtq_gemm_q8", "rtq_gemm_f8", "rtq_block_project", "rtq_dequant_q4",
           "rtq_dequant_q8", "rtq_dequant_f8", "rtq_quantize_q4", "rtq_quantize_q8", "rtq_quantize_f8",
           "rtq_quantize_q4_host", "rtq_quantize_q8_host", "rtq_quantize_f8_host", "rtq_gemm_ex",
           "rtq_block_project_ex", "rtq_block_project_noalloc", "rtq_block_workspace_bytes",
           "rtq_block_project_ws", "rtq_diag_stream_read", "rtq_diag_mfma_loop", "rtq_timing_enable",
           "rtq_timing_read", "rtq_status_string", "rtq_last_error", "rtq_version")

# Arithmetic of a GEMM call (the `math` argument; None runs the library's
# default, MATH_SPLIT_BF16, through the plain entry points).
MATH_SPLIT_BF16, MATH_FP32_MFMA, MATH_BF16, MATH_SPLIT_F16 = 0, 1, 2, 3
MATHS = {"split": MATH_SPLIT_BF16, "fp32": MATH_FP32_MFMA, "bf16": MATH_BF16, "split16": MATH_SPLIT_F16}


class RtqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class _Proj(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("payload", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("x", ctypes.c_void_p), ("y", ctypes.c_void_p), ("bias", ctypes.c_void_p)]


class _Block(ctypes.Structure):
    _fields_ = [(n, _Proj) for n in PROJ_NAMES]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads librtq.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m weight_only_quantized_rtq_amd.build`")
    lib = ctypes.CDLL(path)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32
    for name in ("rtq_gemm_q4", "rtq_gemm_q8"):
        f = getattr(lib, name)
        f.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
        f.restype = ctypes.c_int
    lib.rtq_gemm_f8.argtypes = [vp, vp, vp, i64, i64, i64, vp]
    lib.rtq_gemm_f8.restype = ctypes.c_int
    for name in ("rtq_dequant_f8", "rtq_quantize_f8"):
        f = getattr(lib, name)
        f.argtypes = [vp, vp, i64, i64, vp]
        f.restype = ctypes.c_int
    lib.rtq_block_project.argtypes = [ctypes.POINTER(_Block), i32, i64, vp]
    lib.rtq_block_project.restype = ctypes.c_int
    for name in ("rtq_dequant_q4", "rtq_dequant_q8", "rtq_quantize_q4", "rtq_quantize_q8"):
        f = getattr(lib, name)
        f.argtypes = [vp, vp, vp, i64, i64, vp]
        f.restype = ctypes.c_int
    for name in ("rtq_quantize_q4_host", "rtq_quantize_q8_host"):
        f = getattr(lib, name)
        f.argtypes = [vp, vp, vp, i64, i64, i32]
        f.restype = ctypes.c_int
    lib.rtq_quantize_f8_host.argtypes = [vp, vp, i64, i64, i32]
    lib.rtq_quantize_f8_host.restype = ctypes.c_int
    lib.rtq_gemm_ex.argtypes = [i32, vp, vp, vp, vp, i64, i64, i64, i32, vp]
    lib.rtq_gemm_ex.restype = ctypes.c_int
    lib.rtq_block_project_ex.argtypes = [ctypes.POINTER(_Block), i32, i64, i32, vp]
    lib.rtq_block_project_ex.restype = ctypes.c_int
    lib.rtq_block_project_noalloc.argtypes = [ctypes.POINTER(_Block), i32, i64, i32, vp]
    lib.rtq_block_project_noalloc.restype = ctypes.c_int
    lib.rtq_block_workspace_bytes.argtypes = [ctypes.POINTER(_Block), i32, i64, i32, ctypes.POINTER(i64)]
    lib.rtq_block_workspace_bytes.restype = ctypes.c_int
    lib.rtq_block_project_ws.argtypes = [ctypes.POINTER(_Block), i32, i64, i32, vp, i64, vp]
    lib.rtq_block_project_ws.restype = ctypes.c_int
    lib.rtq_diag_stream_read.argtypes = [vp, i64, i32, i32, vp, vp]
    lib.rtq_diag_stream_read.restype = ctypes.c_int
    lib.rtq_diag_mfma_loop.argtypes = [i32, i64, i32, vp, ctypes.POINTER(ctypes.c_double), vp]
    lib.rtq_diag_mfma_loop.restype = ctypes.c_int
    lib.rtq_timing_enable.argtypes = [i32]
    lib.rtq_timing_enable.restype = ctypes.c_int
    lib.rtq_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    lib.rtq_timing_read.restype = ctypes.c_int
    lib.rtq_status_string.argtypes = [ctypes.c_int]
    lib.rtq_status_string.restype = ctypes.c_char_p
    lib.rtq_last_error.argtypes = []
    lib.rtq_last_error.restype = ctypes.c_char_p
    lib.rtq_version.argtypes = []
    lib.rtq_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def version() -> str:
    return load_library().rtq_version().decode()


def diag_stream_read(buf: torch.Tensor, unroll: int = 8, blocks: int = 4096, sink=None, stream=None) -> None:
    """Streaming read of a whole device tensor (rtq_diag_stream_read)."""
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    _check(load_library().rtq_diag_stream_read(_ptr(buf), buf.numel() * buf.element_size(), unroll, blocks,
                                                _ptr(sink), _stream(stream)))


def diag_mfma_loop(kind: int, iters: int, blocks: int = 1024, sink=None, stream=None) -> float:
    """Back-to-back matrix instructions (rtq_diag_mfma_loop): kind 0 fp16,
    1 bf16, 2 fp32. Returns the launch's floating-point operations."""
    if sink is None:
        sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    flops = ctypes.c_double(0.0)
    _check(load_library().rtq_diag_mfma_loop(kind, iters, blocks, _ptr(sink), ctypes.byref(flops), _stream(stream)))
    return flops.value


def timing_enable(on: bool = True) -> None:
    """Bracket every main GEMM kernel launch with HIP events (rtq_timing_enable)."""
    _check(load_library().rtq_timing_enable(1 if on else 0))


def timing_read() -> tuple[float, int]:
    """(summed kernel ms, number of timed launches) since the last enable/read."""
    ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
    _check(load_library().rtq_timing_read(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def _check(status: int) -> None:
    if status != 0:
        raise RtqError(status, load_library().rtq_last_error().decode())


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, dtype: torch.dtype, name: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.device.index != torch.cuda.current_device():
        # the library launches on the current device's streams
        raise ValueError(f"{name} is on {t.device}, the current device is cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


@dataclass
class Q4Weight:
    payload: torch.Tensor   # uint8 [N, K/2]
    pairs: torch.Tensor     # float16 [N, K/32, 2]: (scale, min)

    @property
    def N(self) -> int:
        return self.payload.shape[0]

    @property
    def K(self) -> int:
        return self.payload.shape[1] * 2

    fmt = FMT_Q4

    @property
    def scale_tensor(self) -> torch.Tensor:
        return self.pairs

    def validate(self) -> None:
        _need(self.payload, torch.uint8, "payload")
        _need(self.pairs, torch.float16, "pairs")
        if self.payload.dim() != 2 or tuple(self.pairs.shape) != (self.N, self.K // Q4_GROUP, 2):
            raise ValueError(f"int4 weight shapes disagree: payload {tuple(self.payload.shape)}, "
                             f"pairs {tuple(self.pairs.shape)}")


@dataclass
class Q8Weight:
    payload: torch.Tensor   # int8 [N, K]
    scale: torch.Tensor     # float32 [N]

    @property
    def N(self) -> int:
        return self.payload.shape[0]

    @property
    def K(self) -> int:
        return self.payload.shape[1]

    fmt = FMT_Q8

    @property
    def scale_tensor(self) -> torch.Tensor:
        return self.scale

    def validate(self) -> None:
        _need(self.payload, torch.int8, "payload")
        _need(self.scale, torch.float32, "scale")
        if self.payload.dim() != 2 or tuple(self.scale.shape) != (self.N,):
            raise ValueError(f"int8 weight shapes disagree: payload {tuple(self.payload.shape)}, "
                             f"scale {tuple(self.scale.shape)}")


@dataclass
class F8Weight:
    payload: torch.Tensor   # uint8 [N, K]: E4M3 codes (a float8_e4m3fn tensor viewed as bytes)

    @property
    def N(self) -> int:
        return self.payload.shape[0]

    @property
    def K(self) -> int:
        return self.payload.shape[1]

    fmt = FMT_F8
    scale_tensor = None

    def validate(self) -> None:
        _need(self.payload, torch.uint8, "payload")
        if self.payload.dim() != 2:
            raise ValueError(f"FP8 weight must be [N, K], got {tuple(self.payload.shape)}")


def weight_from_tensors(payload: torch.Tensor, scale: torch.Tensor | None = None):
    """Format detection from the payload dtype, as the engine's loader does
    (int4 card, "Usage": the format is read off the tensor dtypes): uint8 ->
    int4, int8 -> int8, float8_e4m3fn (FP8 card, "FP8 Format") -> FP8."""
    if payload.dtype == torch.float8_e4m3fn:
        return F8Weight(payload.view(torch.uint8))
    if payload.dtype == torch.uint8:
        return Q4Weight(payload, scale)
    if payload.dtype == torch.int8:
        return Q8Weight(payload, scale)
    raise TypeError(f"payload dtype {payload.dtype} is not a quantized format")


def _gemm(x: torch.Tensor, w, y: torch.Tensor | None, stream, math: int | None = None) -> torch.Tensor:
    lib = load_library()
    w.validate()
    _need(x, torch.float32, "x")
    if x.dim() != 2 or x.shape[1] != w.K:
        raise ValueError(f"x must be [M, {w.K}], got {tuple(x.shape)}")
    M = x.shape[0]
    if y is None:
        y = torch.empty((M, w.N), dtype=torch.float32, device=x.device)
    else:
        _need(y, torch.float32, "y")
        if tuple(y.shape) != (M, w.N):
            raise ValueError(f"y must be [{M}, {w.N}], got {tuple(y.shape)}")
    if math is not None:
        _check(lib.rtq_gemm_ex(w.fmt, _ptr(x), _ptr(w.payload), _ptr(w.scale_tensor), _ptr(y), M, w.N, w.K,
                               int(math), _stream(stream)))
        return y
    if w.fmt == FMT_F8:
        _check(lib.rtq_gemm_f8(_ptr(x), _ptr(w.payload), _ptr(y), M, w.N, w.K, _stream(stream)))
        return y
    fn = lib.rtq_gemm_q4 if w.fmt == FMT_Q4 else lib.rtq_gemm_q8
    _check(fn(_ptr(x), _ptr(w.payload), _ptr(w.scale_tensor), _ptr(y), M, w.N, w.K, _stream(stream)))
    return y


def gemm_q4(x: torch.Tensor, w: Q4Weight, y: torch.Tensor | None = None, stream=None,
            math: int | None = None) -> torch.Tensor:
    """y = x . dequant(w)^T for an int4 weight (rtq_gemm_q4)."""
    if not isinstance(w, Q4Weight):
        raise TypeError("gemm_q4 needs a Q4Weight")
    return _gemm(x, w, y, stream, math)


def gemm_q8(x: torch.Tensor, w: Q8Weight, y: torch.Tensor | None = None, stream=None,
            math: int | None = None) -> torch.Tensor:
    """y = x . dequant(w)^T for an int8 weight (rtq_gemm_q8)."""
    if not isinstance(w, Q8Weight):
        raise TypeError("gemm_q8 needs a Q8Weight")
    return _gemm(x, w, y, stream, math)


def gemm_f8(x: torch.Tensor, w: F8Weight, y: torch.Tensor | None = None, stream=None,
            math: int | None = None) -> torch.Tensor:
    """y = x . W^T for an FP8 E4M3 weight (rtq_gemm_f8)."""
    if not isinstance(w, F8Weight):
        raise TypeError("gemm_f8 needs an F8Weight")
    return _gemm(x, w, y, stream, math)


def gemm(x: torch.Tensor, w, y: torch.Tensor | None = None, stream=None, bias=None,
         math: int | None = None) -> torch.Tensor:
    """y = x . W^T (+ bias, fp32 [N], through a one-projection rtq_block_project)."""
    if bias is None:
        return _gemm(x, w, y, stream, math)
    if y is None:
        y = torch.empty((x.shape[0], w.N), dtype=torch.float32, device=x.device)
    block_project([{"wq": Projection(w, x, y, bias)}], x.shape[0], stream, math=math)
    return y


def dequant(w, stream=None) -> torch.Tensor:
    """Dense fp32 W [N, K] (rtq_dequant_q4 / rtq_dequant_q8)."""
    lib = load_library()
    w.validate()
    out = torch.empty((w.N, w.K), dtype=torch.float32, device=w.payload.device)
    if w.fmt == FMT_F8:
        _check(lib.rtq_dequant_f8(_ptr(w.payload), _ptr(out), w.N, w.K, _stream(stream)))
        return out
    fn = lib.rtq_dequant_q4 if w.fmt == FMT_Q4 else lib.rtq_dequant_q8
    _check(fn(_ptr(w.payload), _ptr(w.scale_tensor), _ptr(out), w.N, w.K, _stream(stream)))
    return out


def quantize_q4(W: torch.Tensor, stream=None) -> Q4Weight:
    """int4 group-32 quantization with the min-MSE clip search (rtq_quantize_q4)."""
    lib = load_library()
    _need(W, torch.float32, "W")
    N, K = W.shape
    payload = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
    pairs = torch.empty((N, K // Q4_GROUP, 2), dtype=torch.float16, device=W.device)
    _check(lib.rtq_quantize_q4(_ptr(W), _ptr(payload), _ptr(pairs), N, K, _stream(stream)))
    return Q4Weight(payload, pairs)


def quantize_q8(W: torch.Tensor, stream=None) -> Q8Weight:
    """int8 per-row symmetric quantization (rtq_quantize_q8)."""
    lib = load_library()
    _need(W, torch.float32, "W")
    N, K = W.shape
    q = torch.empty((N, K), dtype=torch.int8, device=W.device)
    scale = torch.empty((N,), dtype=torch.float32, device=W.device)
    _check(lib.rtq_quantize_q8(_ptr(W), _ptr(q), _ptr(scale), N, K, _stream(stream)))
    return Q8Weight(q, scale)


def quantize_f8(W: torch.Tensor, stream=None) -> F8Weight:
    """FP8 E4M3 codes, as a cast to float8_e4m3fn gives them (rtq_quantize_f8)."""
    lib = load_library()
    _need(W, torch.float32, "W")
    N, K = W.shape
    codes = torch.empty((N, K), dtype=torch.uint8, device=W.device)
    _check(lib.rtq_quantize_f8(_ptr(W), _ptr(codes), N, K, _stream(stream)))
    return F8Weight(codes)


def quantize_host(W: torch.Tensor, fmt: str, threads: int = 0):
    """The quantizers on the host (rtq_quantize_q4_host / _q8_host / _f8_host):
    W is a CPU float32 [N, K] tensor; the result holds CPU tensors, bit-identical
    to what quantize() gives on the GPU. Needs no GPU."""
    lib = load_library()
    if W.device.type != "cpu" or W.dtype != torch.float32 or W.dim() != 2:
        raise ValueError(f"W must be a CPU float32 [N, K] tensor, got {W.dtype} {tuple(W.shape)} on {W.device}")
    W = W.contiguous()
    N, K = W.shape
    if fmt == "q4":
        payload = torch.empty((N, K // 2), dtype=torch.uint8)
        pairs = torch.empty((N, K // Q4_GROUP, 2), dtype=torch.float16)
        _check(lib.rtq_quantize_q4_host(_ptr(W), _ptr(payload), _ptr(pairs), N, K, threads))
        return Q4Weight(payload, pairs)
    if fmt == "q8":
        q = torch.empty((N, K), dtype=torch.int8)
        scale = torch.empty((N,), dtype=torch.float32)
        _check(lib.rtq_quantize_q8_host(_ptr(W), _ptr(q), _ptr(scale), N, K, threads))
        return Q8Weight(q, scale)
    if fmt == "f8":
        codes = torch.empty((N, K), dtype=torch.uint8)
        _check(lib.rtq_quantize_f8_host(_ptr(W), _ptr(codes), N, K, threads))
        return F8Weight(codes)
    raise ValueError(f"unknown format {fmt!r}")


def quantize(W: torch.Tensor, fmt: str, stream=None):
    if fmt == "q4":
        return quantize_q4(W, stream)
    if fmt == "q8":
        return quantize_q8(W, stream)
    if fmt == "f8":
        return quantize_f8(W, stream)
    raise ValueError(f"unknown format {fmt!r}")


@dataclass
class Projection:
    """One projection of a block: its weight, the input it reads and the output it writes."""
    weight: object               # Q4Weight | Q8Weight | F8Weight
    x: torch.Tensor              # float32 [M, K]
    y: torch.Tensor              # float32 [M, N]
    bias: torch.Tensor | None = None   # float32 [N], added to every row of y


def pack_blocks(blocks: list[dict[str, Projection]], M: int):
    """Builds the host descriptor array of rtq_block_project. Names missing from
    a block's dict (e.g. a checkpoint without wg) are skipped."""
    if not 1 <= len(blocks) <= MAX_BLOCKS:
        raise ValueError(f"1..{MAX_BLOCKS} blocks per call, got {len(blocks)}")
    arr = (_Block * len(blocks))()
    keep = []
    for b, blk in enumerate(blocks):
        for name in PROJ_NAMES:
            p = blk.get(name)
            if p is None:
                continue
            w = p.weight
            w.validate()
            _need(p.x, torch.float32, f"{name}.x")
            _need(p.y, torch.float32, f"{name}.y")
            if tuple(p.x.shape) != (M, w.K) or tuple(p.y.shape) != (M, w.N):
                raise ValueError(f"block {b} {name}: x {tuple(p.x.shape)} / y {tuple(p.y.shape)} "
                                 f"do not match M={M}, N={w.N}, K={w.K}")
            d = getattr(arr[b], name)
            d.fmt, d.N, d.K, d.reserved = w.fmt, w.N, w.K, 0
            d.payload, d.scale = _ptr(w.payload), _ptr(w.scale_tensor)
            d.x, d.y = _ptr(p.x), _ptr(p.y)
            if p.bias is not None:
                _need(p.bias, torch.float32, f"{name}.bias")
                if tuple(p.bias.shape) != (w.N,):
                    raise ValueError(f"block {b} {name}: bias {tuple(p.bias.shape)} does not match N={w.N}")
                d.bias = _ptr(p.bias)
            else:
                d.bias = None
            keep.append(p)
    return arr, keep


def block_workspace_bytes(blocks: list[dict[str, Projection]], M: int, math: int = MATH_SPLIT_BF16,
                          packed=None) -> int:
    """Workspace bytes block_project(..., workspace=) needs for this call
    (rtq_block_workspace_bytes)."""
    lib = load_library()
    arr, _keep = packed if packed is not None else pack_blocks(blocks, M)
    out = ctypes.c_int64(0)
    _check(lib.rtq_block_workspace_bytes(arr, len(arr), M, int(math), ctypes.byref(out)))
    return out.value


def block_project(blocks: list[dict[str, Projection]], M: int, stream=None, packed=None,
                  math: int | None = None, workspace: torch.Tensor | None = None) -> None:
    """Runs every projection of the given blocks (rtq_block_project, or
    rtq_block_project_ex with the arithmetic `math`, or rtq_block_project_ws
    with a caller-kept device `workspace` tensor of at least
    block_workspace_bytes() bytes). `packed` may hold a pack_blocks() result
    to reuse across calls."""
    lib = load_library()
    arr, _keep = packed if packed is not None else pack_blocks(blocks, M)
    if workspace is not None:
        nbytes = workspace.numel() * workspace.element_size()
        _check(lib.rtq_block_project_ws(arr, len(arr), M, int(MATH_SPLIT_BF16 if math is None else math),
                                        _ptr(workspace), nbytes, _stream(stream)))
        return
    if math is None:
        _check(lib.rtq_block_project(arr, len(arr), M, _stream(stream)))
    else:
        _check(lib.rtq_block_project_ex(arr, len(arr), M, int(math), _stream(stream)))
