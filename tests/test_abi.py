"""CPU-side checks of the C-ABI library: it loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call.
No kernel is launched here."""
import ctypes
import os
import re

import pytest

torch = pytest.importorskip("torch")

import weight_only_quantized_rtq_amd as rtq  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rtq.h")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_FORMAT, ERR_HIP, ERR_OVERLAP = range(7)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rtq.LIB_PATH):
        pytest.fail("librtq.so is not built; run `python -m weight_only_quantized_rtq_amd.build`")
    return rtq.load_library()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(rtq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_symbols() == sorted(rtq.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version_and_status_strings(lib):
    assert rtq.version().startswith("rtq ")
    for s in range(7):
        assert lib.rtq_status_string(s)
    assert lib.rtq_status_string(99) == b"unknown status"


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(rtq, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        rtq.load_library(str(tmp_path / "nope.so"))


A = 0x7f0000000000   # fake, 256-byte aligned device addresses: never dereferenced
B = 0x7f1000000000
C = 0x7f2000000000
D = 0x7f3000000000


def call_q4(lib, x=A, p=B, s=C, y=D, M=80, N=512, K=512):
    return lib.rtq_gemm_q4(x, p, s, y, M, N, K, None)


def call_q8(lib, x=A, p=B, s=C, y=D, M=80, N=512, K=512):
    return lib.rtq_gemm_q8(x, p, s, y, M, N, K, None)


def test_shape_errors(lib):
    assert call_q4(lib, K=48) == ERR_SHAPE
    assert b"multiple" in lib.rtq_last_error()
    assert call_q4(lib, N=0) == ERR_SHAPE
    assert call_q4(lib, K=0) == ERR_SHAPE
    assert call_q4(lib, M=-1) == ERR_SHAPE
    assert call_q4(lib, M=2**31) == ERR_SHAPE
    assert call_q8(lib, N=2**31) == ERR_SHAPE


def test_element_count_limit(lib):
    """Products of the dimensions are capped (2^38 elements per tensor) before
    any byte-range arithmetic, so no overflow reaches the overlap checks."""
    assert call_q4(lib, M=2**29, N=2**29, K=64) == ERR_SHAPE
    assert b"2^38" in lib.rtq_last_error()
    assert call_q8(lib, M=2, N=2**29, K=2**29) == ERR_SHAPE
    assert lib.rtq_dequant_q8(B, C, A, 2**29, 2**29, None) == ERR_SHAPE
    assert lib.rtq_quantize_f8(A, B, 2**29, 2**29, None) == ERR_SHAPE
    assert lib.rtq_quantize_q4(A, B, C, 2**29, 2**29, None) == ERR_SHAPE
    # each dimension below 2^30
    assert call_q4(lib, M=2**30) == ERR_SHAPE and call_q8(lib, N=2**30) == ERR_SHAPE


def test_m_zero_is_a_noop(lib):
    assert call_q4(lib, M=0, x=None, y=None) == OK
    assert call_q8(lib, M=0, x=None, y=None) == OK


def test_null_errors(lib):
    assert call_q4(lib, x=None) == ERR_NULL
    assert call_q4(lib, p=None) == ERR_NULL
    assert call_q8(lib, s=None) == ERR_NULL
    assert call_q8(lib, y=None) == ERR_NULL
    assert b"y is NULL" in lib.rtq_last_error()


def test_alignment_errors(lib):
    assert call_q4(lib, x=A + 4) == ERR_ALIGN
    assert call_q4(lib, y=D + 8) == ERR_ALIGN
    assert call_q8(lib, p=B + 1) == ERR_ALIGN
    assert call_q8(lib, s=C + 2) == ERR_ALIGN


def test_overlap_errors(lib):
    # y = [A, A + 80*512*4) overlaps x
    assert call_q4(lib, y=A + 1024) == ERR_OVERLAP
    assert call_q8(lib, y=B) == ERR_OVERLAP
    # adjacent but disjoint ranges are fine up to the launch, which needs a GPU:
    # not exercised here.


def _block(fmt=rtq.FMT_Q4, N=512, K=512, x=A, p=B, s=C, y=D, reserved=0):
    blk = rtq._Block()
    d = blk.wq
    d.fmt, d.N, d.K, d.reserved = fmt, N, K, reserved
    d.payload, d.scale, d.x, d.y = p, s, x, y
    return blk


def test_block_project_validation(lib):
    arr = (rtq._Block * 1)(_block())
    assert lib.rtq_block_project(arr, 0, 80, None) == ERR_SHAPE
    assert lib.rtq_block_project(arr, 65, 80, None) == ERR_SHAPE
    assert lib.rtq_block_project(None, 1, 80, None) == ERR_NULL
    assert lib.rtq_block_project((rtq._Block * 1)(_block(fmt=7)), 1, 80, None) == ERR_FORMAT
    assert lib.rtq_block_project((rtq._Block * 1)(_block(K=40)), 1, 80, None) == ERR_SHAPE
    assert lib.rtq_block_project((rtq._Block * 1)(_block(reserved=1)), 1, 80, None) == ERR_SHAPE
    assert lib.rtq_block_project((rtq._Block * 1)(_block(y=A)), 1, 80, None) == ERR_OVERLAP
    # two projections writing the same output
    blk = _block()
    blk.wk = blk.wq
    assert lib.rtq_block_project((rtq._Block * 1)(blk), 1, 80, None) == ERR_OVERLAP
    # an output overlapping another projection's input
    blk = _block()
    blk.wo.fmt, blk.wo.N, blk.wo.K = rtq.FMT_Q8, 512, 512
    blk.wo.payload, blk.wo.scale, blk.wo.x, blk.wo.y = B + 2**24, C + 2**24, D, A + 2**30
    assert lib.rtq_block_project((rtq._Block * 1)(blk), 1, 80, None) == ERR_OVERLAP
    # a bias must be 4-byte aligned and is an input: no y may overlap it
    blk = _block()
    blk.wq.bias = C + 2**24 + 2
    assert lib.rtq_block_project((rtq._Block * 1)(blk), 1, 80, None) == ERR_ALIGN
    assert b"bias" in lib.rtq_last_error()
    blk.wq.bias = D + 1024
    assert lib.rtq_block_project((rtq._Block * 1)(blk), 1, 80, None) == ERR_OVERLAP
    # an empty block (no payloads) and M = 0 are no-ops
    assert lib.rtq_block_project((rtq._Block * 1)(), 1, 80, None) == OK
    assert lib.rtq_block_project(arr, 1, 0, None) == OK


def test_quantize_dequant_validation(lib):
    assert lib.rtq_quantize_q4(A, B, C, 4, 40, None) == ERR_SHAPE
    assert lib.rtq_quantize_q4(A, B, None, 4, 64, None) == ERR_NULL
    assert lib.rtq_quantize_q4(A + 4, B, C, 4, 64, None) == ERR_ALIGN
    assert lib.rtq_quantize_q8(A, B, C, -1, 64, None) == ERR_SHAPE
    assert lib.rtq_dequant_q4(B, C, A, 4, 33, None) == ERR_SHAPE
    assert lib.rtq_dequant_q8(None, C, A, 4, 64, None) == ERR_NULL
    assert lib.rtq_dequant_q8(B, C, A, 0, 64, None) == OK


def test_f8_validation(lib):
    assert lib.rtq_gemm_f8(A, B, D, 80, 512, 0, None) == ERR_SHAPE
    assert lib.rtq_gemm_f8(A, None, D, 80, 512, 512, None) == ERR_NULL
    assert lib.rtq_gemm_f8(A, B + 4, D, 80, 512, 512, None) == ERR_ALIGN
    assert lib.rtq_gemm_f8(A, B, A + 1024, 80, 512, 512, None) == ERR_OVERLAP
    assert lib.rtq_gemm_f8(None, B, None, 0, 512, 512, None) == OK
    assert lib.rtq_dequant_f8(None, A, 4, 64, None) == ERR_NULL
    assert lib.rtq_dequant_f8(B, A, 0, 64, None) == OK
    assert lib.rtq_quantize_f8(A + 2, B, 4, 64, None) == ERR_ALIGN
    assert lib.rtq_quantize_f8(A, A + 16, 4, 64, None) == ERR_OVERLAP
    # an FP8 projection needs no scale companion
    blk = _block(fmt=rtq.FMT_F8, s=None)
    assert lib.rtq_block_project((rtq._Block * 1)(blk), 1, 0, None) == OK


def test_math_is_an_argument_checked_per_call(lib):
    """The arithmetic is a per-call argument: an unknown value is rejected
    before anything runs, and no call changes what a later call computes
    (there is no arithmetic state to set)."""
    for name in ("rtq_set_math", "rtq_get_math"):
        with pytest.raises(AttributeError):
            getattr(lib, name)
    for bad in (-1, 4, 7):
        assert lib.rtq_gemm_ex(rtq.FMT_Q4, A, B, C, D, 80, 512, 512, bad, None) == ERR_FORMAT
        assert b"arithmetic" in lib.rtq_last_error()
        blk = _block()
        assert lib.rtq_block_project_ex((rtq._Block * 1)(blk), 1, 80, bad, None) == ERR_FORMAT
    assert lib.rtq_gemm_ex(9, A, B, C, D, 80, 512, 512, rtq.MATH_SPLIT_BF16, None) == ERR_FORMAT
    for m in rtq.MATHS.values():
        # M = 0 is a no-op in every arithmetic; shape errors are reported as before
        assert lib.rtq_gemm_ex(rtq.FMT_Q8, None, B, C, None, 0, 512, 512, m, None) == OK
        assert lib.rtq_gemm_ex(rtq.FMT_Q4, A, B, C, D, 80, 512, 500, m, None) == ERR_SHAPE
        assert lib.rtq_block_project_ex((rtq._Block * 1)(_block(fmt=rtq.FMT_F8, s=None)), 1, 0, m, None) == OK


def test_struct_layout_matches_header(tmp_path):
    """The binding's ctypes mirror of rtq_proj / rtq_block has the layout the C
    compiler gives the header's structs."""
    fields = [f[0] for f in rtq._Proj._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "rtq.h"\nint main(void) {\n'
                   '  printf("%zu %zu", sizeof(rtq_proj), sizeof(rtq_block));\n'
                   + "".join(f'  printf(" %zu", offsetof(rtq_proj, {f}));\n' for f in fields)
                   + "".join(f'  printf(" %zu", offsetof(rtq_block, {n}));\n' for n in rtq.PROJ_NAMES)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    subprocess.run([cc, "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = [ctypes.sizeof(rtq._Proj), ctypes.sizeof(rtq._Block)]
    want += [getattr(rtq._Proj, f).offset for f in fields]
    want += [getattr(rtq._Block, n).offset for n in rtq.PROJ_NAMES]
    assert got == want
    assert [f[0] for f in rtq._Block._fields_] == list(rtq.PROJ_NAMES)


def test_recipes_agree_with_names():
    assert set(rtq.RECIPE_MIXED) == set(rtq.PROJ_NAMES)
    assert {n for n, f in rtq.RECIPE_MIXED.items() if f == "q8"} == {"wo", "w2"}


E = 0x7f4000000000


def _rtj_blocks(n_blocks, M):
    """The RT-J projection set (mixed recipe) with fake, disjoint device
    addresses: every input, payload, scale array and output its own 256 MiB."""
    import synth
    arr = (rtq._Block * n_blocks)()
    addr = E
    for b in range(n_blocks):
        xs = {}
        for name in synth.PROJ_ORDER:
            N, K, xin = synth.BLOCK_SHAPES[name]
            if xin not in xs:
                xs[xin] = addr
                addr += 1 << 28
            d = getattr(arr[b], name)
            d.fmt, d.N, d.K = {"q4": rtq.FMT_Q4, "q8": rtq.FMT_Q8}[rtq.RECIPE_MIXED[name]], N, K
            d.x = xs[xin]
            d.payload, d.scale, d.y = addr, addr + (1 << 28), addr + (2 << 28)
            addr += 3 << 28
    return arr, addr


def _image_bytes(K, M, NL):
    """Limb image of one input as the layout states it: NL planes of 1 KB per
    (group, 16-row block), then the fp32 group sums, then the int32 row
    exponents."""
    G, RB = K // 32, (M + 15) // 16
    return G * RB * 1024 * NL + G * RB * 16 * 4 + RB * 16 * 4


@pytest.mark.parametrize("math,nl", [(rtq.MATH_SPLIT_F16, 2), (rtq.MATH_SPLIT_BF16, 3), (rtq.MATH_BF16, 1)])
def test_workspace_size_query(lib, math, nl):
    """12 blocks at M = 80 (grouped route): four limb images per block plus
    w2's four K-chunk partials, each image 256-byte aligned; the direct route
    (M <= 32) and the fp32 arithmetic need none."""
    arr, _ = _rtj_blocks(12, 80)
    out = ctypes.c_int64(-1)
    assert lib.rtq_block_workspace_bytes(arr, 12, 80, math, ctypes.byref(out)) == OK
    want = 12 * (3 * _image_bytes(512, 80, nl) + _image_bytes(2048, 80, nl)) + 12 * 4 * 80 * 512 * 4
    assert want <= out.value <= want + 48 * 256, (out.value, want)
    for M, m in ((16, math), (80, rtq.MATH_FP32_MFMA), (0, math)):
        arr, _ = _rtj_blocks(12, M)
        assert lib.rtq_block_workspace_bytes(arr, 12, M, m, ctypes.byref(out)) == OK
        assert out.value == 0, (M, m, out.value)
    assert lib.rtq_block_workspace_bytes(arr, 12, 80, math, None) == ERR_NULL
    assert lib.rtq_block_workspace_bytes(arr, 12, 80, 9, ctypes.byref(out)) == ERR_FORMAT


def test_workspace_validation(lib):
    """rtq_block_project_ws rejects, before any HIP call, a workspace that is
    too small, NULL where one is needed, misaligned, overlapping an input or
    an output, or of negative size; a call that needs none takes NULL."""
    math = rtq.MATH_SPLIT_F16
    arr, end = _rtj_blocks(12, 80)
    out = ctypes.c_int64(0)
    assert lib.rtq_block_workspace_bytes(arr, 12, 80, math, ctypes.byref(out)) == OK
    need = out.value
    ws = end + (1 << 28)
    assert lib.rtq_block_project_ws(arr, 12, 80, math, ws, need - 1, None) == ERR_SHAPE
    assert b"needs" in lib.rtq_last_error()
    assert lib.rtq_block_project_ws(arr, 12, 80, math, None, need, None) == ERR_NULL
    assert lib.rtq_block_project_ws(arr, 12, 80, math, ws + 128, need, None) == ERR_ALIGN
    assert lib.rtq_block_project_ws(arr, 12, 80, math, ws, -1, None) == ERR_SHAPE
    assert lib.rtq_block_project_ws(arr, 12, 80, math, arr[0].wq.y, need, None) == ERR_OVERLAP
    assert lib.rtq_block_project_ws(arr, 12, 80, math, arr[3].w1.payload, need, None) == ERR_OVERLAP
    assert lib.rtq_block_project_ws(arr, 12, 0, math, None, 0, None) == OK      # M = 0: a no-op


def test_small_calls_take_shorter_k_chunks(lib):
    """A call with few workgroups that runs the finish pass anyway (a w2-shaped
    K = 2048 projection) walks K in shorter chunks (16, then 8, then 4 groups
    while it has fewer than 256 workgroups), and its workspace holds those
    chunks' partials; a call that would need the finish pass only for that
    keeps whole 16-group chunks."""
    M = 80
    out = ctypes.c_int64(-1)
    # one 512 x 512 int4 projection: no finish pass otherwise, one chunk
    arr = (rtq._Block * 1)(_block(N=512, K=512))
    assert lib.rtq_block_workspace_bytes(arr, 1, M, rtq.MATH_SPLIT_F16, ctypes.byref(out)) == OK
    assert out.value == (_image_bytes(512, M, 2) + 255) // 256 * 256, out.value
    # one 512 x 2048 int8 projection: 2 column tiles, chunks of 4 groups (16 chunks, 32 workgroups)
    arr = (rtq._Block * 1)(_block(fmt=rtq.FMT_Q8, N=512, K=2048))
    assert lib.rtq_block_workspace_bytes(arr, 1, M, rtq.MATH_SPLIT_F16, ctypes.byref(out)) == OK
    assert out.value == (_image_bytes(2048, M, 2) + 255) // 256 * 256 + 16 * M * 512 * 4, out.value
    # the 12-block set fills the GPU with 408 workgroups: 16-group chunks, only w2 split
    arr12, _ = _rtj_blocks(12, M)
    assert lib.rtq_block_workspace_bytes(arr12, 12, M, rtq.MATH_SPLIT_F16, ctypes.byref(out)) == OK
    images = 12 * (3 * ((_image_bytes(512, M, 2) + 255) // 256 * 256) + (_image_bytes(2048, M, 2) + 255) // 256 * 256)
    assert out.value == images + 12 * 4 * M * 512 * 4, out.value
