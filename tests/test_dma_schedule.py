"""The split kernels' DMA schedule (x stages and weight chunks streamed into
LDS rings), checked on the host.

`DmaSchedule` in gemm_split.hip decides which x stage and weight chunk each
iteration issues and how many of a wave's loads may still be in flight at the
top of each step. The kernels `static_assert` its `verify()`, a replay of the
schedule with an in-order completion model. Here the struct is compiled from
the kernel source with g++ and:
  * `verify()` holds for every (XL, WL, NX, NWC) the kernels instantiate and
    for a few deeper leads;
  * `verify()` fails for planted mistakes: a wait that leaves one load too
    many in flight, a chunk issued one step early, an x stage issued two steps
    ahead into a two-slot ring, a prologue that skips an x stage, and a wait
    count that ignores the order of a step's stage and chunk (waits stricter
    than needed are rejected too), the constant steady-state wait used on the
    first step, where the prologue's loads are still in flight, the head's
    large-GS wait constants taken for too short a K walk, and the tail's wait
    constants with the step parity swapped.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "weight_only_quantized_rtq_amd", "csrc", "gemm_split.hip")

# (XL, WL, NX, NWC) of the instantiated kernels: grouped small-M kernel (eight
# waves, TM = 1..5 row tiles, 1..3 limbs: NX = ceil(TM*NL/8) + 1, two column
# tiles per wave) and the large-M kernel with one or two limbs (four waves,
# eight row tiles: NX = 2*NL + 1), all with XL = WL = 1.
USED = sorted({(1, 1, (tm * nl + 7) // 8 + 1, 2) for tm in range(1, 6) for nl in (1, 2, 3)} |
              {(1, 1, 3, 2), (1, 1, 5, 2)})
DEEPER = [(2, 1, 3, 2), (2, 2, 4, 4), (3, 2, 3, 2), (4, 2, 2, 2), (3, 3, 3, 4)]

MUTANTS = {
    "wait_one_too_many": ("        return n;\n", "        return n + 1;\n"),
    "chunk_one_step_early": ("return i >= 2 && (i & 1) == 0 && i + 2 * WL < GS;",
                             "return i >= 1 && (i & 1) == 1 && i + 1 + 2 * WL < GS;"),
    "stage_two_ahead": ("return i >= 1 && i + XL < GS; }", "return i >= 1 && i + XL + 1 < GS; }"),
    "prologue_skips_stage": ("return need <= XL && need < GS; }", "return need < XL && need < GS; }"),
    "chunk_before_stage_in_key": ("return c <= WL ? 4 * c : 4096 + 2 * (2 * c - 2 * WL) + 1; }",
                                  "return c <= WL ? 4 * c : 4096 + 2 * (2 * c - 2 * WL) - 1; }"),
    "steady_from_first_step": ("static constexpr int kSteadyLo = kPrologue + 1;",
                               "static constexpr int kSteadyLo = 0;"),
    "head_constant_too_early": ("static constexpr int kBig = 2 * kPrologue + 3;",
                                "static constexpr int kBig = kPrologue;"),
    "tail_parity_swapped": ("return allowed(2 * kPrologue + 2 + parity, 2 * kPrologue + 3 + parity + r); }",
                            "return allowed(2 * kPrologue + 3 - parity, 2 * kPrologue + 4 - parity + r); }"),
}


def schedule_source() -> str:
    text = open(SRC).read()
    a = text.index("template <int XL, int WL, int NX, int NWC>\nstruct DmaSchedule")
    b = text.index("\n};\n", a) + 4
    return text[a:b].replace("__host__ __device__ ", "")


def run_verify(struct: str, configs, tmp_path) -> list:
    calls = ", ".join(f"(int)DmaSchedule<{xl}, {wl}, {nx}, {nwc}>::verify()" for xl, wl, nx, nwc in configs)
    prog = "#include <cstdio>\n" + struct + "\nint main() {\n    const int r[] = {" + calls + "};\n" \
        "    for (int v : r) std::printf(\"%d\\n\", v);\n}\n"
    cpp, exe = tmp_path / "sched.cpp", tmp_path / "sched"
    cpp.write_text(prog)
    subprocess.run(["g++", "-std=c++17", "-O1", str(cpp), "-o", str(exe)], check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    return [int(v) for v in out]


pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")


def test_schedule_of_every_instantiated_kernel_verifies(tmp_path):
    assert run_verify(schedule_source(), USED + DEEPER, tmp_path) == [1] * (len(USED) + len(DEEPER))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_schedule_mistake_fails_verify(name, tmp_path):
    before, after = MUTANTS[name]
    src = schedule_source()
    assert src.count(before) == 1, name
    res = run_verify(src.replace(before, after), USED, tmp_path)
    assert 0 in res, (name, res)
