"""HBM traffic of the main GEMM kernels, as read by rocprofv3 hardware counters.

Each record holds FETCH_SIZE and WRITE_SIZE (KiB per dispatch, averaged over
the profiled dispatches), the calibration factor that maps each counter to
bytes (from a plain copy kernel of known size, profiled in the same way) and
the SHA-256 of the kernel sources the counters were taken on. `lookup` returns
None once those sources have changed: stale counters describe another kernel.
"""
from __future__ import annotations

import hashlib
import os
import re

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
# The recorded kernels (split_grouped_kernel, split_gemm_kernel) and the host
# code that routes a call to them. The direct small-M kernel's file is left
# out: the recorded workloads (M = 80 and 65536) never take it.
KERNEL_SOURCES = ("gemm_split.hip", "gemm.hip", "rtq_internal.h", "rtq_device.h", "split_device.h")

# (workload, math) -> record; filled from the counter runs described in the
# profiles folder.
RECORDS: dict = {
    # split_grouped_kernel<5, 2> (two fp16 limbs, eight waves), 12 blocks at M = 80: 126 dispatches per counter run
    ("m80", "split16"): {"fetch_kib": 33278.474, "write_kib": 32640.027,
         "fetch_factor": 1.99987, "write_factor": 1.0,
         "algorithmic_bytes": 80658432,
         "sources_sha256": "4fc92872de08e16494f50e5e39f6f77fb1d5ec79f9d1d5e3b0d8d4e0ea03491d"},
    # split_grouped_kernel<5, 3> (exact three-limb split), same workload
    ("m80", "split"): {"fetch_kib": 38914.274, "write_kib": 32640.0,
         "fetch_factor": 1.99987, "write_factor": 1.0,
         "algorithmic_bytes": 80658432,
         "sources_sha256": "4fc92872de08e16494f50e5e39f6f77fb1d5ec79f9d1d5e3b0d8d4e0ea03491d"},
    # split_grouped_kernel<5, 1> (bf16 activations), same workload
    ("m80", "bf16"): {"fetch_kib": 27804.402, "write_kib": 32640.0,
         "fetch_factor": 1.99987, "write_factor": 1.0,
         "algorithmic_bytes": 80658432,
         "sources_sha256": "4fc92872de08e16494f50e5e39f6f77fb1d5ec79f9d1d5e3b0d8d4e0ea03491d"},
    # split_gemm_kernel<1|2, NL>, 12 blocks at M = 65536: 480 dispatches per counter run
    # (5 steps x 96 projections); algorithmic bytes are the per-launch average
    ("m65536", "split16"): {"fetch_kib": 105071.67, "write_kib": 235620.687,
         "fetch_factor": 1.99987, "write_factor": 1.0,
         "algorithmic_bytes": 419840512,
         "sources_sha256": "4fc92872de08e16494f50e5e39f6f77fb1d5ec79f9d1d5e3b0d8d4e0ea03491d"},
    ("m65536", "split"): {"fetch_kib": 182665.95, "write_kib": 241984.573,
         "fetch_factor": 1.99987, "write_factor": 1.0,
         "algorithmic_bytes": 419840512,
         "sources_sha256": "4fc92872de08e16494f50e5e39f6f77fb1d5ec79f9d1d5e3b0d8d4e0ea03491d"},
    ("m65536", "bf16"): {"fetch_kib": 52472.332, "write_kib": 237270.779,
         "fetch_factor": 1.99987, "write_factor": 1.0,
         "algorithmic_bytes": 419840512,
         "sources_sha256": "4fc92872de08e16494f50e5e39f6f77fb1d5ec79f9d1d5e3b0d8d4e0ea03491d"},
}


def _code_only(text: str) -> str:
    """Source text without comments and blank space: what the compiler sees
    (the kernel sources hold no string literals with comment markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def sources_sha256() -> str:
    """SHA-256 of the kernel sources' code (comments and layout ignored)."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(CSRC, name)) as f:
            h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()


def lookup(workload: str, math: str):
    rec = RECORDS.get((workload, math))
    if rec is None or rec["sources_sha256"] != sources_sha256():
        return None
    fetch = rec["fetch_kib"] * 1024 * rec["fetch_factor"]
    write = rec["write_kib"] * 1024 * rec["write_factor"]
    return {"bytes_per_launch": round(fetch + write), "fetch_bytes": round(fetch),
            "write_bytes": round(write), "algorithmic_bytes": rec["algorithmic_bytes"],
            "ratio": round((fetch + write) / rec["algorithmic_bytes"], 4)}


# ---------------------------------------------------------------------------
# Command line: the calibration copy and the summary of counter runs.
#   python -m weight_only_quantized_rtq_amd.traffic copy [--mib 256] [--reps 4]
#       runs a plain device-to-device copy-like kernel (torch.neg) of known size;
#   python -m weight_only_quantized_rtq_amd.traffic summarize FETCH_CSV WRITE_CSV
#       COPY_FETCH_CSV COPY_WRITE_CSV KERNEL_REGEX ALGORITHMIC_BYTES [MIB]
#       prints the per-launch averages and the calibrated record.
# ---------------------------------------------------------------------------
def _copy(mib: int, reps: int) -> None:
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(f"copy: {reps} x {mib} MiB read + {mib} MiB written", flush=True)


def _per_dispatch(csv_path: str, regex: str, counter: str):
    import csv
    import re
    pat = re.compile(regex)
    vals = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and pat.search(r["Kernel_Name"]):
                vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} rows for /{regex}/ in {csv_path}")
    return sum(vals.values()) / len(vals), len(vals)


def _summarize(fetch_csv, write_csv, cfetch_csv, cwrite_csv, regex, algo_bytes, mib=256):
    fetch, nf = _per_dispatch(fetch_csv, regex, "FETCH_SIZE")
    write, nw = _per_dispatch(write_csv, regex, "WRITE_SIZE")
    cf, _ = _per_dispatch(cfetch_csv, r"neg|elementwise", "FETCH_SIZE")
    cw, _ = _per_dispatch(cwrite_csv, r"neg|elementwise", "WRITE_SIZE")
    known = mib * 1024 * 1024
    rec = {"fetch_kib": round(fetch, 3), "write_kib": round(write, 3),
           "fetch_factor": round(known / (cf * 1024), 5), "write_factor": round(known / (cw * 1024), 5),
           "algorithmic_bytes": int(algo_bytes), "dispatches": [nf, nw],
           "copy_fetch_kib": round(cf, 1), "copy_write_kib": round(cw, 1),
           "sources_sha256": sources_sha256()}
    print(rec)


if __name__ == "__main__":
    import sys
    if len(sys.argv) >= 2 and sys.argv[1] == "copy":
        mib = int(sys.argv[sys.argv.index("--mib") + 1]) if "--mib" in sys.argv else 256
        reps = int(sys.argv[sys.argv.index("--reps") + 1]) if "--reps" in sys.argv else 4
        _copy(mib, reps)
    elif len(sys.argv) >= 8 and sys.argv[1] == "summarize":
        _summarize(*sys.argv[2:7], int(sys.argv[7]), *(int(v) for v in sys.argv[8:9]))
    else:
        raise SystemExit(__doc__)
