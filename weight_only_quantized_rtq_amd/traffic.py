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

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
KERNEL_SOURCES = ("gemm_split.hip", "gemm.hip", "rtq_internal.h", "rtq_device.h")

# (workload, math) -> record; filled from the counter runs described in the
# profiles folder.
RECORDS: dict = {}


def sources_sha256() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
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
