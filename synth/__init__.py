"""Seeded synthetic workloads for the RT-J projection GEMM.

This module only draws random numbers and lays them out in the shapes of the
RT-J blocks. It holds none of the quantization or GEMM arithmetic: both the
CPU oracle and the GPU path receive the same fp32 tensors from here and
quantize / contract them independently.

Shapes follow the RT-J configuration printed on the "Backends" page of the
relational-transformers docs (section "Meta": 12 blocks, d_model 512,
d_ff 2048). The pages' own workload is the RelativeDB golden batch (B=5,
S=16, i.e. 80 rows; int4 model card, section "Accuracy"); that batch and the
trained weights are not available, so Gaussian stand-ins of the same shapes
are drawn here: weights ~ N(0, 0.02^2), activations ~ N(0, 1), fp32.

Every tensor comes from its own PCG64 stream keyed by
SeedSequence([20261203, cfg, set, block, slot, role]).
"""
from __future__ import annotations

import hashlib

import numpy as np

SEED_ROOT = 20261203

# RT-J dimensions ("Backends" page, section "Meta").
NUM_BLOCKS = 12
D_MODEL = 512
D_FF = 2048

# Golden-batch row count (int4 model card, section "Accuracy": B=5, S=16).
M_GOLDEN = 5 * 16
# Compute-bound workload: 256 contexts x 256 cells.
M_LARGE = 256 * 256

# Stream slots. Weights 0..7, activations 8..11.
SLOTS = {
    "wq": 0, "wk": 1, "wv": 2, "wg": 3, "wo": 4, "w1": 5, "w3": 6, "w2": 7,
    "x_attn": 8, "x_o": 9, "x_ffn": 10, "h": 11,
}
ROLE_VALUES = 0
ROLE_HEAVY_PICK = 1

# Projection name -> (N out features, K in features, name of the input it reads).
# wq/wk/wv/wg read the attention input, wo the attention output, w1/w3 the FFN
# input and w2 the FFN hidden state (width d_ff).
BLOCK_SHAPES = {
    "wq": (D_MODEL, D_MODEL, "x_attn"),
    "wk": (D_MODEL, D_MODEL, "x_attn"),
    "wv": (D_MODEL, D_MODEL, "x_attn"),
    "wg": (D_MODEL, D_MODEL, "x_attn"),
    "wo": (D_MODEL, D_MODEL, "x_o"),
    "w1": (D_FF, D_MODEL, "x_ffn"),
    "w3": (D_FF, D_MODEL, "x_ffn"),
    "w2": (D_MODEL, D_FF, "h"),
}
PROJ_ORDER = ("wq", "wk", "wv", "wg", "wo", "w1", "w3", "w2")
INPUT_WIDTH = {"x_attn": D_MODEL, "x_o": D_MODEL, "x_ffn": D_MODEL, "h": D_FF}

WEIGHT_STD = np.float32(0.02)
HEAVY_FRACTION = 0.05
HEAVY_FACTOR = np.float32(20.0)


def rng(cfg: int, set_: int, block: int, slot: int, role: int = ROLE_VALUES) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([SEED_ROOT, cfg, set_, block, slot, role]))


def weight(cfg: int, set_: int, block: int, name: str, N: int | None = None, K: int | None = None,
           heavy: str | None = None) -> np.ndarray:
    """fp32 weight [N, K] ~ N(0, 0.02^2).

    heavy="rows": floor(0.05*N) output rows (seeded pick) are multiplied by 20.
    heavy="cols": floor(0.05*K) input columns are multiplied by 20 (about 1.6
    outliers per 32-wide group, which moves the clip search).
    """
    if N is None or K is None:
        N, K, _ = BLOCK_SHAPES[name]
    slot = SLOTS[name]
    w = rng(cfg, set_, block, slot).standard_normal((N, K), dtype=np.float32) * WEIGHT_STD
    if heavy is not None:
        pick_rng = rng(cfg, set_, block, slot, ROLE_HEAVY_PICK)
        if heavy == "rows":
            idx = pick_rng.choice(N, size=int(np.floor(HEAVY_FRACTION * N)), replace=False)
            w[idx, :] *= HEAVY_FACTOR
        elif heavy == "cols":
            idx = pick_rng.choice(K, size=int(np.floor(HEAVY_FRACTION * K)), replace=False)
            w[:, idx] *= HEAVY_FACTOR
        else:
            raise ValueError(f"unknown heavy-tail variant {heavy!r}")
    return w


SHARED_BLOCK = 4095  # block index of activations shared by every block


def activation(cfg: int, block: int, name: str, M: int, K: int | None = None) -> np.ndarray:
    """fp32 activation [M, K] ~ N(0, 1). Use block=SHARED_BLOCK for an input
    shared by all blocks."""
    if K is None:
        K = INPUT_WIDTH[name]
    return rng(cfg, 0, block, SLOTS[name]).standard_normal((M, K), dtype=np.float32)


def uniform_ints(seed: int, shape, lo: int, hi: int, dtype=np.int64) -> np.ndarray:
    """Seeded integers in [lo, hi] (inclusive), for exact-arithmetic cases."""
    g = np.random.default_rng(np.random.SeedSequence([SEED_ROOT, 99, seed]))
    return g.integers(lo, hi + 1, size=shape).astype(dtype)


def uniform_bytes(seed: int, shape) -> np.ndarray:
    g = np.random.default_rng(np.random.SeedSequence([SEED_ROOT, 98, seed]))
    return g.integers(0, 256, size=shape, dtype=np.uint8)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]
