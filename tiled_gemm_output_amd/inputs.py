"""Seeded synthetic inputs for C = A @ B.

This module only draws numbers and stores them in the input formats; it holds
none of the product's arithmetic. Both the GPU tests and the oracle side take
their inputs from here, as raw bit patterns in numpy arrays:

* ``int32`` arrays for the integer path;
* ``uint16`` arrays of IEEE binary16 or bfloat16 bit patterns for the float paths
  (values drawn in float32 and rounded to the 16-bit format, round-to-nearest-even).

Workloads (name -> shape, formats, value law, tile):

* ``worked_9x9`` -- the Mojo puzzle's worked example ("Tiled Matrix Multiplication",
  section 1 "Shared memory allocation"): A[i][j] = 9i + j, B[i][j] = 2(9i + j),
  int32, 3x3 tiles.
* ``square128_f16`` -- M = N = K = 128, fp16 inputs uniform in [-1, 1), fp32
  output, 16x16x32 tiles (the traffic example of "Reading a matrix multiply
  through its tiles", section "Count the repeated reads").
* ``ragged96_bf16`` / ``ragged1000x777x333_bf16`` -- bf16 standard normal inputs,
  tile 64 leaves partial tiles ("Edge tiles still matter").
* ``square4096_bf16`` / ``square8192_bf16`` -- bf16 standard normal, bf16 output.
* ``tall16384x1024x8192_bf16`` / ``skinny128x8192x8192_bf16`` -- bf16 normal with
  variance 1/K, fp32 output.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SEED_BASE = 20261202


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dtype: str          # one of i32, f16_f32, bf16_f32, bf16_bf16, f16_f16
    law: str            # worked | uniform | normal | normal_inv_k
    tile: tuple | None  # forced (tm, tn, tk) or None for the library's choice
    index: int          # seed index

    @property
    def in_kind(self) -> str:
        return self.dtype.split("_")[0]

    @property
    def out_kind(self) -> str:
        return self.dtype.split("_")[-1]


WORKLOADS = {
    w.name: w
    for w in [
        Workload("worked_9x9", 9, 9, 9, "i32", "worked", (3, 3, 3), 1),
        Workload("square128_f16", 128, 128, 128, "f16_f32", "uniform", (16, 16, 32), 2),
        Workload("ragged96_bf16", 96, 96, 96, "bf16_f32", "normal", (64, 64, 64), 3),
        Workload("ragged1000x777x333_bf16", 1000, 777, 333, "bf16_f32", "normal", (64, 64, 64), 4),
        Workload("square4096_bf16", 4096, 4096, 4096, "bf16_bf16", "normal", None, 5),
        Workload("square8192_bf16", 8192, 8192, 8192, "bf16_bf16", "normal", None, 6),
        Workload("tall16384x1024x8192_bf16", 16384, 1024, 8192, "bf16_f32", "normal_inv_k", None, 7),
        Workload("skinny128x8192x8192_bf16", 128, 8192, 8192, "bf16_f32", "normal_inv_k", None, 8),
    ]
}


def seeds(index: int) -> tuple[int, int]:
    """(seed for A, seed for B) of workload ``index``."""
    return SEED_BASE + index, SEED_BASE + index + 100


def worked_example() -> tuple[np.ndarray, np.ndarray]:
    """The 9x9 matrices printed on the Mojo puzzle page: A = 9i + j, B = 2A."""
    i = np.arange(9, dtype=np.int32)[:, None]
    j = np.arange(9, dtype=np.int32)[None, :]
    a = (9 * i + j).astype(np.int32)
    return a, (2 * a).astype(np.int32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (nearest, ties to even); return uint16 bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_bits(x: np.ndarray, kind: str) -> np.ndarray:
    if kind == "bf16":
        return f32_to_bf16_bits(x)
    if kind == "f16":
        return f32_to_f16_bits(x)
    raise ValueError(kind)


def draw(shape, law: str, kind: str, seed: int, k: int = 1) -> np.ndarray:
    """One seeded matrix of ``shape`` under ``law``, stored as ``kind`` bits."""
    rng = np.random.default_rng(seed)
    if law == "uniform":
        x = rng.random(shape, dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
    elif law == "normal":
        x = rng.standard_normal(shape, dtype=np.float32)
    elif law == "normal_inv_k":
        x = rng.standard_normal(shape, dtype=np.float32) * np.float32(1.0 / np.sqrt(k))
    elif law == "small_int":
        x = rng.integers(-8, 9, size=shape).astype(np.float32)
    else:
        raise ValueError(law)
    return to_bits(x, kind)


def make(w: Workload | str) -> tuple[np.ndarray, np.ndarray]:
    """Host inputs (A, B) of a workload, dense row-major."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    if w.law == "worked":
        return worked_example()
    sa, sb = seeds(w.index)
    a = draw((w.M, w.K), w.law, w.in_kind, sa, w.K)
    b = draw((w.K, w.N), w.law, w.in_kind, sb, w.K)
    return a, b


def random_case(M: int, N: int, K: int, kind: str, seed: int, law: str = "normal"):
    """Inputs for an ad-hoc shape (sweeps and edge cases)."""
    if kind == "i32":
        rng = np.random.default_rng(seed)
        a = rng.integers(-(2**31), 2**31, size=(M, K), dtype=np.int64).astype(np.int32)
        b = rng.integers(-(2**31), 2**31, size=(K, N), dtype=np.int64).astype(np.int32)
        return a, b
    return draw((M, K), law, kind, seed, max(K, 1)), draw((K, N), law, kind, seed + 1, max(K, 1))


def sample_rows_cols(M: int, N: int, seed: int, block: int = 128):
    """Rows/columns checked at full size: one seeded row per ``block`` rows plus the
    first and last row; the same for columns."""
    rng = np.random.default_rng(seed)
    rows = sorted({0, M - 1} | {int(b0 + rng.integers(0, min(block, M - b0))) for b0 in range(0, M, block)})
    cols = sorted({0, N - 1} | {int(b0 + rng.integers(0, min(block, N - b0))) for b0 in range(0, N, block)})
    return np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)
