"""Oracle for C = A @ B -- TEST INFRASTRUCTURE ONLY.

A plain, slow CPU reference (``oracle.c``) and thin numpy-facing wrappers over it.
Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package; the GPU library never does, and the two share no code.

What each function follows (page and section; the C source states the details):

* ``gemm``/``gemm_rows``/``gemm_cols`` -- the plain product
  C[i][j] = sum_k A[i][k] * B[k][j] (Mojo GPU puzzles, "Tiled Matrix
  Multiplication", section 3: standard A x B, not A x B^T). 16-bit float inputs
  are decoded exactly, summed in binary64 in ascending k and rounded once (RNE)
  to the output format; int32 sums wrap modulo 2^32.
* ``ops`` -- 2*M*N*K ("Reading a matrix multiply through its tiles", opening).
* ``traffic_elems``/``traffic_bytes`` -- the no-reuse traffic of the
  output-stationary loop, summed tile by tile over actual edge ranges (same page,
  "Count the repeated reads" and "Edge tiles still matter").
* ``footprint_bytes`` -- one tile step's working set (same page, "What fits in
  local storage?"; the printed formulas were lost, the three 1 KiB values fix them).
* ``tile_range``/``tile_count`` -- ragged tile ranges (Helion matmul page, the
  ``hl.tile`` paragraph: 10 by 4 gives 0:4, 4:8, 8:10).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

I32, F16, BF16, F32, F64 = 0, 1, 2, 3, 4
_KIND_NAMES = {"i32": I32, "f16": F16, "bf16": BF16, "f32": F32, "f64": F64}
_OUT_NP = {I32: np.int32, F16: np.uint16, BF16: np.uint16, F32: np.float32, F64: np.float64}

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-pthread", "-Wall"]


def compile_source(src: str, out: str) -> str:
    """Compile an oracle C source into a shared library (gcc, no fast-math, no FMA)."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build() -> str:
    """Compile oracle.c into liboracle.so next to it."""
    return compile_source(SOURCE, LIBRARY)


def default_threads() -> int:
    return os.cpu_count() or 1


def _kind(k) -> int:
    return _KIND_NAMES[k] if isinstance(k, str) else int(k)


def _check_in(a: np.ndarray, in_kind: int) -> np.ndarray:
    want = np.int32 if in_kind == I32 else np.uint16
    if a.dtype != want:
        raise TypeError("oracle input must be %s bit patterns, got %s" % (want.__name__, a.dtype))
    if a.ndim != 2 or a.strides[1] != a.itemsize or a.strides[0] % a.itemsize or a.strides[0] < 0:
        raise ValueError("oracle inputs must be 2-D with unit column stride")
    return a


def _ld(a: np.ndarray) -> int:
    return max(a.strides[0] // a.itemsize, a.shape[1])


class Oracle:
    """ctypes view of one build of the oracle library."""

    def __init__(self, path: str = LIBRARY):
        if path == LIBRARY and not os.path.exists(path):
            build()
        lib = ctypes.CDLL(path)
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        p64 = ctypes.POINTER(ctypes.c_int64)
        sig = {
            "oracle_decode_f16": ([ctypes.c_uint16], ctypes.c_double),
            "oracle_decode_bf16": ([ctypes.c_uint16], ctypes.c_double),
            "oracle_encode_f16": ([ctypes.c_double], ctypes.c_uint16),
            "oracle_encode_bf16": ([ctypes.c_double], ctypes.c_uint16),
            "oracle_encode_f32": ([ctypes.c_double], ctypes.c_uint32),
            "oracle_gemm": ([i64, i64, i64, vp, i64, vp, i64, ci, vp, i64, ci, ci], ci),
            "oracle_gemm_rows": ([i64, i64, i64, vp, i64, vp, i64, ci, p64, i64, vp, ci, ci], ci),
            "oracle_gemm_cols": ([i64, i64, i64, vp, i64, vp, i64, ci, p64, i64, vp, ci, ci], ci),
            "oracle_ops": ([i64, i64, i64], i64),
            "oracle_tile_count": ([i64, i64], i64),
            "oracle_tile_range": ([i64, i64, i64, p64, p64], None),
            "oracle_traffic_elems": ([i64, i64, i64, i64, i64, i64, ci, p64], None),
            "oracle_traffic_bytes": ([i64, i64, i64, i64, i64, i64, i64, i64, ci, p64], None),
            "oracle_footprint_bytes": ([i64, i64, i64, i64, i64, p64], None),
        }
        for name, (args, res) in sig.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = res
        self.lib = lib
        self.path = path

    # ---- the product -----------------------------------------------------
    def gemm(self, a: np.ndarray, b: np.ndarray, in_kind, out_kind, threads: int | None = None) -> np.ndarray:
        """C = A @ B for 2-D arrays of bit patterns (uint16 for f16/bf16, int32 for i32).

        Returns int32 for i32, uint16 bit patterns for f16/bf16 outputs, float32 for
        f32 and float64 for the unrounded binary64 sums (f64)."""
        ik, ok = _kind(in_kind), _kind(out_kind)
        a, b = _check_in(a, ik), _check_in(b, ik)
        M, K = a.shape
        K2, N = b.shape
        if K != K2:
            raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
        c = np.zeros((M, N), dtype=_OUT_NP[ok])
        rc = self.lib.oracle_gemm(M, N, K, a.ctypes.data, _ld(a), b.ctypes.data, _ld(b), ik,
                                  c.ctypes.data, N, ok, threads or default_threads())
        if rc != 0:
            raise ValueError("oracle_gemm rejected its arguments")
        return c

    def gemm_rows(self, a, b, rows, in_kind, out_kind, threads: int | None = None) -> np.ndarray:
        """Rows ``rows`` of A @ B, shape (len(rows), N)."""
        ik, ok = _kind(in_kind), _kind(out_kind)
        a, b = _check_in(a, ik), _check_in(b, ik)
        M, K = a.shape
        N = b.shape[1]
        r = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.zeros((len(r), N), dtype=_OUT_NP[ok])
        rc = self.lib.oracle_gemm_rows(M, N, K, a.ctypes.data, _ld(a), b.ctypes.data, _ld(b), ik,
                                       r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), len(r),
                                       out.ctypes.data, ok, threads or default_threads())
        if rc != 0:
            raise ValueError("oracle_gemm_rows rejected its arguments")
        return out

    def gemm_cols(self, a, b, cols, in_kind, out_kind, threads: int | None = None) -> np.ndarray:
        """Columns ``cols`` of A @ B, shape (M, len(cols))."""
        ik, ok = _kind(in_kind), _kind(out_kind)
        a, b = _check_in(a, ik), _check_in(b, ik)
        M, K = a.shape
        N = b.shape[1]
        cc = np.ascontiguousarray(cols, dtype=np.int64)
        out = np.zeros((M, len(cc)), dtype=_OUT_NP[ok])
        rc = self.lib.oracle_gemm_cols(M, N, K, a.ctypes.data, _ld(a), b.ctypes.data, _ld(b), ik,
                                       cc.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), len(cc),
                                       out.ctypes.data, ok, threads or default_threads())
        if rc != 0:
            raise ValueError("oracle_gemm_cols rejected its arguments")
        return out

    # ---- formats ---------------------------------------------------------
    def decode(self, bits, kind) -> np.ndarray:
        """Exact binary64 values of 16-bit patterns (f16 or bf16)."""
        f = self.lib.oracle_decode_f16 if _kind(kind) == F16 else self.lib.oracle_decode_bf16
        flat = np.asarray(bits, dtype=np.uint16).ravel()
        return np.array([f(int(x)) for x in flat], dtype=np.float64).reshape(np.shape(bits))

    def encode(self, values, kind) -> np.ndarray:
        """RNE encoding of binary64 values to f16/bf16 (uint16 bits) or f32 (uint32 bits)."""
        k = _kind(kind)
        f = {F16: self.lib.oracle_encode_f16, BF16: self.lib.oracle_encode_bf16, F32: self.lib.oracle_encode_f32}[k]
        dt = np.uint32 if k == F32 else np.uint16
        flat = np.asarray(values, dtype=np.float64).ravel()
        return np.array([f(float(x)) for x in flat], dtype=dt).reshape(np.shape(values))

    # ---- the pages' counts -------------------------------------------------
    def ops(self, M: int, N: int, K: int) -> int:
        return int(self.lib.oracle_ops(M, N, K))

    def tile_count(self, D: int, t: int) -> int:
        return int(self.lib.oracle_tile_count(D, t))

    def tile_range(self, i: int, t: int, D: int) -> tuple[int, int]:
        lo, hi = ctypes.c_int64(), ctypes.c_int64()
        self.lib.oracle_tile_range(i, t, D, ctypes.byref(lo), ctypes.byref(hi))
        return lo.value, hi.value

    def traffic_elems(self, M, N, K, tm, tn, tk, padded=False) -> tuple[int, int, int]:
        out = (ctypes.c_int64 * 3)()
        self.lib.oracle_traffic_elems(M, N, K, tm, tn, tk, int(bool(padded)), out)
        return out[0], out[1], out[2]

    def traffic_bytes(self, M, N, K, tm, tn, tk, s_in, s_out, padded=False) -> tuple[int, int, int]:
        out = (ctypes.c_int64 * 3)()
        self.lib.oracle_traffic_bytes(M, N, K, tm, tn, tk, s_in, s_out, int(bool(padded)), out)
        return out[0], out[1], out[2]

    def footprint_bytes(self, tm, tn, tk, s_in, s_acc=4) -> tuple[int, int, int]:
        out = (ctypes.c_int64 * 3)()
        self.lib.oracle_footprint_bytes(tm, tn, tk, s_in, s_acc, out)
        return out[0], out[1], out[2]


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from oracle.c (compiled on first use if absent)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
