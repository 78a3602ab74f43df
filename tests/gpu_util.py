"""Helpers of the GPU parity tests: device buffers laid out with a chosen leading
dimension and pointer offset, a sentinel-filled C whose untouched elements are
checked after the call, and the accuracy rule.

Accuracy rule for floating-point outputs (the method accumulates in fp32; the
oracle sums exactly in binary64 and rounds once to the output format, giving R):
  * elementwise: |C - R| <= max(2e-3 * max|R|, one unit in the last place of R
    in the output format) -- a different fp32 summation order can flip the final
    rounding of an output by one unit;
  * normwise, for fp32 outputs: max |C - R| / max |R| <= 2e-3. (For bf16/f16
    outputs one such flip near max|R| alone is 2^-8 / 2^-11 relative, so there
    the normwise figure is reported, not asserted.)
Integer outputs and integer-valued float inputs (exact in fp32 in any order) must
match bit for bit.
"""
from __future__ import annotations

import numpy as np

from tiled_gemm_output_amd import tgemm

TOL = 2e-3
OUT_KIND = {tgemm.I32_I32: "i32", tgemm.F16_F32: "f32", tgemm.BF16_F32: "f32", tgemm.BF16_BF16: "bf16",
            tgemm.F16_F16: "f16"}
IN_KIND = {tgemm.I32_I32: "i32", tgemm.F16_F32: "f16", tgemm.BF16_F32: "bf16", tgemm.BF16_BF16: "bf16",
           tgemm.F16_F16: "f16"}
SENTINEL = {2: 0x7FA5, 4: 0x7FC0DEAD}  # NaN patterns no finite product produces


def _torch():
    import torch

    return torch


def int_dtype(nbytes):
    t = _torch()
    return t.int16 if nbytes == 2 else t.int32


def np_int(nbytes):
    return np.int16 if nbytes == 2 else np.int32


class DevMatrix:
    """rows x cols matrix at element offset ``off`` of a device buffer, row stride ``ld``."""

    def __init__(self, host: np.ndarray | None, rows: int, cols: int, ld: int, off: int, nbytes: int, fill=None):
        torch = _torch()
        self.rows, self.cols, self.ld, self.off, self.nbytes = rows, cols, max(ld, 1), off, nbytes
        total = off + (rows - 1) * self.ld + cols if rows > 0 and cols > 0 else off + 1
        total += 8  # guard elements after the matrix
        fill = SENTINEL[nbytes] if fill is None else fill
        self.fill = np.array(fill, dtype=np.int64).astype(np_int(nbytes)).item()
        self.buf = torch.full((total,), self.fill, dtype=int_dtype(nbytes), device="cuda")
        if host is not None and rows > 0 and cols > 0:
            src = torch.from_numpy(np.ascontiguousarray(host).view(np_int(nbytes))).cuda()
            self.view().copy_(src)

    def view(self):
        return self.buf.as_strided((self.rows, self.cols), (self.ld, 1), self.off)

    @property
    def ptr(self) -> int:
        return self.buf.data_ptr() + self.off * self.nbytes

    def host(self) -> np.ndarray:
        if self.rows == 0 or self.cols == 0:
            return np.zeros((self.rows, self.cols), dtype=np_int(self.nbytes))
        return self.view().cpu().numpy()

    def untouched_outside(self) -> bool:
        """Every element outside the matrix window still holds the fill value."""
        torch = _torch()
        mask = torch.ones_like(self.buf, dtype=torch.bool)
        if self.rows > 0 and self.cols > 0:
            mask.as_strided((self.rows, self.cols), (self.ld, 1), self.off).fill_(False)
        return bool((self.buf[mask] == self.fill).all().item())


def run(h, a: np.ndarray, b: np.ndarray, dtype: int, lda=None, ldb=None, ldc=None, offs=(0, 0, 0), stream=None,
        op_a=tgemm.OP_N, op_b=tgemm.OP_N, ab_fill=0):
    """Copy A, B to the device with the given layout, run gemm_run (gemm_run_op when an
    operand is to be supplied transposed: then its transpose is what is stored, with
    row stride lda / ldb), return (C host bits, C DevMatrix). a is the M x K op(A),
    b the K x N op(B). ab_fill: bit pattern of the A and B buffers around the matrices
    (row padding, offsets, guard elements)."""
    torch = _torch()
    M, K = a.shape
    N = b.shape[1]
    ib = 4 if dtype == tgemm.I32_I32 else 2
    ob = tgemm.OUT_BYTES[dtype]
    sa = np.ascontiguousarray(a.T) if op_a == tgemm.OP_T else a
    sb = np.ascontiguousarray(b.T) if op_b == tgemm.OP_T else b
    lda = sa.shape[1] if lda is None else lda
    ldb = sb.shape[1] if ldb is None else ldb
    ldc = N if ldc is None else ldc
    da = DevMatrix(sa, sa.shape[0], sa.shape[1], lda, offs[0], ib, fill=ab_fill)
    db = DevMatrix(sb, sb.shape[0], sb.shape[1], ldb, offs[1], ib, fill=ab_fill)
    dc = DevMatrix(None, M, N, ldc, offs[2], ob)
    s = stream if stream is not None else torch.cuda.current_stream()
    if op_a == tgemm.OP_N and op_b == tgemm.OP_N:
        st = tgemm.gemm_run(h, M, N, K, da.ptr, da.ld, db.ptr, db.ld, dc.ptr, dc.ld, dtype, s.cuda_stream)
    else:
        st = tgemm.gemm_run_op(h, op_a, op_b, M, N, K, da.ptr, da.ld, db.ptr, db.ld, dc.ptr, dc.ld, dtype,
                               s.cuda_stream)
    tgemm.check(st, "gemm_run")
    torch.cuda.synchronize()
    return dc.host(), dc


def values(bits: np.ndarray, kind: str) -> np.ndarray:
    """Float values of output bits (f32 / bf16 / f16), as float64."""
    if kind == "f32":
        return np.asarray(bits).view(np.float32).astype(np.float64)
    if kind == "f16":
        return np.asarray(bits).view(np.uint16).view(np.float16).astype(np.float64)
    if kind == "bf16":
        u = np.asarray(bits).view(np.uint16).astype(np.uint32) << 16
        return u.view(np.float32).astype(np.float64)
    raise ValueError(kind)


def ulp(r: np.ndarray, kind: str) -> np.ndarray:
    """Spacing of the output format at |r| (the unit in the last place)."""
    p, emin = {"f32": (24, -126), "bf16": (8, -126), "f16": (11, -14)}[kind]
    a = np.abs(r)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, emin)
    return np.exp2(e - (p - 1))


def compare(c_bits: np.ndarray, ref_bits: np.ndarray, kind: str, tol: float = TOL) -> dict:
    """Apply the accuracy rule; returns the statistics (raises AssertionError on failure)."""
    if kind == "i32":
        bad = int(np.sum(c_bits.view(np.int32) != ref_bits.view(np.int32)))
        assert bad == 0, "%d int32 mismatches" % bad
        return {"mismatches": 0}
    c = values(c_bits, kind)
    r = values(ref_bits, kind)
    assert np.all(np.isfinite(c)), "non-finite outputs (unwritten elements?)"
    scale = float(np.max(np.abs(r))) if r.size else 0.0
    err = np.abs(c - r)
    norm = float(err.max() / scale) if r.size and scale > 0 else float(err.max() if r.size else 0.0)
    allowed = np.maximum(tol * scale, ulp(r, kind))
    worst = int(np.sum(err > allowed))
    flips = int(np.sum(c_bits != ref_bits))
    assert worst == 0, "%d elements beyond max(tol*max|R|, 1 ulp); normwise %.3g" % (worst, norm)
    if kind == "f32":
        assert norm <= tol or scale == 0.0, "normwise error %.3g > %.3g" % (norm, tol)
    return {"normwise": norm, "differing": flips, "scale": scale}
