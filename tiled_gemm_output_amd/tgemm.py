"""ctypes binding of libtgemm.so (include/tgemm.h). Argument marshalling only.

The function names are those of the C ABI. Every call goes to the HIP library;
there is no fallback: if libtgemm.so has not been built, loading raises.

    h = gemm_create()
    gemm_run(h, M, N, K, a_ptr, lda, b_ptr, ldb, c_ptr, ldc, BF16_BF16, stream)
    gemm_destroy(h)

``run_tensors`` marshals torch tensors (device pointer, row stride, current stream).
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libtgemm.so")

# gemm_status_t
(OK, ERR_INVALID_ARG, ERR_UNSUPPORTED_DTYPE, ERR_NO_DEVICE, ERR_ARCH, ERR_HIP, ERR_OUT_OF_MEMORY, ERR_UNSUPPORTED_TILE,
 ERR_SCRATCH_TOO_SMALL) = range(9)
# gemm_op_t
OP_N, OP_T = 0, 1
# gemm_dtype_t
I32_I32, F16_F32, BF16_F32, BF16_BF16, F16_F16 = range(5)
DTYPES = {"i32": I32_I32, "f16_f32": F16_F32, "bf16_f32": BF16_F32, "bf16_bf16": BF16_BF16, "f16_f16": F16_F16}
IN_BYTES = {I32_I32: 4, F16_F32: 2, BF16_F32: 2, BF16_BF16: 2, F16_F16: 2}
OUT_BYTES = {I32_I32: 4, F16_F32: 4, BF16_F32: 4, BF16_BF16: 2, F16_F16: 2}
KERNEL_NAMES = {0: "none", 1: "zero_fill", 2: "int32_valu", 3: "mfma_16x16x32_one_wave", 4: "mfma_macro_tile"}

EXPORTS = ["gemm_create", "gemm_run", "gemm_run_op", "gemm_run_op_noalloc", "gemm_tune", "gemm_destroy", "gemm_set_tile", "gemm_set_split_k",
           "gemm_set_repack",
           "gemm_check_args", "gemm_check_args_op", "gemm_plan", "gemm_plan_op", "gemm_model", "gemm_status_string"]


class GemmPlan(ctypes.Structure):
    _fields_ = [("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32), ("tile_k", ctypes.c_int32),
                ("threads", ctypes.c_int32), ("vector_loads", ctypes.c_int32), ("kernel", ctypes.c_int32),
                ("grid", ctypes.c_int64), ("lds_bytes", ctypes.c_int32), ("split_k", ctypes.c_int32),
                ("stages", ctypes.c_int32), ("tail_split_k", ctypes.c_int32), ("tail_m0", ctypes.c_int32),
                ("repack", ctypes.c_int32)]

    def as_dict(self) -> dict:
        d = {name: getattr(self, name) for name, _ in self._fields_}
        d["kernel_name"] = KERNEL_NAMES.get(self.kernel, "?")
        return d


class GemmModel(ctypes.Structure):
    _fields_ = [("flops", ctypes.c_double), ("executed_flops", ctypes.c_double), ("bytes_a", ctypes.c_double),
                ("bytes_b", ctypes.c_double), ("bytes_c", ctypes.c_double), ("bytes_workspace", ctypes.c_double),
                ("compulsory_bytes", ctypes.c_double), ("tiles", ctypes.c_int64), ("k_steps", ctypes.c_int64),
                ("footprint_bytes", ctypes.c_int64), ("lds_bytes", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class GemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s: %s" % (where, gemm_status_string(status)))
        self.status = status


_lib = None


def load(path: str = LIBRARY):
    """Load libtgemm.so (raises if it is missing: there is no other implementation)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libtgemm.so is not built (%s); run python -m tiled_gemm_output_amd.build" % path)
    lib = ctypes.CDLL(path)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32
    lib.gemm_create.argtypes = [ctypes.POINTER(vp)]
    lib.gemm_create.restype = i32
    lib.gemm_run.argtypes = [vp, i64, i64, i64, vp, i64, vp, i64, vp, i64, i32, vp]
    lib.gemm_run.restype = i32
    lib.gemm_run_op.argtypes = [vp, i32, i32, i64, i64, i64, vp, i64, vp, i64, vp, i64, i32, vp]
    lib.gemm_run_op.restype = i32
    lib.gemm_run_op_noalloc.argtypes = [vp, i32, i32, i64, i64, i64, vp, i64, vp, i64, vp, i64, i32, vp]
    lib.gemm_run_op_noalloc.restype = i32
    lib.gemm_tune.argtypes = [vp, i32, i32, i64, i64, i64, vp, i64, vp, i64, vp, i64, i32, vp, i32,
                              ctypes.POINTER(GemmPlan)]
    lib.gemm_tune.restype = i32
    lib.gemm_destroy.argtypes = [vp]
    lib.gemm_destroy.restype = i32
    lib.gemm_set_tile.argtypes = [vp, i32, i32, i32]
    lib.gemm_set_tile.restype = i32
    lib.gemm_set_split_k.argtypes = [vp, i32]
    lib.gemm_set_split_k.restype = i32
    lib.gemm_set_repack.argtypes = [vp, i32]
    lib.gemm_set_repack.restype = i32
    lib.gemm_check_args.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, i32]
    lib.gemm_check_args.restype = i32
    lib.gemm_check_args_op.argtypes = [i32, i32, i64, i64, i64, vp, i64, vp, i64, vp, i64, i32]
    lib.gemm_check_args_op.restype = i32
    lib.gemm_plan.argtypes = [vp, i64, i64, i64, vp, i64, vp, i64, vp, i64, i32, ctypes.POINTER(GemmPlan)]
    lib.gemm_plan.restype = i32
    lib.gemm_plan_op.argtypes = [vp, i32, i32, i64, i64, i64, vp, i64, vp, i64, vp, i64, i32, ctypes.POINTER(GemmPlan)]
    lib.gemm_plan_op.restype = i32
    lib.gemm_model.argtypes = [ctypes.POINTER(GemmPlan), i64, i64, i64, i32, ctypes.POINTER(GemmModel)]
    lib.gemm_model.restype = i32
    lib.gemm_status_string.argtypes = [i32]
    lib.gemm_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def gemm_status_string(status: int) -> str:
    return load().gemm_status_string(int(status)).decode()


def check(status: int, where: str = "tgemm") -> None:
    if status != OK:
        raise GemmError(status, where)


def gemm_create():
    """A handle (c_void_p) on the current HIP device."""
    h = ctypes.c_void_p()
    check(load().gemm_create(ctypes.byref(h)), "gemm_create")
    return h


def gemm_destroy(h) -> int:
    return load().gemm_destroy(h)


def gemm_set_tile(h, tm: int, tn: int, tk: int) -> int:
    return load().gemm_set_tile(h, tm, tn, tk)


def gemm_set_split_k(h, splits: int) -> int:
    return load().gemm_set_split_k(h, splits)


def gemm_set_repack(h, mode: int) -> int:
    return load().gemm_set_repack(h, mode)


def gemm_run(h, M, N, K, A, lda, B, ldb, C, ldc, dtype, stream=None) -> int:
    return load().gemm_run(h, M, N, K, A, lda, B, ldb, C, ldc, int(dtype), stream)


def gemm_run_op(h, op_a, op_b, M, N, K, A, lda, B, ldb, C, ldc, dtype, stream=None) -> int:
    return load().gemm_run_op(h, int(op_a), int(op_b), M, N, K, A, lda, B, ldb, C, ldc, int(dtype), stream)


def gemm_run_op_noalloc(h, op_a, op_b, M, N, K, A, lda, B, ldb, C, ldc, dtype, stream=None) -> int:
    return load().gemm_run_op_noalloc(h, int(op_a), int(op_b), M, N, K, A, lda, B, ldb, C, ldc, int(dtype), stream)


def gemm_tune(h, op_a, op_b, M, N, K, A, lda, B, ldb, C, ldc, dtype, stream=None, iters: int = 5) -> dict:
    """Measure the candidate plans for this shape and keep the fastest in the handle
    (blocks until the timed launches have run); returns that plan."""
    p = GemmPlan()
    check(load().gemm_tune(h, int(op_a), int(op_b), M, N, K, A, lda, B, ldb, C, ldc, int(dtype), stream, int(iters),
                           ctypes.byref(p)), "gemm_tune")
    return p.as_dict()


def gemm_check_args(M, N, K, A, lda, B, ldb, C, ldc, dtype) -> int:
    return load().gemm_check_args(M, N, K, A, lda, B, ldb, C, ldc, int(dtype))


def gemm_check_args_op(op_a, op_b, M, N, K, A, lda, B, ldb, C, ldc, dtype) -> int:
    return load().gemm_check_args_op(int(op_a), int(op_b), M, N, K, A, lda, B, ldb, C, ldc, int(dtype))


def gemm_plan(h, M, N, K, A, lda, B, ldb, C, ldc, dtype) -> dict:
    p = GemmPlan()
    check(load().gemm_plan(h, M, N, K, A, lda, B, ldb, C, ldc, int(dtype), ctypes.byref(p)), "gemm_plan")
    return p.as_dict()


def gemm_plan_op(h, op_a, op_b, M, N, K, A, lda, B, ldb, C, ldc, dtype) -> dict:
    p = GemmPlan()
    check(load().gemm_plan_op(h, int(op_a), int(op_b), M, N, K, A, lda, B, ldb, C, ldc, int(dtype), ctypes.byref(p)),
          "gemm_plan_op")
    return p.as_dict()


def gemm_model(plan, M, N, K, dtype) -> dict:
    """Counts of a plan (a dict from gemm_plan / gemm_plan_op, or the plan fields)."""
    p = GemmPlan(**{name: int(plan.get(name, 0)) for name, _ in GemmPlan._fields_})
    m = GemmModel()
    check(load().gemm_model(ctypes.byref(p), M, N, K, int(dtype), ctypes.byref(m)), "gemm_model")
    return m.as_dict()


def tensor_args(a, b, c):
    """(M, N, K, A, lda, B, ldb, C, ldc) of three 2-D device tensors with unit column stride."""
    for t in (a, b, c):
        if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
            raise ValueError("tensors must be 2-D with unit column stride")
    M, K = a.shape
    N = b.shape[1]
    if b.shape[0] != K or tuple(c.shape) != (M, N):
        raise ValueError("shape mismatch: A %s, B %s, C %s" % (tuple(a.shape), tuple(b.shape), tuple(c.shape)))
    ld = lambda t: max(t.stride(0), t.shape[1], 1)  # noqa: E731
    return M, N, K, a.data_ptr(), ld(a), b.data_ptr(), ld(b), c.data_ptr(), ld(c)


def current_stream():
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def run_tensors(h, a, b, c, dtype, stream=None) -> None:
    """C = A @ B on torch device tensors (16-bit float tensors may be passed as
    int16/uint16 views of the bits)."""
    M, N, K, A, lda, B, ldb, C, ldc = tensor_args(a, b, c)
    s = stream if stream is not None else current_stream()
    check(gemm_run(h, M, N, K, A, lda, B, ldb, C, ldc, dtype, s), "gemm_run")


class Gemm:
    """Owns one handle; ``with Gemm() as g: g.run(a, b, c, BF16_BF16)``."""

    def __init__(self):
        self.h = gemm_create()

    def set_tile(self, tm: int, tn: int, tk: int) -> None:
        check(gemm_set_tile(self.h, tm, tn, tk), "gemm_set_tile")

    def set_split_k(self, splits: int) -> None:
        check(gemm_set_split_k(self.h, splits), "gemm_set_split_k")

    def plan(self, a, b, c, dtype) -> dict:
        return gemm_plan(self.h, *tensor_args(a, b, c), dtype)

    def run(self, a, b, c, dtype, stream=None) -> None:
        run_tensors(self.h, a, b, c, dtype, stream)

    def tune(self, a, b, c, dtype, stream=None, iters: int = 5) -> dict:
        """gemm_tune on row-major tensors (see include/tgemm.h)."""
        M, N, K, A, lda, B, ldb, C, ldc = tensor_args(a, b, c)
        s = stream if stream is not None else current_stream()
        return gemm_tune(self.h, OP_N, OP_N, M, N, K, A, lda, B, ldb, C, ldc, dtype, s, iters)

    def close(self) -> None:
        if self.h is not None:
            gemm_destroy(self.h)
            self.h = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
