"""``matmul(a, b) -> c`` on torch device tensors.

The contract is that of the Helion matmul page (the page that writes the tiled
kernel with ``hl.tile``): ``a`` is M x K, ``b`` is K x N, and the result is a new
M x N tensor of ``a``'s dtype, accumulated in an fp32 tile
(fp16 -> fp16, bf16 -> bf16; int32 -> int32, exact modulo 2^32). Tile sizes are
chosen by the library. Every step of the product runs in libtgemm.so; this module
only maps tensors to the C entry point's arguments:

* a row-major view (unit column stride) is passed as stored (``GEMM_OP_N``); a
  column-major view, e.g. ``w.t()`` of a row-major ``w``, is passed as its
  row-major transpose (``GEMM_OP_T``), so transposed operands cost no copy;
* the result is allocated with ``torch.empty`` (device memory only) unless
  ``out`` is given; the work is enqueued on the current stream of ``a``'s device,
  through a library handle of that host thread, device and stream.

Other strides raise ``ValueError``: nothing is copied or converted here.
"""
from __future__ import annotations

import threading

from . import tgemm

# One handle per host thread, device and stream. A handle is single-threaded, and the
# calls that use its workspaces (split-K partial tiles, operand copies) must be ordered:
# calls on one stream are, and calls on different streams (a graph capture runs on a
# stream of its own) get different handles, so they never share a workspace.
_local = threading.local()


def _handle(device_index: int, stream: int):
    import torch

    hs = getattr(_local, "handles", None)
    if hs is None:
        hs = _local.handles = {}
    key = (device_index, stream)
    g = hs.get(key)
    if g is None:
        with torch.cuda.device(device_index):
            g = hs[key] = tgemm.Gemm()
    return g.h


def _dtype_code(in_dtype, out_dtype):
    import torch

    table = {
        (torch.bfloat16, torch.bfloat16): tgemm.BF16_BF16,
        (torch.bfloat16, torch.float32): tgemm.BF16_F32,
        (torch.float16, torch.float16): tgemm.F16_F16,
        (torch.float16, torch.float32): tgemm.F16_F32,
        (torch.int32, torch.int32): tgemm.I32_I32,
    }
    code = table.get((in_dtype, out_dtype))
    if code is None:
        raise TypeError("matmul: unsupported input/output dtypes %s -> %s (inputs bf16, fp16 or int32; output "
                        "the input dtype, or float32 for 16-bit float inputs)" % (in_dtype, out_dtype))
    return code


def operand_form(t, name: str = "operand"):
    """(op, leading dimension) of a 2-D tensor: GEMM_OP_N for a row-major view,
    GEMM_OP_T for a column-major one (its transpose is row-major in memory)."""
    rows, cols = t.shape
    s0, s1 = t.stride()
    if (cols <= 1 or s1 == 1) and (rows <= 1 or s0 >= cols):
        return tgemm.OP_N, (s0 if rows > 1 else max(cols, 1))
    if (rows <= 1 or s0 == 1) and (cols <= 1 or s1 >= rows):
        return tgemm.OP_T, (s1 if cols > 1 else max(rows, 1))
    raise ValueError("matmul: %s with shape %s and strides %s is neither row- nor column-major; pass a "
                     "contiguous tensor" % (name, tuple(t.shape), tuple(t.stride())))


def matmul(a, b, *, out_dtype=None, out=None):
    """C = a @ b computed by the tiled GEMM library.

    a: M x K and b: K x N CUDA/HIP tensors of one dtype (bfloat16, float16 or int32)
    on one device. out_dtype: the result dtype (default a.dtype; float32 is also
    accepted for 16-bit float inputs). out: optional M x N tensor with unit column
    stride to write into (its dtype decides the result dtype). Returns C."""
    import torch

    if not (isinstance(a, torch.Tensor) and isinstance(b, torch.Tensor)):
        raise TypeError("matmul: a and b must be torch tensors")
    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("matmul: a and b must be 2-D, got %d-D and %d-D" % (a.dim(), b.dim()))
    if a.shape[1] != b.shape[0]:
        raise ValueError("matmul: inner dimensions differ: a %s, b %s" % (tuple(a.shape), tuple(b.shape)))
    if a.dtype != b.dtype:
        raise TypeError("matmul: a and b must share a dtype, got %s and %s" % (a.dtype, b.dtype))
    if a.device.type != "cuda" or b.device != a.device:
        raise ValueError("matmul: a and b must be on one GPU device, got %s and %s" % (a.device, b.device))
    M, K = a.shape
    N = b.shape[1]
    if out is not None:
        if out_dtype is not None and out.dtype != out_dtype:
            raise TypeError("matmul: out has dtype %s, out_dtype is %s" % (out.dtype, out_dtype))
        out_dtype = out.dtype
        if tuple(out.shape) != (M, N) or out.device != a.device:
            raise ValueError("matmul: out must be a %d x %d tensor on %s" % (M, N, a.device))
        if N > 1 and out.stride(1) != 1 or (M > 1 and out.stride(0) < N):
            raise ValueError("matmul: out must have unit column stride and row stride >= N")
    elif out_dtype is None:
        out_dtype = a.dtype
    code = _dtype_code(a.dtype, out_dtype)
    op_a, lda = operand_form(a, "a")
    op_b, ldb = operand_form(b, "b")
    c = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=a.device)
    ldc = c.stride(0) if M > 1 else max(N, 1)
    dev = a.device.index if a.device.index is not None else torch.cuda.current_device()
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream().cuda_stream
        h = _handle(dev, stream)
        st = tgemm.gemm_run_op(h, op_a, op_b, M, N, K, a.data_ptr(), lda, b.data_ptr(), ldb, c.data_ptr(), ldc,
                               code, stream)
    tgemm.check(st, "gemm_run_op")
    return c
