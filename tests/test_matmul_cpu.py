"""matmul(a, b): argument checks that run before any GPU call, and the operand
form chosen for each stride pattern (host logic only)."""
import pytest

torch = pytest.importorskip("torch")

from tiled_gemm_output_amd import tgemm  # noqa: E402
from tiled_gemm_output_amd.matmul import _dtype_code, matmul, operand_form  # noqa: E402


def test_operand_form():
    w = torch.empty(64, 48)
    assert operand_form(w) == (tgemm.OP_N, 48)
    assert operand_form(w.t()) == (tgemm.OP_T, 48)        # 48 x 64 view, stored 64 x 48
    assert operand_form(w[:, :40]) == (tgemm.OP_N, 48)     # row stride beyond the row length
    assert operand_form(w[:40].t()) == (tgemm.OP_T, 48)
    assert operand_form(torch.empty(1, 7)) == (tgemm.OP_N, 7)
    assert operand_form(torch.empty(7, 1)) == (tgemm.OP_N, 1)
    assert operand_form(torch.empty(0, 5)) == (tgemm.OP_N, 5)
    with pytest.raises(ValueError):
        operand_form(w[:, ::2])                            # column stride 2
    with pytest.raises(ValueError):
        operand_form(torch.empty(4, 6, 8)[:, :, 0])        # strides (48, 8)


def test_dtype_table():
    assert _dtype_code(torch.bfloat16, torch.bfloat16) == tgemm.BF16_BF16
    assert _dtype_code(torch.bfloat16, torch.float32) == tgemm.BF16_F32
    assert _dtype_code(torch.float16, torch.float16) == tgemm.F16_F16
    assert _dtype_code(torch.float16, torch.float32) == tgemm.F16_F32
    assert _dtype_code(torch.int32, torch.int32) == tgemm.I32_I32
    for pair in [(torch.float32, torch.float32), (torch.int32, torch.float32), (torch.bfloat16, torch.float16)]:
        with pytest.raises(TypeError):
            _dtype_code(*pair)


def test_argument_errors_before_any_gpu_call():
    a = torch.empty(8, 4, dtype=torch.bfloat16)
    b = torch.empty(4, 5, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="one GPU device"):
        matmul(a, b)                                        # host tensors
    with pytest.raises(ValueError, match="inner dimensions"):
        matmul(a, torch.empty(5, 5, dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="share a dtype"):
        matmul(a, b.half())
    with pytest.raises(ValueError, match="2-D"):
        matmul(a[0], b)
    with pytest.raises(TypeError):
        matmul([1], b)
