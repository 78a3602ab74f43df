"""The vendor comparison tool's command line (host only; the timing itself needs a GPU)."""
import pytest

from tiled_gemm_output_amd import vendor_compare as vc


def test_default_shapes():
    shapes, op = vc.parse_args([])
    assert shapes == vc.DEFAULT_SHAPES and (8192, 8192, 8192) in shapes and op == "nn"
    assert all(len(s) == 3 and min(s) >= 1 for s in shapes)


def test_named_shapes():
    shapes, op = vc.parse_args(["--shape", "4096,4096,4096", "--shape", "128,8192,8192", "--op", "nt"])
    assert shapes == [(4096, 4096, 4096), (128, 8192, 8192)] and op == "nt"


@pytest.mark.parametrize("bad", ["1,2", "0,4,4", "a,b,c"])
def test_bad_shape_refused(bad):
    with pytest.raises(SystemExit):
        vc.parse_args(["--shape", bad])
