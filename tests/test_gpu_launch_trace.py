"""launch_trace.py's run mode on the GPU: every launch timed, in order, on a small product."""
import pytest

from tiled_gemm_output_amd import launch_trace

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def test_run_mode_times_every_launch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    t = launch_trace.run("ragged1000x777x333_bf16", 12)
    per = t["launches"]
    assert [p["launch"] for p in per] == list(range(1, 13))
    assert all(p["us"] > 0 for p in per)
    assert all(b["start_ms"] >= a["start_ms"] for a, b in zip(per, per[1:]))  # back to back, in order
    assert t["flops"] == 2.0 * 1000 * 777 * 333 and t["tile"] == [64, 64, 64]
    assert "| 1-1 |" in launch_trace.table(t, t["flops"])
