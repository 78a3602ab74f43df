"""gemm_model (the library's count of what a planned call requests and executes)
pinned to the oracle's tile walk of the pages' traffic count and to the values
the pages print. Host-only: no GPU needed."""
import ctypes

import numpy as np
import pytest

import oracle
from tiled_gemm_output_amd import tgemm

S_IN = {tgemm.I32_I32: 4, tgemm.F16_F32: 2, tgemm.BF16_F32: 2, tgemm.BF16_BF16: 2, tgemm.F16_F16: 2}


@pytest.fixture(scope="module")
def o():
    return oracle.get()


def auto_plan(M, N, K, dtype):
    return tgemm.gemm_plan(None, M, N, K, ctypes.c_void_p(1 << 20), max(K, 1), ctypes.c_void_p(1 << 21), max(N, 1),
                           ctypes.c_void_p(1 << 22), max(N, 1), dtype)


def forced_plan(tm, tn, tk, kernel=4, split_k=1, lds=0, stages=2):
    return {"tile_m": tm, "tile_n": tn, "tile_k": tk, "threads": 64, "vector_loads": 1, "kernel": kernel,
            "grid": 0, "lds_bytes": lds, "split_k": split_k, "stages": stages}


def test_page_values():
    """The traffic example (128^3, 16x16x32, fp16 in, fp32 C): 576 KiB; the edge
    tile counts at tile 64 over actual ranges."""
    m = tgemm.gemm_model(forced_plan(16, 16, 32, kernel=3), 128, 128, 128, tgemm.F16_F32)
    assert m["bytes_a"] + m["bytes_b"] + m["bytes_c"] == 589824 == 576 * 1024
    assert (m["bytes_a"], m["bytes_b"], m["bytes_c"]) == (262144, 262144, 65536)
    assert m["flops"] == 4194304 and m["tiles"] == 64 and m["k_steps"] == 4
    assert m["footprint_bytes"] == 3 * 1024  # 1 KiB each for the A, B and C tiles
    m = tgemm.gemm_model(forced_plan(64, 64, 64), 96, 96, 96, tgemm.BF16_F32)
    assert m["bytes_a"] + m["bytes_b"] + m["bytes_c"] == 110592
    m = tgemm.gemm_model(forced_plan(64, 64, 64), 1000, 777, 333, tgemm.BF16_F32)
    assert m["bytes_a"] + m["bytes_b"] + m["bytes_c"] == 20045712


def shapes():
    rng = np.random.default_rng(11)
    out = [(128, 128, 128), (96, 96, 96), (1000, 777, 333), (8192, 8192, 8192), (128, 8192, 8192), (1, 1, 1),
           (9, 9, 9), (0, 5, 5), (5, 5, 0)]
    out += [tuple(int(x) for x in rng.integers(1, 3000, size=3)) for _ in range(30)]
    return out


@pytest.mark.parametrize("shape", shapes(), ids=str)
def test_model_matches_oracle_walk(o, shape):
    """bytes_a/b/c equal the oracle's actual-range tile walk for the library's own
    plan and for every forced tile; flops equal 2MNK; the working set equals the
    oracle's footprint formula."""
    M, N, K = shape
    for dtype in (tgemm.BF16_BF16, tgemm.F16_F32, tgemm.I32_I32):
        plans = [auto_plan(M, N, K, dtype)]
        if M * N * K > 1 << 36:
            pass  # the oracle walks every (tile, K-step): only the library's own plan at the largest size
        elif dtype != tgemm.I32_I32:
            plans += [forced_plan(16, 16, 32, kernel=3)] + [forced_plan(*t) for t in
                                                            [(64, 64, 64), (128, 128, 64), (256, 128, 64),
                                                             (256, 256, 64)]]
        else:
            plans += [forced_plan(3, 3, 3, kernel=2), forced_plan(32, 8, 7, kernel=2)]
        for p in plans:
            m = tgemm.gemm_model(p, M, N, K, dtype)
            assert m["flops"] == o.ops(M, N, K)
            s_out = tgemm.OUT_BYTES[dtype]
            if p["kernel"] < 2:
                assert m["bytes_a"] == m["bytes_b"] == 0 and m["bytes_c"] == s_out * M * N
                continue
            tm, tn, tk = p["tile_m"], p["tile_n"], p["tile_k"]
            ref = o.traffic_bytes(M, N, K, tm, tn, tk, S_IN[dtype], s_out)
            assert (m["bytes_a"], m["bytes_b"], m["bytes_c"]) == tuple(float(x) for x in ref), (p, dtype)
            assert m["footprint_bytes"] == sum(o.footprint_bytes(tm, tn, tk, S_IN[dtype]))
            assert m["tiles"] == o.tile_count(M, tm) * o.tile_count(N, tn)
            assert m["compulsory_bytes"] == S_IN[dtype] * (M * K + K * N) + s_out * M * N


def test_executed_work_and_split_workspace():
    # 8192^3 at 256x256x64: 128 K-steps: executed == algorithmic
    m = tgemm.gemm_model(forced_plan(256, 256, 64), 8192, 8192, 8192, tgemm.BF16_BF16)
    assert m["executed_flops"] == m["flops"] and m["bytes_workspace"] == 0
    # 96^3 at tile 64: 2x2 tiles of 64x64 over K = 2 steps of 64 -> 128^2 x 128 x 2
    m = tgemm.gemm_model(forced_plan(64, 64, 64), 96, 96, 96, tgemm.BF16_F32)
    assert m["executed_flops"] == 2 * 128 * 128 * 128
    # 3 K-steps, the last one partial (150 = 2 x 64 + 22): 3 steps of MFMAs, no zero steps
    m = tgemm.gemm_model(forced_plan(64, 64, 64), 64, 64, 150, tgemm.BF16_F32)
    assert m["executed_flops"] == 2 * 64 * 64 * 64 * 3
    # split-K: 128 K-steps in 4 slices of 32; fp32 partials written and read: 2 x 4 x S x M x N
    p = auto_plan(128, 8192, 8192, tgemm.BF16_F32)
    m = tgemm.gemm_model(p, 128, 8192, 8192, tgemm.BF16_F32)
    assert p["split_k"] == 4 and m["bytes_workspace"] == 2 * 4 * 4 * 128 * 8192
    assert m["executed_flops"] == m["flops"]
    # 4 stages: 18 K-steps, whatever the stage count
    m = tgemm.gemm_model(forced_plan(128, 128, 64, stages=4), 1792, 1792, 1096, tgemm.BF16_BF16)
    assert m["executed_flops"] == 2 * (14 * 128) ** 2 * 64 * 18
    # 7 K-steps in slices of 3, 3, 1: 7 steps in all
    m = tgemm.gemm_model(forced_plan(64, 64, 64, split_k=3), 64, 64, 7 * 64, tgemm.BF16_F32)
    assert m["executed_flops"] == 2 * 64 * 64 * 64 * 7


def test_model_rejects_bad_plans():
    with pytest.raises(tgemm.GemmError):
        tgemm.gemm_model(forced_plan(0, 64, 64), 64, 64, 64, tgemm.BF16_F32)
    with pytest.raises(tgemm.GemmError):
        tgemm.gemm_model(forced_plan(64, 64, 64, kernel=9), 64, 64, 64, tgemm.BF16_F32)
    with pytest.raises(tgemm.GemmError):
        tgemm.gemm_model(forced_plan(64, 64, 64), -1, 64, 64, tgemm.BF16_F32)
    with pytest.raises(tgemm.GemmError):
        tgemm.gemm_model(forced_plan(64, 64, 64), 64, 64, 64, 7)


def test_model_of_a_tail_split():
    """executed_flops and the workspace of a plan with a split-K tail: the tiles of
    rows [0, tail_m0) over the whole K range, each tail tile in S slices that
    together cover the same K-tiles."""
    for M, N, K, dtype in [(6000, 6000, 6000, tgemm.BF16_BF16), (4352, 4096, 1024, tgemm.BF16_F32),
                           (7000, 7000, 7000, tgemm.F16_F16)]:
        p = auto_plan(M, N, K, dtype)
        assert p["tail_split_k"] > 1
        m = tgemm.gemm_model(p, M, N, K, dtype)
        tm, tn, tk, S = p["tile_m"], p["tile_n"], p["tile_k"], p["tail_split_k"]
        nk = -(-K // tk)

        def slice_steps(splits):
            per = -(-nk // splits)
            return sum(min(per, nk - lo) for lo in range(0, nk, per))

        tiles_n = -(-N // tn)
        main_tiles = (p["tail_m0"] // tm) * tiles_n
        tail_tiles = (-(-M // tm)) * tiles_n - main_tiles
        want = 2 * tm * tn * tk * (main_tiles * slice_steps(1) + tail_tiles * slice_steps(S))
        assert m["executed_flops"] == want
        copies = (4 * M * K if p["repack"] & 1 else 0) + (4 * K * N if p["repack"] & 2 else 0)  # read + write
        assert m["bytes_workspace"] == 8 * S * (M - p["tail_m0"]) * N + copies
        assert m["flops"] == 2 * M * N * K
