"""Time the library's automatic plan beside torch.matmul (the vendor BLAS) on the same
device tensors: bf16 inputs N(0, 1), bf16 output, dense row-major operands. Context only:
the vendor library is not a target and no part of the product path calls it.

Each product is captured in a HIP graph of several launches (so that the host's launch
loop does not set the rate), replayed three times; the median replay gives the time per
launch. The library is timed before and after the vendor library and the better of the
two is kept (the card's clock drifts under sustained load). The library's result is also
checked against a float32 product of the same inputs (normwise error, which for a bf16
output is about one rounding of the output).

    python -m tiled_gemm_output_amd.vendor_compare                 # the default shape list
    python -m tiled_gemm_output_amd.vendor_compare --shape 4096,4096,4096 --shape 128,8192,8192
    python -m tiled_gemm_output_amd.vendor_compare --op nt        # B stored N x K (weights), C = A @ B^T
"""
from __future__ import annotations

import argparse

DEFAULT_SHAPES = [(8192, 8192, 8192), (4096, 4096, 4096), (2048, 2048, 2048), (1024, 1024, 1024), (3072, 3072, 3072),
                  (6144, 6144, 6144), (5120, 5120, 5120), (1536, 8192, 8192), (8192, 1536, 8192), (4096, 14336, 4096),
                  (4096, 4096, 14336), (14336, 4096, 4096), (512, 4096, 4096), (256, 8192, 8192), (128, 16384, 4096),
                  (16384, 128, 4096), (2000, 3000, 4000), (7000, 5000, 3000), (3333, 2222, 1111), (1000, 1000, 16000),
                  (384, 384, 32768), (12288, 12288, 1024)]


def graph_time_us(torch, fn, iters: int) -> float:
    """Median of three replays of a graph holding `iters` calls of fn, per call."""
    g = torch.cuda.CUDAGraph()
    fn()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for _ in range(iters):
            fn()
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1000.0 / iters)
    return sorted(times)[1]


def compare(shapes, op: str = "nn", seed: int = 0):
    """op: the stored forms of A and B ("t": A stored K x M, or B stored N x K)."""
    import torch

    from . import tgemm

    torch.manual_seed(seed)
    h = tgemm.gemm_create()
    ta, tb = op[0] == "t", op[1] == "t"
    rows = []
    try:
        for M, N, K in shapes:
            sa = torch.randn(*((K, M) if ta else (M, K)), device="cuda").to(torch.bfloat16)  # as stored
            sb = torch.randn(*((N, K) if tb else (K, N)), device="cuda").to(torch.bfloat16)
            a, b = (sa.t() if ta else sa), (sb.t() if tb else sb)  # the logical M x K and K x N views
            c = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
            flops = 2.0 * M * N * K
            iters = max(3, min(50, int(2e11 / flops)))

            def ours():
                tgemm.check(tgemm.gemm_run_op(h, tgemm.OP_T if ta else tgemm.OP_N, tgemm.OP_T if tb else tgemm.OP_N,
                                              M, N, K, sa.data_ptr(), sa.stride(0), sb.data_ptr(), sb.stride(0),
                                              c.data_ptr(), N, tgemm.BF16_BF16, tgemm.current_stream()), "gemm_run_op")

            vendor = lambda: torch.matmul(a, b)  # noqa: E731
            for _ in range(3):
                ours()
                vendor()
            t1 = graph_time_us(torch, ours, iters)
            tv = graph_time_us(torch, vendor, iters)
            t2 = graph_time_us(torch, ours, iters)
            ours()
            ref = torch.matmul(a.float(), b.float())
            torch.cuda.synchronize()
            err = ((c.float() - ref).abs().max() / ref.abs().max()).item()
            p = tgemm.gemm_plan_op(h, tgemm.OP_T if ta else tgemm.OP_N, tgemm.OP_T if tb else tgemm.OP_N, M, N, K,
                                   sa.data_ptr(), sa.stride(0), sb.data_ptr(), sb.stride(0), c.data_ptr(), N,
                                   tgemm.BF16_BF16)
            t = min(t1, t2)
            rows.append({"shape": (M, N, K), "op": op, "ours_us": t, "vendor_us": tv, "ours_tflops": flops / t / 1e6,
                         "vendor_tflops": flops / tv / 1e6, "vendor_over_ours": tv / t, "err": err,
                         "plan": "%dx%d, %d K-slices, %d stages%s" % (p["tile_m"], p["tile_n"], p["split_k"], p["stages"],
                                                                     ", tail in %d" % p["tail_split_k"] if p["tail_split_k"] else "")})
            r = rows[-1]
            print("%5dx%5dx%5d  ours %8.1f us (%5.0f TF)  vendor %8.1f us (%5.0f TF)  vendor/ours %.3f  %s  err %.1e" % (
                M, N, K, r["ours_us"], r["ours_tflops"], r["vendor_us"], r["vendor_tflops"], r["vendor_over_ours"], r["plan"],
                r["err"]), flush=True)
    finally:
        tgemm.gemm_destroy(h)
    return rows


def parse_args(argv=None):
    """(shapes, op) of a command line (the default shape list when it names none)."""
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--shape", action="append", default=[], help="M,N,K (repeatable; default: a built-in list)")
    ap.add_argument("--op", choices=["nn", "nt", "tn", "tt"], default="nn",
                    help="stored forms: t = that operand is stored transposed (A as K x M, B as N x K)")
    args = ap.parse_args(argv)
    shapes = []
    for s in args.shape:
        try:
            dims = tuple(int(x) for x in s.split(","))
        except ValueError:
            dims = ()
        if len(dims) != 3 or min(dims) < 1:
            ap.error("--shape takes three positive integers M,N,K, got %r" % s)
        shapes.append(dims)
    return shapes or list(DEFAULT_SHAPES), args.op


def main(argv=None) -> None:
    shapes, op = parse_args(argv)
    compare(shapes, op)


if __name__ == "__main__":
    main()
