"""GPU parity of matmul(a, b) (the Helion-style tensor entry point) against the
oracle: result dtype, transposed views passed without copies, out=, streams and
the empty cases."""
import numpy as np
import pytest

import oracle
from tests import gpu_util as G
from tiled_gemm_output_amd import inputs, tgemm

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "i32": torch.int32}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def o():
    return oracle.get()


def dev(bits, kind):
    """Device tensor of the given element kind holding these bits."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16 if kind != "i32" else np.int32))
    return t.view(TORCH[kind]).cuda()


def host_bits(t):
    return t.cpu().view(torch.int16 if t.element_size() == 2 else torch.int32).numpy()


def matmul(*args, **kw):
    from tiled_gemm_output_amd.matmul import matmul as mm

    return mm(*args, **kw)


@pytest.mark.parametrize("kind,out_kind", [("bf16", "bf16"), ("f16", "f16"), ("bf16", "f32"), ("f16", "f32"),
                                           ("i32", "i32")])
@pytest.mark.parametrize("shape", [(1000, 777, 333), (256, 512, 1024), (1, 1, 1), (64, 8, 4096)], ids=str)
def test_matmul_dtypes(o, kind, out_kind, shape):
    M, N, K = shape
    a, b = inputs.random_case(M, N, K, kind, seed=M + N + K)
    out_dtype = None if out_kind == kind else torch.float32
    c = matmul(dev(a, kind), dev(b, kind), out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert c.shape == (M, N) and c.dtype == (TORCH[kind] if out_dtype is None else torch.float32)
    ref = o.gemm(a, b, kind, out_kind)
    if kind == "i32":
        assert np.array_equal(host_bits(c), ref.view(np.int32))
    else:
        G.compare(host_bits(c), ref.view(np.int16 if out_kind != "f32" else np.int32), out_kind)


@pytest.mark.parametrize("ta,tb", [(False, True), (True, False), (True, True)])
def test_matmul_transposed_views(o, ta, tb):
    """x.t() views go through as transposed operands (no copy): the result is the
    oracle's product of the logical matrices."""
    M, N, K = 300, 264, 520
    a, b = inputs.random_case(M, N, K, "bf16", seed=3)
    da = dev(np.ascontiguousarray(a.T), "bf16").t() if ta else dev(a, "bf16")
    db = dev(np.ascontiguousarray(b.T), "bf16").t() if tb else dev(b, "bf16")
    assert da.shape == (M, K) and db.shape == (K, N)
    c = matmul(da, db)
    torch.cuda.synchronize()
    G.compare(host_bits(c), o.gemm(a, b, "bf16", "bf16").view(np.int16), "bf16")


def test_matmul_out_and_stream(o):
    M, N, K = 200, 136, 1000
    a, b = inputs.random_case(M, N, K, "f16", seed=4)
    big = torch.full((M, N + 24), float("nan"), dtype=torch.float32, device="cuda")
    out = big[:, 8:8 + N]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c = matmul(dev(a, "f16"), dev(b, "f16"), out=out)
    s.synchronize()
    assert c.data_ptr() == out.data_ptr()
    G.compare(host_bits(out.contiguous()), o.gemm(a, b, "f16", "f32").view(np.int32), "f32")
    assert torch.isnan(big[:, :8]).all() and torch.isnan(big[:, 8 + N:]).all()


def test_matmul_empty_and_zero_k():
    z = matmul(torch.empty(0, 16, dtype=torch.bfloat16, device="cuda"),
               torch.empty(16, 8, dtype=torch.bfloat16, device="cuda"))
    assert z.shape == (0, 8)
    c = matmul(torch.empty(5, 0, dtype=torch.bfloat16, device="cuda"),
               torch.empty(0, 7, dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert c.shape == (5, 7) and not c.float().abs().sum().item()


def test_matmul_rejects_strided_views():
    a = torch.zeros(64, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        matmul(a[:, ::2], a[:32])


def test_matmul_split_k_on_two_streams(o):
    """Two split-K products (each tile's K range in slices whose fp32 partial tiles go
    to a workspace) enqueued on two streams with no synchronization between them:
    each stream's calls go through a handle of their own, so neither overwrites the
    other's partial tiles. Both results match the oracle."""
    M, N, K = 128, 8192, 8192
    p = tgemm.gemm_plan(None, M, N, K, 1 << 20, K, 1 << 30, N, 1 << 34, N, tgemm.BF16_F32)
    assert p["split_k"] > 1, p
    cases = [inputs.random_case(M, N, K, "bf16", seed=s) for s in (11, 12)]
    d = [(dev(a, "bf16"), dev(b, "bf16")) for a, b in cases]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            c1 = matmul(*d[0], out_dtype=torch.float32)
        with torch.cuda.stream(s2):
            c2 = matmul(*d[1], out_dtype=torch.float32)
        outs.append((c1, c2))
    torch.cuda.synchronize()
    refs = [o.gemm(a, b, "bf16", "f32").view(np.int32) for a, b in cases]
    for c1, c2 in outs:
        G.compare(host_bits(c1), refs[0], "f32")
        G.compare(host_bits(c2), refs[1], "f32")
