"""Host allocation failures at the C interface (CPU only).

tests/c_abi/alloc_fail_client.cpp replaces the process's operator new with one that
throws std::bad_alloc on an armed countdown, and stands in for the device queries of
gemm_create (one gfx950 device), so that gemm_create and gemm_tune reach their host
allocations without a GPU. Every such failure must come back as
GEMM_ERR_OUT_OF_MEMORY (no exception crosses the C interface) and leave no block
allocated.
"""
import os
import subprocess

import pytest

from tiled_gemm_output_amd import tgemm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")


def test_allocation_failures_return_out_of_memory(tmp_path):
    if not os.path.exists(tgemm.LIBRARY) or not os.path.exists(CLANGXX):
        pytest.skip("libtgemm.so or the ROCm compiler is missing (run the build first)")
    libdir = os.path.dirname(tgemm.LIBRARY)
    exe = str(tmp_path / "alloc_fail_client")
    cmd = [CLANGXX, "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"),
           "-I" + os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi", "alloc_fail_client.cpp"),
           "-o", exe, "-rdynamic", "-L" + libdir, "-ltgemm", "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + libdir, "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "alloc_fail_client: ok" in r.stdout, r.stdout + r.stderr
