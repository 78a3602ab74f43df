"""The C ABI from C: tests/c_abi/abi_client.c is compiled with gcc against
include/tgemm.h and linked with libtgemm.so (no C++, no Python in the caller).
Host mode (argument checks, plans, counts) runs anywhere; GPU mode multiplies on
the device and compares exactly with a host product."""
import os
import shutil
import subprocess

import pytest

from tiled_gemm_output_amd import tgemm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "abi_client.c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_client(tmp_path) -> str:
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    if not os.path.exists(tgemm.LIBRARY):
        pytest.skip("libtgemm.so is not built")
    exe = str(tmp_path / "abi_client")
    libdir = os.path.dirname(tgemm.LIBRARY)
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"),
           "-I" + os.path.join(ROOT, "include"), SRC, "-o", exe, "-L" + libdir, "-ltgemm",
           "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + libdir,
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


def test_c_client_host(tmp_path):
    exe = build_client(tmp_path)
    r = subprocess.run([exe, "host"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_client host: ok" in r.stdout


@pytest.mark.gpu
def test_c_client_gpu(tmp_path):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    exe = build_client(tmp_path)
    r = subprocess.run([exe, "gpu"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_client gpu: ok" in r.stdout
