"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- The oracle (oracle/oracle.c) with gcc's sanitizers, driven by tests/c_abi/oracle_client.c:
  every entry point on empty, ragged and padded cases, every kind, several thread counts.
- The library's host side (csrc/api.hip: argument checks, planning, counts, status strings)
  recompiled with the sanitizers on its host code only (its device part, the scratch array
  of the allocation-free entry point, is built as usual) and linked with the already built
  kernel objects;
  the C client tests/c_abi/abi_client.c, built with the same compiler's sanitizers, runs its
  host checks and a sweep of 13,005 plans over shapes, paddings, odd addresses, operand forms
  and dtypes. No device code is instrumented and no GPU is used.
Any report ends the program with a non-zero status (-fno-sanitize-recover).
"""
import os
import shutil
import subprocess

import pytest

from tiled_gemm_output_amd import tgemm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tiled_gemm_output_amd", "csrc")
BUILD = os.path.join(ROOT, "tiled_gemm_output_amd", "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
# host-only instrumentation flags for the HIP compiler driver
HOST_SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=all".split()
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr)
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_client")
    run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-ffp-contract=off", "-pthread", os.path.join(ROOT, "oracle", "oracle.c"),
         os.path.join(ROOT, "tests", "c_abi", "oracle_client.c"), "-lm", "-o", exe])
    out = run([exe], env=ENV, timeout=120)
    assert "oracle_client: ok" in out


def test_host_library_under_sanitizers(tmp_path):
    objs = [os.path.join(BUILD, f) for f in sorted(os.listdir(BUILD))] if os.path.isdir(BUILD) else []
    objs = [o for o in objs if o.endswith(".o") and os.path.basename(o) != "api.o"]
    if not objs or not os.path.exists(HIPCC) or not os.path.exists(CLANG):
        pytest.skip("kernel objects or the ROCm compilers are missing (run the build first)")
    api = str(tmp_path / "api_san.o")
    run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
         "-fno-omit-frame-pointer", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, *HOST_SAN, "-c",
         os.path.join(CSRC, "api.hip"), "-o", api])
    lib = str(tmp_path / "libtgemm_san.so")
    run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, api, *objs])
    exe = str(tmp_path / "abi_client_san")
    client_flags = ["-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    run([CLANG, *client_flags, "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"),
         "-I" + os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi", "abi_client.c"), "-o", exe,
         "-L" + str(tmp_path), "-ltgemm_san", "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
         "-Wl,-rpath," + str(tmp_path), "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    assert "abi_client host: ok" in run([exe, "host"], env=ENV, timeout=120)
    assert "abi_client sweep: ok" in run([exe, "sweep"], env=ENV, timeout=300)


def test_plan_sweep_uninstrumented(tmp_path):
    """The same sweep against the built library itself."""
    from tests.test_c_abi import build_client

    exe = build_client(tmp_path)
    assert os.path.exists(tgemm.LIBRARY)
    assert "abi_client sweep: ok" in run([exe, "sweep"], timeout=300)
