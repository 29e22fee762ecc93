"""The CPU oracle and the C-ABI validation code under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only; no GPU needed).

Two drivers in tests/sanitize: oracle_driver.c runs every oracle function on small seeded inputs
(a ragged batch with a one-token sequence, full and tiny budgets, SnapKV with c past n);
abi_driver.c calls the library's entry points with invalid or unsupported arguments, which the
library rejects before any HIP call, and its host-side queries at the edges of their ranges.
The library's host code is built with the sanitizers (device code as usual); both drivers exit 0
only when every call returns and every code is the documented one, and the sanitizers abort on
the first finding."""
import os
import shutil
import subprocess

import pytest

from query_aware_sparse_index_amd.build_lib import SOURCES   # every source file of the library

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "query_aware_sparse_index_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "qasi_oracle.c"),
          "-lm", "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert "oracle sanitizer run: ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not available")
def test_abi_validation_under_sanitizers(tmp_path):
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
             "-I", os.path.join(ROOT, "include")]
    procs = [subprocess.Popen([HIPCC, *flags, "-c", os.path.join(CSRC, s), "-o", str(tmp_path / (s + ".o"))],
                              stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True) for s in SOURCES]
    for p, s in zip(procs, SOURCES):
        out, errs = p.communicate(timeout=600)
        assert p.returncode == 0, f"{s}: {errs}"
    lib = str(tmp_path / "libqasi_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[str(tmp_path / (s + ".o")) for s in SOURCES], "-o", lib])
    exe = str(tmp_path / "abi_driver")
    _run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", os.path.join(SAN, "abi_driver.c"),
          lib, "-Wl,-rpath," + str(tmp_path), "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert "C-ABI sanitizer run: ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
