"""Sanitizer builds of the host code (CPU only): the oracle and the C ABI's host side.

* The oracle (oracle/conv_oracle.c) is compiled with AddressSanitizer and
  UndefinedBehaviorSanitizer into tests/sanitize/oracle_check.c, which runs it on
  random small problems with every buffer allocated at exactly its size.
* The library's host side (descriptor validation, extents, path choice,
  backward-data planning, the measured-selection table: csrc/convfwd_api.cpp) is
  compiled with AddressSanitizer + UndefinedBehaviorSanitizer, and separately with
  ThreadSanitizer, and linked with the library's kernel objects into
  tests/sanitize/abi_fuzz.cpp, which drives random (valid and invalid) descriptors
  through every host-side entry point from several threads.  Every call it makes
  returns before a launch, so no GPU is needed.

Any sanitizer report fails the run (non-zero exit).
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"
KOBJ = os.path.join(ROOT, "implicit_gemm_conv_amd", "_build")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout[-4000:]}\n{res.stderr[-4000:]}"
    return res.stdout


def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_check")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", os.path.join(SAN, "oracle_check.c"), "-o", exe, "-lm"])
    out = _run([exe, "3000"], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0"})
    assert "0 failures" in out, out


def _kernel_objects():
    objs = sorted(glob.glob(os.path.join(KOBJ, "k_*.hip.o")))
    if not objs:
        from implicit_gemm_conv_amd import build as hip_build
        hip_build.build()
        objs = sorted(glob.glob(os.path.join(KOBJ, "k_*.hip.o")))
    return objs


@pytest.mark.parametrize("san", ["address,undefined", "thread"])
def test_abi_host_side_under_sanitizers(tmp_path, san):
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang++ not available")
    objs = _kernel_objects()
    flags = ["-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", f"-fsanitize={san}"]
    if san != "thread":
        flags.append("-fno-sanitize-recover=all")
    api = str(tmp_path / "api.o")
    main = str(tmp_path / "main.o")
    exe = str(tmp_path / "abi_fuzz")
    _run([CLANG, *flags, "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-c",
          os.path.join(ROOT, "implicit_gemm_conv_amd", "csrc", "convfwd_api.cpp"), "-o", api])
    _run([CLANG, *flags, "-c", os.path.join(SAN, "abi_fuzz.cpp"), "-o", main])
    _run([CLANG, f"-fsanitize={san}", main, api, *objs, "-o", exe, "-L/opt/rocm/lib", "-lamdhip64",
          "-lpthread", "-Wl,-rpath,/opt/rocm/lib"])
    env = {**os.environ, "TSAN_OPTIONS": "halt_on_error=1", "ASAN_OPTIONS": "detect_leaks=0"}
    out = _run([exe, "8", "20000"], env=env, timeout=300)
    assert "0 inconsistent answers" in out, out
