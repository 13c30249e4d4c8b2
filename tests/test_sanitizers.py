"""Sanitizer builds run on the CPU.

1. The oracle (oracle/oracle.c) compiled with gcc under AddressSanitizer and
   UndefinedBehaviorSanitizer (plus float-cast-overflow and float-divide-by-zero) and driven
   through every entry point on exactly-sized buffers (tests/native/oracle_sanitize.c).
2. The host side of the C ABI (rotated_bit_linear_amd/csrc/api.cpp: validation, planner,
   workspace sizes, the event pool) compiled by hipcc with the same sanitizers on its host side,
   linked against the library's kernel objects, and driven with rejected arguments and
   empty extents (tests/native/abi_sanitize.cpp); no kernel is launched.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN = "address,undefined"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
          f"-fsanitize={SAN},float-cast-overflow,float-divide-by-zero", "-fno-sanitize-recover=all",
          "-Wall", "-Wno-unknown-pragmas", os.path.join(ROOT, "oracle", "oracle.c"),
          os.path.join(NATIVE, "oracle_sanitize.c"), "-o", exe, "-lm"])
    r = _run([exe], env=ENV, timeout=300)
    assert "ok" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm compilers not found")
def test_c_abi_host_side_under_asan_ubsan(tmp_path):
    from rotated_bit_linear_amd import build as hip_build
    kernel_objs = hip_build.kernel_objects()
    inc = os.path.join(ROOT, "include")
    # every -fsanitize= applies to the host side only (-Xarch_host); api.cpp keeps its device
    # part (the allocation-free entry point's scratch array), the test program has none
    san = ["-O1", "-g", "-std=c++17", "-fPIC", "-Xarch_host", f"-fsanitize={SAN}", "-Xarch_host",
           "-fno-sanitize-recover=all", "-I", inc]
    api_o, drv_o, exe = (str(tmp_path / n) for n in ("api.o", "drv.o", "abi_sanitize"))
    _run([HIPCC, "-x", "hip", "--offload-arch=gfx950", *san, "-c",
          os.path.join(ROOT, "rotated_bit_linear_amd", "csrc", "api.cpp"), "-o", api_o])
    _run([HIPCC, "-x", "hip", "--offload-host-only", *san, "-c", os.path.join(NATIVE, "abi_sanitize.cpp"), "-o", drv_o])
    _run([CLANGXX, f"-fsanitize={SAN}", drv_o, api_o, *kernel_objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert "ok" in r.stdout
