"""The C ABI from a native program (tests/native/abi_smoke.cpp, built by the build step):
no Python binding, no torch; device memory from hipMalloc.  The program runs in a child
process and checks that the component calls and cr_linear_nvfp4 (staged, two-stream and
short-batch paths) give the same bits, that the W4A8 / W4A4 layer calls equal their
components (the E2M3 form equal to the nibble form, a repacked E2M3 weight equal to a
directly prepared one), and that argument errors come back as statuses."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "abi_smoke")


def test_native_abi_program():
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: run the build step first")
    print("\n[case] native C-ABI program tests/native/abi_smoke", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=180)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, (r.returncode, r.stderr[-2000:])
    assert "abi_smoke: all cases ok" in r.stdout
