"""Builds the native C-ABI test program tests/native/abi_smoke against the in-tree
libconvrot.so (hipcc, gfx950 host/device toolchain; the program itself has no kernels)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_smoke.cpp")
EXE = os.path.join(HERE, "abi_smoke")
LIBDIR = os.path.join(ROOT, "rotated_bit_linear_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    tmp = EXE + ".tmp"
    cmd = [HIPCC, "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"), SRC, "-o", tmp,
           "-L", LIBDIR, "-lconvrot", "-Wl,-rpath,$ORIGIN/../../rotated_bit_linear_amd"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"native test build failed:\n{r.stderr}")
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
