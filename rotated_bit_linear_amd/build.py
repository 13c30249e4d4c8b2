"""Builds the gfx950 HIP library rotated_bit_linear_amd/libconvrot.so with hipcc.

Every translation unit is compiled for gfx950 only, with FP contraction off (the
preparation kernels must evaluate each IEEE operation as written) and packed-FP32
instructions disabled.
"""
import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libconvrot.so")
SOURCES = ["api.cpp", "quant_act.hip", "prep_weight.hip", "gemm_s8.hip", "gemm_fused.hip", "gemm_s8s4.hip", "gemm_e2m3.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def kernel_objects() -> list[str]:
    """Object files of the kernel sources (every source but api.cpp), compiled if missing;
    the sanitizer test links them under a host-only, instrumented build of api.cpp."""
    os.makedirs(BUILD, exist_ok=True)
    out = []
    for src in SOURCES:
        if src == "api.cpp":
            continue
        obj = os.path.join(BUILD, src + ".o")
        out.append(obj if os.path.exists(obj) else _compile(src))
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
