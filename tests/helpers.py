"""Shared helpers of the GPU parity tests (host-side comparisons only)."""
import sys

import numpy as np
import torch

import synth

TOL = {synth.DT_BF16: 1e-3, synth.DT_FP16: 1e-3, synth.DT_FP32: 1e-5}


def say(msg: str):
    """Name the case about to run on the GPU (flushed before the launch)."""
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def out_f64(arr, dtype: int) -> np.ndarray:
    """Oracle or GPU output (uint16 bit patterns for bf16/fp16) as float64."""
    if isinstance(arr, torch.Tensor):
        arr = arr.detach().cpu()
        if dtype in (synth.DT_BF16, synth.DT_FP16):
            return arr.double().numpy()
        return arr.double().numpy()
    if dtype == synth.DT_BF16:
        return torch.from_numpy(arr.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    if dtype == synth.DT_FP16:
        return arr.view(np.float16).astype(np.float64)
    return arr.astype(np.float64)


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    num = np.linalg.norm((got - ref).ravel())
    den = np.linalg.norm(ref.ravel())
    return float(num / den) if den > 0 else float(num)


def assert_bits_equal(got: np.ndarray, ref: np.ndarray, what: str):
    if not np.array_equal(got, ref):
        bad = np.argwhere(got != ref)
        first = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {ref.size} differ; first at {first}: "
                             f"got {got[first]!r} want {ref[first]!r}")


def out_bits(arr, dtype: int) -> np.ndarray:
    """Output (torch tensor, or oracle array with bf16/fp16 as uint16 bit patterns) as raw
    bit patterns: uint16 for bf16/fp16, uint32 for fp32, int32 for the accumulator."""
    if isinstance(arr, torch.Tensor):
        arr = arr.detach().cpu().contiguous()
        if dtype in (synth.DT_BF16, synth.DT_FP16):
            return arr.view(torch.int16).numpy().view(np.uint16)
        if dtype == synth.DT_FP32:
            return arr.view(torch.int32).numpy().view(np.uint32)
        return arr.numpy()
    arr = np.ascontiguousarray(arr)
    return arr.view(np.uint32) if dtype == synth.DT_FP32 else arr


def check_output(got, ref, dtype: int, what: str) -> float:
    """The output bar (relative L2 within TOL[dtype] against the oracle's output rounded to
    the same dtype), then the stronger property the kernels are built to: the epilogue does
    the oracle's operations in the oracle's order, so every output bit is identical."""
    err = rel_l2(out_f64(got, dtype), out_f64(ref, dtype))
    assert err <= TOL[dtype], (what, err)
    assert_bits_equal(out_bits(got, dtype), out_bits(ref, dtype), f"{what} (bits)")
    return err
