"""Every int32 sum of the GEMMs at the layers' full sizes, checked with Freivalds' method.

The sampled-row tests compare a few hundred rows of an output with the oracle.  Here the
whole M x N int32 result C of one launch is checked through two identities of integer
matrices, evaluated exactly on the CPU:
    C r   == A (B^T r)        for a seeded vector r over the N columns,
    s^T C == (s^T A) B^T      for a seeded vector s over the M rows.
A and B are the integer codes the GEMM was given (drawn here, uniform over the code range).
Every entry of r and s is a nonzero integer in [-64, 64], so a single wrong or unwritten
element of C always changes both sides (C is filled with a sentinel first), and several
wrong elements pass only if they cancel in both seeded combinations at once.  The sums are
below 2^50, so float64 arithmetic is exact in any order and numpy's float64 products serve.

Shapes: QKV [21504, 5376] and FFN-down [5376, 14336] at M = 19989, for the INT8 GEMM, the
W4A8 GEMM (s8 x packed s4), the W4A4 nibble GEMM (s4 x s4) and the W4A4 E2M3 GEMM; and a
ragged long-K case (M 4999, N 5000, K_pad 20224) for the INT8 GEMM.
"""
import numpy as np
import pytest
import torch

import oracle
import rotated_bit_linear_amd as rbl
from helpers import dev, say

pytestmark = pytest.mark.gpu

CHUNK = 2048


def _rows_dot(x: np.ndarray, v: np.ndarray) -> np.ndarray:
    """x @ v for an integer matrix x and an integer-valued float64 vector v (exact)."""
    out = np.empty(x.shape[0])
    for i in range(0, x.shape[0], CHUNK):
        out[i:i + CHUNK] = x[i:i + CHUNK].astype(np.float64) @ v
    return out


def _cols_dot(u: np.ndarray, x: np.ndarray) -> np.ndarray:
    """u @ x for an integer-valued float64 vector u and an integer matrix x (exact)."""
    acc = np.zeros(x.shape[1])
    for i in range(0, x.shape[0], CHUNK):
        acc += u[i:i + CHUNK] @ x[i:i + CHUNK].astype(np.float64)
    return acc


def _nonzero(g: np.random.Generator, n: int) -> np.ndarray:
    v = g.integers(1, 65, size=n) * np.where(g.integers(0, 2, size=n) == 1, 1, -1)
    return v.astype(np.float64)


def _check(c_dev: torch.Tensor, a: np.ndarray, b: np.ndarray, seed: int, what: str):
    g = np.random.default_rng(seed)
    M, N = c_dev.shape
    r, s = _nonzero(g, N), _nonzero(g, M)
    c = c_dev.cpu().numpy()
    lhs_r = _rows_dot(c, r)
    rhs_r = _rows_dot(a, _cols_dot(r, b))
    bad = np.flatnonzero(lhs_r != rhs_r)
    assert bad.size == 0, f"{what}: C r differs in {bad.size} of {M} rows (first {bad[:8].tolist()})"
    lhs_s = _cols_dot(s, c)
    rhs_s = _rows_dot(b, _cols_dot(s, a))
    bad = np.flatnonzero(lhs_s != rhs_s)
    assert bad.size == 0, f"{what}: s^T C differs in {bad.size} of {N} columns (first {bad[:8].tolist()})"


SHAPES = [("qkv", 19989, 21504, 5376), ("ffn_down", 19989, 5376, 14336)]


@pytest.mark.parametrize("name,M,N,Kp", SHAPES, ids=[s[0] for s in SHAPES])
def test_every_int32_sum_at_layer_size(name, M, N, Kp):
    g = np.random.default_rng(M + 7 * N + Kp)
    acc = torch.empty(M, N, dtype=torch.int32, device=dev())

    a8 = g.integers(-127, 128, size=(M, Kp), dtype=np.int8)
    b8 = g.integers(-127, 128, size=(N, Kp), dtype=np.int8)
    ad8 = torch.from_numpy(a8).to(dev())
    say(f"{name}: cr_gemm_s8_rowscale int32 out M={M} N={N} K_pad={Kp}")
    acc.fill_(0x5A5A5A5A)
    rbl.cr_gemm_s8_rowscale(ad8, None, torch.from_numpy(b8).to(dev()), None, acc)
    torch.cuda.synchronize()
    _check(acc, a8, b8, 1, f"{name} s8 x s8")
    del b8

    b4 = g.integers(-7, 8, size=(N, Kp), dtype=np.int8)
    bd4 = torch.from_numpy(oracle.pack_s4(b4)).to(dev())
    say(f"{name}: cr_gemm_s8s4_rowscale int32 out M={M} N={N} K_pad={Kp}")
    acc.fill_(0x5A5A5A5A)
    rbl.cr_gemm_s8s4_rowscale(ad8, None, bd4, None, acc)
    torch.cuda.synchronize()
    _check(acc, a8, b4, 2, f"{name} s8 x s4")
    del ad8, a8

    a4 = g.integers(-7, 8, size=(M, Kp), dtype=np.int8)
    say(f"{name}: cr_gemm_s4s4_rowscale int32 out M={M} N={N} K_pad={Kp}")
    acc.fill_(0x5A5A5A5A)
    rbl.cr_gemm_s4s4_rowscale(torch.from_numpy(oracle.pack_s4(a4)).to(dev()), None, bd4, None, acc)
    torch.cuda.synchronize()
    _check(acc, a4, b4, 3, f"{name} s4 x s4")
    del bd4

    say(f"{name}: cr_gemm_e2m3_rowscale int32 out M={M} N={N} K_pad={Kp}")
    acc.fill_(0x5A5A5A5A)
    rbl.cr_gemm_e2m3_rowscale(torch.from_numpy(oracle.pack_e2m3(a4)).to(dev()), None,
                              torch.from_numpy(oracle.pack_e2m3(b4)).to(dev()), None, acc, K_pad=Kp)
    torch.cuda.synchronize()
    _check(acc, a4, b4, 4, f"{name} E2M3 x E2M3")


def test_every_int32_sum_ragged_long_k():
    M, N, Kp = 4999, 5000, 20224
    g = np.random.default_rng(11)
    a8 = g.integers(-127, 128, size=(M, Kp), dtype=np.int8)
    b8 = g.integers(-127, 128, size=(N, Kp), dtype=np.int8)
    acc = torch.empty(M, N, dtype=torch.int32, device=dev())
    acc.fill_(0x5A5A5A5A)
    say(f"ragged: cr_gemm_s8_rowscale int32 out M={M} N={N} K_pad={Kp}")
    rbl.cr_gemm_s8_rowscale(torch.from_numpy(a8).to(dev()), None, torch.from_numpy(b8).to(dev()), None, acc)
    torch.cuda.synchronize()
    _check(acc, a8, b8, 5, "ragged s8 x s8")
