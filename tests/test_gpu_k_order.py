"""The GEMMs' K direction: the 32 workgroups an XCD runs at once form a generation, and every
other generation walks K from the end (its int32 sums must equal the forward ones). On grids
of at least 2 x 8 x 32 tiles, every XCD runs generations in both directions. The int32 sums
of the S8, W4A8, W4A4 nibble and E2M3 GEMMs are compared with the oracle's in full on rows
that cover every row of tiles. The K_pad values give step counts that leave every remainder
of the 2- and 3-stage rings.
"""
import numpy as np
import pytest
import torch

import oracle
import rotated_bit_linear_amd as rbl
from helpers import assert_bits_equal, dev, say

pytestmark = pytest.mark.gpu

# (M, N, K_pad): 16 x 32 = 512 and 8 x 66 = 528 and 20 x 30 = 600 tiles
CASES = [(4096, 8192, 1280), (2048, 16896, 768), (5100, 7680, 1024)]


def _rows(M: int) -> np.ndarray:
    """Every 16th row, the rows around each 256-row tile edge, and the M tail."""
    r = set(range(0, M, 16)) | set(range(max(0, M - 32), M))
    r |= {t * 256 + d for t in range((M + 255) // 256) for d in (255,) if t * 256 + d < M}
    return np.array(sorted(r))


@pytest.mark.parametrize("M,N,Kp", CASES, ids=[f"M{c[0]}-N{c[1]}-K{c[2]}" for c in CASES])
def test_both_k_directions_give_exact_sums(M, N, Kp):
    g = np.random.default_rng(M + N + Kp)
    a8 = g.integers(-127, 128, size=(M, Kp), dtype=np.int8)
    b8 = g.integers(-127, 128, size=(N, Kp), dtype=np.int8)
    a4 = g.integers(-7, 8, size=(M, Kp), dtype=np.int8)
    b4 = g.integers(-7, 8, size=(N, Kp), dtype=np.int8)
    r = _rows(M)
    rd = torch.from_numpy(r).to(dev())
    ad8, bd8 = torch.from_numpy(a8).to(dev()), torch.from_numpy(b8).to(dev())
    pa4, pb4 = oracle.pack_s4(a4), oracle.pack_s4(b4)
    ad4, bd4 = torch.from_numpy(pa4).to(dev()), torch.from_numpy(pb4).to(dev())
    ad6 = torch.from_numpy(oracle.pack_e2m3(a4)).to(dev())
    bd6 = torch.from_numpy(oracle.pack_e2m3(b4)).to(dev())
    acc = torch.empty(M, N, dtype=torch.int32, device=dev())

    want8 = oracle.gemm_s8(np.ascontiguousarray(a8[r]), b8)
    want84 = oracle.gemm_s8s4(np.ascontiguousarray(a8[r]), pb4)
    want44 = oracle.gemm_s4s4(np.ascontiguousarray(pa4[r]), pb4, Kp)
    for what, run, want in (
            ("cr_gemm_s8_rowscale", lambda: rbl.cr_gemm_s8_rowscale(ad8, None, bd8, None, acc), want8),
            ("cr_gemm_s8s4_rowscale", lambda: rbl.cr_gemm_s8s4_rowscale(ad8, None, bd4, None, acc), want84),
            ("cr_gemm_s4s4_rowscale", lambda: rbl.cr_gemm_s4s4_rowscale(ad4, None, bd4, None, acc), want44),
            ("cr_gemm_e2m3_rowscale", lambda: rbl.cr_gemm_e2m3_rowscale(ad6, None, bd6, None, acc, K_pad=Kp), want44)):
        say(f"{what} M={M} N={N} K_pad={Kp} int32 out ({(M + 255) // 256 * ((N + 255) // 256)} tiles)")
        acc.fill_(0x5A5A5A5A)
        run()
        torch.cuda.synchronize()
        assert_bits_equal(acc[rd].cpu().numpy(), want, f"{what} int32 sums on {len(r)} rows")
