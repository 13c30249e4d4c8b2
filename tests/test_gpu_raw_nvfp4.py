"""GPU parity on NVFP4 bytes drawn directly (no encoder), through the C ABI.

The synthetic encoder only emits the scale bytes and codes that a bell-shaped weight needs
(a narrow band of positive E4M3 exponents, never the -0 code).  Here every code byte is
uniformly random (all 16 nibbles, code 8 = -0 included), every finite E4M3 byte (negative,
subnormal and every exponent) is a block scale, the global scale is not a power of two, K
is ragged (an odd K leaves a padding nibble) and the row padding of both byte arrays holds
garbage, NaN scale bytes included.  The first 254 weight rows each use one scale byte for
the whole row (so every byte's decode decides that row's codes); the others mix all bytes.

Checked bit for bit against the oracle: S8 codes and scales of the weight preparation
(natural and block-transposed order, one-pass, two-pass and forced two-pass), the row
maxima, the int32 sums of the decode-inside-GEMM kernel (row maxima given and found in the
kernel), and cr_linear_nvfp4's outputs on both of its paths (short batch: decode inside the
GEMM; longer: staged S8 tiles, serial and on two streams, chunked by a small tile bound).
"""
import numpy as np
import pytest
import torch

import oracle
import rotated_bit_linear_amd as rbl
import synth
from helpers import assert_bits_equal, check_output, dev, say

pytestmark = pytest.mark.gpu


def _block_transposed(codes: np.ndarray) -> np.ndarray:
    r, kp = codes.shape
    return codes.reshape(r, kp // 256, 16, 16).transpose(0, 1, 3, 2).reshape(r, kp).copy()


CASES = [(300, 999, 0.0137), (264, 20000, 1.0 / 3.0), (270, 4111, 7.1e-37)]


def _x(M, K, seed, scale):
    """bf16 X [M, ld] with a 16-byte row stride ld and garbage in the columns past K."""
    ld = (K + 7) // 8 * 8 + 8
    full = torch.randn(M, ld, generator=torch.Generator().manual_seed(seed)) * scale
    full[:, K:] = 3e4
    return full.to(torch.bfloat16)


def _weight(N, K, g):
    nb = (K + 15) // 16
    return synth.raw_nvfp4(N, K, seed=N + K, ld_codes=(K + 1) // 2 // 16 * 16 + 48, ld_sf=nb + 7, g=g)


@pytest.mark.parametrize("N,K,g", CASES, ids=[f"N{c[0]}-K{c[1]}" for c in CASES])
def test_raw_bytes_weight_prep_and_amax(N, K, g):
    p = _weight(N, K, g)
    assert ((p.codes.numpy() & 15) == 8).any() and ((p.codes.numpy() >> 4) == 8).any()
    nb = (K + 15) // 16
    assert len(np.unique(p.sf.numpy()[:, :nb])) == 254
    cd, sfd = p.codes.to(dev()), p.sf.to(dev())
    gs = torch.tensor([p.g], dtype=torch.float32, device=dev())
    rq, rs = oracle.prep_weight_nvfp4(p.codes.numpy(), p.sf.numpy(), p.g, K)
    ra = oracle.weight_amax_nvfp4(p.codes.numpy(), p.sf.numpy(), p.g, K)
    for flags in (0, rbl.CR_FLAG_BLOCK_TRANSPOSED, rbl.CR_FLAG_FORCE_TWO_PASS,
                  rbl.CR_FLAG_FORCE_TWO_PASS | rbl.CR_FLAG_BLOCK_TRANSPOSED):
        say(f"raw NVFP4 bytes: cr_prep_weight_nvfp4 N={N} K={K} g={p.g!r} flags={flags}")
        q, s = rbl.prep_weight_nvfp4(cd, sfd, gs, K, flags=flags)
        torch.cuda.synchronize()
        want = _block_transposed(rq) if flags & rbl.CR_FLAG_BLOCK_TRANSPOSED else rq
        assert_bits_equal(q.cpu().numpy(), want, f"w_s8 flags={flags}")
        assert_bits_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32), f"w_scale flags={flags}")
    for flags in (0, rbl.CR_FLAG_FORCE_TWO_PASS):
        say(f"raw NVFP4 bytes: cr_weight_amax_nvfp4 N={N} K={K} flags={flags}")
        a = rbl.weight_amax_nvfp4(cd, sfd, gs, K, flags=flags)
        torch.cuda.synchronize()
        assert_bits_equal(a.cpu().numpy().view(np.uint32), ra.view(np.uint32), f"w_amax flags={flags}")


@pytest.mark.parametrize("N,K,g", CASES[:2], ids=[f"N{c[0]}-K{c[1]}" for c in CASES[:2]])
def test_raw_bytes_fused_gemm_int32(N, K, g):
    p = _weight(N, K, g)
    cd, sfd = p.codes.to(dev()), p.sf.to(dev())
    gs = torch.tensor([p.g], dtype=torch.float32, device=dev())
    M = 37
    xf = _x(M, K, K, 3.0)
    rq, rs = oracle.quant_act(synth.bits_u16(xf), synth.DT_BF16, K)
    rqw, _ = oracle.prep_weight_nvfp4(p.codes.numpy(), p.sf.numpy(), p.g, K)
    racc = oracle.gemm_s8(rq, rqw)
    bt = rbl.CR_FLAG_BLOCK_TRANSPOSED
    qx, sx = rbl.quant_act(xf.to(dev())[:, :K], K, flags=bt)
    amax = rbl.weight_amax_nvfp4(cd, sfd, gs, K)
    for am in (amax, None):
        say(f"raw NVFP4 bytes: cr_gemm_nvfp4_fused int32 M={M} N={N} K={K} "
            f"amax={'given' if am is not None else 'in-kernel'}")
        acc = torch.empty(M, N, dtype=torch.int32, device=dev())
        rbl.cr_gemm_nvfp4_fused(qx, sx, cd, sfd, gs, am, K, acc, flags=bt)
        torch.cuda.synchronize()
        assert_bits_equal(acc.cpu().numpy(), racc, "int32 accumulator")


@pytest.mark.parametrize("M", [48, 100])
def test_raw_bytes_layer_both_paths(M):
    """M = 48: activation prep + decode-inside-GEMM; M = 100: staged S8 tiles (the default
    bound, and a 256 KiB bound that splits the weight in two chunks, serial and two-stream)."""
    N, K, g = CASES[0]
    p = _weight(N, K, g)
    cd, sfd = p.codes.to(dev()), p.sf.to(dev())
    gs = torch.tensor([p.g], dtype=torch.float32, device=dev())
    xf = _x(M, K, M, 2.0)
    xf[3, :K] = 0.0
    xd = xf.to(dev())[:, :K]
    aux = torch.cuda.Stream()
    assert (rbl.cr_linear_nvfp4_plan(M, N, K)[1] == 0) == (M <= 64)   # no chunks: decode inside the GEMM
    for odt in (synth.DT_FP32, synth.DT_BF16):
        ref = oracle.linear_nvfp4(synth.bits_u16(xf), synth.DT_BF16, K, False, p.codes.numpy(), p.sf.numpy(),
                                  p.g, odt)
        runs = [(0, None), (256 * 1024, None), (256 * 1024, aux)] if M > 64 else [(0, None), (0, aux)]
        for mt, st in runs:
            say(f"raw NVFP4 bytes: cr_linear_nvfp4 M={M} N={N} K={K} out={odt} max_tile={mt} aux={st is not None}")
            out = rbl.linear_nvfp4(xd, cd, sfd, gs, K, out_dtype=synth.TORCH_DTYPE[odt], max_tile_bytes=mt,
                                   aux_stream=st)
            torch.cuda.synchronize()
            check_output(out, ref, odt, f"layer output out={odt} max_tile={mt}")
