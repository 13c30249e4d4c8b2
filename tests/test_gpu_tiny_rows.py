"""GPU parity on rows so small that the quantizer's reciprocal 127/a is not a finite FP32
value (max |y| below ~3.7e-37), and on rows just above that range.

The row quantizer (ComfyUI Turing Utils README, "Load ConvRot DiT ..." bullet: rows
quantized to S8 with an FP32 scale) takes such a row as its exact copy scaled by 2^64; the
oracle's reading is pinned by the power-of-two invariance and the fp64 error bound on
the CPU.  Here the GPU's codes, scales, row maxima and int32 sums must equal the oracle's
bit for bit, for activations (bf16, fp32; one-pass, several-rows-per-workgroup, two-pass,
SwiGLU) and for NVFP4 weights with a tiny global scale (staged and decode-inside-GEMM).
"""
import numpy as np
import pytest
import torch

import oracle
import rotated_bit_linear_amd as rbl
import synth
from helpers import assert_bits_equal, dev, say

pytestmark = pytest.mark.gpu

DT_T = {synth.DT_BF16: torch.bfloat16, synth.DT_FP32: torch.float32}

# per-row multipliers: below the reciprocal's range (normal and subnormal elements), one
# subnormal element, just above the range (finite reciprocal, still the small-row branch),
# and an ordinary row
ROW_SCALES = [1e-38, 1e-40, None, 1e-36, 1e-33, 1.0]


def _tiny_x(M, cols, dt, seed):
    """[M, ld] with ld the next 16-byte multiple of the row (ordinary garbage past cols)."""
    g = torch.Generator().manual_seed(seed)
    per16 = 16 // (4 if dt == synth.DT_FP32 else 2)
    ld = (cols + per16 - 1) // per16 * per16
    x = torch.randn(M, ld, generator=g)
    for r in range(M):
        sc = ROW_SCALES[r % len(ROW_SCALES)]
        if sc is None:
            x[r, :cols] = 0.0
            x[r, (7 * r) % cols] = 1e-39
        else:
            x[r, :cols] *= sc
    return x.to(DT_T[dt])


def _host(x, dt):
    return x.contiguous().numpy() if dt == synth.DT_FP32 else synth.bits_u16(x)


ACT_CASES = [(synth.DT_FP32, 12, 777, 0), (synth.DT_BF16, 12, 5376, 0), (synth.DT_BF16, 6, 14336, 0),
             (synth.DT_FP32, 6, 20000, 0), (synth.DT_BF16, 6, 3000, rbl.CR_FLAG_FORCE_TWO_PASS),
             (synth.DT_BF16, 6, 5376, rbl.CR_FLAG_BLOCK_TRANSPOSED)]


@pytest.mark.parametrize("dt,M,K,flags", ACT_CASES, ids=[f"dt{c[0]}-M{c[1]}-K{c[2]}-f{c[3]}" for c in ACT_CASES])
def test_quant_act_tiny_rows(dt, M, K, flags):
    x = _tiny_x(M, K, dt, M + K)
    say(f"cr_quant_act tiny rows dt={dt} M={M} K={K} flags={flags}")
    q, s = rbl.quant_act(x.to(dev()), K, flags=flags)
    torch.cuda.synchronize()
    rq, rs = oracle.quant_act(_host(x, dt), dt, K)
    if flags & rbl.CR_FLAG_BLOCK_TRANSPOSED:       # column 16t + j of a block holds element 16j + t
        kp = rq.shape[1]
        perm = np.arange(kp).reshape(-1, 16, 16).transpose(0, 2, 1).reshape(-1)
        rq = rq[:, perm]
    assert_bits_equal(q.cpu().numpy(), rq, "x_s8 (tiny rows)")
    assert_bits_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32), "x_scale (tiny rows)")


@pytest.mark.parametrize("dt,F", [(synth.DT_FP32, 1000), (synth.DT_BF16, 14336)])
def test_quant_act_swiglu_tiny_rows(dt, F):
    M = 6
    g = torch.Generator().manual_seed(F)
    h = torch.randn(M, 2 * F, generator=g)
    h[0] *= 1e-20                                   # swish(a) b ~ a b / 2 ~ 1e-40
    h[1, :F] *= 1e-30                               # gate tiny, value ordinary: ~1e-30
    h[2, F:] *= 1e-37                               # value tiny: ~1e-37
    h[3] *= 1e-19
    h = h.to(DT_T[dt])
    for flags in (0, rbl.CR_FLAG_FORCE_TWO_PASS):
        say(f"cr_quant_act_swiglu tiny rows dt={dt} F={F} flags={flags}")
        q, s = rbl.quant_act(h.to(dev()), F, swiglu=True, flags=flags)
        torch.cuda.synchronize()
        rq, rs = oracle.quant_act(_host(h, dt), dt, F, swiglu=True)
        assert (rs[:4] < 3.7e-37 / 127).any()        # at least one row below the reciprocal's range
        assert_bits_equal(q.cpu().numpy(), rq, "x_s8 (swiglu, tiny rows)")
        assert_bits_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32), "x_scale (swiglu, tiny rows)")


@pytest.mark.parametrize("gscale", [1e-41, 2e-39, 3e-36])
def test_weight_tiny_global_scale(gscale):
    """Decoded weights E2M1 * E4M3 * g with a tiny g: weight preparation, row maxima and the
    decode-inside-GEMM int32 sums against the oracle."""
    N, K, M = 70, 1300, 33
    gen = torch.Generator().manual_seed(N + K)
    p = synth.nvfp4_encode(0.02 * torch.randn(N, K, generator=gen), garbage_seed=N)
    gt = float(np.float32(gscale))
    gs = torch.tensor([gt], dtype=torch.float32, device=dev())
    cd, sfd = p.codes.to(dev()), p.sf.to(dev())
    rqw, rsw = oracle.prep_weight_nvfp4(p.codes.numpy(), p.sf.numpy(), gt, K)
    ra = oracle.weight_amax_nvfp4(p.codes.numpy(), p.sf.numpy(), gt, K)
    if gscale < 1e-40:
        assert (ra < 3.7e-37).all()                  # every row below the reciprocal's range
    else:
        assert (ra > 3.7e-37).all() and (ra < 2.0 ** -104).all()     # finite reciprocal, small-row branch
    for flags in (0, rbl.CR_FLAG_FORCE_TWO_PASS):
        say(f"cr_prep_weight_nvfp4 / cr_weight_amax_nvfp4 tiny g={gt:.3e} flags={flags}")
        qw, sw = rbl.prep_weight_nvfp4(cd, sfd, gs, K, flags=flags)
        am = rbl.weight_amax_nvfp4(cd, sfd, gs, K, flags=flags)
        torch.cuda.synchronize()
        assert_bits_equal(qw.cpu().numpy(), rqw, "w_s8 (tiny g)")
        assert_bits_equal(sw.cpu().numpy().view(np.uint32), rsw.view(np.uint32), "w_scale (tiny g)")
        assert_bits_equal(am.cpu().numpy().view(np.uint32), ra.view(np.uint32), "w_amax (tiny g)")
    x = (torch.randn(M, K + 4, generator=gen) * 2).to(torch.bfloat16)      # 16-byte row stride
    rq, _ = oracle.quant_act(synth.bits_u16(x), synth.DT_BF16, K)
    acc_ref = oracle.gemm_s8(rq, rqw)
    qx, sx = rbl.quant_act(x.to(dev()), K)
    for given in (True, False):
        say(f"cr_gemm_nvfp4_fused tiny g={gt:.3e} M={M} N={N} K={K} amax={'given' if given else 'in-kernel'}")
        acc = torch.empty(M, N, dtype=torch.int32, device=dev())
        rbl.cr_gemm_nvfp4_fused(qx, sx, cd, sfd, gs, am if given else None, K, acc)
        torch.cuda.synchronize()
        assert_bits_equal(acc.cpu().numpy(), acc_ref, "int32 accumulator (fused, tiny g)")
