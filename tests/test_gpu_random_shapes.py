"""Seeded random shapes through every entry point, against the oracle (C ABI, GPU).

Each case draws M, N, K (ragged, with K sometimes past the two-pass threshold), input and
output dtypes, padded row strides with garbage in the padding, a column order, and an
optional pre-scale and bias, then checks the S8 codes and scales bit for bit, the int32
accumulator bit for bit, and the outputs within the output tolerance.  The layer call is
repeated under a small tile bound (1-3 tile heights), serially or with a second stream, and
must give the same bits."""
import numpy as np
import pytest
import torch

import oracle
import rotated_bit_linear_amd as rbl
import synth
from helpers import assert_bits_equal, check_output, dev, say

pytestmark = pytest.mark.gpu

DT_T = {synth.DT_BF16: torch.bfloat16, synth.DT_FP16: torch.float16, synth.DT_FP32: torch.float32}


def _case(i):
    r = np.random.default_rng(1000 + i)
    M = int(r.choice([1, 2, 7, 31, 33, 64, 65, 129, 257, 300]))
    N = int(r.choice([1, 5, 32, 100, 255, 256, 257, 513]))
    K = int(r.choice([1, 15, 16, 17, 255, 256, 257, 1000, 5376, 16385, 20000]))
    xdt = int(r.choice([synth.DT_BF16, synth.DT_FP16, synth.DT_FP32]))
    odt = int(r.choice([synth.DT_BF16, synth.DT_FP16, synth.DT_FP32]))
    swiglu = bool(r.random() < 0.3)
    order = int(r.choice([0, rbl.CR_FLAG_BLOCK_TRANSPOSED]))
    extra = bool(r.random() < 0.4)
    return M, N, K, xdt, odt, swiglu, order, extra


CASES = [_case(i) for i in range(120)]


def _ids(c):
    M, N, K, xdt, odt, swiglu, order, extra = c
    return f"M{M}-N{N}-K{K}-x{xdt}-o{odt}-{'sw' if swiglu else 'x'}-ord{order}-{'pb' if extra else 'np'}"


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_random_shape_all_entry_points(case):
    M, N, K, xdt, odt, swiglu, order, extra = case
    seed = M * 7919 + N * 31 + K
    g = torch.Generator().manual_seed(seed)
    cols = 2 * K if swiglu else K
    esize = 4 if xdt == synth.DT_FP32 else 2
    mult = 16 // esize
    ld = (cols + mult - 1) // mult * mult + mult                  # padded, 16-byte row stride
    x = torch.randn(M, ld, generator=g) * 2
    x[:, cols:] = 3e4                                             # garbage past the row
    x = x.to(DT_T[xdt])
    xb = x.numpy() if xdt == synth.DT_FP32 else synth.bits_u16(x)
    wf = 0.02 * torch.randn(N, K, generator=g)
    p = synth.nvfp4_encode(wf, ld_codes=((K + 1) // 2 + 15) // 16 * 16 + 16, ld_sf=(K + 15) // 16 + 3,
                           garbage_seed=seed)
    gs = torch.tensor([p.g], dtype=torch.float32, device=dev())
    cd, sd = p.codes.to(dev()), p.sf.to(dev())
    pre = (torch.rand(K, generator=g) + 0.5) if extra else None
    bias = torch.randn(N, generator=g) if extra else None
    kp = rbl.padded_k(K)

    # oracle (natural order) and its block-transposed view
    rq, rs = oracle.quant_act(xb, xdt, K, swiglu=swiglu, pre_scale=None if pre is None else pre.numpy())
    rqw, rsw = oracle.prep_weight_nvfp4(p.codes.numpy(), p.sf.numpy(), p.g, K)
    acc = oracle.gemm_s8(rq, rqw)

    def view(codes):
        if order == 0:
            return codes
        r_, c_ = codes.shape
        return codes.reshape(r_, c_ // 256, 16, 16).transpose(0, 1, 3, 2).reshape(r_, c_)

    say(f"random case {_ids(case)}: activation + weight preparation")
    qx, sx = rbl.quant_act(x.to(dev()), K, swiglu=swiglu, flags=order,
                           pre_scale=None if pre is None else pre.to(dev()))
    qw, sw = rbl.prep_weight_nvfp4(cd, sd, gs, K, flags=order)
    torch.cuda.synchronize()
    assert_bits_equal(qx.cpu().numpy(), view(rq), "x_s8")
    assert_bits_equal(sx.cpu().numpy().view(np.uint32), rs.view(np.uint32), "x_scale")
    assert_bits_equal(qw.cpu().numpy(), view(rqw), "w_s8")
    assert_bits_equal(sw.cpu().numpy().view(np.uint32), rsw.view(np.uint32), "w_scale")

    say(f"random case {_ids(case)}: GEMM, fused GEMM, layer")
    ci = torch.empty(M, N, dtype=torch.int32, device=dev())
    rbl.cr_gemm_s8_rowscale(qx, sx, qw, sw, ci)
    cf = torch.empty(M, N, dtype=torch.int32, device=dev())
    rbl.cr_gemm_nvfp4_fused(qx, sx, cd, sd, gs, None, K, cf, flags=order)
    tdt = synth.TORCH_DTYPE[odt]
    bd = None if bias is None else bias.to(dev())
    y = rbl.gemm_s8_rowscale(qx, sx, qw, sw, out_dtype=tdt, bias=bd)
    yl = rbl.linear_nvfp4(x.to(dev()), cd, sd, gs, K, out_dtype=tdt, swiglu=swiglu,
                          pre_scale=None if pre is None else pre.to(dev()), bias=bd)
    # the same layer under a small tile bound (weight chunks of 1-3 tile heights, chosen
    # by the chunk planner), staged serially or on a second stream: the same bits
    rr = np.random.default_rng(seed + 99)
    bound = int(rr.integers(1, 4)) * 256 * kp
    aux = torch.cuda.Stream() if rr.random() < 0.5 else None
    yb = rbl.linear_nvfp4(x.to(dev()), cd, sd, gs, K, out_dtype=tdt, swiglu=swiglu, max_tile_bytes=bound,
                          aux_stream=aux, pre_scale=None if pre is None else pre.to(dev()), bias=bd)
    torch.cuda.synchronize()
    assert torch.equal(yb, yl), f"layer output under a {bound}-byte tile bound differs"
    if aux is not None:
        del aux
    assert_bits_equal(ci.cpu().numpy(), acc, "int32 accumulator")
    assert_bits_equal(cf.cpu().numpy(), acc, "int32 accumulator (decode inside the GEMM)")
    ref = oracle.epilogue(acc, rs, rsw, odt, bias=None if bias is None else bias.numpy())
    for got, what in ((y, "GEMM output"), (yl, "layer output")):
        check_output(got, ref, odt, what)
