"""The largest accepted K_pad (133120 = 520 blocks, the int32 limit 127^2 K_pad < 2^31) on the
GPU, against the oracle: the worst-case accumulator through both GEMMs, two-pass
preparation of 520-block rows, and the layer on both of its paths."""
import numpy as np
import pytest
import torch

import oracle
import rotated_bit_linear_amd as rbl
import synth
from helpers import assert_bits_equal, check_output, dev, say

pytestmark = pytest.mark.gpu

KMAX = rbl.CR_MAX_K_PAD


def test_gemm_worst_case_accumulator_at_max_k():
    """Codes of +-127 everywhere: |acc| reaches 127^2 * 133120 = 2147092480, next to 2^31."""
    M, N = 300, 260
    g = torch.Generator().manual_seed(5)
    a = torch.randint(-127, 128, (M, KMAX), generator=g, dtype=torch.int32).to(torch.int8)
    b = torch.randint(-127, 128, (N, KMAX), generator=g, dtype=torch.int32).to(torch.int8)
    a[0] = 127
    a[1] = -127
    b[0] = 127
    b[N - 1] = 127
    acc = oracle.gemm_s8(a.numpy(), b.numpy())
    assert acc[0, 0] == 127 * 127 * KMAX and acc[1, 0] == -127 * 127 * KMAX
    say(f"cr_gemm_s8_rowscale int32 M={M} N={N} K_pad={KMAX}")
    c = torch.empty(M, N, dtype=torch.int32, device=dev())
    rbl.cr_gemm_s8_rowscale(a.to(dev()), None, b.to(dev()), None, c)
    torch.cuda.synchronize()
    assert_bits_equal(c.cpu().numpy(), acc, "int32 accumulator at the largest K_pad")


def test_preparation_and_layer_at_max_k():
    K = KMAX - 100                                      # ragged: K_pad is still 133120
    g = torch.Generator().manual_seed(6)
    w = 0.02 * torch.randn(40, K, generator=g)
    w[3] = 0.0
    p = synth.nvfp4_encode(w, garbage_seed=6)
    gs = torch.tensor([p.g], dtype=torch.float32, device=dev())
    cd, sd = p.codes.to(dev()), p.sf.to(dev())
    x = (torch.randn(70, KMAX, generator=g) * 2).to(torch.bfloat16)      # row stride 133120
    x[:, K:] = 1e4                                                        # garbage past K
    x[5] = 0.0
    xb = synth.bits_u16(x)

    say(f"preparation at K={K} (K_pad {KMAX}, two-pass rows of 520 blocks)")
    qx, sx = rbl.quant_act(x.to(dev()), K)
    qw, sw = rbl.prep_weight_nvfp4(cd, sd, gs, K)
    am = rbl.weight_amax_nvfp4(cd, sd, gs, K)
    torch.cuda.synchronize()
    rq, rs = oracle.quant_act(xb, synth.DT_BF16, K)
    rqw, rsw = oracle.prep_weight_nvfp4(p.codes.numpy(), p.sf.numpy(), p.g, K)
    ram = oracle.weight_amax_nvfp4(p.codes.numpy(), p.sf.numpy(), p.g, K)
    assert_bits_equal(qx.cpu().numpy(), rq, "x_s8")
    assert_bits_equal(sx.cpu().numpy().view(np.uint32), rs.view(np.uint32), "x_scale")
    assert_bits_equal(qw.cpu().numpy(), rqw, "w_s8")
    assert_bits_equal(sw.cpu().numpy().view(np.uint32), rsw.view(np.uint32), "w_scale")
    assert_bits_equal(am.cpu().numpy().view(np.uint32), ram.view(np.uint32), "w_amax")

    acc = oracle.gemm_s8(rq, rqw)
    for M in (70, 3):                                   # staged path, then decode inside the GEMM
        say(f"cr_linear_nvfp4 M={M} N=40 K={K}")
        y = rbl.linear_nvfp4(x[:M].contiguous().to(dev()), cd, sd, gs, K, out_dtype=torch.float32)
        ci = torch.empty(M, 40, dtype=torch.int32, device=dev())
        rbl.cr_gemm_nvfp4_fused(qx[:M], sx[:M], cd, sd, gs, None, K, ci)
        torch.cuda.synchronize()
        assert_bits_equal(ci.cpu().numpy(), acc[:M], "int32 accumulator (decode inside the GEMM)")
        ref = oracle.epilogue(acc[:M], rs[:M], rsw, synth.DT_FP32)
        check_output(y, ref, synth.DT_FP32, f"layer output M={M}")


def test_two_pass_rows_beyond_the_grid_cap():
    """Forced two-pass preparation of 70000 rows: more rows than two-pass workgroups
    (65536), so workgroups loop over rows; every row bit-exact."""
    M, K = 70000, 300
    g = torch.Generator().manual_seed(8)
    x = (torch.randn(M, 304, generator=g) * 2).to(torch.bfloat16)     # 16-byte row stride
    x[:, K:] = 1e4
    x[7] = 0.0
    say(f"cr_quant_act forced two-pass M={M} K={K}")
    q, s = rbl.quant_act(x.to(dev()), K, flags=rbl.CR_FLAG_FORCE_TWO_PASS)
    w = 0.02 * torch.randn(M, 256, generator=g)
    p = synth.nvfp4_encode(w, garbage_seed=8)
    gs = torch.tensor([p.g], dtype=torch.float32, device=dev())
    say(f"cr_weight_amax_nvfp4 forced two-pass N={M} K=256")
    am = rbl.weight_amax_nvfp4(p.codes.to(dev()), p.sf.to(dev()), gs, 256, flags=rbl.CR_FLAG_FORCE_TWO_PASS)
    torch.cuda.synchronize()
    rq, rs = oracle.quant_act(synth.bits_u16(x), synth.DT_BF16, K)
    assert_bits_equal(q.cpu().numpy(), rq, "x_s8")
    assert_bits_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32), "x_scale")
    ra = oracle.weight_amax_nvfp4(p.codes.numpy(), p.sf.numpy(), p.g, 256)
    assert_bits_equal(am.cpu().numpy().view(np.uint32), ra.view(np.uint32), "w_amax")
