"""GPU parity of the W4A8 variant (4-bit rotated weight rows, 8-bit activations) against the
oracle, through the C ABI.

* cr_quant_weight_w4: packed codes and scales bit-exact for bf16/fp16/fp32 weights, ragged K,
  rows of one block per lane group, of several rows per workgroup and two-pass rows, forced
  two-pass, zero rows and rows small enough for the 2^64 extension, natural and
  block-transposed order.
* cr_gemm_s8s4_rowscale: int32 sums bit-exact on ragged shapes whose step counts cover every
  remainder of the three-stage ring, at the largest accepted K_pad with extreme codes, every
  output dtype with and without bias, columns past N untouched (odd and 16-byte ldc).
* cr_linear_w4a8: outputs bit-identical to the oracle's layer (plain and SwiGLU input, both
  orders, bias).
"""
import numpy as np
import pytest
import torch

import oracle
import rotated_bit_linear_amd as rbl
import synth
from helpers import assert_bits_equal, check_output, dev, say

pytestmark = pytest.mark.gpu

BT = rbl.CR_FLAG_BLOCK_TRANSPOSED


def _block_transposed(codes: np.ndarray) -> np.ndarray:
    r, kp = codes.shape
    return codes.reshape(r, kp // 256, 16, 16).transpose(0, 1, 3, 2).reshape(r, kp).copy()


def _dense(N, K, dt, seed, ld=None):
    """Weight [N, ld] of dtype dt (garbage past K), with a zero row and two tiny rows."""
    g = torch.Generator().manual_seed(seed)
    ld = ld or (K + 7) // 8 * 8
    w = torch.randn(N, ld, generator=g) * 0.02
    w[:, K:] = 1e4
    if N > 3:
        w[1, :K] = 0.0
        w[2, :K] *= 1e-36            # 127/a would overflow for 8-bit codes; 7/a stays finite
    if N > 5 and dt == synth.DT_FP32:
        w[4, :K] *= 1e-37            # 7/a overflows: the 2^64 extension
    return w.to(synth.TORCH_DTYPE[dt])


def _host(w, dt):
    return w.contiguous().numpy() if dt == synth.DT_FP32 else synth.bits_u16(w)


W_CASES = [(synth.DT_BF16, 300, 1000), (synth.DT_FP16, 97, 5376), (synth.DT_FP32, 64, 20000),
           (synth.DT_BF16, 40, 16384), (synth.DT_FP32, 21, 17), (synth.DT_BF16, 70, 14336),
           (synth.DT_FP16, 33, 25000)]


@pytest.mark.parametrize("dt,N,K", W_CASES, ids=[f"dt{c[0]}-N{c[1]}-K{c[2]}" for c in W_CASES])
def test_quant_weight_w4_bit_exact(dt, N, K):
    w = _dense(N, K, dt, N + K)
    rp, rs = oracle.quant_weight_w4(_host(w, dt), dt, K)
    kp = rp.shape[1] * 2
    codes = oracle.unpack_s4(rp, kp)
    rp_bt = oracle.pack_s4(_block_transposed(codes))
    for flags in (0, BT, rbl.CR_FLAG_FORCE_TWO_PASS, rbl.CR_FLAG_FORCE_TWO_PASS | BT):
        say(f"cr_quant_weight_w4 dt={dt} N={N} K={K} flags={flags}")
        p, s = rbl.quant_weight_w4(w.to(dev())[:, :K] if w.shape[1] != K else w.to(dev()), K, flags=flags)
        torch.cuda.synchronize()
        assert_bits_equal(p.cpu().numpy(), rp_bt if flags & BT else rp, f"w_s4 flags={flags}")
        assert_bits_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32), f"w_scale flags={flags}")


# K_pad / 128 steps: 2, 6, 8, 10, 22, 42, 112, 158 (every remainder modulo the 3-stage ring)
G_CASES = [(64, 256, 256), (300, 700, 768), (1, 1, 1024), (513, 255, 1280), (257, 300, 2816),
           (600, 520, 5376), (260, 300, 14336), (77, 129, 20224)]


@pytest.mark.parametrize("M,N,Kp", G_CASES, ids=[f"M{c[0]}-N{c[1]}-K{c[2]}" for c in G_CASES])
def test_gemm_s8s4_int32_exact_and_epilogues(M, N, Kp):
    g = torch.Generator().manual_seed(M * 7 + N + Kp)
    a = torch.randint(-127, 128, (M, Kp), generator=g, dtype=torch.int32).to(torch.int8)
    q = torch.randint(-7, 8, (N, Kp), generator=g, dtype=torch.int32).to(torch.int8)
    b = torch.from_numpy(oracle.pack_s4(q.numpy()))
    sa = torch.rand(M, generator=g) * 1e-2
    sb = torch.rand(N, generator=g) * 1e-2
    sa[0] = 0.0
    bias = torch.randn(N, generator=g)
    acc = oracle.gemm_s8s4(a.numpy(), b.numpy())
    ad, bd, sad, sbd, biasd = a.to(dev()), b.to(dev()), sa.to(dev()), sb.to(dev()), bias.to(dev())
    for ldc in (N + 9, (N + 7) // 8 * 8 + 8):
        for odt in (synth.DT_I32, synth.DT_BF16, synth.DT_FP16, synth.DT_FP32):
            for with_bias in ((False,) if odt == synth.DT_I32 else (False, True)):
                tdt = synth.TORCH_DTYPE[odt]
                full = torch.full((M, ldc), 7, dtype=tdt, device=dev())
                c = full[:, :N]
                say(f"cr_gemm_s8s4_rowscale M={M} N={N} K_pad={Kp} out={odt} ldc={ldc} bias={with_bias}")
                rbl.cr_gemm_s8s4_rowscale(ad, sad, bd, sbd, c, bias=biasd if with_bias else None)
                torch.cuda.synchronize()
                fc = full.cpu()
                assert (fc[:, N:] == 7).all(), "columns past N were written"
                if odt == synth.DT_I32:
                    assert_bits_equal(fc[:, :N].numpy(), acc, "int32 accumulator")
                else:
                    ref = oracle.epilogue(acc, sa.numpy(), sb.numpy(), odt,
                                          bias=bias.numpy() if with_bias else None)
                    check_output(fc[:, :N], ref, odt, f"W4A8 GEMM out={odt} bias={with_bias}")


def test_gemm_s8s4_worst_case_accumulator():
    """The largest accepted K_pad with codes +-127 and +-7: |sum| = 127 * 7 * 133120, and the
    kernel's internal sums are 16 times that (below 2^31)."""
    Kp = rbl.CR_MAX_K_PAD
    a = torch.full((3, Kp), 127, dtype=torch.int8)
    a[1] = -127
    a[2, ::2] = -127
    q = torch.full((5, Kp), 7, dtype=torch.int8)
    q[1] = -7
    q[3, 1::2] = -7
    q[4] = 0
    b = torch.from_numpy(oracle.pack_s4(q.numpy()))
    acc = oracle.gemm_s8s4(a.numpy(), b.numpy())
    assert int(np.abs(acc).max()) == 127 * 7 * Kp
    say(f"cr_gemm_s8s4_rowscale worst-case accumulator K_pad={Kp}")
    c = torch.empty(3, 5, dtype=torch.int32, device=dev())
    rbl.cr_gemm_s8s4_rowscale(a.to(dev()), None, b.to(dev()), None, c)
    torch.cuda.synchronize()
    assert_bits_equal(c.cpu().numpy(), acc, "int32 accumulator at the K_pad limit")


L_CASES = [(300, 700, 1000, synth.DT_BF16, False, 0), (65, 300, 5376, synth.DT_FP16, False, BT),
           (130, 256, 3000, synth.DT_BF16, True, BT), (33, 100, 20000, synth.DT_BF16, False, 0)]


@pytest.mark.parametrize("M,N,K,dt,swiglu,flags", L_CASES,
                         ids=[f"M{c[0]}-N{c[1]}-K{c[2]}-sw{int(c[4])}-f{c[5]}" for c in L_CASES])
def test_linear_w4a8_against_oracle(M, N, K, dt, swiglu, flags):
    wl = synth.Workload("w4a8", M, N, K, dt, (synth.DT_BF16,), M + N, swiglu=swiglu, outlier_frac=0.01)
    x = synth.make_activation(wl)
    w = _dense(N, K, synth.DT_FP32, N * 3 + K)
    rp, rs = oracle.quant_weight_w4(_host(w, synth.DT_FP32), synth.DT_FP32, K)
    say(f"cr_quant_weight_w4 for the layer N={N} K={K} flags={flags}")
    p, s = rbl.quant_weight_w4(w.to(dev())[:, :K], K, flags=flags)
    bias = torch.randn(N, generator=torch.Generator().manual_seed(N)).float()
    xb = synth.bits_u16(x) if dt != synth.DT_FP32 else x.numpy()
    for odt in (synth.DT_BF16, synth.DT_FP32):
        for with_bias in (False, True):
            say(f"cr_linear_w4a8 M={M} N={N} K={K} swiglu={swiglu} flags={flags} out={odt} bias={with_bias}")
            y = rbl.linear_w4a8(x.to(dev()), p, s, K, out_dtype=synth.TORCH_DTYPE[odt], swiglu=swiglu,
                                bias=bias.to(dev()) if with_bias else None, flags=flags)
            torch.cuda.synchronize()
            ref = oracle.linear_w4a8(xb, dt, K, swiglu, rp, rs, odt, bias=bias.numpy() if with_bias else None)
            check_output(y, ref, odt, f"W4A8 layer out={odt} bias={with_bias}")
