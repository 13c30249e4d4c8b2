"""GPU parity of the W4A4 variant (4-bit rotated rows on both operands) against the oracle,
through the C ABI.

* cr_quant_act_w4: packed codes and scales bit-exact for bf16/fp16/fp32 activations and
  SwiGLU inputs, ragged K, every row form (several rows per workgroup, one row, two-pass),
  forced two-pass, zero rows and rows small enough for the 2^64 extension, natural and
  block-transposed order.
* cr_gemm_s4s4_rowscale: int32 sums bit-exact on ragged shapes whose step counts cover every
  remainder of the three-stage ring, at the largest accepted K_pad with extreme codes, every
  output dtype with and without bias, columns past N untouched (odd and 16-byte ldc).
* cr_linear_w4a4: outputs bit-identical to the oracle's layer (plain and SwiGLU input, both
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
DT_T = {synth.DT_BF16: torch.bfloat16, synth.DT_FP16: torch.float16, synth.DT_FP32: torch.float32}


def _block_transposed(codes: np.ndarray) -> np.ndarray:
    r, kp = codes.shape
    return codes.reshape(r, kp // 256, 16, 16).transpose(0, 1, 3, 2).reshape(r, kp).copy()


def _bt_packed(p: np.ndarray) -> np.ndarray:
    kp = p.shape[1] * 2
    return oracle.pack_s4(_block_transposed(oracle.unpack_s4(p, kp)))


def _act(M, width, dt, seed):
    """Activation [M, ld] of dtype dt over `width` used columns (garbage past them), with a
    zero row and tiny rows."""
    g = torch.Generator().manual_seed(seed)
    ld = (width + 7) // 8 * 8 + 8
    x = torch.randn(M, ld, generator=g) * 2.0
    x[:, width:] = 1e4
    if M > 3:
        x[1, :width] = 0.0
        x[2, :width] *= 1e-36 if dt == synth.DT_FP32 else 1e-4
    if M > 5 and dt == synth.DT_FP32:
        x[4, :width] *= 1e-37            # 7/a overflows: the 2^64 extension
    return x.to(synth.TORCH_DTYPE[dt])


def _host(x, dt):
    return x.contiguous().numpy() if dt == synth.DT_FP32 else synth.bits_u16(x)


A_CASES = [(synth.DT_BF16, False, 300, 1000), (synth.DT_FP16, False, 97, 5376), (synth.DT_FP32, False, 64, 20000),
           (synth.DT_FP16, False, 30, 20000), (synth.DT_BF16, False, 9, 32768),
           (synth.DT_BF16, False, 40, 16384), (synth.DT_FP32, False, 21, 17), (synth.DT_BF16, True, 70, 14336),
           (synth.DT_FP16, True, 33, 3000), (synth.DT_FP32, True, 9, 20000), (synth.DT_BF16, True, 50, 255)]


@pytest.mark.parametrize("dt,swiglu,M,K", A_CASES,
                         ids=[f"dt{c[0]}-sw{int(c[1])}-M{c[2]}-K{c[3]}" for c in A_CASES])
def test_quant_act_w4_bit_exact(dt, swiglu, M, K):
    width = 2 * K if swiglu else K
    x = _act(M, width, dt, M + K + int(swiglu))
    rp, rs = oracle.quant_act_w4(_host(x, dt), dt, K, swiglu=swiglu)
    rp_bt = _bt_packed(rp)
    xd = x.to(dev())
    for flags in (0, BT, rbl.CR_FLAG_FORCE_TWO_PASS, rbl.CR_FLAG_FORCE_TWO_PASS | BT):
        say(f"cr_quant_act_w4 dt={dt} swiglu={swiglu} M={M} K={K} flags={flags}")
        p, s = rbl.quant_act_w4(xd, K, swiglu=swiglu, flags=flags)
        torch.cuda.synchronize()
        assert_bits_equal(p.cpu().numpy(), rp_bt if flags & BT else rp, f"x_s4 flags={flags}")
        assert_bits_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32), f"x_scale flags={flags}")


# K_pad / 128 steps: 2, 6, 8, 10, 22, 42, 112, 158 (every remainder modulo the 3-stage ring)
G_CASES = [(64, 256, 256), (300, 700, 768), (1, 1, 1024), (513, 255, 1280), (257, 300, 2816),
           (600, 520, 5376), (260, 300, 14336), (77, 129, 20224)]


@pytest.mark.parametrize("M,N,Kp", G_CASES, ids=[f"M{c[0]}-N{c[1]}-K{c[2]}" for c in G_CASES])
def test_gemm_s4s4_int32_exact_and_epilogues(M, N, Kp):
    g = torch.Generator().manual_seed(M * 11 + N + Kp)
    qa = torch.randint(-7, 8, (M, Kp), generator=g, dtype=torch.int32).to(torch.int8)
    qb = torch.randint(-7, 8, (N, Kp), generator=g, dtype=torch.int32).to(torch.int8)
    a = torch.from_numpy(oracle.pack_s4(qa.numpy()))
    b = torch.from_numpy(oracle.pack_s4(qb.numpy()))
    sa = torch.rand(M, generator=g) * 1e-2
    sb = torch.rand(N, generator=g) * 1e-2
    sa[0] = 0.0
    bias = torch.randn(N, generator=g)
    acc = oracle.gemm_s4s4(a.numpy(), b.numpy(), Kp)
    ad, bd, sad, sbd, biasd = a.to(dev()), b.to(dev()), sa.to(dev()), sb.to(dev()), bias.to(dev())
    for ldc in (N + 9, (N + 7) // 8 * 8 + 8):
        for odt in (synth.DT_I32, synth.DT_BF16, synth.DT_FP16, synth.DT_FP32):
            for with_bias in ((False,) if odt == synth.DT_I32 else (False, True)):
                tdt = synth.TORCH_DTYPE[odt]
                full = torch.full((M, ldc), 7, dtype=tdt, device=dev())
                c = full[:, :N]
                say(f"cr_gemm_s4s4_rowscale M={M} N={N} K_pad={Kp} out={odt} ldc={ldc} bias={with_bias}")
                rbl.cr_gemm_s4s4_rowscale(ad, sad, bd, sbd, c, bias=biasd if with_bias else None)
                torch.cuda.synchronize()
                fc = full.cpu()
                assert (fc[:, N:] == 7).all(), "columns past N were written"
                if odt == synth.DT_I32:
                    assert_bits_equal(fc[:, :N].numpy(), acc, "int32 accumulator")
                else:
                    ref = oracle.epilogue(acc, sa.numpy(), sb.numpy(), odt,
                                          bias=bias.numpy() if with_bias else None)
                    check_output(fc[:, :N], ref, odt, f"W4A4 GEMM out={odt} bias={with_bias}")


def test_gemm_s4s4_strided_operands():
    """Row strides beyond K_pad / 2 on both packed operands (only the first K_pad / 2 bytes of
    a row are codes)."""
    M, N, Kp = 300, 260, 1280
    g = torch.Generator().manual_seed(5)
    qa = torch.randint(-7, 8, (M, Kp), generator=g, dtype=torch.int32).to(torch.int8)
    qb = torch.randint(-7, 8, (N, Kp), generator=g, dtype=torch.int32).to(torch.int8)
    a = torch.from_numpy(oracle.pack_s4(qa.numpy()))
    b = torch.from_numpy(oracle.pack_s4(qb.numpy()))
    acc = oracle.gemm_s4s4(a.numpy(), b.numpy(), Kp)
    af = torch.full((M, Kp // 2 + 48), 0x77, dtype=torch.uint8)
    bf = torch.full((N, Kp // 2 + 16), 0x77, dtype=torch.uint8)
    af[:, :Kp // 2] = a
    bf[:, :Kp // 2] = b
    ad, bd = af.to(dev()), bf.to(dev())
    c = torch.empty(M, N, dtype=torch.int32, device=dev())
    say(f"cr_gemm_s4s4_rowscale strided lda={af.shape[1]} ldb={bf.shape[1]}")
    rbl.cr_gemm_s4s4_rowscale(ad[:, :Kp // 2], None, bd[:, :Kp // 2], None, c, K_pad=Kp)
    torch.cuda.synchronize()
    assert_bits_equal(c.cpu().numpy(), acc, "int32 accumulator with row strides")


def test_gemm_s4s4_worst_case_accumulator():
    """The largest accepted K_pad with codes +-7 on both sides: |sum| = 49 * 133120, and the
    kernel's internal sums are 256 times that (below 2^31)."""
    Kp = rbl.CR_MAX_K_PAD
    qa = torch.full((3, Kp), 7, dtype=torch.int8)
    qa[1] = -7
    qa[2, ::2] = -7
    qb = torch.full((5, Kp), 7, dtype=torch.int8)
    qb[1] = -7
    qb[3, 1::2] = -7
    qb[4] = 0
    a = torch.from_numpy(oracle.pack_s4(qa.numpy()))
    b = torch.from_numpy(oracle.pack_s4(qb.numpy()))
    acc = oracle.gemm_s4s4(a.numpy(), b.numpy(), Kp)
    assert int(np.abs(acc).max()) == 49 * Kp
    assert 256 * 49 * Kp < 2 ** 31
    say(f"cr_gemm_s4s4_rowscale worst-case accumulator K_pad={Kp}")
    c = torch.empty(3, 5, dtype=torch.int32, device=dev())
    rbl.cr_gemm_s4s4_rowscale(a.to(dev()), None, b.to(dev()), None, c)
    torch.cuda.synchronize()
    assert_bits_equal(c.cpu().numpy(), acc, "int32 accumulator at the K_pad limit")


L_CASES = [(300, 700, 1000, synth.DT_BF16, False, 0), (65, 300, 5376, synth.DT_FP16, False, BT),
           (130, 256, 3000, synth.DT_BF16, True, BT), (33, 100, 20000, synth.DT_BF16, False, 0),
           (17, 90, 17, synth.DT_FP32, True, 0)]


@pytest.mark.parametrize("M,N,K,dt,swiglu,flags", L_CASES,
                         ids=[f"M{c[0]}-N{c[1]}-K{c[2]}-sw{int(c[4])}-f{c[5]}" for c in L_CASES])
def test_linear_w4a4_against_oracle(M, N, K, dt, swiglu, flags):
    wl = synth.Workload("w4a4", M, N, K, dt, (synth.DT_BF16,), M + N, swiglu=swiglu, outlier_frac=0.01)
    x = synth.make_activation(wl)
    g = torch.Generator().manual_seed(N * 5 + K)
    w = (torch.randn(N, (K + 7) // 8 * 8, generator=g) * 0.02).float()
    rp, rs = oracle.quant_weight_w4(w.numpy(), synth.DT_FP32, K)
    say(f"cr_quant_weight_w4 for the layer N={N} K={K} flags={flags}")
    p, s = rbl.quant_weight_w4(w.to(dev())[:, :K], K, flags=flags)
    bias = torch.randn(N, generator=torch.Generator().manual_seed(N)).float()
    xb = synth.bits_u16(x) if dt != synth.DT_FP32 else x.numpy()
    # rows of 16-byte multiples on the device (a padded tensor, viewed at its used columns)
    cols = x.shape[1]
    xpad = torch.zeros(M, (cols + 7) // 8 * 8 + 8, dtype=x.dtype)
    xpad[:, :cols] = x
    xd = xpad.to(dev())[:, :cols]
    for odt in (synth.DT_BF16, synth.DT_FP32):
        for with_bias in (False, True):
            say(f"cr_linear_w4a4 M={M} N={N} K={K} swiglu={swiglu} flags={flags} out={odt} bias={with_bias}")
            y = rbl.linear_w4a4(xd, p, s, K, out_dtype=synth.TORCH_DTYPE[odt], swiglu=swiglu,
                                bias=bias.to(dev()) if with_bias else None, flags=flags)
            torch.cuda.synchronize()
            ref = oracle.linear_w4a4(xb, dt, K, swiglu, rp, rs, odt, bias=bias.numpy() if with_bias else None)
            check_output(y, ref, odt, f"W4A4 layer out={odt} bias={with_bias}")


# ------------------------------------------------ the E2M3 execution form ----
# The same codes stored as E2M3 fields (6-bit floats of equal value, rows in quads) and
# multiplied on the 6-bit matrix cores: codes, scales, int32 sums and outputs must equal the
# oracle's.  The conveniences zero their outputs first, so the unused rows of a last quad
# compare equal to the oracle's zeros.

def _e2m3(p_nibbles: np.ndarray) -> np.ndarray:
    """The oracle's E2M3 form of the codes of nibble-packed rows."""
    kp = p_nibbles.shape[1] * 2
    return oracle.pack_e2m3(oracle.unpack_s4(p_nibbles, kp))


@pytest.mark.parametrize("dt,swiglu,M,K", A_CASES,
                         ids=[f"dt{c[0]}-sw{int(c[1])}-M{c[2]}-K{c[3]}" for c in A_CASES])
def test_quant_act_w4_e2m3_bit_exact(dt, swiglu, M, K):
    width = 2 * K if swiglu else K
    x = _act(M, width, dt, M + K + int(swiglu))
    rp, rs = oracle.quant_act_w4(_host(x, dt), dt, K, swiglu=swiglu)
    rf, rf_bt = _e2m3(rp), _e2m3(_bt_packed(rp))
    xd = x.to(dev())
    for flags in (0, BT, rbl.CR_FLAG_FORCE_TWO_PASS, rbl.CR_FLAG_FORCE_TWO_PASS | BT):
        say(f"cr_quant_act_w4_e2m3 dt={dt} swiglu={swiglu} M={M} K={K} flags={flags}")
        p, s = rbl.quant_act_w4_e2m3(xd, K, swiglu=swiglu, flags=flags)
        torch.cuda.synchronize()
        assert_bits_equal(p.cpu().numpy(), rf_bt if flags & BT else rf, f"x_f6 flags={flags}")
        assert_bits_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32), f"x_scale flags={flags}")


W_CASES = [(synth.DT_BF16, 300, 1000), (synth.DT_FP16, 97, 5376), (synth.DT_FP32, 64, 20000), (synth.DT_BF16, 37, 20000),
           (synth.DT_FP32, 21, 17), (synth.DT_BF16, 70, 14336)]


@pytest.mark.parametrize("dt,N,K", W_CASES, ids=[f"dt{c[0]}-N{c[1]}-K{c[2]}" for c in W_CASES])
def test_quant_weight_w4_e2m3_bit_exact(dt, N, K):
    w = _act(N, K, dt, 3 * N + K)
    rp, rs = oracle.quant_weight_w4(_host(w, dt), dt, K)
    rf, rf_bt = _e2m3(rp), _e2m3(_bt_packed(rp))
    wd = w.to(dev())
    for flags in (0, BT, rbl.CR_FLAG_FORCE_TWO_PASS | BT):
        say(f"cr_quant_weight_w4_e2m3 dt={dt} N={N} K={K} flags={flags}")
        p, s = rbl.quant_weight_w4_e2m3(wd, K, flags=flags)
        torch.cuda.synchronize()
        assert_bits_equal(p.cpu().numpy(), rf_bt if flags & BT else rf, f"w_f6 flags={flags}")
        assert_bits_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32), f"w_scale flags={flags}")


@pytest.mark.parametrize("dt,N,K", W_CASES, ids=[f"dt{c[0]}-N{c[1]}-K{c[2]}" for c in W_CASES])
def test_repack_w4_e2m3_equals_direct_preparation(dt, N, K):
    """cr_repack_w4_e2m3 of the nibble-form weight equals cr_quant_weight_w4_e2m3 of the same
    dense weight and the oracle's E2M3 packing of the oracle's codes, bit for bit (both
    column orders); a nibble row stride beyond K_pad / 2 is honoured."""
    w = _act(N, K, dt, 5 * N + K)
    rp, _ = oracle.quant_weight_w4(_host(w, dt), dt, K)
    wd = w.to(dev())
    for flags in (0, BT):
        say(f"cr_repack_w4_e2m3 dt={dt} N={N} K={K} flags={flags}")
        p4, _ = rbl.quant_weight_w4(wd, K, flags=flags)
        kp = p4.shape[1] * 2
        wide = torch.full((N, kp // 2 + 32), 0x88, dtype=torch.uint8, device=dev())
        wide[:, :kp // 2] = p4
        f6 = rbl.repack_w4_e2m3(wide[:, :kp // 2], K_pad=kp)
        d6, _ = rbl.quant_weight_w4_e2m3(wd, K, flags=flags)
        torch.cuda.synchronize()
        want = _e2m3(_bt_packed(rp) if flags & BT else rp)
        assert_bits_equal(f6.cpu().numpy(), want, f"repacked fields flags={flags}")
        assert_bits_equal(d6.cpu().numpy(), want, f"directly prepared fields flags={flags}")


@pytest.mark.parametrize("M,N,Kp", G_CASES, ids=[f"M{c[0]}-N{c[1]}-K{c[2]}" for c in G_CASES])
def test_gemm_e2m3_int32_exact_and_epilogues(M, N, Kp):
    g = torch.Generator().manual_seed(M * 13 + N + Kp)
    qa = torch.randint(-7, 8, (M, Kp), generator=g, dtype=torch.int32).to(torch.int8)
    qb = torch.randint(-7, 8, (N, Kp), generator=g, dtype=torch.int32).to(torch.int8)
    a = torch.from_numpy(oracle.pack_e2m3(qa.numpy()))
    b = torch.from_numpy(oracle.pack_e2m3(qb.numpy()))
    sa = torch.rand(M, generator=g) * 1e-2
    sb = torch.rand(N, generator=g) * 1e-2
    sa[0] = 0.0
    bias = torch.randn(N, generator=g)
    acc = oracle.gemm_e2m3(a.numpy(), b.numpy(), Kp, M, N)
    ad, bd, sad, sbd, biasd = a.to(dev()), b.to(dev()), sa.to(dev()), sb.to(dev()), bias.to(dev())
    for ldc in (N + 9, (N + 7) // 8 * 8 + 8):
        for odt in (synth.DT_I32, synth.DT_BF16, synth.DT_FP16, synth.DT_FP32):
            for with_bias in ((False,) if odt == synth.DT_I32 else (False, True)):
                tdt = synth.TORCH_DTYPE[odt]
                full = torch.full((M, ldc), 7, dtype=tdt, device=dev())
                c = full[:, :N]
                say(f"cr_gemm_e2m3_rowscale M={M} N={N} K_pad={Kp} out={odt} ldc={ldc} bias={with_bias}")
                rbl.cr_gemm_e2m3_rowscale(ad, sad, bd, sbd, c, bias=biasd if with_bias else None)
                torch.cuda.synchronize()
                fc = full.cpu()
                assert (fc[:, N:] == 7).all(), "columns past N were written"
                if odt == synth.DT_I32:
                    assert_bits_equal(fc[:, :N].numpy(), acc, "int32 accumulator")
                else:
                    ref = oracle.epilogue(acc, sa.numpy(), sb.numpy(), odt,
                                          bias=bias.numpy() if with_bias else None)
                    check_output(fc[:, :N], ref, odt, f"E2M3 GEMM out={odt} bias={with_bias}")


def test_gemm_e2m3_strided_operands_and_worst_case():
    """Quad strides beyond 3 K_pad on both operands; and the largest accepted K_pad with codes
    +-7 (|sum| = 49 * 133120 < 2^23: the fp32 sums stay exact)."""
    M, N, Kp = 300, 260, 1280
    g = torch.Generator().manual_seed(6)
    qa = torch.randint(-7, 8, (M, Kp), generator=g, dtype=torch.int32).to(torch.int8)
    qb = torch.randint(-7, 8, (N, Kp), generator=g, dtype=torch.int32).to(torch.int8)
    a = torch.from_numpy(oracle.pack_e2m3(qa.numpy()))
    b = torch.from_numpy(oracle.pack_e2m3(qb.numpy()))
    acc = oracle.gemm_e2m3(a.numpy(), b.numpy(), Kp, M, N)
    lf = 3 * Kp
    af = torch.full(((M + 3) // 4, lf + 48), 0x3F, dtype=torch.uint8)
    bf = torch.full(((N + 3) // 4, lf + 16), 0x3F, dtype=torch.uint8)
    af[:, :lf] = a
    bf[:, :lf] = b
    c = torch.empty(M, N, dtype=torch.int32, device=dev())
    say(f"cr_gemm_e2m3_rowscale strided lda={af.shape[1]} ldb={bf.shape[1]}")
    rbl.cr_gemm_e2m3_rowscale(af.to(dev())[:, :lf], None, bf.to(dev())[:, :lf], None, c, K_pad=Kp)
    torch.cuda.synchronize()
    assert_bits_equal(c.cpu().numpy(), acc, "int32 accumulator with row strides")

    Kp = rbl.CR_MAX_K_PAD
    qa = torch.full((3, Kp), 7, dtype=torch.int8)
    qa[1] = -7
    qa[2, ::2] = -7
    qb = torch.full((5, Kp), 7, dtype=torch.int8)
    qb[1] = -7
    qb[3, 1::2] = -7
    qb[4] = 0
    a = torch.from_numpy(oracle.pack_e2m3(qa.numpy()))
    b = torch.from_numpy(oracle.pack_e2m3(qb.numpy()))
    acc = oracle.gemm_e2m3(a.numpy(), b.numpy(), Kp, 3, 5)
    assert int(np.abs(acc).max()) == 49 * Kp
    say(f"cr_gemm_e2m3_rowscale worst-case accumulator K_pad={Kp}")
    c = torch.empty(3, 5, dtype=torch.int32, device=dev())
    rbl.cr_gemm_e2m3_rowscale(a.to(dev()), None, b.to(dev()), None, c)
    torch.cuda.synchronize()
    assert_bits_equal(c.cpu().numpy(), acc, "int32 accumulator at the K_pad limit")


@pytest.mark.parametrize("M,N,K,dt,swiglu,flags", L_CASES,
                         ids=[f"M{c[0]}-N{c[1]}-K{c[2]}-sw{int(c[4])}-f{c[5]}" for c in L_CASES])
def test_linear_w4a4_e2m3_against_oracle(M, N, K, dt, swiglu, flags):
    """The layer on the 6-bit matrix cores equals the oracle's W4A4 layer bit for bit (and
    so the nibble-form layer)."""
    wl = synth.Workload("w4a4", M, N, K, dt, (synth.DT_BF16,), M + N, swiglu=swiglu, outlier_frac=0.01)
    x = synth.make_activation(wl)
    g = torch.Generator().manual_seed(N * 5 + K)
    w = (torch.randn(N, (K + 7) // 8 * 8, generator=g) * 0.02).float()
    rp, rs = oracle.quant_weight_w4(w.numpy(), synth.DT_FP32, K)
    say(f"cr_quant_weight_w4_e2m3 for the layer N={N} K={K} flags={flags}")
    p, s = rbl.quant_weight_w4_e2m3(w.to(dev())[:, :K], K, flags=flags)
    bias = torch.randn(N, generator=torch.Generator().manual_seed(N)).float()
    xb = synth.bits_u16(x) if dt != synth.DT_FP32 else x.numpy()
    cols = x.shape[1]
    xpad = torch.zeros(M, (cols + 7) // 8 * 8 + 8, dtype=x.dtype)
    xpad[:, :cols] = x
    xd = xpad.to(dev())[:, :cols]
    for odt in (synth.DT_BF16, synth.DT_FP32):
        for with_bias in (False, True):
            say(f"cr_linear_w4a4_e2m3 M={M} N={N} K={K} swiglu={swiglu} flags={flags} out={odt} bias={with_bias}")
            y = rbl.linear_w4a4_e2m3(xd, p, s, K, out_dtype=synth.TORCH_DTYPE[odt], swiglu=swiglu,
                                     bias=bias.to(dev()) if with_bias else None, flags=flags)
            torch.cuda.synchronize()
            ref = oracle.linear_w4a4(xb, dt, K, swiglu, rp, rs, odt, bias=bias.numpy() if with_bias else None)
            check_output(y, ref, odt, f"W4A4 E2M3 layer out={odt} bias={with_bias}")


# ------------------------------------------------------ seeded random shapes ----
# M, N, K, dtypes, SwiGLU, order and bias drawn per case; activations with padded strides and
# garbage past the used columns; the nibble-form and E2M3-form layers, their activation codes
# and the GEMMs' int32 sums against the oracle, bit for bit.

def _rcase(i):
    r = np.random.default_rng(2000 + i)
    M = int(r.choice([1, 2, 7, 31, 33, 64, 65, 129, 257, 300]))
    N = int(r.choice([1, 5, 32, 100, 255, 256, 257, 513]))
    K = int(r.choice([1, 15, 17, 255, 256, 257, 1000, 5376, 16385, 20000]))
    xdt = int(r.choice([synth.DT_BF16, synth.DT_FP16, synth.DT_FP32]))
    odt = int(r.choice([synth.DT_BF16, synth.DT_FP16, synth.DT_FP32]))
    swiglu = bool(r.random() < 0.3)
    order = int(r.choice([0, BT]))
    with_bias = bool(r.random() < 0.4)
    return M, N, K, xdt, odt, swiglu, order, with_bias


R_CASES = [_rcase(i) for i in range(40)]


@pytest.mark.parametrize("case", R_CASES, ids=[f"M{c[0]}-N{c[1]}-K{c[2]}-x{c[3]}-o{c[4]}-sw{int(c[5])}-f{c[6]}-b{int(c[7])}"
                                              for c in R_CASES])
def test_random_shapes_both_forms(case):
    M, N, K, xdt, odt, swiglu, flags, with_bias = case
    seed = M * 7919 + N * 31 + K + 5
    g = torch.Generator().manual_seed(seed)
    cols = 2 * K if swiglu else K
    ld = (cols + 7) // 8 * 8 + 8
    x = torch.randn(M, ld, generator=g) * 1.5
    x[:, cols:] = 3e3
    x = x.to(DT_T[xdt])
    w = (torch.randn(N, (K + 7) // 8 * 8, generator=g) * 0.02).float()
    bias = torch.randn(N, generator=g).float() if with_bias else None
    xh = _host(x, xdt)
    rp, rs = oracle.quant_weight_w4(w.numpy(), synth.DT_FP32, K)
    ap, as_ = oracle.quant_act_w4(xh, xdt, K, swiglu=swiglu)
    ref = oracle.linear_w4a4(xh, xdt, K, swiglu, rp, rs, odt, bias=None if bias is None else bias.numpy())
    acc = oracle.gemm_s4s4(ap, rp, rp.shape[1] * 2)
    xd, wd = x.to(dev()), w.to(dev())[:, :K]
    bd = None if bias is None else bias.to(dev())
    say(f"W4A4 random case {case}")
    # nibble form
    p, s = rbl.quant_weight_w4(wd, K, flags=flags)
    q, qs = rbl.quant_act_w4(xd, K, swiglu=swiglu, flags=flags)
    y = rbl.linear_w4a4(xd, p, s, K, out_dtype=DT_T[odt], swiglu=swiglu, bias=bd, flags=flags)
    c = torch.empty(M, N, dtype=torch.int32, device=dev())
    rbl.cr_gemm_s4s4_rowscale(q, None, p, None, c)
    # E2M3 form
    p6, s6 = rbl.quant_weight_w4_e2m3(wd, K, flags=flags)
    q6, qs6 = rbl.quant_act_w4_e2m3(xd, K, swiglu=swiglu, flags=flags)
    y6 = rbl.linear_w4a4_e2m3(xd, p6, s6, K, out_dtype=DT_T[odt], swiglu=swiglu, bias=bd, flags=flags)
    c6 = torch.empty(M, N, dtype=torch.int32, device=dev())
    rbl.cr_gemm_e2m3_rowscale(q6, None, p6, None, c6)
    torch.cuda.synchronize()
    want_q = _bt_packed(ap) if flags & BT else ap
    assert_bits_equal(q.cpu().numpy(), want_q, "activation nibbles")
    assert_bits_equal(q6.cpu().numpy(), _e2m3(want_q), "activation E2M3 fields")
    assert_bits_equal(qs.cpu().numpy().view(np.uint32), as_.view(np.uint32), "activation scales")
    assert_bits_equal(qs6.cpu().numpy().view(np.uint32), as_.view(np.uint32), "activation scales (E2M3 call)")
    assert_bits_equal(c.cpu().numpy(), acc, "int32 sums, nibble form")
    assert_bits_equal(c6.cpu().numpy(), acc, "int32 sums, E2M3 form")
    check_output(y, ref, odt, "W4A4 layer, nibble form")
    check_output(y6, ref, odt, "W4A4 layer, E2M3 form")


def test_empty_extents_are_no_ops():
    """M = 0 or N = 0 through every W4A4 call: nothing written, no error."""
    x = torch.randn(4, 512, device=dev()).to(torch.bfloat16)
    w = torch.randn(8, 512, device=dev())
    p, s = rbl.quant_weight_w4(w, 512)
    p6, s6 = rbl.quant_weight_w4_e2m3(w, 512)
    out = torch.full((4, 8), 7.0, device=dev())
    say("W4A4 empty extents")
    for fn, wp, ws in ((rbl.cr_linear_w4a4, p, s), (rbl.cr_linear_w4a4_e2m3, p6, s6)):
        fn(x[:0], 512, False, wp, ws, out[:0], None)                  # no rows: no workspace needed
        fn(x, 512, False, wp[:0], ws[:0], out[:, :0], None)            # no columns
    q = torch.empty(0, 256, dtype=torch.uint8, device=dev())
    rbl.cr_quant_act_w4(x[:0], 512, False, q, torch.empty(0, device=dev()))
    rbl.cr_quant_act_w4_e2m3(x[:0], 512, False, torch.empty(0, 1536, dtype=torch.uint8, device=dev()),
                             torch.empty(0, device=dev()))
    torch.cuda.synchronize()
    assert (out == 7.0).all()
