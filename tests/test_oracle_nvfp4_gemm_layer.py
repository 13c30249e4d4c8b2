"""Pins of the oracle's NVFP4 decode, int32 GEMM, epilogue and the composed layer.

NVFP4 (modelpad.app glossary: a 4-bit float format that needs scale factors; the README
keeps weights packed and decodes them for the S8 route): a hand-worked packed row,
exactness for power-of-two global scales (checked against a float64 decode built from
torch's E4M3 conversion), agreement with the synthetic checkpoint encoder (nearest value,
idempotence) and indifference to serialized padding.
GEMM: numpy int64 matmul.  Epilogue: float64 product within binary32 rounding, then
torch/numpy narrowing.  Layer: composition, rotation invariance and the error band the
pages print for this route (tests/golden/pages_accuracy.txt).
"""
import os

import numpy as np
import pytest
import torch

import synth

E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6])
E4M3 = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def decode_f64(codes, sf, g, K):
    """float64 reference decode (exact when g is a power of two)."""
    n = codes.shape[0]
    kp = 256 * ((K + 255) // 256)
    k = np.arange(K)
    byte = codes[:, k // 2]
    nib = np.where(k % 2 == 0, byte & 15, byte >> 4)
    w = np.zeros((n, kp))
    w[:, :K] = E2M1[nib] * E4M3[sf[:, k // 16]] * g
    return w


def test_decode_hand_worked_row(orc):
    # K = 3: byte 0 = 0x92 -> k0 code 2 (1.0), k1 code 9 (-0.5); byte 1 = 0xF7 -> k2 code 7 (6.0),
    # the high nibble is padding.  Scale byte 0x40 = 2^(8-7) = 2.0, g = 0.25.
    codes = np.array([[0x92, 0xF7] + [0xAB] * 14], np.uint8)
    sf = np.array([[0x40] + [0x7F] * 15], np.uint8)     # padding scales are NaN bytes: ignored
    w = orc.nvfp4_decode(codes, sf, 0.25, 3)
    assert w.shape == (1, 256)
    assert w[0, :3].tolist() == [0.5, -0.25, 3.0]
    assert (w[0, 3:] == 0).all()


def test_decode_exact_for_power_of_two_g(orc):
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 256, (32, 160), dtype=np.uint8)
    sf = rng.integers(0, 0x7F, (32, 32), dtype=np.uint8)   # finite positive E4M3 bytes
    for g in (1.0, 2.0 ** -7, 2.0 ** 5):
        for K in (320, 300, 17):
            got = orc.nvfp4_decode(codes, sf, g, K).astype(np.float64)
            assert np.array_equal(got, decode_f64(codes, sf, g, K))


def _all_codes_all_scales():
    """Rows of 16 elements holding codes 0..15 in order (byte j = code 2j | code 2j+1 << 4),
    one row per finite E4M3 scale byte (every byte but 0x7F and 0xFF, the NaNs)."""
    scales = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], np.uint8)
    row = np.array([(2 * j) | ((2 * j + 1) << 4) for j in range(8)], np.uint8)
    codes = np.tile(row, (len(scales), 1))
    return codes, scales[:, None].copy()


# global scales that are not powers of two: decimal fractions, 1/3, one that puts products
# in the subnormal range, one near the top of the range (largest products overflow to inf),
# and the synthetic encoder's g for a 0.02 * N(0, 1) weight
NON_DYADIC_G = [np.float32(0.0137), np.float32(1.0 / 3.0), np.float32(3.3e-43 * 1e4), np.float32(1.7e-41),
                np.float32(1.9e35), np.float32(7.1e-37)]


def _encoder_g():
    w = 0.02 * torch.randn(64, 512, generator=torch.Generator().manual_seed(0))
    return np.float32(synth.nvfp4_encode(w).g)


def test_decode_non_dyadic_g_is_one_rounding_of_the_exact_product(orc):
    """value = fp32(E2M1 * E4M3) * g with the first product exact (at most 2 + 4 significant
    bits), so the decode is the exact product E2M1 * E4M3 * g rounded once to binary32.  That
    product has at most 2 + 4 + 24 significant bits and is exact in float64; numpy's float64
    -> float32 cast rounds it to nearest even, subnormals and overflow included.  E2M1 comes
    from its closed form, E4M3 from torch's float8_e4m3fn; every code (with -0, code 8) meets
    every finite scale byte (negative and subnormal ones included)."""
    codes, sf = _all_codes_all_scales()
    gs = NON_DYADIC_G + [_encoder_g()]
    assert all(np.frexp(np.float64(g))[0] != 0.5 for g in gs), "every g must be a non-power of two"
    for g in gs:
        dec = orc.nvfp4_decode(codes, sf, float(g), 16)[:, :16]
        exact = E2M1[None, :] * E4M3[sf[:, 0]][:, None] * np.float64(g)      # exact in float64
        with np.errstate(over="ignore"):
            want = exact.astype(np.float32)
        assert np.array_equal(dec.view(np.uint32), want.view(np.uint32)), f"g={g!r}"
        # zero codes give +-0 with the sign of the product (code 8 is -0)
        assert np.array_equal(np.signbit(dec[:, 8]), np.signbit(want[:, 8]))


def test_decode_pin_rejects_double_rounding(orc):
    """The pin above has teeth: E2M1 * (E4M3 * g), which rounds the scale product first,
    differs from one rounding of the exact product for some code, scale byte and g above."""
    codes, sf = _all_codes_all_scales()
    e2m1 = E2M1.astype(np.float32)
    differs = 0
    for g in NON_DYADIC_G:
        with np.errstate(over="ignore"):
            wrong = e2m1[None, :] * (E4M3[sf[:, 0]].astype(np.float32)[:, None] * np.float32(g))
            want = (E2M1[None, :] * E4M3[sf[:, 0]][:, None] * np.float64(g)).astype(np.float32)
        differs += int(np.count_nonzero(wrong.view(np.uint32) != want.view(np.uint32)))
    assert differs > 0


def test_decode_matches_synthetic_encoder(orc):
    g0 = torch.Generator().manual_seed(7)
    w = 0.02 * torch.randn(64, 1000, generator=g0)
    p = synth.nvfp4_encode(w, garbage_seed=11)
    dec = orc.nvfp4_decode(p.codes.numpy(), p.sf.numpy(), p.g, 1000).astype(np.float64)
    assert (dec[:, 1000:] == 0).all()
    # every decoded value is the nearest grid value of its block: error <= half the largest step
    scale = E4M3[p.sf.numpy()[:, np.arange(1000) // 16]] * p.g
    err = np.abs(dec[:, :1000] - w.double().numpy())
    assert (err <= scale * 1.0 + 1e-12).all()                     # max E2M1 step is 2
    rel = np.linalg.norm(dec[:, :1000] - w.double().numpy()) / np.linalg.norm(w.double().numpy())
    assert 0.05 < rel < 0.15                                      # 4-bit grid: ~9% relative error
    # idempotence: re-encoding decoded values reproduces them exactly
    p2 = synth.nvfp4_encode(torch.from_numpy(dec[:, :1000]).float())
    dec2 = orc.nvfp4_decode(p2.codes.numpy(), p2.sf.numpy(), p2.g, 1000).astype(np.float64)
    assert p2.g == p.g          # the largest element is a grid value, so amax is unchanged
    assert np.array_equal(dec2, dec)


def test_decode_ignores_serialized_padding(orc):
    g0 = torch.Generator().manual_seed(8)
    w = 0.02 * torch.randn(16, 301, generator=g0)
    a = synth.nvfp4_encode(w, ld_codes=192, ld_sf=48, garbage_seed=1)
    b = synth.nvfp4_encode(w, ld_codes=192, ld_sf=48, garbage_seed=2)
    assert not torch.equal(a.codes, b.codes)
    da = orc.nvfp4_decode(a.codes.numpy(), a.sf.numpy(), a.g, 301)
    db = orc.nvfp4_decode(b.codes.numpy(), b.sf.numpy(), b.g, 301)
    assert np.array_equal(da, db)
    qa, sa = orc.prep_weight_nvfp4(a.codes.numpy(), a.sf.numpy(), a.g, 301)
    qb, sb = orc.prep_weight_nvfp4(b.codes.numpy(), b.sf.numpy(), b.g, 301)
    assert np.array_equal(qa, qb) and np.array_equal(sa, sb)


def test_gemm_int64_brute_force(orc):
    rng = np.random.default_rng(1)
    for (M, N, K) in [(1, 1, 256), (7, 13, 512), (33, 65, 768)]:
        a = rng.integers(-127, 128, (M, K), dtype=np.int8)
        b = rng.integers(-127, 128, (N, K), dtype=np.int8)
        ref = a.astype(np.int64) @ b.astype(np.int64).T
        assert np.array_equal(orc.gemm_s8(a, b).astype(np.int64), ref)
    a = np.full((2, 133120), 127, np.int8)          # largest K_pad without int32 overflow
    assert orc.gemm_s8(a, -a)[0, 0] == -(127 * 127 * 133120)


def test_epilogue(orc):
    rng = np.random.default_rng(2)
    acc = rng.integers(-2 ** 24, 2 ** 24, (9, 11)).astype(np.int32)
    sx = rng.uniform(1e-4, 1e-1, 9).astype(np.float32)
    sw = rng.uniform(1e-5, 1e-2, 11).astype(np.float32)
    f32 = orc.epilogue(acc, sx, sw, synth.DT_FP32)
    ref = acc.astype(np.float64) * sx[:, None].astype(np.float64) * sw[None, :].astype(np.float64)
    assert np.abs(f32 - ref).max() <= np.abs(ref).max() * 2.0 ** -22
    bf = orc.epilogue(acc, sx, sw, synth.DT_BF16)
    assert np.array_equal(bf, torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    hf = orc.epilogue(acc, sx, sw, synth.DT_FP16)
    assert np.array_equal(hf, f32.astype(np.float16).view(np.uint16))
    assert np.array_equal(orc.epilogue(acc, sx, sw, synth.DT_I32), acc)


def _layer_parts(orc, x_bits, x_dtype, K, swiglu, wt):
    qx, sx = orc.quant_act(x_bits, x_dtype, K, swiglu)
    qw, sw = orc.prep_weight_nvfp4(wt.codes.numpy(), wt.sf.numpy(), wt.g, K)
    return qx, sx, qw, sw


def test_layer_is_composition_of_steps(orc):
    w = synth.WORKLOADS["tiny"]
    x = synth.make_activation(w)
    wt = synth.make_weight_nvfp4(w)
    xb = synth.bits_u16(x)
    qx, sx, qw, sw = _layer_parts(orc, xb, w.x_dtype, w.K, False, wt)
    ref = orc.epilogue(orc.gemm_s8(qx, qw), sx, sw, synth.DT_BF16)
    out = orc.linear_nvfp4(xb, w.x_dtype, w.K, False, wt.codes.numpy(), wt.sf.numpy(), wt.g, synth.DT_BF16)
    assert np.array_equal(out, ref)
    # activation preparation is the chain load -> rotate -> quantize
    q2, s2 = orc.row_quant(orc.convrot256(orc.act_load(xb, w.x_dtype, w.K)))
    assert np.array_equal(q2, qx) and np.array_equal(s2, sx)


def test_k_padding_and_ld_garbage(orc):
    rng = np.random.default_rng(3)
    K = 300
    x = torch.from_numpy(rng.standard_normal((8, 320)).astype(np.float32)).to(torch.bfloat16)
    xb = synth.bits_u16(x)
    x_clean = xb.copy()
    x_clean[:, K:] = 0
    q1, s1 = orc.quant_act(xb, synth.DT_BF16, K)          # row stride 320, garbage past K
    q2, s2 = orc.quant_act(np.ascontiguousarray(x_clean[:, :K]), synth.DT_BF16, K)
    assert q1.shape == (8, 512)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)
    assert np.array_equal(orc.act_load(xb, synth.DT_BF16, K)[:, K:], np.zeros((8, 512 - K), np.float32))


def test_swiglu_activation_halves(orc):
    rng = np.random.default_rng(4)
    F = 256
    h = torch.from_numpy(rng.standard_normal((4, 2 * F)).astype(np.float32)).to(torch.bfloat16)
    got = orc.act_load(synth.bits_u16(h), synth.DT_BF16, F, swiglu=True).astype(np.float64)
    hd = h.double()
    ref = (torch.nn.functional.silu(hd[:, :F]) * hd[:, F:]).numpy()
    assert np.allclose(got, ref, rtol=1e-6, atol=1e-12)


def test_zero_and_tiny_rows(orc):
    w = synth.Workload("t", 16, 256, 600, synth.DT_FP16, (synth.DT_FP16,), 9,
                       zero_row_frac=0.125, tiny_row_frac=0.125)
    x = synth.make_activation(w)
    zero, tiny = synth.special_rows(w)
    assert len(zero) == 2 and len(tiny) == 2
    xb = synth.bits_u16(x)
    qx, sx = orc.quant_act(xb, w.x_dtype, w.K)
    assert (sx[zero.numpy()] == 0).all() and (qx[zero.numpy()] == 0).all()
    assert (sx[tiny.numpy()] > 0).all() and (np.abs(qx[tiny.numpy()]).max(axis=1) == 127).all()
    wt = synth.make_weight_nvfp4(w)
    out = orc.linear_nvfp4(xb, w.x_dtype, w.K, False, wt.codes.numpy(), wt.sf.numpy(), wt.g, synth.DT_FP32)
    assert (out[zero.numpy()] == 0).all()


def _pages_band():
    path = os.path.join(os.path.dirname(__file__), "golden", "pages_accuracy.txt")
    vals = {}
    for line in open(path):
        if line.strip() and not line.startswith("#"):
            k, v = line.split()
            vals[k] = float(v)
    return vals


@pytest.mark.parametrize("kind", ["qkv", "ffn_down", "longk"])
def test_error_band_vs_decoded_weights(orc, kind):
    """Relative L2 of the quantized route against the fp64 product with the decoded NVFP4
    weights lies near the pages' 1.31% / 1.39% (plausibility, not parity), and rotation
    beats the unrotated control when outlier channels are present."""
    band = _pages_band()
    base = synth.WORKLOADS[kind]
    w = synth.Workload(kind + "_small", 256, 512, base.K, base.x_dtype, (synth.DT_FP32,), base.seed,
                       swiglu=base.swiglu, outlier_frac=base.outlier_frac)
    x = synth.make_activation(w)
    wt = synth.make_weight_nvfp4(w)
    xb = synth.bits_u16(x)
    out = orc.linear_nvfp4(xb, w.x_dtype, w.K, w.swiglu, wt.codes.numpy(), wt.sf.numpy(), wt.g,
                           synth.DT_FP32).astype(np.float64)
    xf = orc.act_load(xb, w.x_dtype, w.K, w.swiglu).astype(np.float64)
    wd = orc.nvfp4_decode(wt.codes.numpy(), wt.sf.numpy(), wt.g, w.K).astype(np.float64)
    ref = xf @ wd.T
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert 0.010 < rel < 0.016, rel
    assert abs(rel - band["ffn_down" if w.swiglu else "qkv"]) < 0.004
    # unrotated control: same quantizer without ConvRot256
    qx, sx = orc.row_quant(xf.astype(np.float32))
    qw, sw = orc.row_quant(wd.astype(np.float32))
    ctl = orc.epilogue(orc.gemm_s8(qx, qw), sx, sw, synth.DT_FP32).astype(np.float64)
    rel_ctl = np.linalg.norm(ctl - ref) / np.linalg.norm(ref)
    if w.outlier_frac > 0:
        assert rel_ctl > 2.5 * rel
