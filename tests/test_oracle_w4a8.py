"""Pins of the oracle's W4A8 variant (4-bit rotated weights, 8-bit activations).

The pages name W4A8 among the ConvRot formats (ComfyUI Turing Utils README, opening
paragraph and section "Nodes", bullet "Load ConvRot DiT") but do not describe it; the oracle
takes the W8A8 method with 4-bit weight rows (levels -7..7, scale a/7).  Parity against the
pages' own W4A8 implementation is therefore unpinned; what is pinned here is that the
oracle computes that reading:

* packing: a hand-worked unit of 64 codes, and the round trip over all nibble values;
* quantizer: a closed-form row (reciprocal 1, ties to even), the error bound
  |y - q s| <= s/2, full use of +-7, zero rows, invariance under power-of-two scaling
  (tiny rows included: the 2^64 extension), and the reciprocal (not division) reading on
  rows where the two readings differ;
* weight path: weights built as Q s R (R the normalised Sylvester Hadamard matrix from
  scipy, Q integer codes, s a power of two) come back as exactly Q and s;
* GEMM: numpy int64 products of the unpacked codes;
* layer: the composition, and the error band of 4-bit rows.
"""
import numpy as np
import pytest
import scipy.linalg
import torch

import synth

H256 = scipy.linalg.hadamard(256).astype(np.float64)


def unpack_by_hand(p: np.ndarray, K_pad: int) -> np.ndarray:
    """The format, written from its definition: 32-byte units of 64 codes holding the groups
    of 16 codes G0, G2, G1, G3 in that order; in a group, byte j (0..3) holds codes j and
    4 + j, byte 4 + j codes 8 + j and 12 + j, low nibble first; two's complement nibbles."""
    n = p.shape[0]
    u = p[:, :K_pad // 2].reshape(n, K_pad // 64, 4, 8).astype(np.int16)
    u = u[:, :, [0, 2, 1, 3], :]                     # stored slot -> group: G0 G2 G1 G3
    lo, hi = u & 15, u >> 4
    nib = np.concatenate([lo[..., 0:4], hi[..., 0:4], lo[..., 4:8], hi[..., 4:8]], axis=3)
    return np.where(nib >= 8, nib - 16, nib).reshape(n, K_pad).astype(np.int8)


def test_pack_hand_worked_unit(orc):
    # one unit of 64 codes: G0 below, G1 all 1, G2 all -2, G3 all 3 (the rest of the row 0)
    g0 = [1, 2, 3, 4, -1, -2, -3, -4, 7, -7, 0, 5, 6, -6, -5, 3]
    q = np.zeros((1, 256), np.int8)
    q[0, :64] = g0 + [1] * 16 + [-2] * 16 + [3] * 16
    p = orc.pack_s4(q)
    assert p.shape == (1, 128)
    assert p[0, :32].tolist() == ([0xF1, 0xE2, 0xD3, 0xC4, 0x67, 0xA9, 0xB0, 0x35]   # G0
                                  + [0xEE] * 8                                       # G2: -2 = 0xE
                                  + [0x11] * 8                                       # G1
                                  + [0x33] * 8)                                      # G3
    assert (p[0, 32:] == 0).all()


def test_pack_round_trip(orc):
    rng = np.random.default_rng(0)
    q = rng.integers(-8, 8, (5, 512), dtype=np.int8)
    p = orc.pack_s4(q)
    assert p.shape == (5, 256)
    assert np.array_equal(orc.unpack_s4(p, 512), q)
    assert np.array_equal(unpack_by_hand(p, 512), q)


def test_quantizer_closed_form_row(orc):
    # a = 7 gives r = 7/7 = 1 exactly, so q = rint(y) with ties to even, s = 1
    y = np.zeros((1, 256), np.float32)
    y[0, :8] = [7.0, 2.5, 3.5, -0.5, 1.5, -2.5, 0.49999997, 6.5]
    q, s = orc.row_quant_s4(y)
    assert s[0] == 1.0
    assert q[0, :8].tolist() == [7, 2, 4, 0, 2, -2, 0, 6]
    assert (q[0, 8:] == 0).all()


def test_quantizer_bound_range_zero_rows(orc):
    rng = np.random.default_rng(1)
    y = (rng.standard_normal((64, 768)) * rng.uniform(1e-3, 1e3, (64, 1))).astype(np.float32)
    y[5] = 0.0
    q, s = orc.row_quant_s4(y)
    assert s[5] == 0.0 and (q[5] == 0).all()
    live = np.arange(64) != 5
    assert (np.abs(q[live]).max(axis=1) == 7).all()
    assert np.abs(q).max() <= 7
    err = np.abs(y.astype(np.float64) - q.astype(np.float64) * s[:, None].astype(np.float64))
    assert (err[live] <= s[live, None] / 2 * (1 + 2.0 ** -20)).all()
    # s = a / 7 with a the row maximum, one rounding
    a = np.abs(y).max(axis=1)
    assert np.array_equal(s[live], (a[live] / np.float32(7.0)).astype(np.float32))


@pytest.mark.parametrize("j", [-135, -120, -30, -7, 5, 40])
def test_quantizer_power_of_two_invariance(orc, j):
    # rows of multiples of 2^-10 below 2^1: every scaled copy down to 2^-145 is exact, so
    # j = -135 reaches rows whose 7/a overflows (the 2^64 extension) and j = -120 rows whose
    # scale is subnormal
    rng = np.random.default_rng(2)
    y = (rng.integers(-2000, 2001, (16, 512)) * 2.0 ** -10).astype(np.float32)
    q, s = orc.row_quant_s4(y)
    y2 = (y.astype(np.float64) * 2.0 ** j).astype(np.float32)
    assert np.array_equal(y2.astype(np.float64), y.astype(np.float64) * 2.0 ** j), "scaling must be exact"
    q2, s2 = orc.row_quant_s4(y2)
    assert np.array_equal(q2, q)
    if j > -100:                                   # s2 normal: s scales exactly
        assert np.array_equal(s2.astype(np.float64), s.astype(np.float64) * 2.0 ** j)


def test_quantizer_takes_the_rounded_reciprocal(orc):
    """q = rint(y * RN(7/a)), not rint(RN(7 y / a)): values placed within a few ulps of the
    half-integer code boundaries, where the two readings (evaluated in float64 with explicit
    binary32 roundings) give different codes for some of them; the oracle gives the first."""
    rng = np.random.default_rng(3)
    for _ in range(50):
        a = np.float32(rng.uniform(1.0, 2.0))
        r = np.float32(np.float64(7.0) / np.float64(a))
        ys = []
        for k in range(7):
            y0 = np.float32((k + 0.5) * np.float64(a) / 7.0)
            for d in range(-4, 5):
                ys.append(np.float32(y0 + np.float32(d) * np.spacing(y0)))
        y = np.array([a] + ys + [-v for v in ys], np.float32)
        recip = np.rint((y.astype(np.float64) * np.float64(r)).astype(np.float32).astype(np.float64))
        div = np.rint((7.0 * y.astype(np.float64) / np.float64(a)).astype(np.float32).astype(np.float64))
        if (recip != div).any():
            row = np.zeros((1, 256), np.float32)
            row[0, :len(y)] = y
            q, _ = orc.row_quant_s4(row)
            assert np.array_equal(q[0, :len(y)].astype(np.float64), np.clip(recip, -7, 7))
            assert not np.array_equal(q[0, :len(y)].astype(np.float64), np.clip(div, -7, 7))
            return
    raise AssertionError("no row where the two readings differ was found")


def _exact_weight(N, K_pad, seed, s_exp=-6):
    """W = (Q s) R block by block, R = H/16: its rotation is exactly Q s."""
    rng = np.random.default_rng(seed)
    Q = rng.integers(-7, 8, (N, K_pad)).astype(np.int8)
    Q[np.arange(N), rng.integers(0, K_pad, N)] = 7          # every row reaches the top level
    s = 2.0 ** s_exp
    W = np.zeros((N, K_pad))
    for b in range(0, K_pad, 256):
        W[:, b:b + 256] = (Q[:, b:b + 256].astype(np.float64) * s) @ (H256 / 16.0)
    W32 = W.astype(np.float32)
    assert np.array_equal(W32.astype(np.float64), W)            # exactly representable
    return Q, np.float32(s), W32


def test_weight_path_recovers_exact_codes(orc):
    for K_pad in (256, 768):
        Q, s, W = _exact_weight(40, K_pad, K_pad)
        p, sc = orc.quant_weight_w4(W, synth.DT_FP32, K_pad)
        assert p.shape == (40, K_pad // 2)
        assert np.array_equal(unpack_by_hand(p, K_pad), Q)
        assert (sc == s).all()


def test_weight_path_pads_k_and_ignores_garbage(orc):
    rng = np.random.default_rng(4)
    w = rng.standard_normal((9, 320)).astype(np.float32)
    w_garbage = w.copy()
    w_garbage[:, 300:] = 1e6
    p1, s1 = orc.quant_weight_w4(w[:, :300].copy(), synth.DT_FP32, 300)
    p2, s2 = orc.quant_weight_w4(w_garbage, synth.DT_FP32, 300)
    assert p1.shape == (9, 256)
    assert np.array_equal(p1, p2) and np.array_equal(s1, s2)


def test_gemm_s8s4_int64_brute_force(orc):
    rng = np.random.default_rng(5)
    for (M, N, K_pad) in [(1, 1, 256), (7, 13, 512), (33, 65, 1280)]:
        a = rng.integers(-127, 128, (M, K_pad), dtype=np.int8)
        q = rng.integers(-7, 8, (N, K_pad), dtype=np.int8)
        p = orc.pack_s4(q)
        ref = a.astype(np.int64) @ q.astype(np.int64).T
        assert np.array_equal(orc.gemm_s8s4(a, p).astype(np.int64), ref)


def test_layer_composition_and_error_band(orc):
    """The layer equals its steps; against the float64 product x W^T its error is the band
    of 4-bit rows of Gaussian weights (step a/7 with a about 4 sigma: roughly 16 %)."""
    g = torch.Generator().manual_seed(6)
    M, N, K = 96, 320, 1000
    x = torch.randn(M, K, generator=g).to(torch.bfloat16)
    w = (0.02 * torch.randn(N, K, generator=g)).float()
    xb = synth.bits_u16(x)
    p, sw = orc.quant_weight_w4(w.numpy(), synth.DT_FP32, K)
    y = orc.linear_w4a8(xb, synth.DT_BF16, K, False, p, sw, synth.DT_FP32)
    qx, sx = orc.quant_act(xb, synth.DT_BF16, K)
    acc = orc.gemm_s8s4(qx, p)
    assert np.array_equal(y, orc.epilogue(acc, sx, sw, synth.DT_FP32))
    ref = x.double().numpy() @ w.double().numpy().T
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert 0.10 < rel < 0.22, rel
    # with the 8-bit weights of the same values the error is an order of magnitude lower
    from oracle import act_load, convrot256, row_quant
    q8, s8 = row_quant(convrot256(act_load(w.numpy(), synth.DT_FP32, K)))
    y8 = orc.epilogue(orc.gemm_s8(qx, q8), sx, s8, synth.DT_FP32)
    assert np.linalg.norm(y8 - ref) / np.linalg.norm(ref) < rel / 5


# ------------------------------------------------------------------ W4A4 ----
# The README's third ConvRot format, W4A4, read the same way: 4-bit rows on both sides.

def test_w4a4_activation_path_recovers_exact_codes(orc):
    """Activations built as Q s R come back as exactly Q and s (the weight pin above, through
    the activation loader, bf16 input: the values below are exact in bf16)."""
    Q, s, X = _exact_weight(24, 512, 9, s_exp=-3)
    xb = torch.from_numpy(X).to(torch.bfloat16)
    assert np.array_equal(xb.float().numpy(), X)
    p, sc = orc.quant_act_w4(synth.bits_u16(xb), synth.DT_BF16, 512)
    assert np.array_equal(unpack_by_hand(p, 512), Q)
    assert (sc == s).all()


def test_w4a4_swiglu_is_swiglu_then_4bit_rows(orc):
    rng = np.random.default_rng(10)
    h = rng.standard_normal((6, 600)).astype(np.float32)
    p, s = orc.quant_act_w4(h, synth.DT_FP32, 300, swiglu=True)
    y = orc.convrot256(orc.act_load(h, synth.DT_FP32, 300, swiglu=True))
    q, s2 = orc.row_quant_s4(y)
    assert np.array_equal(unpack_by_hand(p, 512), q) and np.array_equal(s, s2)


def test_gemm_s4s4_int64_brute_force(orc):
    rng = np.random.default_rng(11)
    for (M, N, K_pad) in [(1, 1, 256), (9, 17, 768)]:
        qa = rng.integers(-7, 8, (M, K_pad), dtype=np.int8)
        qb = rng.integers(-7, 8, (N, K_pad), dtype=np.int8)
        ref = qa.astype(np.int64) @ qb.astype(np.int64).T
        assert np.array_equal(orc.gemm_s4s4(orc.pack_s4(qa), orc.pack_s4(qb), K_pad).astype(np.int64), ref)


def test_w4a4_layer_composition_and_error_band(orc):
    """The layer equals its steps; its error against the float64 product is that of 4-bit
    rows on both sides (above the W4A8 band), and the rotation still helps when the
    activations carry outlier channels."""
    g = torch.Generator().manual_seed(12)
    M, N, K = 96, 320, 1024
    x = torch.randn(M, K, generator=g)
    x[:, torch.randperm(K, generator=g)[:10]] *= 20.0            # outlier channels
    x = x.to(torch.bfloat16)
    w = (0.02 * torch.randn(N, K, generator=g)).float()
    xb = synth.bits_u16(x)
    p, sw = orc.quant_weight_w4(w.numpy(), synth.DT_FP32, K)
    y = orc.linear_w4a4(xb, synth.DT_BF16, K, False, p, sw, synth.DT_FP32)
    px, sx = orc.quant_act_w4(xb, synth.DT_BF16, K)
    assert np.array_equal(y, orc.epilogue(orc.gemm_s4s4(px, p, K), sx, sw, synth.DT_FP32))
    ref = x.double().numpy() @ w.double().numpy().T
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    y48 = orc.linear_w4a8(xb, synth.DT_BF16, K, False, p, sw, synth.DT_FP32)
    rel48 = np.linalg.norm(y48 - ref) / np.linalg.norm(ref)
    assert rel48 < rel < 0.5, (rel48, rel)
    # the same 4-bit rows without the rotation (plain per-row absmax/7 on both operands)
    def plain(v):
        a = np.abs(v).max(axis=1, keepdims=True)
        return np.clip(np.rint(v / a * 7), -7, 7), a / 7
    qa, sa = plain(x.double().numpy())
    qw, sww = plain(w.double().numpy())
    rel_plain = np.linalg.norm((qa @ qw.T) * sa * sww.T - ref) / np.linalg.norm(ref)
    assert rel < rel_plain / 1.5, (rel, rel_plain)
