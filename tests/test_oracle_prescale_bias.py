"""Pins of the oracle's channel pre-scale and epilogue bias.

Channel pre-scale (ComfyUI Turing Utils README, "Load ConvRot DiT ..." bullet: pre-scales
and SwiGLU run before the rotation, and channel pre-scales keep the unfused order): the
layer input's channel k is multiplied by c[k] after loading (after SwiGLU for the fused
FFN-down input) and before the rotation.  Pinned by brute force on integer rows with
power-of-two scales (everything exact, the rotation taken from scipy's Hadamard matrix and
the quantizer re-derived in numpy float32), by the fused-equals-unfused ordering the pages
state, and by power-of-two invariance.

Bias (MiniMax H3 explainer, "Foundations": y = x W^T + b; glossary "Epilogue": bias fused
at the end of the GEMM): out = ((acc * s_x) * s_w) + b[n] in binary32, then one rounding to
the output type.  Pinned by a closed-form exact case, a float64 error bound and the
zero-bias identity.
"""
import numpy as np
import scipy.linalg

import oracle
import synth

H256 = scipy.linalg.hadamard(256).astype(np.int64)


def _quant_rows_numpy(y: np.ndarray):
    """Row quantization re-derived with numpy float32 operations (one rounding each)."""
    q = np.zeros(y.shape, np.int8)
    s = np.zeros(y.shape[0], np.float32)
    for m in range(y.shape[0]):
        a = np.float32(np.abs(y[m]).max())
        if a == 0:
            continue
        s[m] = np.float32(a / np.float32(127))
        r = np.float32(np.float32(127) / a)
        q[m] = np.clip(np.rint((y[m] * r).astype(np.float32)), -127, 127).astype(np.int8)
    return q, s


def test_prescale_brute_force_channelwise_before_rotation():
    rng = np.random.default_rng(11)
    M, K = 5, 300                                   # K_pad 512: a partial second block
    x = rng.integers(-100, 101, (M, K)).astype(np.float32)
    c = (2.0 ** rng.integers(-2, 3, K)).astype(np.float32)       # per-channel powers of two
    q, s = oracle.quant_act(x, oracle.DT_FP32, K, pre_scale=c)
    # exact reference: (x * c) padded, times H / 16 per 256-block, all exact in int64 / 4
    xc4 = np.zeros((M, 512), np.int64)
    xc4[:, :K] = (x.astype(np.float64) * c * 4).astype(np.int64)   # c >= 1/4: integers
    y = np.concatenate([(xc4[:, b * 256:(b + 1) * 256] @ H256) for b in range(2)], axis=1)
    y = (y.astype(np.float64) / 64.0).astype(np.float32)          # / 4 / 16, exact
    rq, rs = _quant_rows_numpy(y)
    assert np.array_equal(q, rq)
    assert np.array_equal(s.view(np.uint32), rs.view(np.uint32))
    # the pre-scale changes the codes, and the same scales applied after the rotation
    # (to the rotated columns) give other codes than applying them before it
    q_none, _ = oracle.quant_act(x, oracle.DT_FP32, K)
    assert not np.array_equal(q, q_none)
    x4 = np.zeros((M, 512), np.int64)
    x4[:, :K] = (x * 4).astype(np.int64)
    y_after = np.concatenate([(x4[:, b * 256:(b + 1) * 256] @ H256) for b in range(2)], axis=1)
    c_pad = np.ones(512)
    c_pad[:K] = c
    y_after = (y_after.astype(np.float64) * c_pad / 64.0).astype(np.float32)
    q_after, _ = _quant_rows_numpy(y_after)
    assert not np.array_equal(q, q_after)


def test_prescale_after_swiglu_matches_unfused_order():
    rng = np.random.default_rng(12)
    M, F = 4, 700
    h = rng.standard_normal((M, 2 * F)).astype(np.float32)
    c = rng.uniform(0.3, 3.0, F).astype(np.float32)               # not powers of two
    fused_q, fused_s = oracle.quant_act(h, oracle.DT_FP32, F, swiglu=True, pre_scale=c)
    sw = oracle.swiglu(h[:, :F], h[:, F:])                        # unfused: SwiGLU first,
    unf_q, unf_s = oracle.quant_act(sw, oracle.DT_FP32, F, pre_scale=c)   # then the pre-scale
    assert np.array_equal(fused_q, unf_q)
    assert np.array_equal(fused_s.view(np.uint32), unf_s.view(np.uint32))
    # scaling the value half instead (before the product) is a different operation: on a
    # row where value * c overflows but (swish(gate) * value) * c does not, only the
    # SwiGLU-first order keeps a finite row scale
    h1 = np.zeros((1, 2 * F), np.float32)
    h1[0, 0], h1[0, F] = -2.0, 3e38
    c1 = np.ones(F, np.float32)
    c1[0] = 4.0
    _, s_first = oracle.quant_act(h1, oracle.DT_FP32, F, swiglu=True, pre_scale=c1)
    hv = h1.copy()
    with np.errstate(over="ignore"):
        hv[0, F] = np.float32(hv[0, F]) * np.float32(4.0)      # inf
    _, s_value = oracle.quant_act(hv, oracle.DT_FP32, F, swiglu=True)
    assert np.isfinite(s_first[0]) and not np.isfinite(s_value[0])


def test_prescale_uniform_power_of_two_scales_only_the_row_scale():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((6, 1000)).astype(np.float32)
    q0, s0 = oracle.quant_act(x, oracle.DT_FP32, 1000)
    for j in (-3, 1, 5):
        c = np.full(1000, 2.0 ** j, np.float32)
        q, s = oracle.quant_act(x, oracle.DT_FP32, 1000, pre_scale=c)
        assert np.array_equal(q, q0)
        assert np.array_equal(s, (s0 * np.float32(2.0 ** j)).astype(np.float32))
    ones = np.ones(1000, np.float32)
    q1, s1 = oracle.quant_act(x, oracle.DT_FP32, 1000, pre_scale=ones)
    assert np.array_equal(q1, q0) and np.array_equal(s1.view(np.uint32), s0.view(np.uint32))


def test_prescale_step_leaves_padding_zero():
    buf = np.zeros((2, 512), np.float32)
    buf[:, :300] = 1.5
    out = oracle.act_prescale(buf, 300, np.full(300, 2.0, np.float32))
    assert np.all(out[:, :300] == 3.0) and np.all(out[:, 300:] == 0.0)


def test_bias_closed_form_exact():
    acc = np.array([[3, -5, 0, 1 << 20]], np.int32)
    sx = np.array([0.25], np.float32)
    sw = np.array([2.0, 0.5, 8.0, 2.0 ** -10], np.float32)
    b = np.array([1.0, -0.375, 3.0, -1.0], np.float32)
    out = oracle.epilogue(acc, sx, sw, oracle.DT_FP32, bias=b)
    assert np.array_equal(out, np.array([[2.5, -1.0, 3.0, 255.0]], np.float32))
    out16 = oracle.epilogue(acc, sx, sw, oracle.DT_BF16, bias=b)
    assert np.array_equal(out16, np.array([[0x4020, 0xBF80, 0x4040, 0x437F]], np.uint16))


def test_bias_float64_bound_and_zero_bias():
    rng = np.random.default_rng(14)
    M, N = 40, 70
    acc = rng.integers(-2 ** 20, 2 ** 20, (M, N)).astype(np.int32)
    sx = rng.uniform(1e-4, 1e-2, M).astype(np.float32)
    sw = rng.uniform(1e-4, 1e-2, N).astype(np.float32)
    b = rng.standard_normal(N).astype(np.float32)
    out = oracle.epilogue(acc, sx, sw, oracle.DT_FP32, bias=b).astype(np.float64)
    ref = acc.astype(np.float64) * sx[:, None] * sw[None, :] + b[None, :]
    prod = np.abs(acc.astype(np.float64) * sx[:, None] * sw[None, :])
    bound = (prod * 2.0 ** -23) + np.abs(ref) * 2.0 ** -24 + 1e-30
    assert np.all(np.abs(out - ref) <= bound)
    # a bias added to the wrong axis (m instead of n) breaks the bound
    wrong = acc.astype(np.float64) * sx[:, None] * sw[None, :] + b[:M, None]
    assert not np.all(np.abs(out - wrong) <= bound)
    # zero bias: identical values (nonzero accumulators, so no signed-zero question)
    acc_nz = np.where(acc == 0, 1, acc).astype(np.int32)
    o0 = oracle.epilogue(acc_nz, sx, sw, oracle.DT_BF16)
    oz = oracle.epilogue(acc_nz, sx, sw, oracle.DT_BF16, bias=np.zeros(N, np.float32))
    assert np.array_equal(o0, oz)


def test_linear_ex_composes_steps():
    w = synth.WORKLOADS["tiny"]
    x = synth.make_activation(w)
    p = synth.make_weight_nvfp4(w)
    xb = synth.bits_u16(x)
    rng = np.random.default_rng(15)
    c = rng.uniform(0.5, 2.0, w.K).astype(np.float32)
    b = rng.standard_normal(w.N).astype(np.float32)
    y = oracle.linear_nvfp4(xb, w.x_dtype, w.K, False, p.codes.numpy(), p.sf.numpy(), p.g, synth.DT_FP32,
                            pre_scale=c, bias=b)
    qx, sx = oracle.quant_act(xb, w.x_dtype, w.K, pre_scale=c)
    qw, sw = oracle.prep_weight_nvfp4(p.codes.numpy(), p.sf.numpy(), p.g, w.K)
    ref = oracle.epilogue(oracle.gemm_s8(qx, qw), sx, sw, synth.DT_FP32, bias=b)
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))
