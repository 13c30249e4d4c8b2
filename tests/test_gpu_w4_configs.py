"""GPU parity of the W4A8 and W4A4 variants at the pages' shapes: QKV [21504, 5376] and
FFN-down [5376, 14336] with its fused SwiGLU, both at M = 19989. They run in the launch
configuration the benchmark times: a dense 0.02 * N(0, 1) weight prepared once, and the
block-transposed column order.

Full checks, bit-exact against the oracle:
* every 4-bit code and row scale of the weight, in the nibble form and in the E2M3 form;
* every code and scale of the activation in both forms.

Sampled checks, on a seeded sample of rows that always holds the M tail:
* the int32 sums of the three GEMMs (s8 x s4, s4 x s4, E2M3 x E2M3), each launched over
  the whole M x N and read through its raw-accumulator output;
* the bf16 outputs of cr_linear_w4a8, cr_linear_w4a4 and cr_linear_w4a4_e2m3 against the
  oracle's epilogue.

Every output element: the two W4A4 layers agree, and each layer call equals its component
GEMM on the operands checked in full above.
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
SAMPLE_ROWS = 384


def _block_transposed(codes: np.ndarray) -> np.ndarray:
    r, kp = codes.shape
    return codes.reshape(r, kp // 256, 16, 16).transpose(0, 1, 3, 2).reshape(r, kp).copy()


def _bt_codes(p_nibbles: np.ndarray) -> np.ndarray:
    """The oracle's codes of nibble-packed rows, in block-transposed order (int8 [n, K_pad])."""
    return _block_transposed(oracle.unpack_s4(p_nibbles, 2 * p_nibbles.shape[1]))


@pytest.mark.parametrize("name", ["qkv", "ffn_down"])
def test_w4_variants_at_config_size(name):
    w = synth.WORKLOADS[name]
    kp = w.K_pad
    x = synth.make_activation(w)
    wf = synth.make_weight_f32(w)
    xb = synth.bits_u16(x)
    xd = x.to(dev())

    # ---- the weight in both forms, in full ----
    say(f"{name}: cr_quant_weight_w4 / cr_quant_weight_w4_e2m3 N={w.N} K={w.K} block-transposed")
    wd = wf.to(dev())
    p4, s4 = rbl.quant_weight_w4(wd, w.K, flags=BT)
    p6, s6 = rbl.quant_weight_w4_e2m3(wd, w.K, flags=BT)
    torch.cuda.synchronize()
    del wd
    rpw, rsw = oracle.quant_weight_w4(wf.numpy(), synth.DT_FP32, w.K)
    del wf
    cw = _bt_codes(rpw)
    assert_bits_equal(p4.cpu().numpy(), oracle.pack_s4(cw), f"{name} w_s4")
    assert_bits_equal(p6.cpu().numpy(), oracle.pack_e2m3(cw), f"{name} w_f6")
    del cw
    assert_bits_equal(s4.cpu().numpy().view(np.uint32), rsw.view(np.uint32), f"{name} w_scale")
    assert_bits_equal(s6.cpu().numpy().view(np.uint32), rsw.view(np.uint32), f"{name} w_scale (E2M3 form)")

    # ---- the 4-bit activation in both forms, in full ----
    say(f"{name}: cr_quant_act_w4 / cr_quant_act_w4_e2m3 M={w.M} K={w.K} swiglu={w.swiglu}")
    qa4, sa4 = rbl.quant_act_w4(xd, w.K, swiglu=w.swiglu, flags=BT)
    qa6, sa6 = rbl.quant_act_w4_e2m3(xd, w.K, swiglu=w.swiglu, flags=BT)
    torch.cuda.synchronize()
    rpx, rsx4 = oracle.quant_act_w4(xb, w.x_dtype, w.K, swiglu=w.swiglu)
    cx = _bt_codes(rpx)
    assert_bits_equal(qa4.cpu().numpy(), oracle.pack_s4(cx), f"{name} x_s4")
    assert_bits_equal(qa6.cpu().numpy(), oracle.pack_e2m3(cx), f"{name} x_f6")
    del cx
    assert_bits_equal(sa4.cpu().numpy().view(np.uint32), rsx4.view(np.uint32), f"{name} x_scale (4-bit)")
    assert_bits_equal(sa6.cpu().numpy().view(np.uint32), rsx4.view(np.uint32), f"{name} x_scale (E2M3 form)")

    # ---- int32 sums of the three GEMMs over the whole M x N, checked on sampled rows ----
    rows = synth.sample_rows(w.M, SAMPLE_ROWS, w.seed)
    r = rows.numpy()
    rd = rows.to(dev())
    say(f"{name}: cr_quant_act (S8, for W4A8) M={w.M} K={w.K}")
    qx8, sx8 = rbl.quant_act(xd, w.K, swiglu=w.swiglu, flags=BT)
    rqx8, rsx8 = oracle.quant_act(xb, w.x_dtype, w.K, swiglu=w.swiglu)
    assert_bits_equal(sx8.cpu().numpy().view(np.uint32), rsx8.view(np.uint32), f"{name} x_scale (S8)")
    want = {
        "s8 x s4": oracle.gemm_s8s4(np.ascontiguousarray(rqx8[r]), rpw),
        "s4 x s4": oracle.gemm_s4s4(np.ascontiguousarray(rpx[r]), rpw, kp),
    }
    want["E2M3 x E2M3"] = want["s4 x s4"]
    acc = torch.empty(w.M, w.N, dtype=torch.int32, device=dev())
    for what, run in (("s8 x s4", lambda: rbl.cr_gemm_s8s4_rowscale(qx8, None, p4, None, acc)),
                      ("s4 x s4", lambda: rbl.cr_gemm_s4s4_rowscale(qa4, None, p4, None, acc)),
                      ("E2M3 x E2M3", lambda: rbl.cr_gemm_e2m3_rowscale(qa6, None, p6, None, acc))):
        say(f"{name}: {what} GEMM, int32 out, M={w.M} N={w.N} K_pad={kp}")
        acc.fill_(0x5A5A5A5A)
        run()
        torch.cuda.synchronize()
        assert_bits_equal(acc[rd].cpu().numpy(), want[what], f"{name} {what} int32 sums")
    # the layer calls' outputs, compared in full below: the component GEMMs on these operands
    comp8 = torch.empty(w.M, w.N, dtype=torch.bfloat16, device=dev())
    comp4 = torch.empty_like(comp8)
    rbl.cr_gemm_s8s4_rowscale(qx8, sx8, p4, s4, comp8)
    rbl.cr_gemm_s4s4_rowscale(qa4, sa4, p4, s4, comp4)
    del acc, qx8, qa4, qa6

    # ---- the three layers (bf16 out), sampled against the oracle; W4A4 forms equal ----
    say(f"{name}: cr_linear_w4a8 M={w.M} N={w.N} K={w.K}")
    y8 = rbl.linear_w4a8(xd, p4, s4, w.K, swiglu=w.swiglu, flags=BT)
    torch.cuda.synchronize()
    ref8 = oracle.epilogue(want["s8 x s4"], rsx8[r], rsw, synth.DT_BF16)
    assert torch.equal(y8, comp8), f"{name}: cr_linear_w4a8 and its component GEMM differ"
    del comp8
    err = check_output(y8[rd].cpu(), ref8, synth.DT_BF16, f"{name} W4A8 out")
    print(f"{name} W4A8: rows checked={len(r)} rel_l2={err:.3e}, bit-identical")
    del y8
    say(f"{name}: cr_linear_w4a4 M={w.M} N={w.N} K={w.K}")
    y4 = rbl.linear_w4a4(xd, p4, s4, w.K, swiglu=w.swiglu, flags=BT)
    say(f"{name}: cr_linear_w4a4_e2m3 M={w.M} N={w.N} K={w.K}")
    y6 = rbl.linear_w4a4_e2m3(xd, p6, s6, w.K, swiglu=w.swiglu, flags=BT)
    torch.cuda.synchronize()
    assert torch.equal(y4, y6), f"{name}: the two W4A4 forms differ"
    assert torch.equal(y4, comp4), f"{name}: cr_linear_w4a4 and its component GEMM differ"
    ref4 = oracle.epilogue(want["s4 x s4"], rsx4[r], rsw, synth.DT_BF16)
    err = check_output(y4[rd].cpu(), ref4, synth.DT_BF16, f"{name} W4A4 out")
    print(f"{name} W4A4 (both forms): rows checked={len(r)} rel_l2={err:.3e}, bit-identical")
