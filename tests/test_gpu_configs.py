"""GPU parity at the five workload sizes (tiny, QKV M=4096, QKV M=19989, FFN-down with
SwiGLU M=19989, long-K fp16) and at the block's other linear shapes (out_proj, fc1), in the
launch configurations of the benchmark (cr_linear_nvfp4, default tile bound, weight
preparation serial and on a second stream); and the block's MLP as a chain (fc1 -> SwiGLU ->
fc2).

Full checks: every S8 code and row scale of the activation and of the weight, bit-exact;
every output element of the layer call equal to the same call with serial staging and to
the component GEMM on those operands.
Sampled checks: the layer output on a seeded sample of rows that always holds the M tail
and every zero/tiny row, against the oracle's int32 GEMM and epilogue on those rows.
"""
import numpy as np
import pytest
import torch

import oracle
import rotated_bit_linear_amd as rbl
import synth
from helpers import assert_bits_equal, check_output, dev, say

pytestmark = pytest.mark.gpu

SAMPLE_ROWS = 512


def host_bits(x: torch.Tensor, dt: int) -> np.ndarray:
    return x.contiguous().numpy() if dt == synth.DT_FP32 else synth.bits_u16(x)


@pytest.mark.parametrize("name", ["tiny", "qkv_m4096", "qkv", "ffn_down", "longk", "out_proj", "ffn_up"])
def test_workload_parity(name):
    w = synth.WORKLOADS[name]
    x = synth.make_activation(w)
    p = synth.make_weight_nvfp4(w)
    xb = host_bits(x, w.x_dtype)
    gs = torch.tensor([p.g], dtype=torch.float32, device=dev())
    xd, cd, sd = x.to(dev()), p.codes.to(dev()), p.sf.to(dev())
    aux = torch.cuda.Stream()

    say(f"{name}: cr_quant_act{'_swiglu' if w.swiglu else ''} M={w.M} K={w.K}")
    qx, sx = rbl.quant_act(xd, w.K, swiglu=w.swiglu)
    say(f"{name}: cr_prep_weight_nvfp4 N={w.N} K={w.K}")
    qw, sw = rbl.prep_weight_nvfp4(cd, sd, gs, w.K)
    outs = {}
    for odt in w.out_dtypes:
        say(f"{name}: cr_linear_nvfp4 M={w.M} N={w.N} K={w.K} out={odt} (default tiles, aux stream)")
        outs[odt] = rbl.linear_nvfp4(xd, cd, sd, gs, w.K, out_dtype=synth.TORCH_DTYPE[odt], swiglu=w.swiglu,
                                     aux_stream=aux)
    # every output element: the layer call (weight chunks on the second stream) equals the
    # same call with serial staging, and the component GEMM on the separately prepared
    # operands, which are checked in full against the oracle below
    say(f"{name}: cr_linear_nvfp4 serial staging, cr_gemm_s8_rowscale on the components")
    for odt, out in outs.items():
        serial = rbl.linear_nvfp4(xd, cd, sd, gs, w.K, out_dtype=synth.TORCH_DTYPE[odt], swiglu=w.swiglu)
        assert torch.equal(serial, out), f"{name} out={odt}: serial and two-stream staging differ"
        del serial
        comp = rbl.gemm_s8_rowscale(qx, sx, qw, sw, out_dtype=synth.TORCH_DTYPE[odt])
        assert torch.equal(comp, out), f"{name} out={odt}: layer call and component GEMM differ"
        del comp
    torch.cuda.synchronize()

    rqx, rsx = oracle.quant_act(xb, w.x_dtype, w.K, swiglu=w.swiglu)
    assert_bits_equal(qx.cpu().numpy(), rqx, f"{name} x_s8")
    assert_bits_equal(sx.cpu().numpy().view(np.uint32), rsx.view(np.uint32), f"{name} x_scale")
    del qx
    rqw, rsw = oracle.prep_weight_nvfp4(p.codes.numpy(), p.sf.numpy(), p.g, w.K)
    assert_bits_equal(qw.cpu().numpy(), rqw, f"{name} w_s8")
    assert_bits_equal(sw.cpu().numpy().view(np.uint32), rsw.view(np.uint32), f"{name} w_scale")
    del qw

    zero, tiny = synth.special_rows(w)
    rows = synth.sample_rows(w.M, SAMPLE_ROWS, w.seed, torch.cat([zero, tiny]))
    if w.M <= 64:
        rows = torch.arange(w.M)
    r = rows.numpy()
    acc = oracle.gemm_s8(np.ascontiguousarray(rqx[r]), rqw)
    for odt, out in outs.items():
        ref = oracle.epilogue(acc, rsx[r], rsw, odt)
        got = out[rows.to(dev())].cpu()
        err = check_output(got, ref, odt, f"{name} out={odt}")
        print(f"{name} out={odt}: rows checked={len(r)} rel_l2={err:.3e}, bit-identical")
        if len(zero):
            assert (out[zero.to(dev())] == 0).all()


def test_mlp_chain_fc1_swiglu_fc2():
    """fc1 writes H [M, 28672] in bf16 through cr_linear_nvfp4; the FFN-down layer reads it
    through its fused SwiGLU.  The oracle runs the same chain on a seeded sample of rows
    (rows are independent): its own fc1 output rows, rounded to bf16, feed its FFN-down."""
    up, down = (synth.WORKLOADS[n] for n in synth.MLP_CHAIN)
    assert up.N == 2 * down.K and up.M == down.M
    x = synth.make_activation(up)
    pu, pd = synth.make_weight_nvfp4(up), synth.make_weight_nvfp4(down)
    gu = torch.tensor([pu.g], dtype=torch.float32, device=dev())
    gd = torch.tensor([pd.g], dtype=torch.float32, device=dev())
    aux = torch.cuda.Stream()
    say(f"chain: fc1 cr_linear_nvfp4 M={up.M} N={up.N} K={up.K}")
    h = rbl.linear_nvfp4(x.to(dev()), pu.codes.to(dev()), pu.sf.to(dev()), gu, up.K,
                         out_dtype=torch.bfloat16, aux_stream=aux)
    say(f"chain: FFN-down cr_linear_nvfp4 swiglu M={down.M} N={down.N} F={down.K}")
    y = rbl.linear_nvfp4(h, pd.codes.to(dev()), pd.sf.to(dev()), gd, down.K,
                         out_dtype=torch.bfloat16, swiglu=True, aux_stream=aux)
    torch.cuda.synchronize()

    rows = synth.sample_rows(up.M, SAMPLE_ROWS, up.seed, torch.empty(0, dtype=torch.long))
    r = rows.numpy()
    rqwu, rswu = oracle.prep_weight_nvfp4(pu.codes.numpy(), pu.sf.numpy(), pu.g, up.K)
    qx, sx = oracle.quant_act(synth.bits_u16(x[rows]), up.x_dtype, up.K)
    h_ref = oracle.epilogue(oracle.gemm_s8(qx, rqwu), sx, rswu, synth.DT_BF16)   # bf16 bits
    del rqwu
    h_got = synth.bits_u16(h[rows.to(dev())].cpu())
    h_same = float(np.mean(h_got == h_ref))
    rqwd, rswd = oracle.prep_weight_nvfp4(pd.codes.numpy(), pd.sf.numpy(), pd.g, down.K)
    qh, sh = oracle.quant_act(np.ascontiguousarray(h_ref), synth.DT_BF16, down.K, swiglu=True)
    y_ref = oracle.epilogue(oracle.gemm_s8(qh, rqwd), sh, rswd, synth.DT_BF16)
    got = y[rows.to(dev())].cpu()
    print(f"chain: rows checked={len(r)} fc1 bf16 outputs identical={h_same:.6f}")
    assert_bits_equal(h_got, h_ref, "fc1 output (bf16 bits)")
    err = check_output(got, y_ref, synth.DT_BF16, "chain output")
    print(f"chain: final rel_l2={err:.3e}, bit-identical")


def _block_transposed(codes: np.ndarray) -> np.ndarray:
    r, kp = codes.shape
    return codes.reshape(r, kp // 256, 16, 16).transpose(0, 1, 3, 2).reshape(r, kp).copy()


def test_qkv_at_the_pages_16mib_tile_bound():
    """QKV at M = 19989 with S8 weight tiles bounded by 16 MiB (the pages' bound: 7 chunks of
    3072 rows, two tiles alternating, preparation on a second stream).  The call's own
    workspace is read back afterwards: its S8 activation (block-transposed order) and row
    scales bit-exact in full, its last weight tile (chunk 6, rows 18432..21503) bit-exact;
    the output equals the default bound's bit for bit and the oracle's on sampled rows."""
    w = synth.WORKLOADS["qkv"]
    bound = 16 << 20
    R, nch = rbl.cr_linear_nvfp4_plan(w.M, w.N, w.K, bound)
    assert (R, nch) == (3072, 7)
    x = synth.make_activation(w)
    p = synth.make_weight_nvfp4(w)
    gs = torch.tensor([p.g], dtype=torch.float32, device=dev())
    xd, cd, sd = x.to(dev()), p.codes.to(dev()), p.sf.to(dev())
    aux = torch.cuda.Stream()
    ws = torch.empty(rbl.cr_linear_nvfp4_workspace_bytes(w.M, w.N, w.K, bound), dtype=torch.uint8, device=dev())
    out = torch.empty(w.M, w.N, dtype=torch.bfloat16, device=dev())
    say(f"qkv: cr_linear_nvfp4 M={w.M} N={w.N} K={w.K} max_tile_bytes=16 MiB, aux stream")
    rbl.cr_linear_nvfp4(xd, w.K, False, cd, sd, gs, out, ws, bound, aux_stream=aux)
    say("qkv: cr_linear_nvfp4 default tile bound")
    ref_default = rbl.linear_nvfp4(xd, cd, sd, gs, w.K, aux_stream=aux)
    say("qkv: cr_linear_nvfp4 max_tile_bytes=16 MiB, serial staging (separate workspace)")
    serial = rbl.linear_nvfp4(xd, cd, sd, gs, w.K, max_tile_bytes=bound)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_default), "16 MiB and default tile bounds differ"
    assert torch.equal(serial, out), "16 MiB bound: serial and two-stream staging differ"
    del serial

    kp = w.K_pad
    up = lambda v: (v + 255) // 256 * 256   # noqa: E731  (the workspace's 256-byte regions)
    host = ws.cpu().numpy()
    x_s8 = host[:w.M * kp].view(np.int8).reshape(w.M, kp)
    off = up(w.M * kp)
    x_scale = host[off:off + 4 * w.M].view(np.float32)
    off = up(off + 4 * w.M)
    tiles = []
    for _ in range(2):
        t = host[off:off + R * kp].view(np.int8).reshape(R, kp)
        off = up(off + R * kp)
        s = host[off:off + 4 * R].view(np.float32)
        off = up(off + 4 * R)
        tiles.append((t, s))
    rqx, rsx = oracle.quant_act(synth.bits_u16(x), w.x_dtype, w.K)
    assert_bits_equal(x_s8, _block_transposed(rqx), "x_s8 in the workspace (block-transposed)")
    assert_bits_equal(x_scale.view(np.uint32), rsx.view(np.uint32), "x_scale in the workspace")
    last = nch - 1                            # chunk 6 went to tile 6 % 2 = 0
    n0, rows = last * R, w.N - last * R
    rqw, rsw = oracle.prep_weight_nvfp4(p.codes.numpy()[n0:], p.sf.numpy()[n0:], p.g, w.K)
    t, s = tiles[last % 2]
    assert_bits_equal(t[:rows], _block_transposed(rqw), "last S8 weight tile")
    assert_bits_equal(s[:rows].view(np.uint32), rsw.view(np.uint32), "last weight tile scales")

    rows_m = synth.sample_rows(w.M, SAMPLE_ROWS, w.seed, torch.empty(0, dtype=torch.long)).numpy()
    rqw_all, rsw_all = oracle.prep_weight_nvfp4(p.codes.numpy(), p.sf.numpy(), p.g, w.K)
    acc = oracle.gemm_s8(np.ascontiguousarray(rqx[rows_m]), rqw_all)
    ref = oracle.epilogue(acc, rsx[rows_m], rsw_all, synth.DT_BF16)
    err = check_output(out[torch.from_numpy(rows_m).to(dev())].cpu(), ref, synth.DT_BF16, "qkv at 16 MiB")
    print(f"qkv at the 16 MiB bound: rows checked={len(rows_m)} rel_l2={err:.3e}, bit-identical")


def test_ffn_down_at_the_pages_16mib_tile_bound():
    """FFN-down with its SwiGLU at M = 19989 with S8 weight tiles bounded by 16 MiB: the plan
    takes 7 chunks of 768 rows (237-tile GEMMs, one round of workgroups each) instead of
    1024-row chunks.  The output equals the default bound's and serial staging's bit for bit,
    and the oracle's on sampled rows (their SwiGLU, rotation and quantization computed row
    by row)."""
    w = synth.WORKLOADS["ffn_down"]
    bound = 16 << 20
    R, nch = rbl.cr_linear_nvfp4_plan(w.M, w.N, w.K, bound)
    assert (R, nch) == (768, 7)
    x = synth.make_activation(w)
    p = synth.make_weight_nvfp4(w)
    gs = torch.tensor([p.g], dtype=torch.float32, device=dev())
    xd, cd, sd = x.to(dev()), p.codes.to(dev()), p.sf.to(dev())
    aux = torch.cuda.Stream()
    ws = torch.empty(rbl.cr_linear_nvfp4_workspace_bytes(w.M, w.N, w.K, bound), dtype=torch.uint8, device=dev())
    out = torch.empty(w.M, w.N, dtype=torch.bfloat16, device=dev())
    say(f"ffn_down: cr_linear_nvfp4 swiglu M={w.M} N={w.N} K={w.K} max_tile_bytes=16 MiB, aux stream")
    rbl.cr_linear_nvfp4(xd, w.K, True, cd, sd, gs, out, ws, bound, aux_stream=aux)
    say("ffn_down: cr_linear_nvfp4 default tile bound")
    ref_default = rbl.linear_nvfp4(xd, cd, sd, gs, w.K, swiglu=True, aux_stream=aux)
    say("ffn_down: cr_linear_nvfp4 max_tile_bytes=16 MiB, serial staging")
    serial = rbl.linear_nvfp4(xd, cd, sd, gs, w.K, swiglu=True, max_tile_bytes=bound)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_default), "16 MiB and default tile bounds differ"
    assert torch.equal(serial, out), "16 MiB bound: serial and two-stream staging differ"
    del serial

    rows_m = synth.sample_rows(w.M, SAMPLE_ROWS, w.seed, torch.empty(0, dtype=torch.long)).numpy()
    xs = np.ascontiguousarray(synth.bits_u16(x)[rows_m])
    rqx, rsx = oracle.quant_act(xs, w.x_dtype, w.K, swiglu=True)
    rqw, rsw = oracle.prep_weight_nvfp4(p.codes.numpy(), p.sf.numpy(), p.g, w.K)
    ref = oracle.epilogue(oracle.gemm_s8(rqx, rqw), rsx, rsw, synth.DT_BF16)
    err = check_output(out[torch.from_numpy(rows_m).to(dev())].cpu(), ref, synth.DT_BF16, "ffn_down at 16 MiB")
    print(f"ffn_down at the 16 MiB bound: rows checked={len(rows_m)} rel_l2={err:.3e}, bit-identical")
