"""GPU parity of the decode-inside-GEMM path (cr_weight_amax_nvfp4, cr_gemm_nvfp4_fused)
against the oracle, through the C ABI.

Row maxima: bit-exact against the oracle's rotated-row maxima (one-pass, two-pass and
forced two-pass rows, padded strides with garbage).  Fused GEMM: int32 sums bit-exact
against the oracle's GEMM of the oracle's codes; outputs within the output tolerance of the
oracle's epilogue and bit-identical to the two-step GPU path (weight preparation, then
cr_gemm_s8_rowscale[_bias]); columns past N untouched; both activation column orders.
"""
import numpy as np
import pytest
import torch

import oracle
import rotated_bit_linear_amd as rbl
import synth
from helpers import assert_bits_equal, check_output, dev, say

pytestmark = pytest.mark.gpu


def _weight(N, K, seed, padded=False):
    g = torch.Generator().manual_seed(seed)
    w = 0.02 * torch.randn(N, K, generator=g)
    w[N // 3] = 0.0                                     # a zero row
    if padded:
        return synth.nvfp4_encode(w, ld_codes=(K + 1) // 2 // 16 * 16 + 32, ld_sf=(K + 15) // 16 + 5,
                                  garbage_seed=seed)
    return synth.nvfp4_encode(w, garbage_seed=seed)


def _x(M, K, seed):
    """bf16 X [M, ld] (ld a multiple of 8 elements, garbage in columns K..ld-1)."""
    g = torch.Generator().manual_seed(seed)
    ld = (K + 7) // 8 * 8 + 8
    x = torch.randn(M, ld, generator=g) * 2
    x[:, K:] = 1e4
    if M >= 4:
        x[1, :K] = 0.0                                  # a zero activation row
        x[2] *= 1e-4
    return x.to(torch.bfloat16)


AMAX_CASES = [(40, 300, False), (300, 5376, False), (21, 20000, False), (33, 1000, True), (5, 16, False),
              (70, 14336, False)]


@pytest.mark.parametrize("N,K,forced", AMAX_CASES, ids=[f"N{c[0]}-K{c[1]}-{'f' if c[2] else 'a'}" for c in AMAX_CASES])
def test_weight_amax_bit_exact(N, K, forced):
    p = _weight(N, K, N + K, padded=True)
    gs = torch.tensor([p.g], dtype=torch.float32, device=dev())
    say(f"cr_weight_amax_nvfp4 N={N} K={K} forced_two_pass={forced}")
    a = rbl.weight_amax_nvfp4(p.codes.to(dev()), p.sf.to(dev()), gs, K,
                              flags=rbl.CR_FLAG_FORCE_TWO_PASS if forced else 0)
    torch.cuda.synchronize()
    ref = oracle.weight_amax_nvfp4(p.codes.numpy(), p.sf.numpy(), p.g, K)
    assert_bits_equal(a.cpu().numpy().view(np.uint32), ref.view(np.uint32), "w_amax")


FUSED_CASES = [(1, 32, 256), (5, 40, 300), (32, 300, 1000), (33, 64, 512), (64, 257, 768),
               (100, 300, 5376), (128, 96, 16), (200, 100, 1300), (300, 70, 2048)]


@pytest.mark.parametrize("M,N,K", FUSED_CASES, ids=[f"M{c[0]}-N{c[1]}-K{c[2]}" for c in FUSED_CASES])
def test_gemm_fused_against_oracle(M, N, K):
    p = _weight(N, K, 7 * N + K, padded=(N % 2 == 0))
    x = _x(M, K, M + K)
    gs = torch.tensor([p.g], dtype=torch.float32, device=dev())
    cd, sfd = p.codes.to(dev()), p.sf.to(dev())
    say(f"cr_weight_amax_nvfp4 + prep N={N} K={K}")
    amax = rbl.weight_amax_nvfp4(cd, sfd, gs, K)
    rq, rs = oracle.quant_act(synth.bits_u16(x), synth.DT_BF16, K)
    rqw, rsw = oracle.prep_weight_nvfp4(p.codes.numpy(), p.sf.numpy(), p.g, K)
    acc = oracle.gemm_s8(rq, rqw)
    bias = torch.randn(N, generator=torch.Generator().manual_seed(N)).float()
    bd = bias.to(dev())
    for order in (0, rbl.CR_FLAG_BLOCK_TRANSPOSED):
        qx, sx = rbl.quant_act(x.to(dev()), K, flags=order)
        qw, sw = rbl.prep_weight_nvfp4(cd, sfd, gs, K, flags=order)     # two-step reference, same order
        ldc = N + 9
        for odt in (synth.DT_I32, synth.DT_BF16, synth.DT_FP16, synth.DT_FP32):
            for with_bias in ((False,) if odt == synth.DT_I32 else (False, True)):
                tdt = synth.TORCH_DTYPE[odt]
                full = torch.full((M, ldc), 7, dtype=tdt, device=dev())
                c = full[:, :N]
                # row maxima given, or found by the kernel's own first pass (alternating)
                am = amax if (odt + int(with_bias) + order) % 2 == 0 else None
                say(f"cr_gemm_nvfp4_fused M={M} N={N} K={K} order={order} out={odt} bias={with_bias} "
                    f"amax={'given' if am is not None else 'in-kernel'}")
                rbl.cr_gemm_nvfp4_fused(qx, sx, cd, sfd, gs, am, K, c, bias=bd if with_bias else None,
                                        flags=order)
                two = torch.empty(M, N, dtype=tdt, device=dev())
                if with_bias:
                    rbl.cr_gemm_s8_rowscale_bias(qx, sx, qw, sw, bd, two)
                else:
                    rbl.cr_gemm_s8_rowscale(qx, sx, qw, sw, two)
                torch.cuda.synchronize()
                fc = full.cpu()
                assert (fc[:, N:] == 7).all(), "columns past N were written"
                assert torch.equal(fc[:, :N], two.cpu()), "fused and two-step outputs differ"
                if odt == synth.DT_I32:
                    assert_bits_equal(fc[:, :N].numpy(), acc, "int32 accumulator")
                else:
                    ref = oracle.epilogue(acc, rs, rsw, odt, bias=bias.numpy() if with_bias else None)
                    check_output(fc[:, :N], ref, odt, f"fused GEMM out={odt} bias={with_bias}")


@pytest.mark.parametrize("M", [1, 128])
def test_gemm_fused_qkv_shape_sampled(M):
    """The QKV weight [21504, 5376] at a short batch, in the order and launch the layer uses;
    the oracle covers a seeded sample of 512 weight rows (with the last 32) for all M rows."""
    w = synth.WORKLOADS["qkv_m128"]
    p = synth.make_weight_nvfp4(w)
    x = synth.make_activation(w)[:M].contiguous()
    gs = torch.tensor([p.g], dtype=torch.float32, device=dev())
    cd, sfd = p.codes.to(dev()), p.sf.to(dev())
    bt = rbl.CR_FLAG_BLOCK_TRANSPOSED
    say(f"qkv shape M={M}: amax + quant_act + cr_gemm_nvfp4_fused (bf16 out)")
    amax = rbl.weight_amax_nvfp4(cd, sfd, gs, w.K)
    qx, sx = rbl.quant_act(x.to(dev()), w.K, flags=bt)
    out = rbl.gemm_nvfp4_fused(qx, sx, cd, sfd, gs, amax, w.K, flags=bt)
    out2 = rbl.gemm_nvfp4_fused(qx, sx, cd, sfd, gs, None, w.K, flags=bt)       # in-kernel row maxima
    acc = torch.empty(M, w.N, dtype=torch.int32, device=dev())
    rbl.cr_gemm_nvfp4_fused(qx, sx, cd, sfd, gs, amax, w.K, acc, flags=bt)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "given and in-kernel row maxima give different outputs"
    rows = synth.sample_rows(w.N, 512, 77)
    ci, si = p.codes.numpy()[rows.numpy()], p.sf.numpy()[rows.numpy()]
    ra = oracle.weight_amax_nvfp4(ci, si, p.g, w.K)
    assert_bits_equal(amax.cpu().numpy()[rows.numpy()].view(np.uint32), ra.view(np.uint32), "w_amax (sample)")
    rq, rs = oracle.quant_act(synth.bits_u16(x), synth.DT_BF16, w.K)
    rqw, rsw = oracle.prep_weight_nvfp4(ci, si, p.g, w.K)
    racc = oracle.gemm_s8(rq, rqw)
    assert_bits_equal(acc.cpu().numpy()[:, rows.numpy()], racc, "int32 accumulator (sampled columns)")
    ref = oracle.epilogue(racc, rs, rsw, synth.DT_BF16)
    check_output(out.cpu()[:, rows], ref, synth.DT_BF16, "fused GEMM output (sampled columns)")


LAYER_CASES = [(1, 300, 1000, False), (17, 520, 5376, False), (64, 256, 700, True), (64, 100, 20000, False),
               (65, 300, 1000, False)]


@pytest.mark.parametrize("M,N,K,swiglu", LAYER_CASES, ids=[f"M{c[0]}-N{c[1]}-K{c[2]}-{'sw' if c[3] else 'x'}"
                                                           for c in LAYER_CASES])
def test_layer_short_batch(M, N, K, swiglu):
    """cr_linear_nvfp4 at short batches (the decode-inside-GEMM path up to 64 rows, the
    staged path at 65): serial and two-stream runs identical, equal to the oracle's layer,
    with and without channel pre-scale and bias."""
    w = synth.Workload("t", M, N, K, synth.DT_BF16, (synth.DT_BF16,), 31, swiglu=swiglu, outlier_frac=0.01)
    x = synth.make_activation(w)
    p = synth.make_weight_nvfp4(w)
    xd, cd, sd = x.to(dev()), p.codes.to(dev()), p.sf.to(dev())
    gs = torch.tensor([p.g], dtype=torch.float32, device=dev())
    g = torch.Generator().manual_seed(M + N)
    c = (torch.rand(K, generator=g) + 0.5).to(torch.float32)
    bias = torch.randn(N, generator=g)
    aux = torch.cuda.Stream()
    assert rbl.cr_linear_nvfp4_plan(M, N, K)[1] == (0 if M <= 64 else 1)
    for extra in (False, True):
        kw = dict(pre_scale=c.to(dev()), bias=bias.to(dev())) if extra else {}
        outs = []
        for use_aux in (False, True):
            say(f"cr_linear_nvfp4 short batch M={M} N={N} K={K} swiglu={swiglu} pre/bias={extra} aux={use_aux}")
            outs.append(rbl.linear_nvfp4(xd, cd, sd, gs, K, out_dtype=torch.float32, swiglu=swiglu,
                                         aux_stream=aux if use_aux else None, **kw))
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1])
        ref = oracle.linear_nvfp4(synth.bits_u16(x), synth.DT_BF16, K, swiglu, p.codes.numpy(), p.sf.numpy(),
                                  p.g, synth.DT_FP32, pre_scale=c.numpy() if extra else None,
                                  bias=bias.numpy() if extra else None)
        check_output(outs[0], ref, synth.DT_FP32, f"short-batch layer output pre/bias={extra}")
