"""GPU parity of each entry point against the CPU oracle on small, ragged inputs.

Bar: S8 codes, row scales and int32 accumulators bit-exact; dequantized outputs within
relative L2 1e-3 (bf16/fp16) or 1e-5 (fp32) of the oracle's output in the same dtype.
Every call goes through the C ABI (rotated_bit_linear_amd's ctypes binding).
"""
import numpy as np
import pytest
import torch

import oracle
import rotated_bit_linear_amd as rbl
import synth
from helpers import assert_bits_equal, check_output, dev, say

pytestmark = pytest.mark.gpu

DT_T = {synth.DT_BF16: torch.bfloat16, synth.DT_FP16: torch.float16, synth.DT_FP32: torch.float32}


def host_bits(x: torch.Tensor, dt: int) -> np.ndarray:
    return x.contiguous().numpy() if dt == synth.DT_FP32 else synth.bits_u16(x)


def make_x(M, cols, dt, seed, ld=None, special=False):
    g = torch.Generator().manual_seed(seed)
    ld = ld or cols
    x = torch.randn(M, ld, generator=g) * 2
    x[:, cols:] = torch.randn(M, ld - cols, generator=g) * 1e4          # garbage past K
    if special and M >= 4:
        x[1, :] = 0.0
        x[2, :cols] *= 1e-4
        x[3, : min(cols, 7)] *= 300.0
    return x.to(DT_T[dt])


# ------------------------------------------------------------------ SwiGLU bits ----

@pytest.mark.parametrize("dt", [synth.DT_BF16, synth.DT_FP16])
def test_swiglu_exhaustive_gate_values(dt):
    F = 65536
    gate = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    g = torch.Generator().manual_seed(5)
    value = torch.randn(F, generator=g).to(DT_T[dt]).view(torch.int16)
    h = torch.cat([gate, value]).view(DT_T[dt]).reshape(1, 2 * F)
    out = torch.empty(1, F, dtype=torch.float32, device=dev())
    say(f"cr_swiglu dtype={dt} F={F} all gate bit patterns")
    rbl.cr_swiglu(h.to(dev()), F, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()[0]
    hb = synth.bits_u16(h)[0]
    conv = oracle.bf16_to_f32 if dt == synth.DT_BF16 else oracle.fp16_to_f32
    ref = oracle.swiglu(conv(hb[:F]), conv(hb[F:]))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert_bits_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32), "swiglu bits")


def test_swiglu_fp32_random_and_edges():
    g = torch.Generator().manual_seed(6)
    F = 1 << 20
    gate = torch.cat([torch.randn(F - 16, generator=g) * 8,
                      torch.tensor([0.0, -0.0, 88.7, -88.7, 89.0, -89.0, 103.9, -103.9, 104.5, -104.5,
                                    1e-30, -1e-30, 3e38, -3e38, 1e-45, -1e-45])])
    value = torch.randn(F, generator=g)
    h = torch.cat([gate, value]).reshape(1, 2 * F)
    out = torch.empty(1, F, dtype=torch.float32, device=dev())
    say("cr_swiglu fp32 random + edge gates")
    rbl.cr_swiglu(h.to(dev()), F, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()[0]
    ref = oracle.swiglu(gate.numpy(), value.numpy())
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert_bits_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32), "swiglu fp32 bits")


def test_swiglu_fp32_every_gate_reaching_the_reciprocal():
    """Every fp32 gate a with 2^-25 <= |a| < 2^7, value 1.0.  This range produces every
    denominator 1 + E(-a) that the refined reciprocal handles (gates outside it give
    d in {1, 2} or take the IEEE-division branch), so the refined reciprocal is checked
    against the oracle's division for all of them.  16 chunks of 2^25 gates."""
    F, M = 8192, 4096
    n = F * M
    h = torch.empty(M, 2 * F, dtype=torch.float32)
    h[:, F:] = 1.0
    hd = torch.empty(M, 2 * F, dtype=torch.float32, device=dev())
    out = torch.empty(M, F, dtype=torch.float32, device=dev())
    ones = np.ones(n, np.float32)
    for c in range(16):
        sign, e0 = c // 8, 102 + 4 * (c % 8)
        start = (sign << 31) | (e0 << 23)
        bits = np.arange(start, start + n, dtype=np.uint64).astype(np.uint32)
        gate = bits.view(np.float32)
        h[:, :F] = torch.from_numpy(gate.reshape(M, F))
        say(f"cr_swiglu fp32 gates sign={sign} exponents {e0}..{e0 + 3}")
        hd.copy_(h)
        rbl.cr_swiglu(hd, F, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy().ravel()
        ref = oracle.swiglu(gate, ones)
        assert_bits_equal(got.view(np.uint32), ref.view(np.uint32), f"swiglu fp32 chunk {c}")


# ------------------------------------------------------------ activation prep ----

ACT_CASES = [
    # dt, M, K, ld, special, forced two-pass
    (synth.DT_BF16, 64, 512, 512, False, False),
    (synth.DT_BF16, 37, 300, 304, True, False),
    (synth.DT_FP16, 33, 1000, 1016, True, False),
    (synth.DT_FP32, 17, 777, 780, True, False),
    (synth.DT_BF16, 5, 16384, 16384, False, False),
    (synth.DT_BF16, 5, 16385, 16392, True, False),    # 65 blocks: one pass, two blocks a group
    (synth.DT_FP16, 3, 20000, 20000, True, False),    # 79 blocks: one pass
    (synth.DT_FP16, 6, 32768, 32768, True, False),    # 128 blocks: one pass, 1024 threads
    (synth.DT_FP32, 4, 32768, 32768, True, False),    # fp32 rows above 64 blocks: two-pass
    (synth.DT_BF16, 4, 32769, 32776, True, False),    # 129 blocks: two-pass by size
    (synth.DT_BF16, 7, 20000, 20000, True, True),     # forced two-pass at 79 blocks
    (synth.DT_BF16, 11, 5376, 5376, True, True),      # forced two-pass
    (synth.DT_FP32, 1, 1, 4, False, False),           # one element
]


@pytest.mark.parametrize("dt,M,K,ld,special,forced", ACT_CASES,
                         ids=[f"dt{c[0]}-M{c[1]}-K{c[2]}-ld{c[3]}{'-tp' if c[5] else ''}" for c in ACT_CASES])
def test_quant_act_bit_exact(dt, M, K, ld, special, forced):
    x = make_x(M, K, dt, seed=M * 7 + K, ld=ld, special=special)
    say(f"cr_quant_act dt={dt} M={M} K={K} ld={ld} forced_two_pass={forced}")
    q, s = rbl.quant_act(x.to(dev()), K, flags=rbl.CR_FLAG_FORCE_TWO_PASS if forced else 0)
    torch.cuda.synchronize()
    rq, rs = oracle.quant_act(host_bits(x, dt), dt, K)
    assert_bits_equal(q.cpu().numpy(), rq, "x_s8")
    assert_bits_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32), "x_scale")


def test_two_pass_equals_one_pass_activation():
    for K in (4000, 25000):      # one block a group; two blocks a group over 49 groups
        x = make_x(50, K, synth.DT_BF16, seed=3, special=True).to(dev())
        for flags in (0, rbl.CR_FLAG_BLOCK_TRANSPOSED):
            say(f"cr_quant_act one-pass vs forced two-pass M=50 K={K} flags={flags}")
            q1, s1 = rbl.quant_act(x, K, flags=flags)
            q2, s2 = rbl.quant_act(x, K, flags=flags | rbl.CR_FLAG_FORCE_TWO_PASS)
            torch.cuda.synchronize()
            assert torch.equal(q1, q2) and torch.equal(s1, s2), (K, flags)


SWI_CASES = [
    (synth.DT_BF16, 32, 14336),
    (synth.DT_BF16, 6, 20000),      # 79 blocks: two-pass by size
    (synth.DT_FP16, 4, 17000),      # 67 blocks, sigma computed
    (synth.DT_BF16, 3, 33000),
    (synth.DT_BF16, 9, 300),        # value half not 16-byte aligned: element loads
    (synth.DT_FP32, 7, 1000),
    (synth.DT_FP16, 5, 640),
    (synth.DT_BF16, 3, 8200),
]


@pytest.mark.parametrize("dt,M,F", SWI_CASES, ids=[f"dt{c[0]}-M{c[1]}-F{c[2]}" for c in SWI_CASES])
def test_quant_act_swiglu_bit_exact(dt, M, F):
    h = make_x(M, 2 * F, dt, seed=F + M, ld=2 * F + (8 if dt != synth.DT_FP32 else 4), special=True)
    for forced in (False, True):
        say(f"cr_quant_act_swiglu dt={dt} M={M} F={F} forced_two_pass={forced}")
        q, s = rbl.quant_act(h.to(dev()), F, swiglu=True, flags=rbl.CR_FLAG_FORCE_TWO_PASS if forced else 0)
        torch.cuda.synchronize()
        rq, rs = oracle.quant_act(host_bits(h, dt), dt, F, swiglu=True)
        assert_bits_equal(q.cpu().numpy(), rq, "x_s8 (swiglu)")
        assert_bits_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32), "x_scale (swiglu)")


# ---------------------------------------------------------------- weight prep ----

# row shapes: one block per lane group (K <= 8192), two (8192 < K <= 16384: 14336 and a
# 33-block row with a tail), two in up to 64 groups (16384 < K <= 32768: 20000, 32768),
# two-pass (K > 32768: 40000), and tiny rows
W_CASES = [(256, 512, None, None), (300, 1000, 512, 80), (97, 20000, None, None), (64, 5376, None, None),
           (1, 17, 16, 5), (40, 14336, None, None), (21, 8200, 4112, 520), (33, 32768, None, None),
           (19, 40000, None, None)]


@pytest.mark.parametrize("N,K,ldc,ldsf", W_CASES, ids=[f"N{c[0]}-K{c[1]}" for c in W_CASES])
def test_prep_weight_bit_exact(N, K, ldc, ldsf):
    g = torch.Generator().manual_seed(N + K)
    w = 0.02 * torch.randn(N, K, generator=g)
    p = synth.nvfp4_encode(w, ld_codes=ldc, ld_sf=ldsf, garbage_seed=N)
    gs = torch.tensor([p.g], dtype=torch.float32, device=dev())
    rq, rs = oracle.prep_weight_nvfp4(p.codes.numpy(), p.sf.numpy(), p.g, K)
    for forced in (False, True):
        say(f"cr_prep_weight_nvfp4 N={N} K={K} ld={p.ld_codes}/{p.ld_sf} forced_two_pass={forced}")
        q, s = rbl.prep_weight_nvfp4(p.codes.to(dev()), p.sf.to(dev()), gs, K,
                                     flags=rbl.CR_FLAG_FORCE_TWO_PASS if forced else 0)
        torch.cuda.synchronize()
        assert_bits_equal(q.cpu().numpy(), rq, "w_s8")
        assert_bits_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32), "w_scale")


# ----------------------------------------------------------------------- GEMM ----

G_CASES = [(64, 256, 512), (300, 700, 768), (1, 1, 256), (513, 255, 1280), (257, 300, 5376), (600, 520, 256)]


@pytest.mark.parametrize("M,N,Kp", G_CASES, ids=[f"M{c[0]}-N{c[1]}-K{c[2]}" for c in G_CASES])
def test_gemm_int32_exact_and_epilogues(M, N, Kp):
    g = torch.Generator().manual_seed(M * N + Kp)
    a = torch.randint(-127, 128, (M, Kp), generator=g, dtype=torch.int32).to(torch.int8)
    b = torch.randint(-127, 128, (N, Kp), generator=g, dtype=torch.int32).to(torch.int8)
    sa = torch.rand(M, generator=g) * 1e-2
    sb = torch.rand(N, generator=g) * 1e-3
    sa[0] = 0.0
    acc = oracle.gemm_s8(a.numpy(), b.numpy())
    ad, bd, sad, sbd = a.to(dev()), b.to(dev()), sa.to(dev()), sb.to(dev())
    # an odd row stride (element stores) and a 16-byte multiple (vector stores, N tail)
    for ldc in (N + 9, (N + 7) // 8 * 8 + 8):
        for odt in (synth.DT_I32, synth.DT_BF16, synth.DT_FP16, synth.DT_FP32):
            tdt = synth.TORCH_DTYPE[odt]
            full = torch.full((M, ldc), 7, dtype=tdt, device=dev())
            c = full[:, :N]
            say(f"cr_gemm_s8_rowscale M={M} N={N} K_pad={Kp} out={odt} ldc={ldc}")
            rbl.cr_gemm_s8_rowscale(ad, sad, bd, sbd, c)
            torch.cuda.synchronize()
            fc = full.cpu()
            assert (fc[:, N:] == 7).all(), "columns past N were written"
            ref = oracle.epilogue(acc, sa.numpy(), sb.numpy(), odt)
            if odt == synth.DT_I32:
                assert_bits_equal(fc[:, :N].numpy(), acc, "int32 accumulator")
            else:
                check_output(fc[:, :N], ref, odt, f"GEMM M={M} N={N} out={odt} ldc={ldc}")


# ---------------------------------------------------------------------- layer ----

def _layer_inputs(M, N, K, dt, swiglu, seed):
    w = synth.Workload("t", M, N, K, dt, (synth.DT_BF16,), seed, swiglu=swiglu, outlier_frac=0.01)
    x = synth.make_activation(w)
    p = synth.make_weight_nvfp4(w)
    return w, x, p


@pytest.mark.parametrize("swiglu", [False, True])
def test_layer_chunking_and_streams_identical(swiglu):
    M, N, K = 300, 1000, 1000
    w, x, p = _layer_inputs(M, N, K, synth.DT_BF16, swiglu, 11)
    xd, cd, sd = x.to(dev()), p.codes.to(dev()), p.sf.to(dev())
    gs = torch.tensor([p.g], dtype=torch.float32, device=dev())
    aux = torch.cuda.Stream()
    outs = []
    for mt, use_aux in [(0, False), (256 * 1024, False), (256 * 1024, True), (512 * 1024, True), (0, True)]:
        say(f"cr_linear_nvfp4 M={M} N={N} K={K} swiglu={swiglu} max_tile={mt} aux={use_aux}")
        outs.append(rbl.linear_nvfp4(xd, cd, sd, gs, K, swiglu=swiglu, max_tile_bytes=mt,
                                     aux_stream=aux if use_aux else None))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    ref = oracle.linear_nvfp4(synth.bits_u16(x), synth.DT_BF16, K, swiglu, p.codes.numpy(), p.sf.numpy(),
                              p.g, synth.DT_BF16)
    check_output(outs[0], ref, synth.DT_BF16, "layer output")


def test_layer_tiny_full():
    w = synth.WORKLOADS["tiny"]
    x = synth.make_activation(w)
    p = synth.make_weight_nvfp4(w)
    gs = torch.tensor([p.g], dtype=torch.float32, device=dev())
    say("cr_linear_nvfp4 tiny 64x256x512 bf16 (and the three steps separately)")
    out = rbl.linear_nvfp4(x.to(dev()), p.codes.to(dev()), p.sf.to(dev()), gs, w.K)
    qx, sx = rbl.quant_act(x.to(dev()), w.K)
    qw, sw = rbl.prep_weight_nvfp4(p.codes.to(dev()), p.sf.to(dev()), gs, w.K)
    acc = torch.empty(w.M, w.N, dtype=torch.int32, device=dev())
    rbl.cr_gemm_s8_rowscale(qx, sx, qw, sw, acc)
    torch.cuda.synchronize()
    xb = synth.bits_u16(x)
    rqx, rsx = oracle.quant_act(xb, w.x_dtype, w.K)
    rqw, rsw = oracle.prep_weight_nvfp4(p.codes.numpy(), p.sf.numpy(), p.g, w.K)
    racc = oracle.gemm_s8(rqx, rqw)
    assert_bits_equal(qx.cpu().numpy(), rqx, "x_s8")
    assert_bits_equal(qw.cpu().numpy(), rqw, "w_s8")
    assert_bits_equal(acc.cpu().numpy(), racc, "acc")
    ref = oracle.epilogue(racc, rsx, rsw, synth.DT_BF16)
    err = check_output(out, ref, synth.DT_BF16, "tiny layer output")
    print(f"tiny: rel_l2={err:.3e}, bit-identical")


# ------------------------------------------------ non-finite inputs stay local ----

NF_CASES = [
    # K, swiglu, forced two-pass: several rows per workgroup, one and two blocks per lane
    # group, SwiGLU one block per group, forced and size-driven two-pass
    (1000, False, False), (10000, False, False), (14336, True, False), (1000, True, True),
    (17000, False, False),
]


@pytest.mark.parametrize("K,swiglu,forced", NF_CASES, ids=[f"K{c[0]}-sw{int(c[1])}-tp{int(c[2])}" for c in NF_CASES])
def test_non_finite_rows_leave_other_rows_exact(K, swiglu, forced):
    """Inputs are assumed finite; a NaN or an infinity leaves its own row's codes, scale and
    outputs unspecified, but every other row stays bit-exact (rows are prepared independently,
    also where several share a workgroup), for activations, SwiGLU, NVFP4 weights (a NaN E4M3
    block scale) and the whole layer."""
    M, N = 70, 300                                       # 70 rows: the layer stages S8 weight tiles
    cols = 2 * K if swiglu else K
    x = make_x(M, cols, synth.DT_BF16, seed=K + 7)
    x[5, 17] = float("nan")
    x[9, cols - 1] = float("inf")
    x[12, cols // 2] = float("-inf")
    x[66, 0] = float("nan")
    bad = [5, 9, 12, 66]
    good = [i for i in range(M) if i not in bad]
    flags = rbl.CR_FLAG_FORCE_TWO_PASS if forced else 0
    say(f"non-finite rows K={K} swiglu={swiglu} forced={forced}: quant_act")
    q, s = rbl.quant_act(x.to(dev()), K, swiglu=swiglu, flags=flags)
    p = synth.nvfp4_encode(0.02 * torch.randn(N, K, generator=torch.Generator().manual_seed(K)))
    sf_bad = p.sf.clone()
    sf_bad[7, 2] = 0x7F                                  # E4M3 NaN
    gs = torch.tensor([p.g], dtype=torch.float32, device=dev())
    say(f"non-finite rows K={K}: prep_weight with a NaN block scale, layer")
    qw, sw = rbl.prep_weight_nvfp4(p.codes.to(dev()), sf_bad.to(dev()), gs, K, flags=flags)
    out = rbl.linear_nvfp4(x.to(dev()), p.codes.to(dev()), p.sf.to(dev()), gs, K, swiglu=swiglu, flags=flags)
    torch.cuda.synchronize()
    xb = synth.bits_u16(x)[good]
    rq, rs = oracle.quant_act(xb, synth.DT_BF16, K, swiglu=swiglu)
    assert_bits_equal(q.cpu().numpy()[good], rq, "x_s8 of the finite rows")
    assert_bits_equal(s.cpu().numpy()[good].view(np.uint32), rs.view(np.uint32), "x_scale of the finite rows")
    wgood = [i for i in range(N) if i != 7]
    rqw, rsw = oracle.prep_weight_nvfp4(p.codes.numpy()[wgood], p.sf.numpy()[wgood], p.g, K)
    assert_bits_equal(qw.cpu().numpy()[wgood], rqw, "w_s8 of the finite rows")
    assert_bits_equal(sw.cpu().numpy()[wgood].view(np.uint32), rsw.view(np.uint32), "w_scale of the finite rows")
    ref = oracle.linear_nvfp4(xb, synth.DT_BF16, K, swiglu, p.codes.numpy(), p.sf.numpy(), p.g, synth.DT_BF16)
    check_output(out.cpu()[good], ref, synth.DT_BF16, "layer output of the finite rows")


# ------------------------------------------------ channel pre-scale and bias ----

PRE_CASES = [
    # dt, M, K, swiglu, forced two-pass
    (synth.DT_BF16, 37, 300, False, False),
    (synth.DT_FP16, 9, 5376, False, False),
    (synth.DT_FP32, 5, 16385, False, False),        # two-pass by size
    (synth.DT_FP16, 3, 20000, True, False),         # SwiGLU fp16 + pre-scale, 79 blocks
    (synth.DT_FP32, 3, 40000, False, False),
    (synth.DT_BF16, 7, 700, True, False),
    (synth.DT_BF16, 4, 14336, True, False),         # 56-block SwiGLU rows: one block per lane group
    (synth.DT_BF16, 4, 14336, False, False),        # 56-block plain rows: two blocks per lane group
    (synth.DT_BF16, 5, 20000, False, False),        # 79-block plain rows: two blocks a group, 40 groups
    (synth.DT_FP16, 3, 32768, False, False),        # 128 blocks: 64 groups, 1024 threads
    (synth.DT_BF16, 6, 1000, False, True),          # forced two-pass
]


@pytest.mark.parametrize("dt,M,K,swiglu,forced", PRE_CASES,
                         ids=[f"dt{c[0]}-M{c[1]}-K{c[2]}{'-swiglu' if c[3] else ''}{'-tp' if c[4] else ''}"
                              for c in PRE_CASES])
def test_quant_act_prescale_bit_exact(dt, M, K, swiglu, forced):
    cols = 2 * K if swiglu else K
    mult = 4 if dt == synth.DT_FP32 else 8           # 16-byte row strides, garbage past the row
    x = make_x(M, cols, dt, seed=M + K + 99, ld=(cols // mult + 1) * mult, special=True)
    g = torch.Generator().manual_seed(K)
    c = (torch.rand(K, generator=g) * 3.75 + 0.25).to(torch.float32)
    say(f"cr_quant_act_ex dt={dt} M={M} K={K} swiglu={swiglu} pre_scale forced_two_pass={forced}")
    q, s = rbl.quant_act(x.to(dev()), K, swiglu=swiglu, pre_scale=c.to(dev()),
                         flags=rbl.CR_FLAG_FORCE_TWO_PASS if forced else 0)
    torch.cuda.synchronize()
    rq, rs = oracle.quant_act(host_bits(x, dt), dt, K, swiglu=swiglu, pre_scale=c.numpy())
    assert_bits_equal(q.cpu().numpy(), rq, "x_s8 (pre-scaled)")
    assert_bits_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32), "x_scale (pre-scaled)")


@pytest.mark.parametrize("M,N,Kp", [(300, 700, 768), (257, 1030, 512)])
def test_gemm_bias(M, N, Kp):
    g = torch.Generator().manual_seed(M + N)
    a = torch.randint(-127, 128, (M, Kp), generator=g, dtype=torch.int32).to(torch.int8)
    b = torch.randint(-127, 128, (N, Kp), generator=g, dtype=torch.int32).to(torch.int8)
    sa = torch.rand(M, generator=g) * 1e-2
    sb = torch.rand(N, generator=g) * 1e-3
    bias = torch.randn(N + 1, generator=g)
    acc = oracle.gemm_s8(a.numpy(), b.numpy())
    ad, bd, sad, sbd = a.to(dev()), b.to(dev()), sa.to(dev()), sb.to(dev())
    biasd = bias.to(dev())
    for off in (0, 1):                              # 16-byte aligned bias, and 4-byte aligned
        bv = biasd[off:off + N]
        for ldc in (N + 9, (N + 7) // 8 * 8 + 8):
            for odt in (synth.DT_BF16, synth.DT_FP16, synth.DT_FP32):
                tdt = synth.TORCH_DTYPE[odt]
                full = torch.full((M, ldc), 7, dtype=tdt, device=dev())
                c = full[:, :N]
                say(f"cr_gemm_s8_rowscale_bias M={M} N={N} K_pad={Kp} out={odt} ldc={ldc} bias+{off}")
                rbl.cr_gemm_s8_rowscale_bias(ad, sad, bd, sbd, bv, c)
                torch.cuda.synchronize()
                fc = full.cpu()
                assert (fc[:, N:] == 7).all(), "columns past N were written"
                ref = oracle.epilogue(acc, sa.numpy(), sb.numpy(), odt, bias=bias[off:off + N].numpy())
                check_output(fc[:, :N], ref, odt, f"GEMM+bias M={M} N={N} out={odt} ldc={ldc}")


@pytest.mark.parametrize("swiglu", [False, True])
def test_layer_prescale_bias(swiglu):
    M, N, K = 300, 1000, 1000
    w, x, p = _layer_inputs(M, N, K, synth.DT_BF16, swiglu, 21)
    g = torch.Generator().manual_seed(21)
    c = (torch.rand(K, generator=g) + 0.5).to(torch.float32)
    bias = torch.randn(N, generator=g)
    xd, cd, sd = x.to(dev()), p.codes.to(dev()), p.sf.to(dev())
    gs = torch.tensor([p.g], dtype=torch.float32, device=dev())
    aux = torch.cuda.Stream()
    outs = []
    for mt, use_aux in [(0, False), (256 * 1024, True)]:
        say(f"cr_linear_nvfp4_ex M={M} N={N} K={K} swiglu={swiglu} pre_scale bias max_tile={mt} aux={use_aux}")
        outs.append(rbl.linear_nvfp4(xd, cd, sd, gs, K, out_dtype=torch.float32, swiglu=swiglu, max_tile_bytes=mt,
                                     aux_stream=aux if use_aux else None, pre_scale=c.to(dev()),
                                     bias=bias.to(dev())))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    ref = oracle.linear_nvfp4(synth.bits_u16(x), synth.DT_BF16, K, swiglu, p.codes.numpy(), p.sf.numpy(),
                              p.g, synth.DT_FP32, pre_scale=c.numpy(), bias=bias.numpy())
    check_output(outs[0], ref, synth.DT_FP32, "layer output (pre-scale, bias)")


# ----------------------------------------------------- block-transposed order ----

def _block_transposed(codes: np.ndarray) -> np.ndarray:
    """Natural-order codes [rows, K_pad] -> block-transposed order: column 16t + j of each
    256-column block holds element 16j + t."""
    r, kp = codes.shape
    return codes.reshape(r, kp // 256, 16, 16).transpose(0, 1, 3, 2).reshape(r, kp).copy()


@pytest.mark.parametrize("dt,M,K,swiglu,forced", [(synth.DT_BF16, 37, 300, False, False),
                                                  (synth.DT_BF16, 6, 700, True, False),
                                                  (synth.DT_FP16, 3, 20000, False, False),
                                                  (synth.DT_BF16, 5, 14336, True, True)])
def test_block_transposed_activation(dt, M, K, swiglu, forced):
    cols = 2 * K if swiglu else K
    x = make_x(M, cols, dt, seed=K + 5, ld=(cols // 8 + 1) * 8, special=True)
    flags = rbl.CR_FLAG_BLOCK_TRANSPOSED | (rbl.CR_FLAG_FORCE_TWO_PASS if forced else 0)
    say(f"cr_quant_act block-transposed dt={dt} M={M} K={K} swiglu={swiglu} forced={forced}")
    q, s = rbl.quant_act(x.to(dev()), K, swiglu=swiglu, flags=flags)
    torch.cuda.synchronize()
    rq, rs = oracle.quant_act(host_bits(x, dt), dt, K, swiglu=swiglu)
    assert_bits_equal(q.cpu().numpy(), _block_transposed(rq), "x_s8 (block-transposed)")
    assert_bits_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32), "x_scale (block-transposed)")


@pytest.mark.parametrize("N,K", [(300, 1000), (40, 20000), (64, 14336)])
def test_block_transposed_weight_and_gemm(N, K):
    g = torch.Generator().manual_seed(N * 3 + K)
    w = 0.02 * torch.randn(N, K, generator=g)
    p = synth.nvfp4_encode(w, garbage_seed=N)
    gs = torch.tensor([p.g], dtype=torch.float32, device=dev())
    say(f"cr_prep_weight_nvfp4 block-transposed N={N} K={K}")
    qt, st = rbl.prep_weight_nvfp4(p.codes.to(dev()), p.sf.to(dev()), gs, K, flags=rbl.CR_FLAG_BLOCK_TRANSPOSED)
    qn, sn = rbl.prep_weight_nvfp4(p.codes.to(dev()), p.sf.to(dev()), gs, K)
    x = make_x(65, K, synth.DT_BF16, seed=K)
    xt, xst = rbl.quant_act(x.to(dev()), K, flags=rbl.CR_FLAG_BLOCK_TRANSPOSED)
    xn, xsn = rbl.quant_act(x.to(dev()), K)
    acc_t = torch.empty(65, N, dtype=torch.int32, device=dev())
    acc_n = torch.empty(65, N, dtype=torch.int32, device=dev())
    say(f"cr_gemm_s8_rowscale int32, both operands block-transposed vs natural, N={N} K={K}")
    rbl.cr_gemm_s8_rowscale(xt, xst, qt, st, acc_t)
    rbl.cr_gemm_s8_rowscale(xn, xsn, qn, sn, acc_n)
    torch.cuda.synchronize()
    rq, rs = oracle.prep_weight_nvfp4(p.codes.numpy(), p.sf.numpy(), p.g, K)
    assert_bits_equal(qt.cpu().numpy(), _block_transposed(rq), "w_s8 (block-transposed)")
    assert_bits_equal(st.cpu().numpy().view(np.uint32), rs.view(np.uint32), "w_scale (block-transposed)")
    assert_bits_equal(acc_t.cpu().numpy(), acc_n.cpu().numpy(), "int32 sums, transposed vs natural order")


# ------------------------------------------------------ rows per workgroup sweep ----

@pytest.mark.parametrize("nb", list(range(1, 65)))
def test_every_short_row_shape_bit_exact(nb):
    """Rows of 1..64 blocks (ragged K = 256 nb - 7): up to 32 blocks several rows share a
    workgroup; SwiGLU rows of 33..64 blocks hold one block per lane group, plain activation
    and weight rows two.
    Activation, SwiGLU, weight and row-maximum preparation, bit-exact against the oracle,
    with a row count that leaves the last set of rows of a workgroup incomplete."""
    K = 256 * nb - 7
    M = 37
    ld = (2 * K + 7) // 8 * 8 + 8
    g = torch.Generator().manual_seed(nb)
    h = (torch.randn(M, ld, generator=g) * 2).to(torch.bfloat16)
    h[3] = 0.0
    hb = synth.bits_u16(h)
    say(f"short rows nb={nb}: quant_act / swiglu")
    q, s = rbl.quant_act(h.to(dev()), K, flags=rbl.CR_FLAG_BLOCK_TRANSPOSED if nb % 2 else 0)
    qs, ss = rbl.quant_act(h.to(dev()), K, swiglu=True)
    w = 0.02 * torch.randn(M + 4, K, generator=g)
    p = synth.nvfp4_encode(w, garbage_seed=nb)
    gs = torch.tensor([p.g], dtype=torch.float32, device=dev())
    say(f"short rows nb={nb}: prep_weight / weight_amax")
    qw, sw = rbl.prep_weight_nvfp4(p.codes.to(dev()), p.sf.to(dev()), gs, K)
    am = rbl.weight_amax_nvfp4(p.codes.to(dev()), p.sf.to(dev()), gs, K)
    torch.cuda.synchronize()
    rq, rs = oracle.quant_act(hb, synth.DT_BF16, K)
    if nb % 2:
        rq = rq.reshape(M, nb, 16, 16).transpose(0, 1, 3, 2).reshape(M, 256 * nb)
    assert_bits_equal(q.cpu().numpy(), rq, "x_s8")
    assert_bits_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32), "x_scale")
    rqs, rss = oracle.quant_act(hb, synth.DT_BF16, K, swiglu=True)
    assert_bits_equal(qs.cpu().numpy(), rqs, "swiglu x_s8")
    assert_bits_equal(ss.cpu().numpy().view(np.uint32), rss.view(np.uint32), "swiglu x_scale")
    rqw, rsw = oracle.prep_weight_nvfp4(p.codes.numpy(), p.sf.numpy(), p.g, K)
    assert_bits_equal(qw.cpu().numpy(), rqw, "w_s8")
    assert_bits_equal(sw.cpu().numpy().view(np.uint32), rsw.view(np.uint32), "w_scale")
    ra = oracle.weight_amax_nvfp4(p.codes.numpy(), p.sf.numpy(), p.g, K)
    assert_bits_equal(am.cpu().numpy().view(np.uint32), ra.view(np.uint32), "w_amax")


# ---------------------------------------------------------------- empty extents ----

def test_empty_batches_and_empty_outputs():
    """M = 0 (an empty batch) and N = 0 (no output columns) through the binding: empty
    results, nothing launched, and the next ordinary call on the stream is unaffected."""
    K, N, M = 700, 300, 40
    g = torch.Generator().manual_seed(9)
    p = synth.nvfp4_encode(0.02 * torch.randn(N, K, generator=g), garbage_seed=9)
    gs = torch.tensor([p.g], dtype=torch.float32, device=dev())
    cd, sfd = p.codes.to(dev()), p.sf.to(dev())
    x = make_x(M, K, synth.DT_BF16, seed=10, ld=704).to(dev())
    say("empty extents: quant_act / prep_weight / gemm / fused / linear with M = 0 or N = 0")
    q0, s0 = rbl.quant_act(x[:0], K)
    h0, hs0 = rbl.quant_act(torch.empty(0, 2 * K, dtype=torch.bfloat16, device=dev()), K, swiglu=True)
    qw0, sw0 = rbl.prep_weight_nvfp4(cd[:0], sfd[:0], gs, K)
    am0 = rbl.weight_amax_nvfp4(cd[:0], sfd[:0], gs, K)
    assert q0.shape == (0, 768) and s0.shape == (0,) and h0.shape == (0, 768) and hs0.shape == (0,)
    assert qw0.shape == (0, 768) and sw0.shape == (0,) and am0.shape == (0,)
    qx, sx = rbl.quant_act(x, K)
    qw, sw = rbl.prep_weight_nvfp4(cd, sfd, gs, K)
    assert rbl.gemm_s8_rowscale(qx[:0], sx[:0], qw, sw).shape == (0, N)
    assert rbl.gemm_s8_rowscale(qx, sx, qw[:0], sw[:0]).shape == (M, 0)
    assert rbl.gemm_nvfp4_fused(qx[:0], sx[:0], cd, sfd, gs, None, K).shape == (0, N)
    assert rbl.gemm_nvfp4_fused(qx, sx, cd[:0], sfd[:0], gs, None, K).shape == (M, 0)
    for rows in (0, 100):                            # empty batch on both paths' sides of 64
        xe = torch.empty(0, 704, dtype=torch.bfloat16, device=dev())[:, :K] if rows == 0 else x
        y = rbl.linear_nvfp4(xe, cd if rows == 0 else cd[:0], sfd if rows == 0 else sfd[:0], gs, K)
        assert y.shape == ((0, N) if rows == 0 else (M, 0))
    y = rbl.linear_nvfp4(x, cd, sfd, gs, K, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.linear_nvfp4(synth.bits_u16(x.cpu()), synth.DT_BF16, K, False, p.codes.numpy(), p.sf.numpy(),
                              p.g, synth.DT_FP32)
    check_output(y, ref, synth.DT_FP32, "layer output")


@pytest.mark.parametrize("F,flags", [(256, 0), (16384, 0), (16384, rbl.CR_FLAG_BLOCK_TRANSPOSED),
                                     (512, rbl.CR_FLAG_FORCE_TWO_PASS)])
def test_quant_act_swiglu_every_bf16_gate(F, flags):
    """Every finite bf16 gate pattern through the fused SwiGLU preparation (whose bf16 sigma
    comes from a table built in LDS): S8 codes and scales bit-exact against the oracle.  The
    value of each element is 2^-e for the gate's exponent e (clamped to +-100), so every
    product stays near 1 and no row overflows in the rotation; inf/NaN patterns are 0."""
    pat = np.arange(65536, dtype=np.uint32)
    gate = (pat << 16).view(np.float32).copy()
    gate[~np.isfinite(gate)] = 0.0
    e = np.clip(((pat >> 7) & 0xFF).astype(np.int64) - 127, -100, 100)
    value = np.ldexp(np.ones(65536), -e).astype(np.float32)
    M = 65536 // F
    h = torch.cat([torch.from_numpy(gate.reshape(M, F)), torch.from_numpy(value.reshape(M, F))], dim=1)
    h = h.to(torch.bfloat16)                        # both exact in bf16
    assert np.array_equal((synth.bits_u16(h)[:, :F].astype(np.uint32) << 16).view(np.float32), gate.reshape(M, F))
    say(f"cr_quant_act_swiglu all bf16 gate patterns F={F} flags={flags}")
    q, s = rbl.quant_act(h.to(dev()), F, swiglu=True, flags=flags)
    torch.cuda.synchronize()
    rq, rs = oracle.quant_act(synth.bits_u16(h), synth.DT_BF16, F, swiglu=True)
    if flags & rbl.CR_FLAG_BLOCK_TRANSPOSED:
        perm = np.arange(rq.shape[1]).reshape(-1, 16, 16).transpose(0, 2, 1).reshape(-1)
        rq = rq[:, perm]
    assert np.isfinite(rs).all()
    assert_bits_equal(q.cpu().numpy(), rq, "x_s8 (all bf16 gates)")
    assert_bits_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32), "x_scale (all bf16 gates)")


@pytest.mark.parametrize("dt", [synth.DT_BF16, synth.DT_FP16])
def test_quant_act_swiglu_two_pass_many_rows(dt):
    """SwiGLU rows of 67 blocks (two passes by size, and forced) in more rows than the device
    holds workgroups at once: with bf16 gates each workgroup builds the sigma table once and
    loops over rows (alternating reduction slots), with fp16 gates sigma is computed."""
    M, F = 700, 17000
    h = make_x(M, 2 * F, dt, seed=71, ld=2 * F + 8, special=True)
    rq, rs = oracle.quant_act(host_bits(h, dt), dt, F, swiglu=True)
    for flags in (0, rbl.CR_FLAG_FORCE_TWO_PASS):
        say(f"cr_quant_act_swiglu many rows dt={dt} M={M} F={F} flags={flags}")
        q, s = rbl.quant_act(h.to(dev()), F, swiglu=True, flags=flags)
        torch.cuda.synchronize()
        assert_bits_equal(q.cpu().numpy(), rq, f"x_s8 (swiglu, many rows, flags={flags})")
        assert_bits_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32), f"x_scale (swiglu, flags={flags})")