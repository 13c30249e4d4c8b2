"""The C-ABI library loads, exports every function include/convrot.h declares, carries
gfx950 code, and validates arguments on the host before anything is enqueued.

No computation runs here: the validation cases use fake (never dereferenced) pointer
values and return before any HIP call; the no-device case runs only where no GPU is
visible.
"""
import ctypes as C

import numpy as np
import pytest
import torch

import rotated_bit_linear_amd as rbl

OK, INV, DT, MIS, BIG, NODEV = 0, 1, 2, 3, 4, 5
A16 = 0x10000          # 16-byte aligned fake device address
ST = None              # default stream


def test_library_exports_header_functions():
    L = rbl.lib()
    names = rbl.header_functions()
    assert set(names) >= {"cr_prep_weight_nvfp4", "cr_quant_act", "cr_quant_act_swiglu",
                          "cr_gemm_s8_rowscale", "cr_linear_nvfp4", "cr_linear_nvfp4_workspace_bytes",
                          "cr_linear_nvfp4_plan", "cr_quant_act_ex", "cr_gemm_s8_rowscale_bias",
                          "cr_linear_nvfp4_ex", "cr_weight_amax_nvfp4", "cr_gemm_nvfp4_fused",
                          "cr_abi_version", "cr_status_string", "cr_padded_k"}
    for n in names:
        assert hasattr(L, n), n


def test_library_holds_gfx950_code():
    blob = open(rbl.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


def test_version_and_helpers():
    L = rbl.lib()
    assert L.cr_abi_version() == rbl.CR_ABI_VERSION
    assert [L.cr_padded_k(k) for k in (0, 1, 256, 257, 20000)] == [0, 256, 256, 512, 20224]
    assert L.cr_status_string(4) == b"CR_ERR_TOO_LARGE"


def qa(x=A16, dt=0, ld_x=512, M=4, K=512, q=A16, ld_q=512, s=A16, flags=0):
    return rbl.lib().cr_quant_act(x, dt, ld_x, M, K, q, ld_q, s, flags, ST)


def test_quant_act_validation():
    assert qa(x=None) == INV
    assert qa(M=-1) == INV
    assert qa(K=0) == INV
    assert qa(dt=3) == DT
    assert qa(ld_x=500) == INV            # ld_x < K
    assert qa(ld_q=256) == INV            # ld_s8 < K_pad
    assert qa(x=A16 + 2) == MIS
    assert qa(ld_x=513, K=512) == MIS      # 1026-byte rows
    assert qa(K=CR_BIG, ld_x=CR_BIG + 16, ld_q=CR_BIG + 256) == BIG
    assert qa(flags=4) == INV
    assert qa(q=A16 + 8) == MIS


CR_BIG = rbl.CR_MAX_K_PAD + 1


def test_swiglu_validation():
    L = rbl.lib()
    assert L.cr_quant_act_swiglu(A16, 0, 1000, 4, 512, A16, 512, A16, 0, ST) == INV   # ld_h < 2F
    assert L.cr_quant_act_swiglu(A16, 0, 1024, 4, 512, A16, 256, A16, 0, ST) == INV   # ld_s8 < F_pad
    assert L.cr_quant_act_swiglu(A16, 3, 1024, 4, 512, A16, 512, A16, 0, ST) == DT


def qx(x=A16, dt=0, ld_x=512, sw=0, M=4, K=512, pre=A16, q=A16, ld_q=512, s=A16, flags=0):
    return rbl.lib().cr_quant_act_ex(x, dt, ld_x, sw, M, K, pre, q, ld_q, s, flags, ST)


def test_quant_act_ex_validation():
    assert qx(pre=A16 + 2) == MIS           # pre-scale must be 4-byte aligned
    assert qx(x=None) == INV
    assert qx(sw=1) == INV                  # SwiGLU needs ld_x >= 2K
    assert qx(sw=1, ld_x=1024, ld_q=256) == INV
    assert qx(dt=3) == DT


def pw(codes=A16, ld=256, sf=A16, ld_sf=32, g=A16, n=8, K=512, q=A16, ld_q=512, s=A16, flags=0):
    return rbl.lib().cr_prep_weight_nvfp4(codes, ld, sf, ld_sf, g, n, K, q, ld_q, s, flags, ST)


def test_prep_weight_validation():
    assert pw(g=None) == INV
    assert pw(n=-1) == INV
    assert pw(ld=200) == INV               # < ceil(K/2)
    assert pw(ld_sf=31) == INV             # < ceil(K/16)
    assert pw(ld=264) == MIS               # not a multiple of 16
    assert pw(codes=A16 + 4) == MIS
    assert pw(K=CR_BIG, ld=CR_BIG, ld_sf=CR_BIG, ld_q=CR_BIG + 256) == BIG
    assert pw(flags=4) == INV
    assert pw(flags=2) != INV              # block-transposed order is a valid flag


def gm(a=A16, lda=512, sa=A16, b=A16, ldb=512, sb=A16, M=8, N=8, K=512, c=A16, dt=0, ldc=8):
    return rbl.lib().cr_gemm_s8_rowscale(a, lda, sa, b, ldb, sb, M, N, K, c, dt, ldc, ST)


def test_gemm_bias_validation():
    L = rbl.lib()

    def gb(bias=A16, dt=0, sa=A16):
        return L.cr_gemm_s8_rowscale_bias(A16, 512, sa, A16, 512, A16, bias, 8, 8, 512, A16, dt, 8, ST)
    assert gb(dt=3) == INV                 # no bias on the raw int32 accumulator
    assert gb(bias=A16 + 2) == MIS
    assert gb(sa=None) == INV


def test_gemm_validation():
    assert gm(K=500, lda=512, ldb=512) == INV      # K_pad not a multiple of 256
    assert gm(sa=None) == INV
    assert gm(ldc=7) == INV
    assert gm(dt=7) == DT
    assert gm(a=A16 + 1) == MIS
    assert gm(lda=520) == MIS
    assert gm(c=A16 + 1) == MIS
    assert gm(K=rbl.CR_MAX_K_PAD + 256, lda=rbl.CR_MAX_K_PAD + 256, ldb=rbl.CR_MAX_K_PAD + 256) == BIG
    # more 256 x 256 tiles than a dispatch's 32-bit work-item count allows (512 threads each)
    big = 1 << 21
    assert gm(M=big, N=big, ldc=big) == BIG
    assert gm(M=big, N=(1 << 21) // 256 * 2, ldc=big) != BIG   # 8192 x 16 tiles: fine


def test_layer_validation_and_workspace():
    L = rbl.lib()
    ws = L.cr_linear_nvfp4_workspace_bytes(65, 256, 512, 0)
    assert ws >= 65 * 512 + 65 * 4 + 256 * 512 + 256 * 4
    big = L.cr_linear_nvfp4_workspace_bytes(19989, 21504, 5376, 16 << 20)
    one = L.cr_linear_nvfp4_workspace_bytes(19989, 21504, 5376, 0)
    assert big < one                            # 16 MiB tiles: two 3072-row tiles
    args = dict(x=A16, dt=0, ldx=512, sw=0, M=65, K=512, w=A16, ldw=256, sf=A16, ldsf=32, g=A16, N=256,
                out=A16, odt=0, ldc=256, ws=0x100000, wsb=ws, mt=0, fl=0)

    def call(**kw):
        a = dict(args, **kw)
        return L.cr_linear_nvfp4(a["x"], a["dt"], a["ldx"], a["sw"], a["M"], a["K"], a["w"], a["ldw"], a["sf"],
                                 a["ldsf"], a["g"], a["N"], a["out"], a["odt"], a["ldc"], a["ws"], a["wsb"],
                                 a["mt"], a["fl"], ST, None)
    assert call(wsb=ws - 1) == BIG
    assert call(ws=0x100010) == MIS                # workspace must be 256-byte aligned
    assert call(odt=3) == DT
    assert call(ldc=255) == INV
    assert call(sw=1) == INV                       # SwiGLU needs ld_x >= 2K
    # the short-batch (decode-inside-GEMM) path validates the same way
    wsf = L.cr_linear_nvfp4_workspace_bytes(64, 256, 512, 0)
    assert wsf == 64 * 512 + 256
    assert call(M=64, wsb=wsf - 1) == BIG
    assert call(M=64, wsb=wsf, ws=0x100010) == MIS
    assert call(M=64, wsb=wsf, odt=3) == DT
    assert call(M=64, wsb=wsf, ldc=255) == INV
    assert call(M=64, wsb=wsf, sw=1) == INV
    assert call(M=64, wsb=wsf, ldw=264) == MIS
    assert call(M=64, wsb=wsf, fl=4) == INV


def test_layer_chunk_plan():
    # Without a device the planner assumes 256 compute units, as on MI355X.
    # QKV (M 19989, N 21504): 79 x 84 tiles take 26 rounds; two halves of 42 tile columns
    # take 13 + 13, so the weight is split and its second half is prepared during the
    # first GEMM.
    assert rbl.cr_linear_nvfp4_plan(19989, 21504, 5376) == (10752, 2)
    assert rbl.cr_linear_nvfp4_plan(4096, 21504, 5376) == (10752, 2)       # 6 rounds = 3 + 3
    # FFN down (N 5376): 79 x 21 tiles take 7 rounds, halves 4 + 4: not split.
    assert rbl.cr_linear_nvfp4_plan(19989, 5376, 14336) == (5376, 1)
    # one tile row of workgroups: a split would double the rounds
    assert rbl.cr_linear_nvfp4_plan(65, 512, 256) == (512, 1)
    assert rbl.cr_linear_nvfp4_plan(8192, 5000, 20000) == (5120, 1)
    # short batches decode the weight inside the GEMM: no chunks, a workspace of the S8
    # activation and its scales (256-byte aligned regions)
    assert rbl.cr_linear_nvfp4_plan(64, 512, 256) == (0, 0)
    assert rbl.cr_linear_nvfp4_plan(1, 21504, 5376) == (0, 0)
    assert rbl.cr_linear_nvfp4_workspace_bytes(64, 512, 256) == 64 * 256 + 256
    assert rbl.cr_linear_nvfp4_workspace_bytes(1, 1, 1) == 256 + 256
    # the tile bound chunks first: 16 MiB / 5376 B per row -> at most 3072 rows; 12 tile
    # columns per chunk take 7 x 4 = 28 rounds, which no lower height beats (3 columns tie)
    assert rbl.cr_linear_nvfp4_plan(19989, 21504, 5376, 16 << 20) == (3072, 7)
    # FFN down under 16 MiB (at most 1170 rows of 14336 bytes): 1024-row chunks take 2
    # rounds each (79 x 4 = 316 tiles), 11 in all; 768-row chunks take 1 each, 7 in all
    assert rbl.cr_linear_nvfp4_plan(19989, 5376, 14336, 16 << 20) == (768, 7)
    # a bound below one tile height still gives one 256-row chunk
    assert rbl.cr_linear_nvfp4_plan(300, 1000, 5376, 1) == (256, 4)
    # an empty layer: no chunks, no workspace
    assert rbl.cr_linear_nvfp4_plan(0, 256, 256) == (0, 0)
    assert rbl.cr_linear_nvfp4_plan(19989, 0, 5376) == (0, 0)
    assert rbl.cr_linear_nvfp4_workspace_bytes(0, 256, 256) == 0
    assert rbl.cr_linear_nvfp4_workspace_bytes(300, 0, 256) == 0
    with pytest.raises(rbl.CrError):
        rbl.cr_linear_nvfp4_plan(-1, 256, 256)
    with pytest.raises(rbl.CrError):
        rbl.cr_linear_nvfp4_plan(1, 256, 0)
    with pytest.raises(rbl.CrError):
        rbl.cr_linear_nvfp4_plan(1, 256, rbl.CR_MAX_K_PAD + 1)


def test_bounded_chunk_plan_takes_fewest_rounds():
    """Under a tile bound, the chunk height is the tallest of those (multiples of 256 rows,
    within the bound) whose GEMMs take the fewest rounds of workgroups over 256 CUs in all,
    checked by enumerating every height on random shapes."""
    rng = np.random.default_rng(7)

    def rounds(tiles):
        return -(-tiles // 256)

    for _ in range(400):
        M = int(rng.integers(65, 40000))
        N = int(rng.integers(1, 30000))
        kp = 256 * int(rng.integers(1, 80))
        bound = int(rng.integers(1, 256 * kp * 40))
        R, nch = rbl.cr_linear_nvfp4_plan(M, N, kp, bound)
        tm, tn = -(-M // 256), -(-N // 256)
        kmax = max(1, bound // kp // 256)
        if kmax >= tn:
            continue                                    # the whole weight fits the bound
        total = {k: (tn // k) * rounds(tm * k) + (rounds(tm * (tn % k)) if tn % k else 0)
                 for k in range(1, kmax + 1)}
        best = min(total.values())
        assert R % 256 == 0 and R // 256 <= kmax, (M, N, kp, bound, R)
        assert total[R // 256] == best, (M, N, kp, bound, R, best)
        assert all(total[k] > best for k in range(R // 256 + 1, kmax + 1)), (M, N, kp, bound, R)
        assert nch == -(-N // R)


def wa(codes=A16, ld=256, sf=A16, ld_sf=32, g=A16, n=8, K=512, a=A16, flags=0):
    return rbl.lib().cr_weight_amax_nvfp4(codes, ld, sf, ld_sf, g, n, K, a, flags, ST)


def test_weight_amax_validation():
    assert wa(a=None) == INV
    assert wa(g=None) == INV
    assert wa(n=-1) == INV
    assert wa(ld=200) == INV               # < ceil(K/2)
    assert wa(ld_sf=31) == INV             # < ceil(K/16)
    assert wa(ld=264) == MIS
    assert wa(a=A16 + 2) == MIS
    assert wa(K=CR_BIG, ld=CR_BIG, ld_sf=CR_BIG) == BIG
    assert wa(flags=4) == INV


def fz(a=A16, lda=512, sa=A16, codes=A16, ld=256, sf=A16, ld_sf=32, g=A16, am=A16, bias=None, M=8, N=40,
       K=512, c=A16, dt=0, ldc=40, flags=0):
    return rbl.lib().cr_gemm_nvfp4_fused(a, lda, sa, codes, ld, sf, ld_sf, g, am, bias, M, N, K, c, dt, ldc,
                                         flags, ST)


def test_gemm_fused_validation():
    assert fz(a=None) == INV
    assert fz(g=None) == INV
    assert fz(am=A16 + 2) == MIS
    assert fz(sa=None) == INV              # scales needed unless int32 out
    assert fz(dt=3, bias=A16) == INV       # no bias on the raw accumulator
    assert fz(dt=7) == DT
    assert fz(M=-1) == INV
    assert fz(N=-1) == INV
    assert fz(lda=256) == INV              # < K_pad
    assert fz(ld=200) == INV
    assert fz(ldc=39) == INV
    assert fz(lda=520) == MIS
    assert fz(c=A16 + 1) == MIS
    assert fz(bias=A16 + 2) == MIS
    assert fz(K=CR_BIG, lda=CR_BIG + 256, ld=CR_BIG, ld_sf=CR_BIG) == BIG
    assert fz(M=128 * 65535 + 1) == BIG    # workgroup rows of 128 activation rows
    n_big = 32 * (0xFFFFFFFF // 256) + 32  # one 32-row band more than 2^32 work-items allow
    assert fz(N=n_big, ldc=n_big) == BIG
    assert fz(flags=4) == INV


def test_empty_extents_are_no_ops():
    """M (or n_rows) = 0 or N = 0: CR_OK with nothing enqueued, buffers of zero size may be
    NULL; the arguments that do not depend on the empty extent are still checked, and K = 0
    or a negative size is still an error.  (Returns before any HIP call: safe without a GPU.)"""
    L = rbl.lib()
    N0 = None
    # activation preparation (plain, SwiGLU, pre-scaled) and the unfused SwiGLU
    assert qa(x=N0, M=0, q=N0, s=N0) == OK
    assert qa(x=N0, M=0, q=N0, s=N0, K=0) == INV
    assert qa(x=N0, M=0, q=N0, s=N0, dt=3) == DT
    assert qa(x=N0, M=0, q=N0, s=N0, flags=4) == INV
    assert qa(x=N0, M=0, q=N0, s=N0, ld_q=256) == INV
    assert L.cr_quant_act_swiglu(N0, 0, 1024, 0, 512, N0, 512, N0, 0, ST) == OK
    assert qx(x=N0, M=0, q=N0, s=N0, pre=N0) == OK
    assert L.cr_swiglu(N0, 0, 1024, 0, 512, N0, 512, ST) == OK
    # weight preparation and row maxima
    assert pw(codes=N0, sf=N0, g=N0, n=0, q=N0, s=N0) == OK
    assert pw(codes=N0, sf=N0, g=N0, n=0, q=N0, s=N0, ld=200) == INV
    assert wa(codes=N0, sf=N0, g=N0, n=0, a=N0) == OK
    # GEMMs: no rows, or no columns
    assert gm(a=N0, sa=N0, M=0, c=N0) == OK
    assert gm(b=N0, sb=N0, N=0, c=N0, ldc=0) == OK
    assert gm(a=N0, sa=N0, M=0, c=N0, dt=7) == DT
    assert gm(a=N0, sa=N0, M=0, c=N0, K=500, lda=512, ldb=512) == INV
    assert gm(M=-1) == INV
    assert fz(a=N0, sa=N0, M=0, c=N0) == OK
    assert fz(codes=N0, sf=N0, g=N0, am=N0, N=0, c=N0, ldc=0) == OK
    # the layer: empty batch or empty output, no workspace
    def layer(x=N0, M=0, N=256, out=N0, ws=N0, wsb=0, odt=0, dt=0, K=512, w=A16, sf=A16, g=A16):
        return L.cr_linear_nvfp4(x, dt, 512, 0, M, K, w, 256, sf, 32, g, N, out, odt, 256, ws, wsb, 0, 0, ST, None)
    assert layer() == OK
    assert layer(M=300, x=A16, N=0, w=N0, sf=N0, g=N0) == OK
    assert layer(odt=3) == DT
    assert layer(dt=5) == DT
    assert layer(K=0) == INV
    assert layer(M=-1) == INV
    assert layer(g=N0) == INV                       # N > 0: the weight is still required
    assert layer(M=300, N=0, w=N0, sf=N0, g=N0) == INV          # M > 0: x is not an empty buffer
    assert layer(x=A16 + 2) == MIS                  # strides and alignment are still checked
    assert L.cr_linear_nvfp4(N0, 0, 513, 0, 0, 512, A16, 256, A16, 32, A16, 256, N0, 0, 256, N0, 0, 0, 0, ST,
                             None) == MIS            # 1026-byte rows
    assert L.cr_linear_nvfp4_ex(N0, 0, 512, 0, 0, 512, N0, A16, 256, A16, 32, A16, 256, N0, N0, 0, 256,
                                N0, 0, 0, 0, ST, None) == OK
