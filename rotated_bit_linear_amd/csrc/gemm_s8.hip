// Row-scaled INT8 GEMM on gfx950 matrix cores: C[m, n] = ((float)sum_k A[m,k] B[n,k])
// * a_scale[m] * b_scale[n], with the dequantization fused into the epilogue so the
// int32 accumulator never reaches memory (ComfyUI Turing Utils README, "Load ConvRot
// DiT ..." bullet: row-scaled INT8 GEMM over the rotated S8 operands; MiniMax H3
// explainer, fused-kernel paragraph: rescaling inside the matmul).
//
// Tiling: a BM x BN output tile per workgroup, WAVES_M x WAVES_N waves, each wave a
// (WT_M/32) x (WT_N/32) grid of v_mfma_i32_32x32x32_i8.  K advances BK bytes per step
// through an LDS ring of STAGES stages filled by direct global->LDS loads
// (global_load_lds_dwordx4: every lane moves 16 bytes, a wave fills 1 KB of LDS), so no
// VGPR staging is needed and STAGES-1 steps are in flight while one is consumed.
// LDS rows hold BK bytes (BK/16 chunks of 16 B); chunk c of row r lives at c ^ swz(r),
// which keeps the 32-row fragment reads bank-conflict free with 32 or 64 banks; the
// global side of each DMA lane picks the chunk that lands in its LDS slot, so every
// group of BK/16 lanes still reads one contiguous BK-byte row segment.
// Software pipeline of one step k (BK/32 slices of 32 along K, ks = 0 .. KS-1):
//   read fragments (k, ks+1) || MFMAs on (k, ks)          for ks < KS-1
//   wait for the own DMA of step k+1, barrier (every wave is past its reads of stage k),
//   DMA of step k+STAGES into stage k, read fragments (k+1, 0) || MFMAs on (k, KS-1)
// so LDS latency, the barrier and the DMA issue all overlap queued MFMA work.
// Tiles are assigned so that all XCDs (workgroup id mod 8 on this part) work on one chip
// block at a time, each on a compact sub-block: L2 reuse inside an XCD, and one MALL-resident
// working set for the whole chip (the XCDs form a 2 x 4 grid over a square chip block, so a
// round of workgroups touches as few distinct operand bands as possible).  Every other
// generation of an XCD's workgroups walks K backwards (gemm::k_reversed).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_common.hpp"
#include "kernels.hpp"

#ifndef CONVROT_GEMM_WAVES_M
#define CONVROT_GEMM_WAVES_M 4
#endif
#ifndef CONVROT_GEMM_WAVES_N
#define CONVROT_GEMM_WAVES_N 2
#endif
#ifndef CONVROT_GEMM_WT_M
#define CONVROT_GEMM_WT_M 64
#endif
#ifndef CONVROT_GEMM_WT_N
#define CONVROT_GEMM_WT_N 128
#endif
#ifndef CONVROT_GEMM_BK
#define CONVROT_GEMM_BK 128
#endif
#ifndef CONVROT_GEMM_STAGES
#define CONVROT_GEMM_STAGES 2
#endif

namespace convrot {

using gemm::v4i;
using gemm::v16i;
using gemm::waitcnt_vm;
using gemm::waitcnt_lgkm0;
using gemm::read_groups;
using gemm::EPI_BYTES;

constexpr int WAVES_M = CONVROT_GEMM_WAVES_M, WAVES_N = CONVROT_GEMM_WAVES_N;
constexpr int WT_M = CONVROT_GEMM_WT_M, WT_N = CONVROT_GEMM_WT_N;
constexpr int FM = WT_M / 32, FN = WT_N / 32;      // MFMA tiles per wave
constexpr int GBM = WAVES_M * WT_M, GBN = WAVES_N * WT_N, GBK = CONVROT_GEMM_BK;
constexpr int GWAVES = WAVES_M * WAVES_N;
constexpr int GTHREADS = 64 * GWAVES;
constexpr int GSTAGES = CONVROT_GEMM_STAGES;
constexpr int KS = GBK / 32;                       // 32-deep MFMA slices per step
constexpr int CPR = GBK / 16;                      // 16-byte chunks per LDS row
constexpr int RPP = 1024 / GBK;                    // rows per 1 KB DMA piece
constexpr int STAGE_A = GBM * GBK, STAGE_B = GBN * GBK;
constexpr int PIECES = (STAGE_A + STAGE_B) / 1024;  // 1 KB DMA pieces per stage
constexpr int PPW = PIECES / GWAVES;                 // pieces per wave per stage
static_assert(GBK == 64 || GBK == 128, "BK is 64 or 128");
static_assert(256 % (GBK * GSTAGES) == 0, "a K_pad multiple of 256 must be whole groups of stages");
static_assert(PIECES % GWAVES == 0 && (STAGE_A / 1024) % PPW == 0, "DMA pieces must split evenly");
static_assert(GSTAGES * (STAGE_A + STAGE_B) <= 160 * 1024, "LDS ring exceeds 160 KB");
static_assert(PPW * (GSTAGES - 1) <= 63, "vmcnt range");
static_assert(KS % 2 == 0, "fragment register sets alternate per slice");

// chunk swizzle of an LDS row: for 4 chunks, rows 0..7 (and 0..15 in pairs) get distinct
// bank groups; for 8 chunks, rows 0..7 and the even/odd rows of 0..15 do.
__device__ __forceinline__ int gswz(int row)
{
    if constexpr (CPR == 4) return ((row >> 1) ^ (row >> 2)) & 3;
    else return (row ^ (row >> 3)) & 7;
}

template <int OUT, bool BIAS>
__global__ __launch_bounds__(GTHREADS, 1)
void gemm_s8_kernel(const int8_t *__restrict__ A, int64_t lda, const float *__restrict__ sa,
                    const int8_t *__restrict__ B, int64_t ldb, const float *__restrict__ sb,
                    const float *__restrict__ bias, int M, int N, int K_pad, void *__restrict__ C,
                    int64_t ldc, int tiles_m, int tiles_n)
{
    __shared__ __attribute__((aligned(1024))) int8_t lA0[STAGE_A];
    __shared__ __attribute__((aligned(1024))) int8_t lA1[STAGE_A];
    __shared__ __attribute__((aligned(1024))) int8_t lB0[STAGE_B];
    __shared__ __attribute__((aligned(1024))) int8_t lB1[STAGE_B];
#if CONVROT_GEMM_STAGES == 4
    __shared__ __attribute__((aligned(1024))) int8_t lA2[STAGE_A];
    __shared__ __attribute__((aligned(1024))) int8_t lA3[STAGE_A];
    __shared__ __attribute__((aligned(1024))) int8_t lB2[STAGE_B];
    __shared__ __attribute__((aligned(1024))) int8_t lB3[STAGE_B];
    int8_t *const stA[GSTAGES] = {lA0, lA1, lA2, lA3};
    int8_t *const stB[GSTAGES] = {lB0, lB1, lB2, lB3};
#else
    int8_t *const stA[GSTAGES] = {lA0, lA1};
    int8_t *const stB[GSTAGES] = {lB0, lB1};
#endif

    // ---- tile id: XCD-aware order (gemm::tile_of) ----
    int tm, tn;
    gemm::tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * GBM, n0 = tn * GBN;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    // ---- DMA assignment: wave w moves pieces w*PPW .. w*PPW+PPW-1 of the stage (A pieces
    //      first, then B), each piece RPP rows x BK bytes; lane p covers row p/CPR of a
    //      piece and the LDS slot p%CPR, which holds logical chunk (p%CPR) ^ swz(row) ----
    const int piece0 = wave * PPW;
    const bool dma_a = piece0 < STAGE_A / 1024;
    const int prow = lane / CPR;
    const int8_t *gsrc[PPW];
#pragma unroll
    for (int j = 0; j < PPW; j++) {
        if (dma_a) {
            const int r = (piece0 + j) * RPP + prow;                          // row inside the tile
            const int chunk = (lane % CPR) ^ gswz(r);
            gsrc[j] = A + (int64_t)min(m0 + r, M - 1) * lda + chunk * 16;     // rows past M: row M-1
        } else {
            const int r = (piece0 - STAGE_A / 1024 + j) * RPP + prow;
            const int chunk = (lane % CPR) ^ gswz(r);
            gsrc[j] = B + (int64_t)min(n0 + r, N - 1) * ldb + chunk * 16;     // (masked at the store)
        }
    }
    const int dma_off = (dma_a ? piece0 : piece0 - STAGE_A / 1024) * 1024;

    // step kt of the K loop reads the operands' step kt, or step last_step - kt when this
    // workgroup walks K backwards (gemm::k_reversed)
    const bool k_rev = gemm::k_reversed(blockIdx.x);
    const int last_step = K_pad / GBK - 1;
    auto issue = [&](int s, int kt) {
        int8_t *dst = (dma_a ? stA[s] : stB[s]) + dma_off;
        const int64_t ko = (int64_t)(k_rev ? last_step - kt : kt) * GBK;
#pragma unroll
        for (int j = 0; j < PPW; j++)
            __builtin_amdgcn_global_load_lds(gsrc[j] + ko, dst + j * 1024, 16, 0, 0);
    };

    // ---- fragment offsets: row = base + (lane & 31), chunk = 2 ks + (lane >> 5) ----
    const int frow = lane & 31, fhalf = lane >> 5;
    int offA[KS][FM], offB[KS][FN];
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
        const int c = 2 * ks + fhalf;
#pragma unroll
        for (int i = 0; i < FM; i++) {
            const int r = wm * WT_M + i * 32 + frow;
            offA[ks][i] = r * GBK + ((c ^ gswz(r)) << 4);
        }
#pragma unroll
        for (int j = 0; j < FN; j++) {
            const int r = wn * WT_N + j * 32 + frow;
            offB[ks][j] = r * GBK + ((c ^ gswz(r)) << 4);
        }
    }

    v16i acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0;

    v4i fa[2][FM], fb[2][FN];
    auto read_frags = [&](int s, int ks, int slot) {
        const int8_t *sA = stA[s];
        const int8_t *sB = stB[s];
#pragma unroll
        for (int i = 0; i < FM; i++) fa[slot][i] = *reinterpret_cast<const v4i *>(sA + offA[ks][i]);
#pragma unroll
        for (int j = 0; j < FN; j++) fb[slot][j] = *reinterpret_cast<const v4i *>(sB + offB[ks][j]);
    };
    // MFMA roles: the weight fragment is the first operand and the activation fragment the
    // second, so D = (W X^T) per 32x32 block and lane l of a block holds output row
    // m = l%32 and the 4-column runs n = 8g + 4(l/32) + q (g, q = 0..3) in registers 4g+q.
    auto mfmas = [&](int slot) {
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
            for (int j = 0; j < FN; j++)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[slot][j], fa[slot][i], acc[i][j], 0, 0, 0);
    };
    // MFMAs number t0 .. t1-1 of a slice (t = i*FN + j)
    auto mfmas_range = [&](int slot, int t0, int t1) {
#pragma unroll
        for (int t = 0; t < FM * FN; t++) {
            if (t < t0 || t >= t1) continue;
            const int i = t / FN, j = t % FN;
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[slot][j], fa[slot][i], acc[i][j], 0, 0, 0);
        }
    };
    // scheduling hints: each slice opens with an MFMA (its operands were read during the
    // previous slice), then the next slice's fragment reads go out two at a time between
    // MFMAs, front-loaded so they land well before that slice starts; after a barrier the
    // DMA issues are spread over the remaining MFMAs
    constexpr int NFR = FM + FN, NMF = FM * FN;
    constexpr int RD_GROUPS = (NFR + 1) / 2;
    static_assert(RD_GROUPS + 1 < NMF, "need more MFMAs than read pairs per slice");
    auto interleave_reads = [&](bool with_dma, int pre) {
        read_groups<0, NFR>();
        if (with_dma) {
            constexpr int rest = NMF - 1 - RD_GROUPS;   // only used after the barrier (pre = 1)
#pragma unroll
            for (int t = 0; t < (PPW < rest ? PPW : rest); t++) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);                   // VMEM (DMA)
            }
            if constexpr (rest > PPW) __builtin_amdgcn_sched_group_barrier(0x008, rest - PPW, 0);
            else if constexpr (PPW > rest) __builtin_amdgcn_sched_group_barrier(0x010, PPW - rest, 0);
        } else if (pre == 0) {
            __builtin_amdgcn_sched_group_barrier(0x008, NMF - RD_GROUPS, 0);
        } else {
            __builtin_amdgcn_sched_group_barrier(0x008, NMF - 1 - RD_GROUPS, 0);
        }
    };
    // wait until this wave's DMA of a step has landed while `younger` later steps, issued
    // after it, may stay in flight (vmcnt counts this wave's outstanding DMAs)
    auto wait_dma = [&](int younger) {
        if (younger >= 3) __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * PPW));
        else if (younger == 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * PPW));
        else if (younger == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(PPW));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    };
    auto barrier = [&]() { gemm::barrier(); };

    // Prologue: every stage is free; steps 0..STAGES-1 are issued, step 0 awaited.
    // In step k the DMAs issued so far cover steps 0..min(k+STAGES-1, nk-1), so before the
    // barrier of step k+1 at most min(k+STAGES-1, nk-1) - (k+1) younger steps are in flight.
    const int nk = K_pad / GBK;   // a multiple of STAGES, >= STAGES (K_pad % 256 == 0)
#pragma unroll
    for (int s = 0; s < GSTAGES; s++) issue(s, s);
    wait_dma(GSTAGES - 1);
    barrier();
    read_frags(0, 0, 0);

    // One step on stage S; the loop runs whole groups of STAGES steps (stage index known at
    // compile time) and only the last group is peeled, which keeps every step free of
    // branches around its LDS reads.  Inside the loop STAGES-2 younger steps are in flight
    // at each barrier and the DMA of step k+STAGES always exists; in the last group
    // (k = nk-STAGES+S) STAGES-2-S remain and nothing new is issued.  The barrier opens the
    // last slice: its fragments were read during the previous slice.
    auto step = [&](auto S_, int kt, int younger, bool do_issue, bool last) {
        constexpr int S = decltype(S_)::value;
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            if (ks < KS - 1) {
                read_frags(S, ks + 1, (ks + 1) & 1);
                mfmas(ks & 1);
                interleave_reads(false, 0);
                __builtin_amdgcn_sched_barrier(0);
            } else if (!last) {
                // the first MFMA consumes this slice's fragments, so every LDS read of
                // stage S has completed before the barrier; it also keeps the matrix pipe
                // busy while the barrier resolves
                mfmas_range(ks & 1, 0, 1);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                wait_dma(younger);
                barrier();
                read_frags((S + 1) % GSTAGES, 0, 0);
                mfmas_range(ks & 1, 1, NMF);
                if (do_issue) issue(S, kt + S + GSTAGES);
                interleave_reads(do_issue, 1);
                __builtin_amdgcn_sched_barrier(0);
            } else {
                mfmas(ks & 1);
            }
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    int kt = 0;
    for (; kt < nk - GSTAGES; kt += GSTAGES) {
        step(I0{}, kt, GSTAGES - 2, true, false);
        step(I1{}, kt, GSTAGES - 2, true, false);
        if constexpr (GSTAGES == 4) {
            step(I2{}, kt, GSTAGES - 2, true, false);
            step(I3{}, kt, GSTAGES - 2, true, false);
        }
    }
    if constexpr (GSTAGES == 4) {
        step(I0{}, kt, 2, false, false);
        step(I1{}, kt, 1, false, false);
        step(I2{}, kt, 0, false, false);
        step(I3{}, kt, 0, false, true);
    } else {
        step(I0{}, kt, 0, false, false);
        step(I1{}, kt, 0, false, true);
    }

    // ---- epilogue through LDS: every wave owns EPI_BYTES of the (now idle) stage ring
    //      (gemm::store_tile); the scales are requested before the barrier so their latency
    //      overlaps the last MFMAs ----
    const int nbase = n0 + wn * WT_N;
    gemm::EpiScales<FM, FN> esc;
    gemm::load_scales<OUT, FM, FN>(esc, sa, sb, m0 + wm * WT_M, nbase, frow, fhalf, M, N);
    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0());
    barrier();                                     // every wave is done with the ring
    // the tile's GBN bias values go through LDS (past the last wave's epilogue tile) rather
    // than 64 more registers per lane
    constexpr int WPA = (GWAVES + 2 * GSTAGES - 1) / (2 * GSTAGES);   // waves per epilogue region
    static_assert(WPA * EPI_BYTES + GBN * 4 <= STAGE_B, "bias area fits beside the epilogue tiles");
    float *const bias_lds = reinterpret_cast<float *>(stB[GSTAGES - 1] + WPA * EPI_BYTES);
    if constexpr (BIAS) {
        const int tid_ = threadIdx.x;
        if (tid_ < GBN) bias_lds[tid_] = (n0 + tid_ < N) ? bias[n0 + tid_] : 0.0f;
        barrier();
    }
    static_assert(WPA * EPI_BYTES <= STAGE_A && WPA * EPI_BYTES <= STAGE_B, "epilogue tile fits the ring");
    int8_t *etile;
    switch (wave / WPA) {          // wave-uniform: a scalar branch
    case 0: etile = lA0; break;
    case 1: etile = lA1; break;
#if CONVROT_GEMM_STAGES == 4
    case 2: etile = lA2; break;
    case 3: etile = lA3; break;
    case 4: etile = lB0; break;
    case 5: etile = lB1; break;
    case 6: etile = lB2; break;
    default: etile = lB3; break;
#else
    case 2: etile = lB0; break;
    default: etile = lB1; break;
#endif
    }
    etile += (wave % WPA) * EPI_BYTES;
    constexpr int ES = (OUT == 0 || OUT == 1) ? 2 : 4;
    const bool vec_ok = (((uintptr_t)C) % 16 == 0) && ((ldc * ES) % 16 == 0);
    const bool interior = vec_ok && m0 + GBM <= M && n0 + GBN <= N;   // uniform fast path
    gemm::store_tile<OUT, BIAS, FM, FN, WT_N>(acc, esc, etile, bias_lds + wn * WT_N, C, ldc, m0 + wm * WT_M,
                                              nbase, M, N, interior, vec_ok, lane);
}

template <int OUT, bool BIAS>
static void launch_one(const dim3 &grid, const dim3 &block, hipStream_t st, const int8_t *A, int64_t lda,
                       const float *sa, const int8_t *B, int64_t ldb, const float *sb, const float *bias,
                       int64_t M, int64_t N, int64_t K_pad, void *C, int64_t ldc, int tiles_m, int tiles_n)
{
    hipLaunchKernelGGL((gemm_s8_kernel<OUT, BIAS>), grid, block, 0, st, A, lda, sa, B, ldb, sb, bias,
                       (int)M, (int)N, (int)K_pad, C, ldc, tiles_m, tiles_n);
}

hipError_t launch_gemm_s8(const int8_t *A, int64_t lda, const float *sa, const int8_t *B, int64_t ldb,
                          const float *sb, const float *bias, int64_t M, int64_t N, int64_t K_pad, void *C,
                          int out_dtype, int64_t ldc, hipStream_t st)
{
    const int tiles_m = (int)((M + GBM - 1) / GBM);
    const int tiles_n = (int)((N + GBN - 1) / GBN);
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(GTHREADS);
    const bool b = bias != nullptr;
    switch (out_dtype) {
    case 0: (b ? launch_one<0, true> : launch_one<0, false>)(grid, block, st, A, lda, sa, B, ldb, sb, bias, M, N, K_pad, C, ldc, tiles_m, tiles_n); break;
    case 1: (b ? launch_one<1, true> : launch_one<1, false>)(grid, block, st, A, lda, sa, B, ldb, sb, bias, M, N, K_pad, C, ldc, tiles_m, tiles_n); break;
    case 2: (b ? launch_one<2, true> : launch_one<2, false>)(grid, block, st, A, lda, sa, B, ldb, sb, bias, M, N, K_pad, C, ldc, tiles_m, tiles_n); break;
    case 3:
        if (b) return hipErrorInvalidValue;   // the raw accumulator takes no bias
        launch_one<3, false>(grid, block, st, A, lda, sa, B, ldb, sb, bias, M, N, K_pad, C, ldc, tiles_m, tiles_n);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace convrot
