// W4A8 GEMM on gfx950 matrix cores: C[m, n] = ((float)sum_k A[m, k] W[n, k]) * a_scale[m]
// * b_scale[n] with A the S8 activation codes and W the 4-bit weight codes (-7..7), stored
// packed two per byte (ComfyUI Turing Utils README: the ConvRot path dispatches W8A8, W4A8
// and W4A4 layers and ships a packed W4A8 kernel; the packed format is this library's own:
// 32-byte units of 64 codes holding the 16-code groups G0, G2, G1, G3, each group's codes
// j and 4 + j, 8 + j and 12 + j sharing a byte, low nibble first).
//
// gfx950 has no 4-bit integer matrix instruction, so the weight codes are widened to bytes
// in registers and fed to v_mfma_i32_32x32x32_i8 with the activation codes.  Widening keeps
// each nibble in the high half of its byte: (byte & 0xF0) read as int8 is 16 q exactly, so
// a nibble pair costs one AND (high nibble) or a shift and an AND (low nibble), with no sign
// extension.  The MFMAs then sum 16 q a; |16 * 7 * 127 * K_pad| < 2^31 for every accepted
// K_pad (<= 133120), and the epilogue shifts the sums back by 4 bits (exact).
//
// Memory: the packed weight is half the bytes of an S8 weight, so a 128-deep step of a
// 256 x 256 tile moves 32 KB of A and 16 KB of W by direct global->LDS loads, and three
// stages (144 KB) fit the 160 KB LDS: two steps are in flight while one is consumed.  A
// lane's weight fragment for two consecutive 32-deep slices is one 16-byte LDS read (the
// G0 G2 | G1 G3 order puts one k-half of both slices side by side), so each slice reads
// 2 KB of activation and 2 KB of weight fragments per wave instead of 2 KB + 4 KB.
// Tile order, waits and the epilogue are those of the S8 x S8 GEMM (gemm_common.hpp).
//
// The W4A4 form (A4 = true) takes the activation codes packed the same way: both operands
// are widened (products 256 qa qb; |256 * 7 * 7 * K_pad| < 2^31 for every accepted K_pad),
// the epilogue shifts by 8 bits, a stage is 16 KB + 16 KB, and the activation fragments of
// a slice pair are one 16-byte read like the weight's.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_common.hpp"
#include "kernels.hpp"

namespace convrot {
namespace {

using gemm::v4i;
using gemm::v16i;
using gemm::EPI_BYTES;

constexpr int W_M = 4, W_N = 2;                 // waves along M (activation rows), N
constexpr int T_M = 64, T_N = 128;              // wave tile
constexpr int F_M = T_M / 32, F_N = T_N / 32;   // 32 x 32 MFMA blocks per wave
constexpr int BM = W_M * T_M, BN = W_N * T_N;   // 256 x 256 workgroup tile
constexpr int BK = 128;                         // K per step
constexpr int NSTAGE = 3;
constexpr int NWAVE = W_M * W_N, NTHREAD = 64 * NWAVE;
constexpr int ROW_B = BK / 2;                   // LDS bytes per weight row of a stage
constexpr int SB = BN * ROW_B;
constexpr int KS = BK / 32;                     // 32-deep slices per step (two per packed read)
static_assert(KS == 4, "the step below reads packed fragments for slices (0, 1) and (2, 3)");

// LDS of one form.  W4A8: the activation stages A0 A1 A2 (32 KB each), then the weight
// stages B0 B1 B2 (16 KB each); a DS instruction adds at most 65535 to its address
// register, so the fragment reads use three address sets: activation rows (+0 for A0,
// +32768 for A1), activation rows + 64 KB (A2), and weight rows + 96 KB (+16384 per
// stage).  W4A4: A0 A1 A2 of 16 KB, then B0 B1 B2, two address sets.
template <bool A4>
struct Ring {
    static constexpr int ROW_A = A4 ? BK / 2 : BK;
    static constexpr int SA = BM * ROW_A, SSTAGE = SA + SB;
    static constexpr int A_BASE = 0, B_BASE = NSTAGE * SA;
    static constexpr int PIECES_A = SA / 1024, PIECES_B = SB / 1024;    // 1 KB DMA pieces per stage
    static constexpr int PPW = (PIECES_A + PIECES_B) / NWAVE;           // pieces per wave per stage
    static constexpr int POOL = NSTAGE * SSTAGE > NWAVE * EPI_BYTES + BN * 4 ? NSTAGE * SSTAGE
                                                                             : NWAVE * EPI_BYTES + BN * 4;
    static_assert((PIECES_A + PIECES_B) % NWAVE == 0, "DMA pieces split evenly over the waves");
    static_assert(POOL <= 160 * 1024, "LDS exceeds 160 KB");
    static_assert(PPW * (NSTAGE - 1) <= 63, "vmcnt range");
};
constexpr int POOL_BYTES = Ring<false>::POOL > Ring<true>::POOL ? Ring<false>::POOL : Ring<true>::POOL;
constexpr int MAX_PPW = Ring<false>::PPW > Ring<true>::PPW ? Ring<false>::PPW : Ring<true>::PPW;

// 16-byte chunk swizzles: activation rows have 8 chunks, weight rows 4 (chunk 2p + h is
// k-half h of slice pair p); both keep 32-row fragment reads free of bank conflicts
__device__ __forceinline__ int swz_a(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int swz_b(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// weight codes of one k-half of a slice (two dwords of a 16-byte fragment read) as bytes
// 16 q, in k order: the low nibbles of d0 (codes 0..3), its high nibbles (4..7), then d1
__device__ __forceinline__ v4i widen(uint32_t d0, uint32_t d1)
{
    constexpr uint32_t hi = 0xF0F0F0F0u;
    return v4i{(int32_t)((d0 << 4) & hi), (int32_t)(d0 & hi), (int32_t)((d1 << 4) & hi), (int32_t)(d1 & hi)};
}

template <int OUT, bool BIAS, bool A4>
__global__ __launch_bounds__(NTHREAD, 1)
void gemm_s8s4_kernel(const int8_t *__restrict__ A, int64_t lda, const float *__restrict__ sa,
                      const uint8_t *__restrict__ B, int64_t ldb, const float *__restrict__ sb,
                      const float *__restrict__ bias, int M, int N, int K_pad, void *__restrict__ C,
                      int64_t ldc, int tiles_m, int tiles_n)
{
    // The pool and the DMA source arrays have types that do not depend on the template
    // parameters: with a dependent operand type the host compilation drops the kernel's
    // launch stub without a diagnostic (the DMA builtin is checked against the host target
    // at instantiation).  One workgroup runs per CU either way.
    using R = Ring<A4>;
    __shared__ __attribute__((aligned(1024))) int8_t pool[POOL_BYTES];

    int tm, tn;
    gemm::tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / W_N, wn = wave % W_N;

    // ---- DMA assignment: wave w moves pieces w*PPW .. w*PPW+PPW-1 of a stage.  Piece
    //      p < PIECES_A: activation rows 8p .. 8p+7 (lane: row lane/8, LDS slot lane%8),
    //      packed activation rows 16p .. 16p+15 in the W4A4 form (as the weight's);
    //      otherwise weight rows 16q .. 16q+15, q = p - PIECES_A (lane: row lane/4, slot
    //      lane%4).  Slot s of row r holds logical chunk s ^ swz(r); rows past M or N read
    //      the last row (their results are never stored). ----
    const int8_t *gsrc[MAX_PPW];        // non-dependent types: see the pool above
    int ldst[MAX_PPW], kstep[MAX_PPW];
#pragma unroll
    for (int j = 0; j < R::PPW; j++) {
        const int p = wave * R::PPW + j;
        if (A4 && p < R::PIECES_A) {
            const int r = 16 * p + (lane >> 2);
            const int chunk = (lane & 3) ^ swz_b(r);
            gsrc[j] = A + (int64_t)min(m0 + r, M - 1) * lda + chunk * 16;
            ldst[j] = R::A_BASE + p * 1024;
            kstep[j] = BK / 2;
        } else if (p < R::PIECES_A) {
            const int r = 8 * p + (lane >> 3);
            const int chunk = (lane & 7) ^ swz_a(r);
            gsrc[j] = A + (int64_t)min(m0 + r, M - 1) * lda + chunk * 16;
            ldst[j] = R::A_BASE + p * 1024;
            kstep[j] = BK;
        } else {
            const int q = p - R::PIECES_A;
            const int r = 16 * q + (lane >> 2);
            const int chunk = (lane & 3) ^ swz_b(r);
            gsrc[j] = reinterpret_cast<const int8_t *>(B) + (int64_t)min(n0 + r, N - 1) * ldb + chunk * 16;
            ldst[j] = R::B_BASE + q * 1024;
            kstep[j] = BK / 2;
        }
    }
    // step kt of the K loop reads the operands' step kt, or step last_step - kt when this
    // workgroup walks K backwards (gemm::k_reversed)
    const bool k_rev = gemm::k_reversed(blockIdx.x);
    const int last_step = K_pad / BK - 1;
    auto issue = [&](int s, int kt) {
        const int64_t ks = k_rev ? last_step - kt : kt;
#pragma unroll
        for (int j = 0; j < R::PPW; j++) {
            const int stage_off = ldst[j] < R::B_BASE ? s * R::SA : s * SB;
            __builtin_amdgcn_global_load_lds(gsrc[j] + ks * kstep[j], pool + ldst[j] + stage_off, 16, 0, 0);
        }
    };

    // ---- fragment offsets inside a stage: row = base + (lane & 31); activation chunk
    //      2 ks + (lane >> 5) of slice ks, weight chunk 2 p + (lane >> 5) of slice pair p ----
    const int frow = lane & 31, fhalf = lane >> 5;
    uint32_t adrA[KS][F_M], adrA2[KS][F_M], adrB[KS / 2][F_N];
#pragma unroll
    for (int ks = 0; ks < KS; ks++)
#pragma unroll
        for (int i = 0; i < F_M; i++) {
            const int r = wm * T_M + i * 32 + frow;
            if constexpr (A4) {
                // packed rows: chunk 2 p + (lane >> 5) of slice pair p (entries ks >= 2 unused)
                adrA[ks][i] = (uint32_t)(uintptr_t)pool + R::A_BASE + r * R::ROW_A + (((2 * (ks & 1) + fhalf) ^ swz_b(r)) << 4);
            } else {
                adrA[ks][i] = (uint32_t)(uintptr_t)pool + R::A_BASE + r * R::ROW_A + (((2 * ks + fhalf) ^ swz_a(r)) << 4);
                adrA2[ks][i] = adrA[ks][i] + 2 * R::SA;
            }
        }
#pragma unroll
    for (int pp = 0; pp < KS / 2; pp++)
#pragma unroll
        for (int j = 0; j < F_N; j++) {
            const int r = wn * T_N + j * 32 + frow;
            adrB[pp][j] = (uint32_t)(uintptr_t)pool + R::B_BASE + r * ROW_B + (((2 * pp + fhalf) ^ swz_b(r)) << 4);
        }

    v16i acc[F_M][F_N];
#pragma unroll
    for (int i = 0; i < F_M; i++)
#pragma unroll
        for (int j = 0; j < F_N; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0;

    v4i fa[2][F_M], fb[2][F_N];      // fragments of even (0) and odd (1) slices
    v4i braw[F_N];                    // weight fragment reads of one slice pair
    v4i araw[F_M];                    // packed activation reads of one slice pair (W4A4)
    // LDS reads of stage s (a compile-time constant at every call, so the stage offset is
    // the instruction's immediate)
    auto lds = [](uint32_t a) { return reinterpret_cast<const __attribute__((address_space(3))) v4i *>(a); };
    auto read_a = [&](int s, int ks, int slot) {
#pragma unroll
        for (int i = 0; i < F_M; i++)
            fa[slot][i] = s == 2 ? *lds(adrA2[ks][i]) : *lds(adrA[ks][i] + s * R::SA);
    };
    auto read_b = [&](int s, int pp) {
#pragma unroll
        for (int j = 0; j < F_N; j++) braw[j] = *lds(adrB[pp][j] + s * SB);
    };
    auto widen_b = [&]() {
#pragma unroll
        for (int j = 0; j < F_N; j++) {
            fb[0][j] = widen((uint32_t)braw[j][0], (uint32_t)braw[j][1]);
            fb[1][j] = widen((uint32_t)braw[j][2], (uint32_t)braw[j][3]);
        }
    };
    // W4A4: packed activation fragments of slice pair pp, and their widening
    auto read_a4 = [&](int s, int pp) {
#pragma unroll
        for (int i = 0; i < F_M; i++) araw[i] = *lds(adrA[pp][i] + s * R::SA);
    };
    auto widen_a = [&]() {
#pragma unroll
        for (int i = 0; i < F_M; i++) {
            fa[0][i] = widen((uint32_t)araw[i][0], (uint32_t)araw[i][1]);
            fa[1][i] = widen((uint32_t)araw[i][2], (uint32_t)araw[i][3]);
        }
    };
    // MFMAs number t0 .. t1-1 of a slice (t = i*F_N + j); weight fragment first, so lane l
    // of block (i, j) holds output row l % 32 (the layout gemm::store_tile expects)
    auto mfmas = [&](int slot, int t0, int t1) {
#pragma unroll
        for (int t = 0; t < F_M * F_N; t++) {
            if (t < t0 || t >= t1) continue;
            const int i = t / F_N, j = t % F_N;
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[slot][j], fa[slot][i], acc[i][j], 0, 0, 0);
        }
    };

    // Prologue: steps 0 .. NSTAGE-1 requested (clamped to the last step), step 0 awaited, its
    // first fragments read.
    const int nk = K_pad / BK;                   // even, >= 2 (K_pad is a multiple of 256)
#pragma unroll
    for (int s = 0; s < NSTAGE; s++) issue(s, min(s, nk - 1));
    __builtin_amdgcn_s_waitcnt(gemm::waitcnt_vm((NSTAGE - 1) * R::PPW));
    gemm::barrier();
    if constexpr (A4) read_a4(0, 0);
    else read_a(0, 0, 0);
    read_b(0, 0);

    // One step k on stage S (= k % 3).  Before its last slice every wave waits for its own
    // DMA of step k+1 and meets the others at the barrier; after it, stage S is free and is
    // refilled with step k+3.  Near the end the refill target is clamped to the last step
    // (k+3 >= nk): those loads re-read valid rows into stages nobody reads again, and keep
    // every step identical (one step in flight beyond k+1 at each barrier), so the waits
    // need no special cases.  The last step refills nothing; the epilogue waits for all
    // loads before reusing the ring.
    constexpr int NMF = F_M * F_N;
    auto step = [&](auto S_, int k) {
        constexpr int S = decltype(S_)::value;
        constexpr int NX = (S + 1) % NSTAGE;
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            if (ks % 2 == 0) {                   // slices ks and ks+1 from the pair's reads
                if constexpr (A4) widen_a();
                widen_b();
            }
            if (ks < KS - 1) {
                if constexpr (A4) {
                    if (ks == 1) read_a4(S, 1);
                } else {
                    read_a(S, ks + 1, (ks + 1) & 1);
                }
                if (ks == 1) read_b(S, 1);
                mfmas(ks & 1, 0, NMF);
                __builtin_amdgcn_sched_barrier(0);
            } else {
                // the first MFMA consumes this slice's fragments, so every LDS read of stage S
                // has completed before the barrier; it also covers part of the wait
                mfmas(ks & 1, 0, 1);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                __builtin_amdgcn_s_waitcnt(gemm::waitcnt_vm(R::PPW));
                gemm::barrier();
                if constexpr (A4) read_a4(NX, 0);
                else read_a(NX, 0, 0);
                read_b(NX, 0);
                mfmas(ks & 1, 1, NMF);
                if (k + 1 < nk) issue(S, min(k + NSTAGE, nk - 1));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    int kt = 0;
    for (; kt + NSTAGE <= nk; kt += NSTAGE) {
        step(C0{}, kt);
        step(C1{}, kt + 1);
        step(C2{}, kt + 2);
    }
    if (kt < nk) step(C0{}, kt);
    if (kt + 1 < nk) step(C1{}, kt + 1);
    __builtin_amdgcn_s_waitcnt(gemm::waitcnt_vm(0));   // the clamped re-reads have landed

    // ---- epilogue (gemm::store_tile) on the idle ring: wave w's tile at w * EPI_BYTES, the
    //      bias values after the eight tiles; the sums are 16 (W4A4: 256) times too large ----
    const int nbase = n0 + wn * T_N;
    gemm::EpiScales<F_M, F_N> esc;
    gemm::load_scales<OUT, F_M, F_N>(esc, sa, sb, m0 + wm * T_M, nbase, frow, fhalf, M, N);
    __builtin_amdgcn_s_waitcnt(gemm::waitcnt_lgkm0());
    gemm::barrier();                             // every wave is done with the ring
    float *const bias_lds = reinterpret_cast<float *>(pool + NWAVE * EPI_BYTES);
    if constexpr (BIAS) {
        if (tid < BN) bias_lds[tid] = (n0 + tid < N) ? bias[n0 + tid] : 0.0f;
        gemm::barrier();
    }
    constexpr int ES = (OUT == 0 || OUT == 1) ? 2 : 4;
    const bool vec_ok = (((uintptr_t)C) % 16 == 0) && ((ldc * ES) % 16 == 0);
    const bool interior = vec_ok && m0 + BM <= M && n0 + BN <= N;
    gemm::store_tile<OUT, BIAS, F_M, F_N, T_N, A4 ? 8 : 4>(acc, esc, pool + wave * EPI_BYTES, bias_lds + wn * T_N, C, ldc,
                                                  m0 + wm * T_M, nbase, M, N, interior, vec_ok, lane);
}

template <int OUT, bool BIAS, bool A4>
void launch_one(const dim3 &grid, hipStream_t st, const int8_t *A, int64_t lda, const float *sa, const uint8_t *B,
                int64_t ldb, const float *sb, const float *bias, int64_t M, int64_t N, int64_t K_pad, void *C,
                int64_t ldc, int tiles_m, int tiles_n)
{
    hipLaunchKernelGGL((gemm_s8s4_kernel<OUT, BIAS, A4>), grid, dim3(NTHREAD), 0, st, A, lda, sa, B, ldb, sb, bias,
                       (int)M, (int)N, (int)K_pad, C, ldc, tiles_m, tiles_n);
}

using LaunchFn = void (*)(const dim3 &, hipStream_t, const int8_t *, int64_t, const float *, const uint8_t *,
                         int64_t, const float *, const float *, int64_t, int64_t, int64_t, void *, int64_t, int, int);

// the instantiation for one output dtype, bias and form (nullptr: no int32 output with bias)
LaunchFn pick(int out_dtype, bool bias, bool a4)
{
    switch (out_dtype) {
    case 0: return bias ? (a4 ? launch_one<0, true, true> : launch_one<0, true, false>)
                        : (a4 ? launch_one<0, false, true> : launch_one<0, false, false>);
    case 1: return bias ? (a4 ? launch_one<1, true, true> : launch_one<1, true, false>)
                        : (a4 ? launch_one<1, false, true> : launch_one<1, false, false>);
    case 2: return bias ? (a4 ? launch_one<2, true, true> : launch_one<2, true, false>)
                        : (a4 ? launch_one<2, false, true> : launch_one<2, false, false>);
    case 3: return bias ? nullptr : (a4 ? launch_one<3, false, true> : launch_one<3, false, false>);
    default: return nullptr;
    }
}

hipError_t launch_form(bool a4, const int8_t *A, int64_t lda, const float *sa, const uint8_t *B, int64_t ldb,
                       const float *sb, const float *bias, int64_t M, int64_t N, int64_t K_pad, void *C,
                       int out_dtype, int64_t ldc, hipStream_t st)
{
    const LaunchFn fn = pick(out_dtype, bias != nullptr, a4);
    if (!fn) return hipErrorInvalidValue;
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    fn(dim3((unsigned)(tiles_m * tiles_n)), st, A, lda, sa, B, ldb, sb, bias, M, N, K_pad, C, ldc, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_s8s4(const int8_t *A, int64_t lda, const float *sa, const uint8_t *B, int64_t ldb,
                            const float *sb, const float *bias, int64_t M, int64_t N, int64_t K_pad, void *C,
                            int out_dtype, int64_t ldc, hipStream_t st)
{
    return launch_form(false, A, lda, sa, B, ldb, sb, bias, M, N, K_pad, C, out_dtype, ldc, st);
}

hipError_t launch_gemm_s4s4(const uint8_t *A, int64_t lda, const float *sa, const uint8_t *B, int64_t ldb,
                            const float *sb, const float *bias, int64_t M, int64_t N, int64_t K_pad, void *C,
                            int out_dtype, int64_t ldc, hipStream_t st)
{
    return launch_form(true, reinterpret_cast<const int8_t *>(A), lda, sa, B, ldb, sb, bias, M, N, K_pad, C,
                             out_dtype, ldc, st);
}

}  // namespace convrot
