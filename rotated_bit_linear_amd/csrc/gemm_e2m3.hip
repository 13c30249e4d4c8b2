// W4A4 GEMM on the gfx950 6-bit floating-point matrix cores: C[m, n] = ((float)sum_k
// A[m, k] W[n, k]) * a_scale[m] * b_scale[n] with A and W 4-bit code rows (-7..7) stored as
// E2M3 fields (ComfyUI Turing Utils README: the ConvRot path dispatches W4A4 layers; the
// layout is this library's own: 96 bytes per 128 codes, each quarter of 32 codes a 192-bit
// field with code e in bits 6e..6e+5, the fields' first 16 bytes in the order Q0 Q2 Q1 Q3
// and then their last 8 bytes in the same order; rows stored in quads, the four rows' units
// of 128 codes side by side).
//
// Why quads: with rows stored one after another a 96-byte step segment of a row straddles
// cache lines, and the DMA's 1 KB requests touched about 18 lines each; the L1 then held
// the address unit back for about 40 % of the kernel's cycles.  Four rows' segments of one
// step are 384 contiguous bytes, three whole lines: 8 lines per request, as for the S8
// GEMM's 128-byte row segments, and the GEMM 10-11 % faster.
//
// Every code -7..7 is an E2M3 number, so v_mfma_f32_32x32x64_f8f6f4 (both operands E2M3)
// forms the products exactly; the fp32 sums are integers below 49 * K_pad < 2^23 for every
// accepted K_pad, so they are exact in any order and convert to the int32 sums exactly.  On
// this chip the instruction multiplies twice as many operand pairs per cycle as the INT8 one,
// and on small codes it draws less power per product.
//
// Tiles: 256 x 256, 8 waves of 64 x 128, a step of 128 codes (two 64-deep slices).  A lane's
// operand for one slice is its row's quarter: 16 bytes of head (one aligned 16-byte LDS read)
// and 8 bytes of tail (one 8-byte read).  A row's 96 bytes of a step are six 16-byte chunks
// (heads of Q0 Q2 Q1 Q3, then the two tail chunks [Q0 Q2] and [Q1 Q3]); the chunks of row r
// sit at LDS positions rotated by one bit of r (rot below), which spreads sixteen consecutive
// rows over all banks for the head reads.  Stages: 24 KB per operand, three stages (144 KB)
// in flight.
// Waits, refills, tile order and the epilogue follow the packed 4-bit GEMM (gemm_s8s4.hip).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_common.hpp"
#include "kernels.hpp"

namespace convrot {
namespace {

using gemm::v16i;
using gemm::EPI_BYTES;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i_ __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int W_M = 4, W_N = 2;                 // waves along M (activation rows), N
constexpr int T_M = 64, T_N = 128;              // wave tile
constexpr int F_M = T_M / 32, F_N = T_N / 32;   // 32 x 32 MFMA blocks per wave
constexpr int BM = W_M * T_M, BN = W_N * T_N;   // 256 x 256 workgroup tile
constexpr int BK = 128;                         // codes per step
constexpr int KS = BK / 64;                     // 64-deep slices per step
constexpr int NSTAGE = 3;
constexpr int NWAVE = W_M * W_N, NTHREAD = 64 * NWAVE;
constexpr int ROW = BK * 3 / 4;                 // 96 bytes of a row per step
constexpr int CHUNKS = ROW / 16;                // 6
constexpr int QUAD_STEP = 4 * ROW;              // a step of four rows stored together: 384 bytes
constexpr int SOP = BM * ROW;                   // one operand's stage: 24 KB
constexpr int A_BASE = 0, B_BASE = NSTAGE * SOP;
constexpr int POOL = 2 * NSTAGE * SOP;
constexpr int PIECES = SOP / 1024;              // 1 KB DMA pieces per operand and stage
constexpr int PPW = 2 * PIECES / NWAVE;         // pieces per wave per stage
static_assert(BM == BN, "one piece layout serves both operands");
static_assert((2 * PIECES) % NWAVE == 0 && PIECES % PPW == 0, "a wave's pieces belong to one operand");
static_assert(POOL <= 160 * 1024, "LDS ring exceeds 160 KB");
static_assert(NWAVE * EPI_BYTES + BN * 4 <= POOL, "epilogue tiles and bias fit the ring");
static_assert(PPW * (NSTAGE - 1) <= 63, "vmcnt range");
static_assert(KS == 2, "the step below has two slices");

// Rotation of row r's chunk positions: chunk c of row r sits at 16-byte slot
// 6 r + (c + rot(r)) mod 6.  The LDS has 64 banks of 4 bytes and a 16-byte read serves 16
// lanes (rows r0 .. r0+15, r0 % 16 == 0) per cycle.  6 r mod 16 is even and repeats after
// 8 rows, so rows r and r + 8 need rotations of different parity; with rot = bit 2 xor bit 3
// of r every aligned group of 16 rows (and of 8, for 32 banks) reads a chunk from 16 (8)
// different bank groups.  The 8-byte tail reads (32 lanes per cycle) meet each bank twice:
// a row's two tail halves share a chunk, so the 32 halves of one slice take only 16 bank
// pairs.
__device__ __forceinline__ int rot(int r) { return ((r >> 2) ^ (r >> 3)) & 1; }

template <int OUT, bool BIAS>
__global__ __launch_bounds__(NTHREAD, 1)
void gemm_e2m3_kernel(const uint8_t *__restrict__ A, int64_t lda, const float *__restrict__ sa,
                      const uint8_t *__restrict__ B, int64_t ldb, const float *__restrict__ sb,
                      const float *__restrict__ bias, int M, int N, int K_pad, void *__restrict__ C,
                      int64_t ldc, int tiles_m, int tiles_n)
{
    __shared__ __attribute__((aligned(1024))) int8_t pool[POOL];

    int tm, tn;
    gemm::tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / W_N, wn = wave % W_N;

    // ---- DMA assignment: wave w moves pieces w*PPW .. w*PPW+PPW-1 of a stage (pieces
    //      0..PIECES-1 activation rows, then weight rows).  Lane l of piece q fills LDS slot
    //      s = 64 q + l of its operand: row s / 6, position s % 6, which holds the row's
    //      chunk (position - rot(row)) mod 6.  Operand rows are stored in quads (row 4q + i
    //      at q * ld + 96 i, its steps 384 bytes apart), so a step of four rows is three whole
    //      128-byte lines.  Rows past M or N read the last row (their results are never
    //      stored). ----
    const uint8_t *gsrc[PPW];
    int ldst[PPW];
    const bool wave_a = wave * PPW < PIECES;
#pragma unroll
    for (int j = 0; j < PPW; j++) {
        const int q = (wave * PPW + j) % PIECES;
        const int s = 64 * q + lane;
        const int r = s / CHUNKS, pos = s % CHUNKS;
        const int chunk = (pos - rot(r) + CHUNKS) % CHUNKS;
        const int64_t rr = wave_a ? min(m0 + r, M - 1) : min(n0 + r, N - 1);
        gsrc[j] = (wave_a ? A : B) + (rr >> 2) * (wave_a ? lda : ldb) + (rr & 3) * ROW + chunk * 16;
        ldst[j] = (wave_a ? A_BASE : B_BASE) + q * 1024;
    }
    // step kt of the K loop reads the operands' step kt, or step last_step - kt when this
    // workgroup walks K backwards (gemm::k_reversed)
    const bool k_rev = gemm::k_reversed(blockIdx.x);
    const int last_step = K_pad / BK - 1;
    auto issue = [&](int s, int kt) {
        const int64_t ks = k_rev ? last_step - kt : kt;
#pragma unroll
        for (int j = 0; j < PPW; j++)
            __builtin_amdgcn_global_load_lds(gsrc[j] + ks * QUAD_STEP, pool + ldst[j] + s * SOP, 16, 0, 0);
    };

    // ---- fragment addresses: row = base + (lane & 31), lane half h = lane >> 5 reads the
    //      head chunk 2h + slice (+16 bytes for slice 1) and 8 bytes of tail chunk 4 + h
    //      (+8 for slice 1) ----
    const int frow = lane & 31, fhalf = lane >> 5;
    uint32_t adrHA[F_M], adrTA[F_M], adrHB[F_N], adrTB[F_N];
#pragma unroll
    for (int i = 0; i < F_M; i++) {
        const int r = wm * T_M + i * 32 + frow;
        const uint32_t row = (uint32_t)(uintptr_t)pool + A_BASE + r * ROW;
        adrHA[i] = row + ((2 * fhalf + rot(r)) << 4);
        adrTA[i] = row + (((4 + fhalf + rot(r)) % CHUNKS) << 4);
    }
#pragma unroll
    for (int j = 0; j < F_N; j++) {
        const int r = wn * T_N + j * 32 + frow;
        const uint32_t row = (uint32_t)(uintptr_t)pool + B_BASE + r * ROW;
        adrHB[j] = row + ((2 * fhalf + rot(r)) << 4);
        adrTB[j] = row + (((4 + fhalf + rot(r)) % CHUNKS) << 4);
    }

    v16f acc[F_M][F_N];
#pragma unroll
    for (int i = 0; i < F_M; i++)
#pragma unroll
        for (int j = 0; j < F_N; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    v4i_ ha[2][F_M], hb[2][F_N];     // heads of even (0) and odd (1) slices
    v2i ta[2][F_M], tb[2][F_N];      // tails
    auto lds16 = [](uint32_t a) { return *reinterpret_cast<const __attribute__((address_space(3))) v4i_ *>(a); };
    auto lds8 = [](uint32_t a) { return *reinterpret_cast<const __attribute__((address_space(3))) v2i *>(a); };
    // fragments of slice ks of stage s into slot ks (compile-time offsets: immediates), in
    // the order the MFMAs below first need them: A0 B0 B1 .. B(F_N-1) A1 .. A(F_M-1)
    auto read_a = [&](int s, int ks, int i) {
        ha[ks][i] = lds16(adrHA[i] + s * SOP + ks * 16);
        ta[ks][i] = lds8(adrTA[i] + s * SOP + ks * 8);
    };
    auto read = [&](int s, int ks) {
        read_a(s, ks, 0);
#pragma unroll
        for (int j = 0; j < F_N; j++) {
            hb[ks][j] = lds16(adrHB[j] + s * SOP + ks * 16);
            tb[ks][j] = lds8(adrTB[j] + s * SOP + ks * 8);
        }
#pragma unroll
        for (int i = 1; i < F_M; i++) read_a(s, ks, i);
    };
    // MFMAs t0 .. t1-1 of slice `slot` (t = i*F_N + j); weight operand first, so lane l of
    // block (i, j) holds output row l % 32 (the layout gemm::store_tile expects).  The two
    // upper dwords of an operand are not read for E2M3 inputs.
    auto mfmas = [&](int slot, int t0, int t1) {
#pragma unroll
        for (int t = 0; t < F_M * F_N; t++) {
            if (t < t0 || t >= t1) continue;
            const int i = t / F_N, j = t % F_N;
            const v8i a = __builtin_shufflevector(hb[slot][j], __builtin_shufflevector(tb[slot][j], tb[slot][j], 0, 1, -1, -1),
                                                  0, 1, 2, 3, 4, 5, -1, -1);
            const v8i b = __builtin_shufflevector(ha[slot][i], __builtin_shufflevector(ta[slot][i], ta[slot][i], 0, 1, -1, -1),
                                                  0, 1, 2, 3, 4, 5, -1, -1);
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][j], 2, 2, 0, 0, 0, 0);
        }
    };

    // Prologue: steps 0 .. NSTAGE-1 requested (clamped to the last step), step 0 awaited, its
    // first slice read.
    const int nk = K_pad / BK;                   // even, >= 2 (K_pad is a multiple of 256)
#pragma unroll
    for (int s = 0; s < NSTAGE; s++) issue(s, min(s, nk - 1));
    __builtin_amdgcn_s_waitcnt(gemm::waitcnt_vm((NSTAGE - 1) * PPW));
    gemm::barrier();
    read(0, 0);

    // One step k on stage S (= k % 3): slice 1's fragments are read while slice 0 multiplies;
    // before slice 1's MFMAs complete every wave waits for its own DMA of step k+1 and meets
    // the others at the barrier, then reads slice 0 of step k+1 and refills stage S with step
    // k+3 (clamped to the last step, as in gemm_s8s4.hip).
    constexpr int NMF = F_M * F_N;
    auto step = [&](auto S_, int k) {
        constexpr int S = decltype(S_)::value;
        constexpr int NX = (S + 1) % NSTAGE;
        read(S, 1);
        mfmas(0, 0, NMF);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(1, 0, 1);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_waitcnt(gemm::waitcnt_vm(PPW));
        gemm::barrier();
        read(NX, 0);
        mfmas(1, 1, NMF);
        if (k + 1 < nk) issue(S, min(k + NSTAGE, nk - 1));
        __builtin_amdgcn_sched_barrier(0);
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

    // ---- epilogue: the exact integer sums as int32, then gemm::store_tile ----
    v16i iacc[F_M][F_N];
#pragma unroll
    for (int i = 0; i < F_M; i++)
#pragma unroll
        for (int j = 0; j < F_N; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) iacc[i][j][r] = (int)acc[i][j][r];
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
    gemm::store_tile<OUT, BIAS, F_M, F_N, T_N, 0>(iacc, esc, pool + wave * EPI_BYTES, bias_lds + wn * T_N, C, ldc,
                                                  m0 + wm * T_M, nbase, M, N, interior, vec_ok, lane);
}

template <int OUT, bool BIAS>
void launch_one(const dim3 &grid, hipStream_t st, const uint8_t *A, int64_t lda, const float *sa, const uint8_t *B,
                int64_t ldb, const float *sb, const float *bias, int64_t M, int64_t N, int64_t K_pad, void *C,
                int64_t ldc, int tiles_m, int tiles_n)
{
    hipLaunchKernelGGL((gemm_e2m3_kernel<OUT, BIAS>), grid, dim3(NTHREAD), 0, st, A, lda, sa, B, ldb, sb, bias,
                       (int)M, (int)N, (int)K_pad, C, ldc, tiles_m, tiles_n);
}

}  // namespace

hipError_t launch_gemm_e2m3(const uint8_t *A, int64_t lda, const float *sa, const uint8_t *B, int64_t ldb,
                            const float *sb, const float *bias, int64_t M, int64_t N, int64_t K_pad, void *C,
                            int out_dtype, int64_t ldc, hipStream_t st)
{
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    const dim3 grid((unsigned)(tiles_m * tiles_n));
    const bool b = bias != nullptr;
    switch (out_dtype) {
    case 0: (b ? launch_one<0, true> : launch_one<0, false>)(grid, st, A, lda, sa, B, ldb, sb, bias, M, N, K_pad, C, ldc, tiles_m, tiles_n); break;
    case 1: (b ? launch_one<1, true> : launch_one<1, false>)(grid, st, A, lda, sa, B, ldb, sb, bias, M, N, K_pad, C, ldc, tiles_m, tiles_n); break;
    case 2: (b ? launch_one<2, true> : launch_one<2, false>)(grid, st, A, lda, sa, B, ldb, sb, bias, M, N, K_pad, C, ldc, tiles_m, tiles_n); break;
    case 3:
        if (b) return hipErrorInvalidValue;
        launch_one<3, false>(grid, st, A, lda, sa, B, ldb, sb, bias, M, N, K_pad, C, ldc, tiles_m, tiles_n);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace convrot
