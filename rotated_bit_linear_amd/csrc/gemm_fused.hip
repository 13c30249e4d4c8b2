// Decode-inside-GEMM for short activation batches: C[m, n] = ((float)sum_k A[m,k] Q[n,k])
// * a_scale[m] * s_w[n] (+ bias[n]), where the weight codes Q and scales s_w are never
// stored: every workgroup decodes its band of NVFP4 weight rows one 256-column block at a
// time, rotates the block (ConvRot256), quantizes it with the row's code multiplier and
// feeds the codes to the matrix cores straight from LDS.
//
// ComfyUI Turing Utils README, "Load ConvRot DiT ..." bullet: weights stay packed NVFP4 in
// memory and are decoded, rotated and quantized per call, then multiplied by the row-scaled
// INT8 GEMM.  The row quantizer needs the row maximum a[n] = max |y[n, :]| over the whole
// padded row before the first block can be quantized.  It is either an input (from the
// row maximum mode of the weight preparation kernel, reusable across calls for a fixed
// weight) or computed by a first pass of this kernel over the workgroup's band (decode and
// rotation only).  The codes are those of the plain definition, bit for bit: each block's
// butterflies are the same IEEE operations in the same order as in the two-step path, and
// the code multiplier is derived from a exactly as there (a = max|z| / 16 is exact, so
// max|z| = 16 a is recovered exactly for every row that takes the folded multiplier).
//
// When this pays: the decode, rotation and quantization cost ~16 vector instructions per
// weight element, against 2 M multiply-adds per element on the matrix cores, so the kernel
// is bound by vector issue as long as M is at most a few hundred rows.  There it saves the
// weight preparation's S8 write and the GEMM's S8 read (2 K_pad bytes per weight element)
// and the wave quantization of a GEMM with few output tiles.  For long batches every
// M-tile would repeat the decode; the two-step path (prepare once, multiply) is the right
// one there.
//
// Tiling: a workgroup owns a band of 32 weight rows (one MFMA column block) and 32 * FM
// activation rows (FM <= 4, one 32-row block per wave).  Per 256-column block b:
//   every wave: decode + rotate + quantize 8 of the band's rows of block b+1 into LDS
//               stage (b+1) & 1 (16 lanes per row-block, 2 rows per lane group);
//   wave w < FM: 8 MFMAs (v_mfma_i32_32x32x32_i8) on block b: weight fragments from LDS
//               stage b & 1, activation fragments read straight from global memory (the
//               activation tile is small and L2-resident, shared by all workgroups);
//   one barrier.
// The K order inside an MFMA slice is a free choice as long as both operands use the same:
// slice ks of a block takes the 16 columns 16 ks .. 16 ks + 15 for lanes 0-31 and
// 128 + 16 ks .. + 15 for lanes 32-63, so each lane reads 128 contiguous activation bytes
// per block and a lane group's lane t (codes of columns 16 t .. 16 t + 15) feeds slice
// t & 7, half t >> 3.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "kernels.hpp"
#include "nvfp4.hpp"
#include "row_prep.hpp"

namespace convrot {

typedef int32_t fz_v4i __attribute__((ext_vector_type(4)));
typedef int32_t fz_v16i __attribute__((ext_vector_type(16)));

constexpr int FZ_N = 32;                              // weight rows per workgroup
constexpr int FZ_THREADS = 256;                       // 4 waves, 16 lane groups
constexpr int FZ_GROUPS = FZ_THREADS / kLanesPerBlock;
constexpr int FZ_RPG = FZ_N / FZ_GROUPS;              // weight rows per lane group: 2
constexpr int FZ_STAGE = FZ_N * 256;                  // S8 codes of one block of the band
constexpr size_t FZ_TILES = (size_t)FZ_GROUPS * kTileStrideF * sizeof(float);
constexpr size_t FZ_LDS = 2 * FZ_STAGE + FZ_TILES + FZ_N * sizeof(float);
static_assert(FZ_RPG * FZ_GROUPS == FZ_N, "band rows split evenly over the lane groups");

// chunk c (16 bytes) of LDS row r of a stage sits at chunk c ^ (r & 15): the 16-byte
// fragment reads (32 rows, one chunk) and the code writes (one row, 16 chunks) are both
// free of bank conflicts
__device__ __forceinline__ int fz_off(int r, int c) { return r * 256 + ((c ^ (r & 15)) << 4); }

template <int FM, int OUT, bool BIAS>
__global__ __launch_bounds__(FZ_THREADS)
void gemm_nvfp4_fused_kernel(const int8_t *__restrict__ A, int64_t lda, const float *__restrict__ sa,
                             NVFP4Loader W, const float *__restrict__ amax, const float *__restrict__ bias,
                             int M, int N, int nb, void *__restrict__ C, int64_t ldc, int natural)
{
    extern __shared__ __attribute__((aligned(16))) int8_t fz_lds[];
    int8_t *const stage0 = fz_lds;
    int8_t *const stage1 = fz_lds + FZ_STAGE;
    float *const tiles = reinterpret_cast<float *>(fz_lds + 2 * FZ_STAGE);
    float *const sw_band = reinterpret_cast<float *>(fz_lds + 2 * FZ_STAGE + FZ_TILES);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = tid >> 4, t = tid & 15;
    float *tile = tiles + grp * kTileStrideF;
    const int n0 = blockIdx.x * FZ_N;
    const int m0 = blockIdx.y * (32 * FM);
    W.gs = *W.g;

    // ---- decode duties: band rows grp + 16 q; rows past N decode as zeros ----
    using Raw = NVFP4Loader::Raw;
    bool live[FZ_RPG];
#pragma unroll
    for (int q = 0; q < FZ_RPG; q++) live[q] = n0 + grp + FZ_GROUPS * q < N;
    auto fetch_block = [&](int b, Raw (&raw)[FZ_RPG]) {
#pragma unroll
        for (int q = 0; q < FZ_RPG; q++) {
            raw[q].w0 = raw[q].w1 = raw[q].sc = 0u;
            if (live[q]) W.fetch((int64_t)(n0 + grp + FZ_GROUPS * q), (int64_t)b * 16 + t, raw[q]);
        }
    };
    RowQuant rq[FZ_RPG];
    if (amax != nullptr) {
#pragma unroll
        for (int q = 0; q < FZ_RPG; q++) {
            const int r = grp + FZ_GROUPS * q;
            rq[q] = row_quant(live[q] ? amax[n0 + r] * 16.0f : 0.0f);
        }
    } else {
        // pass 1: the band rows' maxima over the whole padded row.  Every block of a row
        // is rotated by the same 16-lane group, so the maximum needs no workgroup barrier
        // (the order of z does not matter for it: no transposition back)
        float zm[FZ_RPG];
        Raw raw[FZ_RPG];
#pragma unroll
        for (int q = 0; q < FZ_RPG; q++) zm[q] = 0.0f;
        fetch_block(0, raw);
        for (int b = 0; b < nb; b++) {
            float v[FZ_RPG][16];
#pragma unroll
            for (int q = 0; q < FZ_RPG; q++) W.decode(raw[q], (int64_t)b * 16 + t, NVFP4Loader::Lane{}, v[q]);
            if (b + 1 < nb) fetch_block(b + 1, raw);
#pragma unroll
            for (int q = 0; q < FZ_RPG; q++) {
                hadamard256(v[q], tile, t, false);
#pragma unroll
                for (int i = 0; i < 16; i++) zm[q] = fmaxf(zm[q], fabsf(v[q][i]));
            }
        }
#pragma unroll
        for (int q = 0; q < FZ_RPG; q++) {
            rq[q] = row_quant(group16_max(zm[q]));
        }
    }
#pragma unroll
    for (int q = 0; q < FZ_RPG; q++)
        if (t == 0) sw_band[grp + FZ_GROUPS * q] = rq[q].scale;
    // decode (then request block b+1's bytes), rotate and quantize block b into `dst`
    auto make_block = [&](int b, Raw (&raw)[FZ_RPG], int8_t *dst) {
        float v[FZ_RPG][16];
#pragma unroll
        for (int q = 0; q < FZ_RPG; q++) W.decode(raw[q], (int64_t)b * 16 + t, NVFP4Loader::Lane{}, v[q]);
        if (b + 1 < nb) fetch_block(b + 1, raw);
#pragma unroll
        for (int q = 0; q < FZ_RPG; q++) {
            hadamard256(v[q], tile, t, natural != 0);
            store_codes(v[q], rq[q], dst + fz_off(grp + FZ_GROUPS * q, t));
        }
    };

    // ---- MFMA duties: wave w < FM owns activation rows m0 + 32 w .. +31 ----
    const int frow = lane & 31, fhalf = lane >> 5;
    const bool mma = wave < FM;
    const int8_t *arow = A + (int64_t)min(m0 + 32 * wave + frow, M - 1) * lda + 128 * fhalf;
    fz_v4i af[8];
    auto load_a = [&](int b) {
#pragma unroll
        for (int ks = 0; ks < 8; ks++) af[ks] = *reinterpret_cast<const fz_v4i *>(arow + (int64_t)b * 256 + 16 * ks);
    };
    fz_v16i acc0, acc1;                   // even and odd slices: two independent chains
#pragma unroll
    for (int r = 0; r < 16; r++) acc0[r] = acc1[r] = 0;

    Raw raw[FZ_RPG];
    fetch_block(0, raw);
    if (mma) load_a(0);
    make_block(0, raw, stage0);
    __syncthreads();
    for (int b = 0; b < nb; b++) {
        const int8_t *cur = (b & 1) ? stage1 : stage0;
        int8_t *nxt = (b & 1) ? stage0 : stage1;
        if (mma) {
#pragma unroll
            for (int ks = 0; ks < 8; ks += 2) {
                const fz_v4i b0 = *reinterpret_cast<const fz_v4i *>(cur + fz_off(frow, 8 * fhalf + ks));
                const fz_v4i b1 = *reinterpret_cast<const fz_v4i *>(cur + fz_off(frow, 8 * fhalf + ks + 1));
                acc0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b0, af[ks], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b1, af[ks + 1], acc1, 0, 0, 0);
            }
            if (b + 1 < nb) load_a(b + 1);   // lands while the next block is decoded
        }
        if (b + 1 < nb) make_block(b + 1, raw, nxt);
        __syncthreads();
    }

    // ---- epilogue: lane l holds row m = l % 32 of its block and the columns
    //      n = 8 g + 4 (l / 32) + j of the band in registers 4 g + j ----
    if (!mma) return;
    const int m = m0 + 32 * wave + frow;
    if (m >= M) return;
    constexpr int ES = (OUT == 0 || OUT == 1) ? 2 : 4;
    const float sam = (OUT == 3) ? 0.0f : sa[m];
    int8_t *crow = static_cast<int8_t *>(C) + (int64_t)m * ldc * ES;
    const bool vec_ok = (((uintptr_t)C) % (4 * ES) == 0) && ((ldc * ES) % (4 * ES) == 0);
#pragma unroll
    for (int g = 0; g < 4; g++) {
        const int nl = 8 * g + 4 * fhalf;
        const int n = n0 + nl;
        int32_t a[4];
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            a[j] = acc0[4 * g + j] + acc1[4 * g + j];
            if constexpr (OUT != 3) {
                v[j] = ((float)a[j] * sam) * sw_band[nl + j];
                if constexpr (BIAS) v[j] = v[j] + ((n + j < N) ? bias[n + j] : 0.0f);
            }
        }
        int8_t *dst = crow + (int64_t)n * ES;
        if (vec_ok && n + 4 <= N) {
            if constexpr (OUT == 3) {
                *reinterpret_cast<fz_v4i *>(dst) = fz_v4i{a[0], a[1], a[2], a[3]};
            } else if constexpr (OUT == 2) {
                *reinterpret_cast<float4 *>(dst) = make_float4(v[0], v[1], v[2], v[3]);
            } else if constexpr (OUT == 0) {
                const __hip_bfloat16 h[4] = {__float2bfloat16(v[0]), __float2bfloat16(v[1]),
                                             __float2bfloat16(v[2]), __float2bfloat16(v[3])};
                *reinterpret_cast<uint2 *>(dst) = *reinterpret_cast<const uint2 *>(h);
            } else {
                const __half h[4] = {__float2half(v[0]), __float2half(v[1]), __float2half(v[2]), __float2half(v[3])};
                *reinterpret_cast<uint2 *>(dst) = *reinterpret_cast<const uint2 *>(h);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; j++) {
                if (n + j >= N) continue;
                if constexpr (OUT == 3) reinterpret_cast<int32_t *>(dst)[j] = a[j];
                else if constexpr (OUT == 2) reinterpret_cast<float *>(dst)[j] = v[j];
                else if constexpr (OUT == 0) reinterpret_cast<__hip_bfloat16 *>(dst)[j] = __float2bfloat16(v[j]);
                else reinterpret_cast<__half *>(dst)[j] = __float2half(v[j]);
            }
        }
    }
}

template <int FM, int OUT, bool BIAS>
static void launch_fz(const dim3 &grid, hipStream_t st, const int8_t *A, int64_t lda, const float *sa,
                      const NVFP4Loader &L, const float *amax, const float *bias, int64_t M, int64_t N,
                      int64_t nb, void *C, int64_t ldc, bool natural)
{
    hipLaunchKernelGGL((gemm_nvfp4_fused_kernel<FM, OUT, BIAS>), grid, dim3(FZ_THREADS), FZ_LDS, st, A, lda,
                       sa, L, amax, bias, (int)M, (int)N, (int)nb, C, ldc, natural ? 1 : 0);
}

template <int FM>
static hipError_t launch_fz_fm(hipStream_t st, const int8_t *A, int64_t lda, const float *sa,
                               const NVFP4Loader &L, const float *amax, const float *bias, int64_t M,
                               int64_t N, int64_t nb, void *C, int out_dtype, int64_t ldc, bool natural)
{
    const dim3 grid((unsigned)((N + FZ_N - 1) / FZ_N), (unsigned)((M + 32 * FM - 1) / (32 * FM)));
    const bool b = bias != nullptr;
    switch (out_dtype) {
    case 0: (b ? launch_fz<FM, 0, true> : launch_fz<FM, 0, false>)(grid, st, A, lda, sa, L, amax, bias, M, N, nb, C, ldc, natural); break;
    case 1: (b ? launch_fz<FM, 1, true> : launch_fz<FM, 1, false>)(grid, st, A, lda, sa, L, amax, bias, M, N, nb, C, ldc, natural); break;
    case 2: (b ? launch_fz<FM, 2, true> : launch_fz<FM, 2, false>)(grid, st, A, lda, sa, L, amax, bias, M, N, nb, C, ldc, natural); break;
    case 3:
        if (b) return hipErrorInvalidValue;   // the raw accumulator takes no bias
        launch_fz<FM, 3, false>(grid, st, A, lda, sa, L, amax, bias, M, N, nb, C, ldc, natural);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gemm_nvfp4_fused(const int8_t *A, int64_t lda, const float *sa, const uint8_t *codes,
                                   int64_t ld_codes, const uint8_t *sf, int64_t ld_sf, const float *g,
                                   const float *amax, const float *bias, int64_t M, int64_t N, int64_t K,
                                   void *C, int out_dtype, int64_t ldc, bool transposed, hipStream_t st)
{
    const int64_t nb = (K + 255) / 256;
    const NVFP4Loader L{codes, ld_codes, sf, ld_sf, g, K, 0.0f};
    if (M <= 32) return launch_fz_fm<1>(st, A, lda, sa, L, amax, bias, M, N, nb, C, out_dtype, ldc, !transposed);
    if (M <= 64) return launch_fz_fm<2>(st, A, lda, sa, L, amax, bias, M, N, nb, C, out_dtype, ldc, !transposed);
    return launch_fz_fm<4>(st, A, lda, sa, L, amax, bias, M, N, nb, C, out_dtype, ldc, !transposed);
}

}  // namespace convrot
