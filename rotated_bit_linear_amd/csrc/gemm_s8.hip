// Row-scaled INT8 GEMM on gfx950 matrix cores: C[m, n] = ((float)sum_k A[m,k] B[n,k])
// * a_scale[m] * b_scale[n], with the dequantization fused into the epilogue so the
// int32 accumulator never reaches memory (ComfyUI Turing Utils README, "Load ConvRot
// DiT ..." bullet: row-scaled INT8 GEMM over the rotated S8 operands; MiniMax H3
// explainer, fused-kernel paragraph: rescaling inside the matmul).
//
// Tiling: a 256x256 output tile per workgroup of 4 waves (2x2), each wave 128x128 as a
// 4x4 grid of v_mfma_i32_32x32x32_i8.  K advances 64 bytes per step through two LDS
// stages (register-staged prefetch of the next step while the current one computes).
// LDS rows are 64 bytes (4 chunks of 16 B); chunk c of row r lives at c ^ swz(r) so that
// fragment reads (32 rows, one chunk) and the prefetch writes are bank-conflict free.
// Workgroups are renumbered so that each XCD (workgroup id mod 8 on this part) works on a
// contiguous band of tiles, ordered in groups of 8 M-tiles, for L2 reuse of both operands.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "kernels.hpp"

namespace convrot {

typedef int32_t v4i __attribute__((ext_vector_type(4)));
typedef int32_t v16i __attribute__((ext_vector_type(16)));

constexpr int GBM = 256, GBN = 256, GBK = 64;
constexpr int GTHREADS = 256;
constexpr int GROUP_M = 8;
constexpr int NUM_XCD = 8;

__device__ __forceinline__ int gswz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

template <int OUT>
__device__ __forceinline__ void store_out(void *C, int64_t idx, int32_t acc, float sa, float sb)
{
    if constexpr (OUT == 3) {
        static_cast<int32_t *>(C)[idx] = acc;
    } else {
        const float v = ((float)acc * sa) * sb;
        if constexpr (OUT == 2) {
            static_cast<float *>(C)[idx] = v;
        } else if constexpr (OUT == 0) {
            static_cast<__hip_bfloat16 *>(C)[idx] = __float2bfloat16(v);
        } else {
            static_cast<__half *>(C)[idx] = __float2half(v);
        }
    }
}

template <int OUT>
__global__ __launch_bounds__(GTHREADS, 1)
void gemm_s8_kernel(const int8_t *__restrict__ A, int64_t lda, const float *__restrict__ sa,
                    const int8_t *__restrict__ B, int64_t ldb, const float *__restrict__ sb,
                    int M, int N, int K_pad, void *__restrict__ C, int64_t ldc,
                    int tiles_m, int tiles_n)
{
    __shared__ __attribute__((aligned(16))) int8_t smem[2][(GBM + GBN) * GBK];

    // ---- tile id: XCD-contiguous renumbering, then grouped ordering along M ----
    const int total = tiles_m * tiles_n;
    const int pid = blockIdx.x;
    const int xcd = pid % NUM_XCD, idx = pid / NUM_XCD;
    const int per = total / NUM_XCD, rem = total % NUM_XCD;
    const int lid = (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    const int in_group = GROUP_M * tiles_n;
    const int group = lid / in_group;
    const int first_m = group * GROUP_M;
    const int gsize = min(tiles_m - first_m, GROUP_M);
    const int tm = first_m + (lid % in_group) % gsize;
    const int tn = (lid % in_group) / gsize;
    const int m0 = tm * GBM, n0 = tn * GBN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- global -> register prefetch assignment: 4 chunks of A and 4 of B per thread ----
    const int lrow = tid >> 2, lc = tid & 3;
    const int8_t *pa[4];
    const int8_t *pb[4];
#pragma unroll
    for (int p = 0; p < 4; p++) {
        const int ra = min(m0 + lrow + 64 * p, M - 1);        // rows past M read row M-1
        const int rb = min(n0 + lrow + 64 * p, N - 1);        // (results masked at the store)
        pa[p] = A + (int64_t)ra * lda + lc * 16;
        pb[p] = B + (int64_t)rb * ldb + lc * 16;
    }
    const int st_off = lrow * GBK + ((lc ^ gswz(lrow)) << 4);   // + p * 64 rows * 64 B

    v16i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0;

    uint4 ra_[4], rb_[4];
    auto gload = [&](int kt) {
        const int64_t ko = (int64_t)kt * GBK;
#pragma unroll
        for (int p = 0; p < 4; p++) {
            ra_[p] = *reinterpret_cast<const uint4 *>(pa[p] + ko);
            rb_[p] = *reinterpret_cast<const uint4 *>(pb[p] + ko);
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int p = 0; p < 4; p++) {
            *reinterpret_cast<uint4 *>(&smem[buf][st_off + p * 64 * GBK]) = ra_[p];
            *reinterpret_cast<uint4 *>(&smem[buf][GBM * GBK + st_off + p * 64 * GBK]) = rb_[p];
        }
    };

    // fragment read offsets: row = base + (lane & 31), chunk = 2s + (lane >> 5)
    const int frow = lane & 31, fhalf = lane >> 5;

    const int nk = K_pad / GBK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt++) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        const int8_t *sA = smem[cur];
        const int8_t *sB = smem[cur] + GBM * GBK;
#pragma unroll
        for (int s = 0; s < 2; s++) {
            const int c = 2 * s + fhalf;
            v4i a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int r = wm * 128 + i * 32 + frow;
                a[i] = *reinterpret_cast<const v4i *>(sA + r * GBK + ((c ^ gswz(r)) << 4));
            }
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int r = wn * 128 + j * 32 + frow;
                b[j] = *reinterpret_cast<const v4i *>(sB + r * GBK + ((c ^ gswz(r)) << 4));
            }
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) lstore(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: accumulator element r of lane l is row 8(r/4) + 4(l/32) + r%4, col l%32 ----
    float sbv[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int n = n0 + wn * 128 + j * 32 + frow;
        sbv[j] = (OUT != 3 && n < N) ? sb[n] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int m = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * fhalf + (r & 3);
            if (m >= M) continue;
            const float sav = (OUT != 3) ? sa[m] : 0.0f;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int n = n0 + wn * 128 + j * 32 + frow;
                if (n < N) store_out<OUT>(C, (int64_t)m * ldc + n, acc[i][j][r], sav, sbv[j]);
            }
        }
    }
}

hipError_t launch_gemm_s8(const int8_t *A, int64_t lda, const float *sa, const int8_t *B, int64_t ldb,
                          const float *sb, int64_t M, int64_t N, int64_t K_pad, void *C, int out_dtype,
                          int64_t ldc, hipStream_t st)
{
    const int tiles_m = (int)((M + GBM - 1) / GBM);
    const int tiles_n = (int)((N + GBN - 1) / GBN);
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(GTHREADS);
    switch (out_dtype) {
    case 0: hipLaunchKernelGGL(gemm_s8_kernel<0>, grid, block, 0, st, A, lda, sa, B, ldb, sb, (int)M, (int)N, (int)K_pad, C, ldc, tiles_m, tiles_n); break;
    case 1: hipLaunchKernelGGL(gemm_s8_kernel<1>, grid, block, 0, st, A, lda, sa, B, ldb, sb, (int)M, (int)N, (int)K_pad, C, ldc, tiles_m, tiles_n); break;
    case 2: hipLaunchKernelGGL(gemm_s8_kernel<2>, grid, block, 0, st, A, lda, sa, B, ldb, sb, (int)M, (int)N, (int)K_pad, C, ldc, tiles_m, tiles_n); break;
    case 3: hipLaunchKernelGGL(gemm_s8_kernel<3>, grid, block, 0, st, A, lda, sa, B, ldb, sb, (int)M, (int)N, (int)K_pad, C, ldc, tiles_m, tiles_n); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace convrot
