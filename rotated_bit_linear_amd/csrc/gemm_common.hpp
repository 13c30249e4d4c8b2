// Pieces shared by the row-scaled INT8 GEMMs of this library (S8 x S8 and S8 x packed S4):
// the XCD-aware assignment of output tiles to workgroups, wait and barrier helpers, and the
// epilogue that dequantizes the int32 accumulators with the two row scales and streams the
// tile out through LDS (MiniMax H3 explainer, glossary entries "Epilogue" and "Fused kernel":
// the rescaling runs inside the matmul, the accumulator never reaches memory).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace convrot {
namespace gemm {

typedef int32_t v4i __attribute__((ext_vector_type(4)));
typedef int32_t v16i __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int NUM_XCD = 8;
constexpr int XCD_M = 2, XCD_N = 4;              // the XCDs' grid over a chip block
constexpr int GROUP_M = 8;
static_assert(XCD_M * XCD_N == NUM_XCD, "XCD grid");

constexpr int EPI_STRIDE = 272;                  // bytes per LDS row of the epilogue tile
constexpr int EPI_BYTES = 32 * EPI_STRIDE;       // one 32-row x 256-byte tile per wave

// s_waitcnt immediates (gfx9 encoding) waiting for vmcnt <= n only / lgkmcnt == 0 only.
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14); }
constexpr int waitcnt_lgkm0() { return 15 | (7 << 4) | (0 << 8) | (3 << 14); }

// scheduling groups "1 MFMA, then 2 LDS reads", repeated until NFR reads are placed
template <int T, int NFR>
__device__ __forceinline__ void read_groups()
{
    if constexpr (2 * T < NFR) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                         // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, (2 * T + 1 < NFR) ? 2 : 1, 0); // DS read
        read_groups<T + 1, NFR>();
    }
}

// orders LDS traffic between the lanes of one wave
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// a workgroup barrier the compiler schedules nothing across
__device__ __forceinline__ void barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

// Tile of workgroup pid.  Workgroup pid runs on XCD pid % 8, as its idx-th workgroup there.
// Chip blocks of (XCD_M xa) x (XCD_N xb) tiles: all XCDs work on the same block at the same
// time (its operand bands are fetched once from HBM into the MALL and shared), XCD x on the
// xa x xb sub-block at row x / XCD_N, column x % XCD_N of the block (L2 reuse inside the
// XCD); blocks advance along N so consecutive blocks share their A bands.  With 256 x 256
// tiles the square 16 x 16 block reads 32 operand bands per round of 256 workgroups where a
// 64 x 4 block reads 68: with K_pad = 14336 that is 117 MB instead of 250 MB, which the MALL
// can hold.  Tiles outside whole blocks are split XCD-contiguously afterwards, in groups of
// GROUP_M M-tiles.
__device__ __forceinline__ void tile_of(int pid, int tiles_m, int tiles_n, int &tm, int &tn)
{
    const int xcd = pid % NUM_XCD, idx = pid / NUM_XCD;
    int xa = 8;                                      // largest power of two <= 8 with XCD_M xa <= tiles_m
    while (xa > 1 && XCD_M * xa > tiles_m) xa >>= 1;
    const int xb = 32 / xa;
    const int nbm = tiles_m / (XCD_M * xa), nbn = tiles_n / (XCD_N * xb);
    const int main_per_xcd = nbm * nbn * xa * xb;
    if (idx < main_per_xcd) {
        const int blk = idx / (xa * xb), j = idx % (xa * xb);
        const int bm = blk / nbn, bn = blk % nbn;
        tm = bm * (XCD_M * xa) + (xcd / XCD_N) * xa + j % xa;
        tn = bn * (XCD_N * xb) + (xcd % XCD_N) * xb + j / xa;
    } else {
        const int trem = tiles_m * tiles_n - main_per_xcd * NUM_XCD;
        const int rq = trem / NUM_XCD, rr = trem % NUM_XCD;
        int r = ((xcd < rr) ? xcd * (rq + 1) : rr * (rq + 1) + (xcd - rr) * rq) + (idx - main_per_xcd);
        const int mm = nbm * XCD_M * xa, nn = nbn * XCD_N * xb;
        int h, w, bm0, bn0;
        if (r < mm * (tiles_n - nn)) {              // right strip beside the blocks
            h = mm; w = tiles_n - nn; bm0 = 0; bn0 = nn;
        } else {                                    // bottom strip below them
            r -= mm * (tiles_n - nn);
            h = tiles_m - mm; w = tiles_n; bm0 = mm; bn0 = 0;
        }
        const int in_group = GROUP_M * w;
        const int g = r / in_group;
        const int gsize = min(h - g * GROUP_M, GROUP_M);
        tm = bm0 + g * GROUP_M + (r % in_group) % gsize;
        tn = bn0 + (r % in_group) / gsize;
    }
}

// Whether workgroup pid walks K from the end.  The 32 workgroups an XCD runs at once (one
// per CU, consecutive in tile_of's order) form a generation, and consecutive generations
// share their activation bands.  Odd generations run K backwards, so each generation starts
// on the operand slices that the previous one read last, while they are still in the XCD's
// L2.  The int32 sums are exact in any order.
__device__ __forceinline__ bool k_reversed(int pid) { return ((pid / NUM_XCD) >> 5) & 1; }

// Row and column scales one lane needs in the epilogue: sav[i] for its row of 32-row block
// i, sbv[j][g] for the 4-column run n = 8g + 4(l/32) .. +3 of 32-column block j (16-byte
// loads when aligned).  Requested before the last barrier so their latency overlaps the
// last MFMAs.
template <int FM, int FN>
struct EpiScales {
    float sav[FM];
    float4 sbv[FN][4];
};

template <int OUT, int FM, int FN>
__device__ __forceinline__ void load_scales(EpiScales<FM, FN> &e, const float *__restrict__ sa,
                                            const float *__restrict__ sb, int mbase, int nbase, int frow,
                                            int fhalf, int M, int N)
{
    if constexpr (OUT != 3) {
#pragma unroll
        for (int i = 0; i < FM; i++) {
            const int m = mbase + i * 32 + frow;
            e.sav[i] = (m < M) ? sa[m] : 0.0f;
        }
        const bool sb16 = ((uintptr_t)sb % 16) == 0;
#pragma unroll
        for (int j = 0; j < FN; j++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int n = nbase + j * 32 + 8 * g + 4 * fhalf;
                float4 r;
                if (sb16 && n + 4 <= N) {
                    r = *reinterpret_cast<const float4 *>(sb + n);
                } else {
                    r.x = (n < N) ? sb[n] : 0.0f;
                    r.y = (n + 1 < N) ? sb[n + 1] : 0.0f;
                    r.z = (n + 2 < N) ? sb[n + 2] : 0.0f;
                    r.w = (n + 3 < N) ? sb[n + 3] : 0.0f;
                }
                e.sbv[j][g] = r;
            }
    }
}

// The epilogue of one wave's FM x FN grid of 32 x 32 blocks, after the MFMA roles "weight
// fragment first": lane l of block (i, j) holds output row mbase + 32 i + l % 32 and the
// 4-column runs n = nbase + 32 j + 8 g + 4 (l / 32) + q (g, q = 0..3) in registers 4 g + q.
// Per 32-row block and per 256-byte column chunk, lanes write their dequantized runs to a
// padded LDS tile (etile, EPI_BYTES of this wave's own), then read it back in 16-byte
// pieces, so each global store instruction covers 4 rows x 256 contiguous bytes.
//   out = ((float)acc * sa[m]) * sb[n] (+ bias[n]), one rounding to the output type;
//   OUT: 0 bf16, 1 fp16, 2 fp32, 3 the raw int32 accumulator.  kShift: the accumulators
//   hold 2^kShift times the sums (exactly), shifted back first.  bias_w: this wave's
//   WT_N bias values (in LDS).  interior: the whole tile lies inside M x N and rows allow
//   16-byte stores (a uniform fast path); vec_ok: 16-byte stores are allowed at all.
template <int OUT, bool BIAS, int FM, int FN, int WT_N, int kShift = 0>
__device__ __forceinline__ void store_tile(const v16i (&acc)[FM][FN], const EpiScales<FM, FN> &e, int8_t *etile,
                                           const float *bias_w, void *__restrict__ C, int64_t ldc, int mbase,
                                           int nbase, int M, int N, bool interior, bool vec_ok, int lane)
{
    constexpr int ES = (OUT == 0 || OUT == 1) ? 2 : 4;
    constexpr int NC = 256 / ES;                   // columns per chunk
    constexpr int CHUNKS = WT_N / NC;
    static_assert(WT_N % NC == 0, "wave tile width must be whole 256-byte chunks");
    const int frow = lane & 31, fhalf = lane >> 5;
#pragma unroll
    for (int i = 0; i < FM; i++) {
#pragma unroll
        for (int c = 0; c < CHUNKS; c++) {
#pragma unroll
            for (int jj = 0; jj < NC / 32; jj++) {
                const int j = c * (NC / 32) + jj;
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    const int nl = jj * 32 + 8 * g + 4 * fhalf;   // column inside the chunk
                    int8_t *dst = etile + frow * EPI_STRIDE + nl * ES;
                    const int32_t a0 = acc[i][j][4 * g] >> kShift, a1 = acc[i][j][4 * g + 1] >> kShift;
                    const int32_t a2 = acc[i][j][4 * g + 2] >> kShift, a3 = acc[i][j][4 * g + 3] >> kShift;
                    if constexpr (OUT == 3) {
                        *reinterpret_cast<v4i *>(dst) = v4i{a0, a1, a2, a3};
                    } else {
                        const float4 s4 = e.sbv[j][g];
                        const float sa_i = e.sav[i];
                        float v0 = ((float)a0 * sa_i) * s4.x, v1 = ((float)a1 * sa_i) * s4.y;
                        float v2 = ((float)a2 * sa_i) * s4.z, v3 = ((float)a3 * sa_i) * s4.w;
                        if constexpr (BIAS) {
                            const float4 b4 = *reinterpret_cast<const float4 *>(bias_w + j * 32 + 8 * g + 4 * fhalf);
                            v0 = v0 + b4.x; v1 = v1 + b4.y; v2 = v2 + b4.z; v3 = v3 + b4.w;
                        }
                        if constexpr (OUT == 2) {
                            *reinterpret_cast<float4 *>(dst) = make_float4(v0, v1, v2, v3);
                        } else if constexpr (OUT == 0) {
                            const __hip_bfloat16 h[4] = {__float2bfloat16(v0), __float2bfloat16(v1),
                                                         __float2bfloat16(v2), __float2bfloat16(v3)};
                            *reinterpret_cast<uint2 *>(dst) = *reinterpret_cast<const uint2 *>(h);
                        } else {
                            const __half h[4] = {__float2half(v0), __float2half(v1), __float2half(v2),
                                                 __float2half(v3)};
                            *reinterpret_cast<uint2 *>(dst) = *reinterpret_cast<const uint2 *>(h);
                        }
                    }
                }
            }
            wave_sync();
            // 32 rows x 256 bytes = 512 pieces of 16 B, 8 per lane, 4 rows per instruction
#pragma unroll
            for (int t = 0; t < 8; t++) {
                const int q = lane + 64 * t;
                const int row = q >> 4, cc = q & 15;
                const uint4 v = *reinterpret_cast<const uint4 *>(etile + row * EPI_STRIDE + cc * 16);
                const int mg = mbase + i * 32 + row;
                const int ng = nbase + c * NC + cc * (16 / ES);
                int8_t *out = static_cast<int8_t *>(C) + ((int64_t)mg * ldc + ng) * ES;
                if (interior) {
                    // streaming store: the output is written once and must not evict the
                    // operand tiles other workgroups are still reading from L2
                    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4 *>(out));
                } else if (mg < M) {
                    if (vec_ok && ng + 16 / ES <= N) {
                        __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4 *>(out));
                    } else {
                        const int8_t *vb = reinterpret_cast<const int8_t *>(&v);
#pragma unroll
                        for (int el = 0; el < 16 / ES; el++)
                            if (ng + el < N) {
                                if constexpr (ES == 2) reinterpret_cast<uint16_t *>(out)[el] = reinterpret_cast<const uint16_t *>(vb)[el];
                                else reinterpret_cast<uint32_t *>(out)[el] = reinterpret_cast<const uint32_t *>(vb)[el];
                            }
                    }
                }
            }
            wave_sync();
        }
    }
}

}  // namespace gemm
}  // namespace convrot
