// Diagnostic: the sustained rate of v_mfma_i32_32x32x32_i8 with its operands already in
// registers (no LDS, no global traffic), on random or constant int8 data.
//
// On this part the matrix cores are power-limited: with bits that toggle from one MFMA to
// the next the clock drops well below its peak, so the dense INT8 figure of the data sheet
// is reachable only with constant operands.  The probe measures that ceiling on the device
// at hand, so the GEMM's roofline fraction can be read against what the matrix cores
// sustain on real data as well as against the published peak.  The bell-shaped kind is the
// sum of four uniform bytes (Irwin-Hall), centred and scaled by 7/32: mean 0, standard
// deviation about 32, range -112 .. 111 -- the rotated, row-quantized activations and
// weights of the block's linear layers have standard deviations of 30 to 33.
//
// Shape: 2 workgroups of 4 waves per CU (8 waves, as in the GEMM), each wave cycling
// through 4 A and 4 B fragments (16 bytes per lane each) into 4 independent accumulator
// chains; 16 MFMAs per iteration per wave.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace convrot {

typedef int32_t pm_v4i __attribute__((ext_vector_type(4)));
typedef int32_t pm_v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t pm_hash(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x7feb352dU;
    x ^= x >> 15;
    x *= 0x846ca68bU;
    x ^= x >> 16;
    return x;
}

// four bytes of one operand register; kind 0 constant, 1 uniform, 2 bell-shaped
__device__ __forceinline__ int pm_word(uint32_t seed, int kind)
{
    if (kind == 0) return 0x01010101;
    if (kind == 1) return (int)pm_hash(seed);
    uint32_t w = 0;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const uint32_t h = pm_hash(seed * 4u + q);
        const int sum = (int)(h & 0xff) + (int)((h >> 8) & 0xff) + (int)((h >> 16) & 0xff) + (int)(h >> 24);
        w |= (uint32_t)(uint8_t)(((sum - 510) * 7) >> 5) << (8 * q);
    }
    return (int)w;
}

__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, int kind, int *__restrict__ out)
{
    const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
    pm_v4i a[4], b[4];
#pragma unroll
    for (int f = 0; f < 4; f++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
            a[f][e] = pm_word(gid * 131u + f * 17u + e, kind);
            b[f][e] = pm_word(gid * 977u + f * 29u + e + 7u, kind);
        }
    pm_v16i acc[4];
#pragma unroll
    for (int c = 0; c < 4; c++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[c][r] = 0;
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int s = 0; s < 4; s++)
#pragma unroll
            for (int c = 0; c < 4; c++)
                acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[(s + c) & 3], b[(3 * s + c) & 3], acc[c], 0, 0, 0);
    }
    int total = 0;
#pragma unroll
    for (int c = 0; c < 4; c++)
#pragma unroll
        for (int r = 0; r < 16; r++) total += acc[c][r];
    out[gid] = total;                              // keeps the chains live
}

hipError_t launch_probe_mfma(int cus, int iters, int kind, int *out, hipStream_t st)
{
    hipLaunchKernelGGL(probe_mfma_kernel, dim3((unsigned)(2 * cus)), dim3(256), 0, st, iters, kind, out);
    return hipGetLastError();
}

}  // namespace convrot
