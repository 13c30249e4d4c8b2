// Diagnostic: the sustained rate of v_mfma_i32_32x32x32_i8 with its operands already in
// registers (no LDS, no global traffic), on random or constant int8 data.
//
// On this part the matrix cores are power-limited: with bits that toggle from one MFMA to
// the next the clock drops well below its peak, so the dense INT8 figure of the data sheet
// is reachable only with constant operands.  The probe measures that ceiling on the device
// at hand, so the GEMM's roofline fraction can be read against what the matrix cores
// sustain on real data as well as against the published peak.
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

__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, int random_data, int *__restrict__ out)
{
    const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
    pm_v4i a[4], b[4];
#pragma unroll
    for (int f = 0; f < 4; f++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
            a[f][e] = random_data ? (int)pm_hash(gid * 131u + f * 17u + e) : 0x01010101;
            b[f][e] = random_data ? (int)pm_hash(gid * 977u + f * 29u + e + 7u) : 0x01010101;
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

hipError_t launch_probe_mfma(int cus, int iters, bool random_data, int *out, hipStream_t st)
{
    hipLaunchKernelGGL(probe_mfma_kernel, dim3((unsigned)(2 * cus)), dim3(256), 0, st, iters,
                       random_data ? 1 : 0, out);
    return hipGetLastError();
}

}  // namespace convrot
