// Weight preparation kernel: NVFP4 decode + ConvRot256 + per-row S8 quantization, fused.
//
// ComfyUI Turing Utils README, "Load ConvRot DiT ..." bullet: packed NVFP4 weights stay
// unchanged in memory; for each call a bounded tile of rows is decoded, rotated in FP32
// with the same block rotation as the activations, and quantized to S8 with an FP32 row
// scale; logical K is zero-padded to a multiple of 256 and serialized padding is ignored.
//
// NVFP4 element k of a row: nibble k of the packed row (low nibble of byte k/2 for even
// k), an E2M1 code (sign, 2 exponent bits with bias 1, 1 mantissa bit); its 16-element
// block k/16 has an E4M3 scale byte (sign, 4 exponent bits with bias 7, 3 mantissa bits,
// S.1111.111 = NaN); the tensor has one FP32 global scale g.
// Decoded value = (E2M1 * E4M3, exact in binary32) * g, rounded once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"
#include "row_prep.hpp"

namespace convrot {

// E2M1 magnitude code m (0..7) -> binary32 bits: 0, 0.5, then (1 + m0/2) * 2^(e-1).
__device__ __forceinline__ float e2m1_to_f32(uint32_t code)
{
    const uint32_t m = code & 7u;
    uint32_t bits = (m >= 2u) ? ((m + 252u) << 22) : (m ? 0x3f000000u : 0u);
    bits |= (code & 8u) << 28;
    return __uint_as_float(bits);
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t b)
{
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    float mag;
    if (e == 0u) mag = (float)m * 0x1.0p-9f;                       // subnormal: m/8 * 2^-6
    else if (e == 15u && m == 7u) mag = __builtin_nanf("");
    else mag = __uint_as_float(((e + 120u) << 23) | (m << 20));
    return (b & 0x80u) ? -mag : mag;
}

struct NVFP4Loader {
    const uint8_t *codes;
    int64_t ld_codes;
    const uint8_t *sf;
    int64_t ld_sf;
    const float *g;
    int64_t K;
    // raw bytes of one 16-element segment: 8 code bytes and its block-scale byte
    struct Raw {
        uint32_t w0, w1, sc;
    };
    __device__ __forceinline__ void fetch(int64_t row, int64_t seg, Raw &r) const
    {
        const int64_t k0 = seg * 16;
        r.w0 = r.w1 = r.sc = 0u;
        if (k0 >= K) return;           // pure padding: no byte of the row is read
        r.sc = sf[row * ld_sf + seg];
        const uint8_t *p = codes + row * ld_codes + seg * 8;
        if (k0 + 16 <= K) {
            const uint2 q = *reinterpret_cast<const uint2 *>(p);
            r.w0 = q.x;
            r.w1 = q.y;
            return;
        }
        const int64_t nbytes = (K - k0 + 1) / 2;   // bytes holding elements k0 .. K-1
#pragma unroll
        for (int i = 0; i < 8; i++)
            if (i < nbytes) {
                const uint32_t byte = p[i];
                if (i < 4) r.w0 |= byte << (8 * i);
                else r.w1 |= byte << (8 * (i - 4));
            }
    }
    __device__ __forceinline__ void decode(const Raw &r, int64_t seg, float (&v)[16]) const
    {
        const int64_t k0 = seg * 16;
        const float gs = *g;
        const float sc = e4m3_to_f32(r.sc);
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const uint32_t code = (((i < 8) ? r.w0 : r.w1) >> (4 * (i & 7))) & 15u;
            const float prod = e2m1_to_f32(code) * sc;   // exact
            const float val = prod * gs;
            v[i] = (k0 + i < K) ? val : 0.0f;             // nibbles past K are padding
        }
    }
};

template <int RB>
__global__ __launch_bounds__(512) void prep_weight_kernel(NVFP4Loader ld, int64_t n_rows, int nb, int8_t *__restrict__ out,
                                   int64_t ld_out, float *__restrict__ scale, int two_pass)
{
    row_prep_kernel_body<NVFP4Loader, RB>(ld, n_rows, nb, out, ld_out, scale, two_pass);
}

hipError_t launch_prep_weight(const uint8_t *codes, int64_t ld_codes, const uint8_t *sf, int64_t ld_sf,
                              const float *g, int64_t n_rows, int64_t K, int8_t *w_s8, int64_t ld_s8,
                              float *w_scale, bool two_pass, hipStream_t st)
{
    const int64_t nb = (K + 255) / 256;
    const RowPrepShape s = row_prep_shape(nb, two_pass);
    const size_t lds = row_prep_lds_bytes(s.threads);
    const dim3 grid((unsigned)row_prep_grid(n_rows, s));
    NVFP4Loader L{codes, ld_codes, sf, ld_sf, g, K};
    if (s.rb == 2)
        hipLaunchKernelGGL(prep_weight_kernel<2>, grid, dim3(s.threads), lds, st,
                           L, n_rows, (int)nb, w_s8, ld_s8, w_scale, 0);
    else
        hipLaunchKernelGGL(prep_weight_kernel<1>, grid, dim3(s.threads), lds, st,
                           L, n_rows, (int)nb, w_s8, ld_s8, w_scale, s.two_pass ? 1 : 0);
    return hipGetLastError();
}

}  // namespace convrot
