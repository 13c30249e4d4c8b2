// NVFP4 weight loader of the row engine (decode of one 16-element segment per lane).
//
// NVFP4 element k of a row: nibble k of the packed row (low nibble of byte k/2 for even
// k), an E2M1 code (sign, 2 exponent bits with bias 1, 1 mantissa bit); its 16-element
// block k/16 has an E4M3 scale byte (sign, 4 exponent bits with bias 7, 3 mantissa bits,
// S.1111.111 = NaN); the tensor has one FP32 global scale g.
// Decoded value = (E2M1 * E4M3, exact in binary32) * g, rounded once (ComfyUI Turing Utils
// README, "Load ConvRot DiT ..." bullet: packed NVFP4 weights are decoded per call; logical
// K is zero-padded and serialized padding is ignored).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "row_prep.hpp"

namespace convrot {

typedef float f32x2 __attribute__((ext_vector_type(2)));

// E2M1 codes -> binary32 with the gfx950 conversion instruction: nibbles 2j and 2j+1 of
// `word` (byte j) become .x and .y.  With a scale of 1.0 the result is the exact E2M1
// value; no other scale is used here, since the instruction applies only the exponent of
// its scale operand.
template <int J>
__device__ __forceinline__ f32x2 e2m1_pair(uint32_t word)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, J);
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
    static constexpr bool kLongOnePass = true;
    static constexpr bool kE2M3Fast = true;       // (no E2M3 output from NVFP4 rows)
    static constexpr bool kFetchAfterDecode = false;   // little raw data, cheap decode
    // two-pass rows: loads then decode in place (prefetching the next slice measured 6 %
    // slower on long-K weights: 12 bytes a lane are little to hide)
    static constexpr bool kTwoPassPrefetch = false;
    const uint8_t *codes;
    int64_t ld_codes;
    const uint8_t *sf;
    int64_t ld_sf;
    const float *g;
    int64_t K;
    float gs;      // *g, read once per workgroup
    // raw bytes of one 16-element segment: 8 code bytes and its block-scale byte
    struct Raw {
        uint32_t w0, w1, sc;
    };
    using Lane = PreScaleLane<false>;   // no per-segment constants
    __device__ __forceinline__ Lane lane(int64_t) const { return Lane{}; }
    template <bool kKeep = false>                      // ordinary loads either way
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
        const int nbytes = opaque((int)((K - k0 + 1) / 2));   // bytes holding elements k0 .. K-1
#pragma unroll
        for (int i = 0; i < 8; i++)
            if (i < nbytes) {
                const uint32_t byte = p[i];
                if (i < 4) r.w0 |= byte << (8 * i);
                else r.w1 |= byte << (8 * (i - 4));
            }
    }
    __device__ __forceinline__ void decode(const Raw &r, int64_t seg, const Lane &, float (&v)[16]) const
    {
        const int64_t k0 = seg * 16;
        const float sc = e4m3_to_f32(r.sc);
        f32x2 e[8];
        e[0] = e2m1_pair<0>(r.w0); e[1] = e2m1_pair<1>(r.w0);
        e[2] = e2m1_pair<2>(r.w0); e[3] = e2m1_pair<3>(r.w0);
        e[4] = e2m1_pair<0>(r.w1); e[5] = e2m1_pair<1>(r.w1);
        e[6] = e2m1_pair<2>(r.w1); e[7] = e2m1_pair<3>(r.w1);
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const float prod = ((i & 1) ? e[i >> 1].y : e[i >> 1].x) * sc;   // exact
            v[i] = prod * gs;
        }
        if (k0 + 16 > K) {                                // nibbles past K are padding
            const int rem = opaque((int)(K > k0 ? K - k0 : 0));
#pragma unroll
            for (int i = 0; i < 16; i++)
                if (i >= rem) v[i] = 0.0f;
        }
    }
};

}  // namespace convrot
