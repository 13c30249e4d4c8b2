// Row preparation engine shared by the activation and weight kernels (gfx950).
//
// One workgroup prepares one row: every 256-column block of the row is held by a group
// of 16 lanes, 16 fp32 values per lane; a wave holds 4 blocks.  The block rotation
// (ConvRot256: y = x * H/16, H the Sylvester Walsh-Hadamard matrix, paired on activations
// and weights; ComfyUI Turing Utils README, "Load ConvRot DiT ..." bullet) is evaluated
// with the butterfly stages in the fixed order h = 1, 2, ..., 128:
//   phase A: lane t holds elements 16t..16t+15, stages h = 1..8 run inside the lane;
//   transpose through LDS so lane t holds elements t, t+16, ..., t+240;
//   phase B: stages h = 16..128 run inside the lane;
//   transpose back so lane t again holds 16 contiguous elements.
// Every butterfly is the same IEEE add/sub as in the plain definition, so the butterfly
// output z is bit-identical to the sequential transform whatever the data layout.
//
// The final 1/16 scaling y = z * 0.0625 is folded into the quantization.  With
// a' = max |z| (exact, order-free): a = max |y| = a' * 0.0625 (rounding is monotone);
// r = 127 / a; and when a' >= 2^-100, y * r = z * (r * 0.0625) exactly for every element
// that can round to a nonzero code (scaling by 2^-4 is exact for normal numbers, and
// elements so small that z * 0.0625 is subnormal give |y * r| < 2^-15 either way, hence
// code 0).  Rows with 0 < a' < 2^-100 scale every element as written and then multiply
// it by 2^64 (exact), with r = 127 / (a * 2^64): where 127 / a is a finite FP32 value
// (a >= ~3.7e-37) r is that value times 2^-64 exactly (both lie in the normal range), so
// the products and codes are unchanged, and where it overflows this is the definition of
// the quantizer for such rows (the row's exact copy scaled by 2^64).  Either way the codes
// and the scale a / 127 are those of the definition, bit for bit.
//
// Codes: q = clamp(rint(y * r), -127, 127).  With |y| <= a and r = RN(127 / a),
// |y * r| <= 127 (1 + 2^-24), whose FP32 rounding is at most 127 + 2^-17: rint never
// leaves [-127, 127] for a finite row, so no clamp is evaluated.  Adding 1.5 * 2^23
// rounds to the nearest integer, ties to even, and leaves q in two's complement in the
// low byte of the sum (the sum lies in [2^23, 2^24), where the spacing is 1).
//
// Code order.  Natural: the 16 codes a lane stores are elements 16t .. 16t+15 of its block.
// Block-transposed: the transposition back is skipped and the lane stores the codes of
// elements t, t+16, .., t+240 in that order, i.e. column 16t + j of every 256-column block
// holds element 16j + t.  The same codes, in another column order; a GEMM over two
// operands stored in the same order gives the same int32 sums.
//
// 4-bit codes (the W4A8 weight rows) follow the same rule with L = 7 levels in place of
// 127 (s = a / 7, r = 7 / a, no clamp evaluated: |y * r| <= 7 (1 + 2^-24)); everything said
// above holds with 127 replaced by 7.  They are packed two per byte (quantize_store16_s4,
// code_offset), or stored as E2M3 fields of equal value (quantize_e2m3_16, store_codes).
//
// Rows whose K_pad exceeds 128 blocks (32768 columns; 64 blocks for the SwiGLU loaders,
// which have no one-pass form for longer rows), or when forced, are streamed twice:
// pass 1 rotates every block to find the row maximum, pass 2 reloads, rotates again and
// quantizes (same operations, so the same bits).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdint>
#include <mutex>

namespace convrot {

constexpr int kLanesPerBlock = 16;          // lanes sharing one 256-column block
constexpr int kTileStrideF = 272;           // floats per 16x16 transpose tile (256 + 16 pad)
constexpr int kMaxGroups1 = 60;             // two-pass rows: 960 threads
constexpr int kMaxGroups2 = 32;             // one-pass rows of two blocks per group: 512 threads
constexpr int kMaxGroupsWide = 64;          // one-pass SwiGLU rows, one block per group
constexpr int64_t kTwoPassMaxGrid = 65536;  // workgroups of a two-pass launch (they loop)

// XOR swizzle of 16-byte chunks inside a 16x16 fp32 tile: conflict-free ds_read/ds_write
// for both row-wise (b128) and column-wise (b32) access with 32 or 64 LDS banks.
__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

__device__ __forceinline__ int tile_index(int row, int col)
{
    return row * 16 + (((col >> 2) ^ swz(row)) << 2) + (col & 3);
}

// Orders LDS traffic between the lanes of one wave (LDS operations of a wave execute in
// issue order; the fences stop the compiler from moving accesses across this point).
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// In-lane butterflies over the 4 index bits of a 16-element register array.
__device__ __forceinline__ void butterflies16(float (&v)[16])
{
#pragma unroll
    for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
        for (int j = 0; j < 16; j++) {
            if (j & h) continue;
            float u = v[j], w = v[j + h];
            v[j] = u + w;
            v[j + h] = u - w;
        }
    }
}

// The eight butterfly stages of ConvRot256 on the block held by this lane's 16-lane group
// (the 1/16 scaling is left to the quantization).  `tile` is the group's private 16x16
// LDS tile.  In: v[i] = x[16t + i].  Out: v[i] = z[16t + i] (natural), or v[j] =
// z[16j + t] when !natural (the layout after phase B: the transposition back is skipped).
__device__ __forceinline__ void hadamard256(float (&v)[16], float *tile, int t, bool natural)
{
    butterflies16(v);                                   // stages h = 1, 2, 4, 8
#pragma unroll
    for (int c = 0; c < 4; c++) {                       // row t <- v
        float4 q = make_float4(v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]);
        *reinterpret_cast<float4 *>(tile + t * 16 + ((c ^ swz(t)) << 2)) = q;
    }
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < 16; j++) v[j] = tile[tile_index(j, t)];   // v[j] = x'[16j + t]
    butterflies16(v);                                   // stages h = 16, 32, 64, 128
    wave_lds_sync();
    if (!natural) return;
#pragma unroll
    for (int j = 0; j < 16; j++) tile[tile_index(j, t)] = v[j];
    wave_lds_sync();
#pragma unroll
    for (int c = 0; c < 4; c++) {                       // v <- row t
        float4 q = *reinterpret_cast<const float4 *>(tile + t * 16 + ((c ^ swz(t)) << 2));
        v[4 * c] = q.x; v[4 * c + 1] = q.y; v[4 * c + 2] = q.z; v[4 * c + 3] = q.w;
    }
    wave_lds_sync();
}

// Per-segment channel pre-scales of an activation loader: c[i] multiplies element 16 seg + i
// (1.0 past K, where the element is 0 anyway); an empty struct when there are none.
template <bool kPre> struct PreScaleLane { float c[16]; };
template <> struct PreScaleLane<false> {};

template <bool kPre>
__device__ __forceinline__ PreScaleLane<kPre> load_prescale(const float *pre, int64_t seg, int64_t K)
{
    PreScaleLane<kPre> l;
    if constexpr (kPre) {
        const int64_t k0 = seg * 16;
#pragma unroll
        for (int i = 0; i < 16; i++) l.c[i] = (k0 + i < K) ? pre[k0 + i] : 1.0f;
    }
    return l;
}

// An opaque copy of a per-lane value.  Work that depends on it stays where it is written
// (inside a rarely taken branch) instead of being hoisted out of the row loop, where its
// per-element lane masks would occupy scalar registers for the whole loop.
__device__ __forceinline__ int opaque(int v)
{
    asm volatile("" : "+v"(v));
    return v;
}

// Maxima of non-negative floats (|z| values) taken on their bit patterns: for x, y >= 0 the
// unsigned order of the patterns is the order of the values (+inf included), so an integer
// maximum gives the float maximum exactly, with no NaN canonicalisation.
// Maximum over each row of 16 lanes, in every lane of the row: DPP exchanges within quads
// (lane ^ 1, lane ^ 2), then the half-row mirror (lane i <-> 7 - i) and the row mirror
// (lane i <-> 15 - i), each folded in by v_max_u32.
__device__ __forceinline__ uint32_t group16_umax(uint32_t x)
{
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, true));   // quad_perm 1,0,3,2
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, true));   // quad_perm 2,3,0,1
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, true));  // row_half_mirror
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xF, 0xF, true));  // row_mirror
    return x;
}

__device__ __forceinline__ float group16_max(float a)
{
    return __uint_as_float(group16_umax(__float_as_uint(a)));
}

// Maximum over the wave (every lane active), as a wave-uniform value.
__device__ __forceinline__ uint32_t wave_umax(uint32_t x)
{
    x = group16_umax(x);
    const uint32_t r0 = __builtin_amdgcn_readlane(x, 0), r1 = __builtin_amdgcn_readlane(x, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(x, 32), r3 = __builtin_amdgcn_readlane(x, 48);
    return max(max(r0, r1), max(r2, r3));
}

// Workgroup maximum of non-negative values; every thread gets the result.  `red` holds one
// slot per wave (at most 16 waves): lane i of each 16-lane row reads slot i, and the row
// reduces them.
__device__ __forceinline__ float block_max(float a, float *red)
{
    const uint32_t m = wave_umax(__float_as_uint(a));
    const int w = threadIdx.x >> 6;
    uint32_t *slots = reinterpret_cast<uint32_t *>(red);
    if ((threadIdx.x & 63) == 0) slots[w] = m;
    __syncthreads();
    const int i = threadIdx.x & 15;
    return __uint_as_float(group16_umax(i < (int)(blockDim.x >> 6) ? slots[i] : 0u));
}

// rint(t) in two's complement in the low byte of the result, for |t| < 128 (the
// quantizer's products satisfy |t| <= 127 + 2^-17, so clamping to +-127 is a no-op)
__device__ __forceinline__ uint32_t code_bits(float t)
{
    return __float_as_uint(t + 12582912.0f);
}

// low bytes of a, b, c, d -> bytes 0..3
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);
    const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0c0c0400u);
    return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

// Codes of 16 butterfly outputs z, stored as 16 contiguous bytes: of z * m with
// m = r * 0.0625 (folded), or of ((z * 0.0625) * 2^64) * m with m = 127 / (a * 2^64)
// (kScaleFirst, rows with a' < 2^-100).
template <bool kScaleFirst>
__device__ __forceinline__ void quantize_store16(const float (&z)[16], float m, int8_t *dst)
{
    uint32_t c[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const float y = kScaleFirst ? (z[i] * 0.0625f) * 0x1p64f : z[i];
        c[i] = code_bits(y * m);
    }
    uint4 o;
    o.x = pack_low_bytes(c[0], c[1], c[2], c[3]);
    o.y = pack_low_bytes(c[4], c[5], c[6], c[7]);
    o.z = pack_low_bytes(c[8], c[9], c[10], c[11]);
    o.w = pack_low_bytes(c[12], c[13], c[14], c[15]);
    *reinterpret_cast<uint4 *>(dst) = o;
}

// The same for 4-bit codes (levels -7..7): the 16 codes packed into 8 bytes, byte j
// (j = 0..3) holding codes j and 4 + j and byte 4 + j codes 8 + j and 12 + j, low nibble
// first, two's complement.  With |y| <= a and r = RN(7 / a), |y * r| <= 7 (1 + 2^-24), so
// here too rint stays in range and no clamp is evaluated.
template <bool kScaleFirst>
__device__ __forceinline__ void quantize_store16_s4(const float (&z)[16], float m, int8_t *dst)
{
    uint32_t c[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const float y = kScaleFirst ? (z[i] * 0.0625f) * 0x1p64f : z[i];
        c[i] = code_bits(y * m);
    }
    const uint32_t p0 = pack_low_bytes(c[0], c[1], c[2], c[3]);
    const uint32_t p1 = pack_low_bytes(c[4], c[5], c[6], c[7]);
    const uint32_t p2 = pack_low_bytes(c[8], c[9], c[10], c[11]);
    const uint32_t p3 = pack_low_bytes(c[12], c[13], c[14], c[15]);
    uint2 o;
    o.x = (p0 & 0x0F0F0F0Fu) | ((p1 & 0x0F0F0F0Fu) << 4);
    o.y = (p2 & 0x0F0F0F0Fu) | ((p3 & 0x0F0F0F0Fu) << 4);
    *reinterpret_cast<uint2 *>(dst) = o;
}

// The same 4-bit codes as E2M3 numbers of equal value (kBits == 6, the execution form of the
// W4A4 operands): 16 codes -> 16 six-bit fields = 12 bytes, code i in bits 6i..6i+5 of the
// 96-bit result (w0 = bits 0..31).  q = rint(t) + 0 (round half to even, as code_bits; the
// + 0 turns -0 into +0); for |q| in 0..7 the fp32 bits 20..30 of |q| are (127 + E) * 8 + the
// top three mantissa bits, so (those bits - 1008), clamped at 0, is the E2M3 magnitude
// code ((E + 1) * 8 + mantissa; 0 for q = 0), and bit 31 moves to the E2M3 sign bit 5.
template <bool kScaleFirst>
__device__ __forceinline__ void quantize_e2m3_16(const float (&z)[16], float m, uint32_t &w0, uint32_t &w1,
                                                 uint32_t &w2)
{
    uint32_t w[3] = {0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const float y = kScaleFirst ? (z[i] * 0.0625f) * 0x1p64f : z[i];
        const float q = __builtin_rintf(y * m) + 0.0f;
        const uint32_t u = __float_as_uint(q);
        const uint32_t mag = max((u >> 20) & 0x7FFu, 1008u) - 1008u;
        const uint32_t code = mag | ((u >> 26) & 0x20u);
        const int bit = 6 * i;
        w[bit / 32] |= code << (bit % 32);
        if (bit % 32 > 26) w[bit / 32 + 1] |= code >> (32 - bit % 32);
    }
    w0 = w[0];
    w1 = w[1];
    w2 = w[2];
}

// The same result from two 8-entry byte tables (fewer vector instructions, two more live
// registers): per byte of four codes (rounded as code_bits), bit 3 of the nibble is set
// exactly for q < 0, the low three bits index the table of the code's sign.
template <bool kScaleFirst>
__device__ __forceinline__ void quantize_e2m3_16_tables(const float (&z)[16], float m, uint32_t &w0, uint32_t &w1,
                                                        uint32_t &w2)
{
    uint32_t f[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        uint32_t c[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float y = kScaleFirst ? (z[4 * k + i] * 0.0625f) * 0x1p64f : z[4 * k + i];
            c[i] = code_bits(y * m);
        }
        const uint32_t p = pack_low_bytes(c[0], c[1], c[2], c[3]);
        const uint32_t sel = p & 0x07070707u;
        // E2M3 of 0..7: 0x00 0x08 0x10 0x14 0x18 0x1A 0x1C 0x1E; of -8..-1 (nibble 8..15):
        // (unused) 0x3E 0x3C 0x3A 0x38 0x34 0x30 0x28
        const uint32_t pos = __builtin_amdgcn_perm(0x1E1C1A18u, 0x14100800u, sel);
        const uint32_t neg = __builtin_amdgcn_perm(0x28303438u, 0x3A3C3E00u, sel);
        const uint32_t one = (p >> 3) & 0x01010101u;
        const uint32_t mask = (one << 8) - one;                     // 0xFF in the bytes of negative codes
        const uint32_t e = (neg & mask) | (pos & ~mask);
        f[k] = (e & 0x3Fu) | ((e >> 2) & 0xFC0u) | ((e >> 4) & 0x3F000u) | ((e >> 6) & 0xFC0000u);
    }
    w0 = f[0] | (f[1] << 24);
    w1 = (f[1] >> 8) | (f[2] << 16);
    w2 = (f[2] >> 16) | (f[3] << 8);
}

// The same result from gfx950's conversion of fp32 to packed 6-bit fields (E2M3, scale
// 1): each code is rounded to an integral fp32 value exactly as code_bits rounds it (adding
// and subtracting 1.5 * 2^23, which also turns -0 into +0, the field 0x00), and one
// instruction packs the lane's 16 codes.  Its output interleaves its two sources (field
// 2i from source 0, field 2i + 1 from source 1), so the even codes go to source 0 and the
// odd codes to source 1, with zeros above element 7; fields 0..15, the first three words,
// are the lane's codes in order.  Fewer vector instructions than the tables, but 32
// operand registers: used where the registers allow it (store_codes' kCvt).
template <bool kScaleFirst>
__device__ __forceinline__ void quantize_e2m3_16_cvt(const float (&z)[16], float m, uint32_t &w0, uint32_t &w1,
                                                     uint32_t &w2)
{
    typedef float f32x16 __attribute__((ext_vector_type(16)));
    f32x16 even = {}, odd = {};
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const float y0 = kScaleFirst ? (z[2 * i] * 0.0625f) * 0x1p64f : z[2 * i];
        const float y1 = kScaleFirst ? (z[2 * i + 1] * 0.0625f) * 0x1p64f : z[2 * i + 1];
        even[i] = (y0 * m + 12582912.0f) - 12582912.0f;
        odd[i] = (y1 * m + 12582912.0f) - 12582912.0f;
    }
    const auto f = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(even, odd, 1.0f);
    w0 = f[0];
    w1 = f[1];
    w2 = f[2];
}

// Row constants from a' = max |z|: the scale a / L and the code multiplier, for codes of
// L = 127 (8-bit) or L = 7 (4-bit) levels on each side of zero.
struct RowQuant {
    float scale;    // a / L (0 when a == 0)
    float mult;     // r * 0.0625 (folded) or L / (a * 2^64) (scale first); 0 when a == 0
    bool folded;    // block-uniform
};

// A zero row (a == 0: every z is 0) takes the scale-first branch with multiplier 0, so
// every product is exactly 0 and every code 0; L / 0 is never formed.
template <int kBits = 8>
__device__ __forceinline__ RowQuant row_quant(float zmax)
{
    constexpr float L = kBits == 8 ? 127.0f : 7.0f;
    const float a = zmax * 0.0625f;
    const bool zero = (a == 0.0f);
    RowQuant q;
    q.scale = zero ? 0.0f : a / L;
    q.folded = zmax >= 0x1p-100f;
    q.mult = q.folded ? (L / a) * 0.0625f : (zero ? 0.0f : L / (a * 0x1p64f));
    return q;
}

// Byte offset of the codes of 16-lane group member t in block b of a row: 16 bytes per
// lane for 8-bit codes; for packed 4-bit codes, 8 bytes per lane, the four groups of 16
// codes of each 64-code unit stored in the order G0, G2, G1, G3 (so that a 16-byte read
// holds one lane's codes for two consecutive 32-deep MFMA slices).
template <int kBits>
__device__ __forceinline__ int64_t code_offset(int64_t b, int t)
{
    if constexpr (kBits == 8) return b * 256 + t * 16;
    else return b * 128 + (t >> 2) * 32 + ((((t & 1) << 1) | ((t >> 1) & 1)) << 3);
}

// 8-bit codes of 16 butterfly outputs at dst (16 bytes)
__device__ __forceinline__ void store_codes(const float (&z)[16], const RowQuant &q, int8_t *dst)
{
    if (q.folded) quantize_store16<false>(z, q.mult, dst);
    else quantize_store16<true>(z, q.mult, dst);
}

// Start of row `row`'s codes in an output of row stride ld_out: for E2M3 fields (kBits == 6)
// rows are stored in quads, ld_out bytes per quad, row 4q + i starting 96 i bytes into quad q
// (its 128-code units then follow every 384 bytes, store_codes).
template <int kBits>
__device__ __forceinline__ int8_t *row_base(int8_t *out, int64_t row, int64_t ld_out)
{
    if constexpr (kBits == 6) return out + (row >> 2) * ld_out + (row & 3) * 96;
    else return out + row * ld_out;
}

// Codes of member t of block b stored in the row at `row` (row_base).  kBits == 6 (E2M3
// fields): a 128-code unit is 96 bytes, its quarters' first 16 bytes in the order Q0 Q2 Q1
// Q3, then their last 8 bytes in the same order; member t holds half t & 1 of quarter
// (t >> 1) & 3 of unit t >> 3 of the block: bits 0..95 of the quarter's field (its head's
// bytes 0..11), or bits 96..191 (head bytes 12..15 and the 8-byte tail).  kFast: byte
// tables (or, with kCvt, the conversion instruction) and paired stores; else the arithmetic
// encoding and per-lane stores (fewer registers).
template <int kBits = 8, bool kFast = true, bool kCvt = false>
__device__ __forceinline__ void store_codes(const float (&z)[16], const RowQuant &q, int8_t *row, int64_t b, int t)
{
    if constexpr (kBits == 8) {
        int8_t *dst = row + code_offset<8>(b, t);
        if (q.folded) quantize_store16<false>(z, q.mult, dst);
        else quantize_store16<true>(z, q.mult, dst);
    } else if constexpr (kBits == 4) {
        int8_t *dst = row + code_offset<4>(b, t);
        if (q.folded) quantize_store16_s4<false>(z, q.mult, dst);
        else quantize_store16_s4<true>(z, q.mult, dst);
    } else {
        uint32_t w0, w1, w2;
        if constexpr (kFast && kCvt) {
            if (q.folded) quantize_e2m3_16_cvt<false>(z, q.mult, w0, w1, w2);
            else quantize_e2m3_16_cvt<true>(z, q.mult, w0, w1, w2);
        } else if constexpr (kFast) {
            if (q.folded) quantize_e2m3_16_tables<false>(z, q.mult, w0, w1, w2);
            else quantize_e2m3_16_tables<true>(z, q.mult, w0, w1, w2);
        } else {
            if (q.folded) quantize_e2m3_16<false>(z, q.mult, w0, w1, w2);
            else quantize_e2m3_16<true>(z, q.mult, w0, w1, w2);
        }
        // A row's units are 384 bytes apart (quads); 32-bit offsets from the row keep fewer
        // registers live.  Members t and t ^ 1 (adjacent lanes, the same block of the same
        // row: both store or neither) hold the two halves of one quarter.
        const int g = (t >> 1) & 3, slot = ((g & 1) << 1) | (g >> 1), h = t & 1;
        const int unit = (int)b * 768 + (t >> 3) * 384;
        if constexpr (kFast) {
            // half 1's first word (head bytes 12..15) moves to half 0 by DPP: half 0 stores
            // the whole 16-byte head, half 1 the 8-byte tail (aligned, contiguous in a unit)
            const uint32_t w0_partner = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w0, 0xB1, 0xF, 0xF, true);  // quad_perm 1,0,3,2
            if (h == 0) *reinterpret_cast<uint4 *>(row + unit + 16 * slot) = make_uint4(w0, w1, w2, w0_partner);
            else *reinterpret_cast<uint2 *>(row + unit + 64 + 8 * slot) = make_uint2(w1, w2);
        } else {
            // one dword and one 8-byte store per lane: half 0 writes head bytes 0..3 and 4..11,
            // half 1 head bytes 12..15 and the tail
            const int o0 = unit + 16 * slot + 12 * h;
            const int o1 = h ? unit + 64 + 8 * slot : o0 + 4;
            *reinterpret_cast<uint32_t *>(row + o0) = w0;
            *reinterpret_cast<uint2 *>(row + o1) = make_uint2(w1, w2);
        }
    }
}

// Dynamic LDS of one workgroup: per-group transpose tiles followed by two sets of
// reduction slots (alternating between consecutive rows of the row loop).
__host__ __device__ constexpr size_t row_prep_lds_bytes(int threads)
{
    return (size_t)(threads / kLanesPerBlock) * kTileStrideF * sizeof(float) + 32 * sizeof(float);
}

// Loader concept:
//   static constexpr bool kLongOnePass;              rows of 65-128 blocks are held in one
//                                                    pass, two blocks per lane group in up to
//                                                    64 groups (the 1024-thread kernels)
//   static constexpr bool kE2M3Fast;                 E2M3 codes through byte tables and
//                                                    paired stores (else arithmetic codes and
//                                                    per-lane stores: fewer live registers)
//   static constexpr bool kFetchAfterDecode;         request the next row after decoding
//                                                    this one (else before: two buffers)
//   static constexpr bool kTwoPassPrefetch;          two-pass rows: request the next slice
//                                                    before decoding this one
//   struct Raw;                                      raw bytes of one 16-element segment
//   struct Lane;                                     per-segment constants (same every row)
//   Lane lane(int64_t seg) const;                    read them (once per workgroup)
//   template <bool kKeep> void fetch(int64_t row, int64_t seg, Raw &) const;
//                                                    issue the loads (nothing past K); kKeep:
//                                                    the bytes will be read again soon
//   void decode(const Raw &, int64_t seg, const Lane &, float (&)[16]) const;
//                                                    fp32 elements 16*seg.., zero for k >= K
// Splitting the two lets a workgroup request the next row while it works on this one.

// One pass, several rows per workgroup: the G = blockDim/16 groups hold RB blocks each
// (block grp + r*G in v[r]; requires nb <= RB*G).  Rows blockIdx.x, +gridDim.x, ... are
// processed in turn; the raw bytes of the next row are fetched before the current row is
// decoded, so their latency overlaps the rotation, the reduction and the stores.
template <class Loader, int RB, int kBits = 8>
__device__ __forceinline__ void row_prep_rows(const Loader &ld, int64_t n_rows, int nb,
                                              int8_t *__restrict__ out, int64_t ld_out,
                                              float *__restrict__ scale_out, bool natural, bool amax_only)
{
    extern __shared__ float lds[];
    const int tid = threadIdx.x;
    const int grp = tid >> 4;
    const int t = tid & 15;
    const int G = blockDim.x >> 4;
    float *tile = lds + grp * kTileStrideF;
    float *red = lds + G * kTileStrideF;
    using Raw = typename Loader::Raw;
    typename Loader::Lane lanes[RB];
#pragma unroll
    for (int q = 0; q < RB; q++) {
        const int b = grp + q * G;
        if (b < nb) lanes[q] = ld.lane((int64_t)b * 16 + t);
    }

    auto fetch_row = [&](int64_t r, Raw (&dst)[RB]) {
#pragma unroll
        for (int q = 0; q < RB; q++) {
            const int b = grp + q * G;
            if (b < nb) ld.fetch(r, (int64_t)b * 16 + t, dst[q]);
        }
    };
    // rotation, row maximum, codes and scale of one decoded row
    auto finish = [&](float (&v)[RB][16], int64_t row, int parity) {
        float zmax = 0.0f;
#pragma unroll
        for (int q = 0; q < RB; q++) {
            const int b = grp + q * G;
            if (b < nb) {
                hadamard256(v[q], tile, t, natural);
#pragma unroll
                for (int i = 0; i < 16; i++) zmax = fmaxf(zmax, fabsf(v[q][i]));
            }
        }
        const float zrow = block_max(zmax, red + 16 * parity);
        if (amax_only) {                           // a = max |z * 0.0625|, no codes
            if (tid == 0) scale_out[row] = zrow * 0.0625f;
            return;
        }
        const RowQuant rq = row_quant<kBits>(zrow);
        int8_t *orow = row_base<kBits>(out, row, ld_out);
#pragma unroll
        for (int q = 0; q < RB; q++) {
            const int b = grp + q * G;
            if (b < nb) store_codes<kBits, Loader::kE2M3Fast, true>(v[q], rq, orow, b, t);
        }
        if (tid == 0) scale_out[row] = rq.scale;
    };
    auto process = [&](const Raw (&cur)[RB], int64_t row, int parity) {
        float v[RB][16];
#pragma unroll
        for (int q = 0; q < RB; q++) {
            const int b = grp + q * G;
            if (b < nb) ld.decode(cur[q], (int64_t)b * 16 + t, lanes[q], v[q]);
        }
        finish(v, row, parity);
    };

    int64_t row = blockIdx.x;
    if constexpr (Loader::kFetchAfterDecode) {
        // one buffer: the next row is requested as soon as this row's raw bytes are
        // decoded (fewer live registers; the rotation, reduction and stores of this row
        // cover the latency)
        Raw raw[RB];
        if (row < n_rows) fetch_row(row, raw);
        int parity = 0;
        for (; row < n_rows; row += gridDim.x) {
            float v[RB][16];
#pragma unroll
            for (int q = 0; q < RB; q++) {
                const int b = grp + q * G;
                if (b < nb) ld.decode(raw[q], (int64_t)b * 16 + t, lanes[q], v[q]);
            }
            const int64_t next = row + gridDim.x;
            if (next < n_rows) fetch_row(next, raw);
            finish(v, row, parity);
            parity ^= 1;
        }
    } else if constexpr (RB == 1) {
        // two buffers in turn (the row loop unrolled by two): the next row is requested
        // before this row is decoded, with no register copies
        Raw ra[RB], rb[RB];
        if (row < n_rows) fetch_row(row, ra);
        while (row < n_rows) {
            int64_t next = row + gridDim.x;
            if (next < n_rows) fetch_row(next, rb);
            process(ra, row, 0);
            row = next;
            if (row >= n_rows) break;
            next = row + gridDim.x;
            if (next < n_rows) fetch_row(next, ra);
            process(rb, row, 1);
            row = next;
        }
    } else {
        // one buffer copied forward
        Raw nxt[RB];
        if (row < n_rows) fetch_row(row, nxt);
        int parity = 0;
        for (; row < n_rows; row += gridDim.x) {
            Raw cur[RB];
#pragma unroll
            for (int q = 0; q < RB; q++) cur[q] = nxt[q];
            const int64_t next = row + gridDim.x;
            if (next < n_rows) fetch_row(next, nxt);
            process(cur, row, parity);
            parity ^= 1;
        }
    }
}

// Two passes, one row at a time per workgroup: the row is streamed in slices of G blocks,
// once for the maximum and once for the codes (the same operations both times, so the
// same bits).  `parity` selects the reduction slot set (alternating between consecutive
// rows of a workgroup, so one barrier per row suffices).
template <class Loader, int kBits = 8>
__device__ __forceinline__ void row_prep_two_pass(const Loader &ld, int64_t row, int nb,
                                                  int8_t *__restrict__ out, int64_t ld_out,
                                                  float *__restrict__ scale_out, bool natural,
                                                  bool amax_only, int parity)
{
    extern __shared__ float lds[];
    const int tid = threadIdx.x;
    const int grp = tid >> 4;
    const int t = tid & 15;
    const int G = blockDim.x >> 4;
    float *tile = lds + grp * kTileStrideF;
    float *red = lds + G * kTileStrideF;
    int8_t *orow = row_base<kBits>(out, row, ld_out);

    // Slices are visited twice, pass 1 then pass 2 (once with amax_only).  With
    // Loader::kTwoPassPrefetch the raw bytes of the next visit are requested before this one
    // is decoded, so their latency overlaps the rotation.  Pass 1 loads keep the row in the
    // cache for pass 2.
    using Raw = typename Loader::Raw;
    const int nslices = (nb + G - 1) / G;
    auto fetch_slice = [&](int s, bool first_pass, Raw &r) {
        const int b = s * G + grp;
        if (b < nb) {
            if (first_pass) ld.template fetch<true>(row, (int64_t)b * 16 + t, r);
            else ld.fetch(row, (int64_t)b * 16 + t, r);
        }
    };
    auto decode_slice = [&](int s, const Raw &r, float (&v)[16]) {
        const int b = s * G + grp;
        if (b < nb) {
            const typename Loader::Lane ln = ld.lane((int64_t)b * 16 + t);
            ld.decode(r, (int64_t)b * 16 + t, ln, v);
        } else {
#pragma unroll
            for (int i = 0; i < 16; i++) v[i] = 0.0f;
        }
    };
    // a second raw buffer for the loaders that gain from it (Loader::kTwoPassPrefetch)
    constexpr bool kPrefetch = Loader::kTwoPassPrefetch;
    float v[16];
    float zmax = 0.0f;
    Raw cur{}, nxt{};
    if constexpr (kPrefetch) fetch_slice(0, true, cur);
    for (int s = 0; s < nslices; s++) {
        if constexpr (kPrefetch) {
            if (s + 1 < nslices) fetch_slice(s + 1, true, nxt);
            else if (!amax_only) fetch_slice(0, false, nxt);    // pass 2 starts over
            decode_slice(s, cur, v);
            cur = nxt;
        } else {
            fetch_slice(s, true, cur);
            decode_slice(s, cur, v);
        }
        hadamard256(v, tile, t, natural);
#pragma unroll
        for (int i = 0; i < 16; i++) zmax = fmaxf(zmax, fabsf(v[i]));
    }
    const float zrow = block_max(zmax, red + 16 * parity);
    if (amax_only) {
        if (tid == 0) scale_out[row] = zrow * 0.0625f;
        return;
    }
    const RowQuant rq = row_quant<kBits>(zrow);
    for (int s = 0; s < nslices; s++) {
        const int b = s * G + grp;
        if constexpr (kPrefetch) {
            if (s + 1 < nslices) fetch_slice(s + 1, false, nxt);
            decode_slice(s, cur, v);
            cur = nxt;
        } else {
            fetch_slice(s, false, cur);
            decode_slice(s, cur, v);
        }
        hadamard256(v, tile, t, natural);
        if (b < nb) store_codes<kBits, Loader::kE2M3Fast, true>(v, rq, orow, b, t);
    }
    if (tid == 0) scale_out[row] = rq.scale;
}

// Several short rows per workgroup (nb <= 32 blocks): `rpw` rows of nb blocks are held by
// rpw * nb lane groups at once (group g: row slot g / nb, block g % nb), so that a
// workgroup of up to 64 groups leaves few lanes idle whatever nb is (one row of 21 blocks
// alone would leave 3 of 24 groups idle).  Row maximum: each group reduces its 16 lanes,
// one lane per group writes it to LDS, one barrier, then lane t of each group reads entries
// t and t + 16 of its row and the group reduces them; two alternating slot sets make one
// barrier per set of rows enough.
// The raw bytes of the next set of rows are requested before this set is decoded, or right
// after it is decoded for loaders that prefer one buffer (Loader::kFetchAfterDecode).
template <class Loader, int kBits = 8>
__device__ __forceinline__ void row_prep_multi(const Loader &ld, int64_t n_rows, int nb, int rpw,
                                               int8_t *__restrict__ out, int64_t ld_out,
                                               float *__restrict__ scale_out, bool natural, bool amax_only)
{
    extern __shared__ float lds[];
    const int tid = threadIdx.x;
    const int grp = tid >> 4;
    const int t = tid & 15;
    const int G = blockDim.x >> 4;
    float *tile = lds + grp * kTileStrideF;
    float *red = lds + G * kTileStrideF;               // two sets of G floats
    const int slot = grp / nb, b = grp - slot * nb;
    const bool active = slot < rpw;
    const int64_t seg = (int64_t)b * 16 + t;
    using Raw = typename Loader::Raw;
    typename Loader::Lane lane_c{};
    if (active) lane_c = ld.lane(seg);
    const int64_t step = (int64_t)gridDim.x * rpw;

    auto fetch = [&](int64_t base, Raw &r) {
        const int64_t row = base + slot;
        if (active && row < n_rows) ld.fetch(row, seg, r);
    };
    // every lane decodes: the raw bytes of a lane outside the workgroup's rows were never
    // fetched (zero, so the values are 0), and those of a lane past the last row are the
    // previous row's; neither lane stores anything
    auto decode = [&](const Raw &r, int64_t, float (&v)[16]) { ld.decode(r, seg, lane_c, v); };
    auto finish = [&](float (&v)[16], int64_t base, int parity) {
        const int64_t row = base + slot;
        const bool live = active && row < n_rows;
        hadamard256(v, tile, t, natural);
        float zm = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; i++) zm = fmaxf(zm, fabsf(v[i]));
        zm = group16_max(zm);
        uint32_t *set = reinterpret_cast<uint32_t *>(red + parity * G);
        if (t == 0) set[grp] = __float_as_uint(zm);
        __syncthreads();
        // lane t of a group reads slots t and t + 16 of its row (nb <= 32), and the group
        // reduces them (every lane of a group shares its activity, so the DPP steps stay
        // inside active rows)
        uint32_t zbits = 0;
        if (active) {
            const uint32_t *rs = set + slot * nb;
            if (t < nb) zbits = rs[t];
            if (t + 16 < nb) zbits = max(zbits, rs[t + 16]);
        }
        const float zrow = __uint_as_float(group16_umax(zbits));
        if (amax_only) {                               // a = max |z * 0.0625|, no codes
            if (live && b == 0 && t == 0) scale_out[row] = zrow * 0.0625f;
            return;
        }
        const RowQuant rq = row_quant<kBits>(zrow);
        // the multi-row kernel keeps the byte tables: the conversion's operand registers
        // would halve its workgroups per CU
        if (live) store_codes<kBits, Loader::kE2M3Fast, false>(v, rq, row_base<kBits>(out, row, ld_out), b, t);
        if (live && b == 0 && t == 0) scale_out[row] = rq.scale;
    };

    int64_t base = (int64_t)blockIdx.x * rpw;
    int parity = 0;
    if constexpr (Loader::kFetchAfterDecode) {
        // one buffer: the next set of rows is requested as soon as this set is decoded
        Raw raw{};
        if (base < n_rows) fetch(base, raw);
        for (; base < n_rows; base += step) {
            float v[16];
            decode(raw, base, v);
            if (base + step < n_rows) fetch(base + step, raw);
            finish(v, base, parity);
            parity ^= 1;
        }
    } else {
        // two buffers in turn (unrolled by two): the next set is requested before decoding
        Raw ra{}, rb{};
        if (base < n_rows) fetch(base, ra);
        while (base < n_rows) {
            int64_t next = base + step;
            if (next < n_rows) fetch(next, rb);
            {
                float v[16];
                decode(ra, base, v);
                finish(v, base, parity);
            }
            parity ^= 1;
            base = next;
            if (base >= n_rows) break;
            next = base + step;
            if (next < n_rows) fetch(next, ra);
            {
                float v[16];
                decode(rb, base, v);
                finish(v, base, parity);
            }
            parity ^= 1;
            base = next;
        }
    }
}

// Rows per workgroup for the multi-row form: the count (at most 64 lane groups in all)
// that leaves the fewest idle lanes in the workgroup's last wave, the smallest on ties.
inline int row_prep_multi_rows(int64_t nb)
{
    int best = 1;
    int64_t best_idle = INT64_MAX;
    for (int r = 1; r * nb <= 64; r++) {
        const int64_t groups = r * nb, alloc = (groups + 3) / 4 * 4;
        const int64_t idle_frac_x1000 = (alloc - groups) * 1000 / alloc;
        if (idle_frac_x1000 < best_idle) {
            best_idle = idle_frac_x1000;
            best = r;
        }
    }
    return best;
}

// Dynamic LDS of a multi-row workgroup: per-group transpose tiles and two sets of one
// float per group.
__host__ __device__ constexpr size_t row_prep_multi_lds_bytes(int threads)
{
    return (size_t)(threads / kLanesPerBlock) * (kTileStrideF + 2) * sizeof(float);
}

// Kernel body shared by all loaders (kBits: 8-bit codes, packed 4-bit codes, or 4-bit codes
// as E2M3 fields).
// mode: bit 0 two-pass, bit 1 block-transposed code order, bit 2 row maximum only (the
// row's a = max |y| goes to scale_out; no codes are written and `out` is not used)
template <class Loader, int RB, int kBits = 8>
__device__ __forceinline__ void row_prep_kernel_body(const Loader &ld, int64_t n_rows, int nb,
                                                     int8_t *__restrict__ out, int64_t ld_out,
                                                     float *__restrict__ scale_out, int mode)
{
    const bool natural = (mode & 2) == 0;
    const bool amax_only = (mode & 4) != 0;
    if (mode & 1) {
        int parity = 0;
        for (int64_t row = blockIdx.x; row < n_rows; row += gridDim.x) {
            row_prep_two_pass<Loader, kBits>(ld, row, nb, out, ld_out, scale_out, natural, amax_only, parity);
            parity ^= 1;
        }
    } else {
        row_prep_rows<Loader, RB, kBits>(ld, n_rows, nb, out, ld_out, scale_out, natural, amax_only);
    }
}

// Launch shape of a row of nb blocks.
// * Up to one_pass_groups blocks (32, or 64 for the SwiGLU activation kernel): one block per
//   16-lane group.
// * Up to 64 blocks: two per group (at most 512 threads).
// * For loaders that opt in (kLongOnePass), up to 128 blocks: two per group in up to 64
//   groups.  This is the "wide" form, a kernel bound to 1024 threads and at most 128
//   registers a lane.  The whole row stays in registers, so it is loaded, decoded and
//   rotated once.
// * Beyond that: two passes over slices of at most 60 groups (960 threads), the blocks
//   spread evenly over the slices.
// One block per group keeps fewer values per lane, so a SwiGLU row of 56 blocks runs 14 waves
// of at most 128 registers instead of 7 waves of 144 (1-3 % faster).  Rows with a short
// decode (plain activations, NVFP4 weights) are 2-3 % faster at two blocks per group.  For
// 65-128 blocks, two blocks per group in up to 64 groups (79-91 registers) beat four blocks
// per group in up to 32 (129 registers): twice the lanes per row at the same rows per CU.
// On long-K weights [5000, 20000] the time fell from 0.091 to 0.056 ms.
struct RowPrepShape {
    int threads;   // workgroup size, a multiple of 64
    int rb;        // blocks held per 16-lane group in one-pass mode (1 or 2)
    bool two_pass;
    bool wide;     // two blocks per group beyond 32 groups: the 1024-thread kernel
};

// Launch bound of the kernel instantiation that runs RB blocks per group (the wide form has
// kernels of its own, bound to 1024 threads).
template <int RB>
constexpr int row_prep_max_threads() { return RB == 1 ? 1024 : 512; }

// Longest row (in 256-column blocks) prepared in one pass: two blocks in each of 64 groups.
constexpr int64_t kOnePassMaxBlocks = 4 * kMaxGroups2;

// long_one_pass: the loader takes rows of 65-128 blocks in one pass (the wide form)
inline RowPrepShape row_prep_shape(int64_t nb, bool force_two_pass, int one_pass_groups = kMaxGroups2,
                                   bool long_one_pass = true)
{
    RowPrepShape s{};
    int64_t groups;
    if (!force_two_pass && nb <= one_pass_groups) {
        s.rb = 1;
        groups = nb;
    } else if (!force_two_pass && nb <= 2 * kMaxGroups2) {
        s.rb = 2;
        groups = (nb + 1) / 2;
    } else if (!force_two_pass && long_one_pass && nb <= kOnePassMaxBlocks) {
        s.rb = 2;
        s.wide = true;
        groups = (nb + 1) / 2;
    } else {
        // as few slices as 60 groups allow, with the blocks spread evenly over them
        s.rb = 1;
        s.two_pass = true;
        const int64_t slices = (nb + kMaxGroups1 - 1) / kMaxGroups1;
        groups = (nb + slices - 1) / slices;
    }
    s.threads = (int)(((groups + 3) / 4) * 64);
    return s;
}

// Workgroups of the one-pass row loop: as many as the device holds at once (each then
// works through its rows with the next row always in flight), never more than rows.
// Two-pass launches one workgroup per row.
inline int row_prep_grid(int64_t n_rows, const RowPrepShape &s, const void *kernel, size_t lds)
{
    // two-pass rows: one workgroup per row up to a cap that keeps the dispatch's 32-bit
    // work-item count far from overflow (960 threads x 65536); beyond it workgroups loop
    if (s.two_pass) return (int)(n_rows < kTwoPassMaxGrid ? n_rows : kTwoPassMaxGrid);
    struct Entry { int dev; const void *kernel; int threads; size_t lds; int64_t resident; };
    static std::mutex mu;
    static Entry cache[64];
    static int n_cache = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) { (void)hipGetLastError(); dev = -1; }
    int64_t resident = 0;
    {
        std::lock_guard<std::mutex> lock(mu);
        for (int i = 0; i < n_cache; i++)
            if (cache[i].dev == dev && cache[i].kernel == kernel && cache[i].threads == s.threads && cache[i].lds == lds)
                resident = cache[i].resident;
    }
    if (resident == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
            (void)hipGetLastError();
            cus = 256;
        }
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, s.threads, lds) != hipSuccess || per_cu <= 0) {
            (void)hipGetLastError();
            per_cu = 1;
        }
        resident = (int64_t)cus * per_cu;
        std::lock_guard<std::mutex> lock(mu);
        if (n_cache < 64) cache[n_cache++] = Entry{dev, kernel, s.threads, lds, resident};
    }
    return (int)(n_rows < resident ? n_rows : resident);
}

}  // namespace convrot
