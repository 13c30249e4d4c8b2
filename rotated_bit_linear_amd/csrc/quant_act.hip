// Activation preparation kernels: (optional SwiGLU) + ConvRot256 + per-row S8 quantization.
//
// ComfyUI Turing Utils README, "Load ConvRot DiT ..." bullet: the same block rotation is
// applied to the activations as to the decoded weights, rows are quantized to S8 with an
// FP32 scale, logical K is zero-padded to a multiple of 256 before the rotation, SwiGLU
// runs before the rotation, and K above 16384 streams each row twice.  MiniMax H3
// explainer (modelpad.app), MLP paragraph: the SwiGLU gate is the first half of fc1's
// output and multiplies the swish of itself into the second half.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "kernels.hpp"
#include "row_prep.hpp"

namespace convrot {

// ---------------------------------------------------------------- element loads ----

template <int DT> struct Elem;
template <> struct Elem<0> {   // bf16: the upper half of a binary32
    using T = uint16_t;
    static __device__ __forceinline__ float cvt(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
};
template <> struct Elem<1> {   // fp16: exact widening
    using T = uint16_t;
    static __device__ __forceinline__ float cvt(uint16_t h) { return __half2float(__ushort_as_half(h)); }
};
template <> struct Elem<2> {   // fp32
    using T = float;
    static __device__ __forceinline__ float cvt(float f) { return f; }
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Raw bytes of 16 consecutive elements: 32 bytes for 16-bit types, 64 for fp32.
template <int DT> struct RawSeg {
    u32x4 w[DT == 2 ? 4 : 2];
};

// Fetch elements [k0, k0+16) of a row with logical length K: vector loads when the whole
// segment lies below K and the row permits 16-byte loads (non-temporal: the activation is
// read once; ordinary with kKeep, for the first pass over a row that is read twice),
// element loads for a segment straddling K, nothing at all past K.
template <int DT, bool kKeep = false>
__device__ __forceinline__ void fetch_seg(const typename Elem<DT>::T *row, int64_t k0, int64_t K, bool aligned,
                                          RawSeg<DT> &r)
{
    constexpr int NW = DT == 2 ? 4 : 2;
    if (aligned && k0 + 16 <= K) {
#pragma unroll
        for (int c = 0; c < NW; c++) {
            const u32x4 *src = reinterpret_cast<const u32x4 *>(row + k0) + c;
            if constexpr (kKeep) r.w[c] = *src;
            else r.w[c] = __builtin_nontemporal_load(src);
        }
        return;
    }
#pragma unroll
    for (int c = 0; c < NW; c++) r.w[c] = u32x4{0u, 0u, 0u, 0u};
    if (k0 >= K) return;
    const int rem = opaque((int)(K - k0 < 16 ? K - k0 : 16));   // elements below K
    if constexpr (DT == 2) {
        const uint32_t *p = reinterpret_cast<const uint32_t *>(row + k0);
#pragma unroll
        for (int i = 0; i < 16; i++)
            if (i < rem) r.w[i >> 2][i & 3] = p[i];
    } else {
        const uint16_t *p = reinterpret_cast<const uint16_t *>(row + k0);
#pragma unroll
        for (int i = 0; i < 16; i++)
            if (i < rem) r.w[i >> 3][(i >> 1) & 3] |= (uint32_t)p[i] << (16 * (i & 1));
    }
}

// element i (0..15) of a fetched segment
template <int DT>
__device__ __forceinline__ float seg_elem(const RawSeg<DT> &r, int i)
{
    if constexpr (DT == 2) {
        return __uint_as_float(r.w[i >> 2][i & 3]);
    } else {
        const uint32_t w = r.w[i >> 3][(i >> 1) & 3];
        return Elem<DT>::cvt((uint16_t)((i & 1) ? (w >> 16) : (w & 0xffffu)));
    }
}

template <int DT>
__device__ __forceinline__ void decode_seg(const RawSeg<DT> &r, float (&v)[16])
{
#pragma unroll
    for (int i = 0; i < 16; i++) v[i] = seg_elem<DT>(r, i);
}

// ------------------------------------------------------ reproducible exponential ----

// E(x) ~ exp(x) from IEEE basic operations only: Cody & Waite (1980) reduction
// x = k ln2 + r, k = rint(x log2 e), ln2 = C1 + C2 with C1 holding 15 significant bits,
// then the degree-7 Taylor polynomial of exp(r) in Horner form with fused multiply-adds,
// then the exact scaling by 2^k.  Coefficients: RN(1/n!).  By definition E(x) = +inf for
// x > 89 and E(x) = 0 for x < -104.
//
// The steps are evaluated on x clamped to [-200, 200] with no further selects: inside
// [-104, 89] nothing changes; for x in (89, 200] the reduction gives k >= 128 with
// p >= 1.32 (k = 128) or p >= 0.70 (k > 128), so p * 2^k overflows to +inf; for x in
// [-200, -104) it gives p * 2^k < 2^-150, which rounds to 0.  A NaN argument gives NaN
// or, if the clamp returns a bound, a finite value; the callers below only use E(-a)
// inside a product with a, which is NaN either way.
__device__ __forceinline__ float repro_exp_nan_free(float x)
{
    const float kLog2e = 0x1.715476p+0f;
    const float kC1 = 0x1.62e4p-1f;
    const float kC2 = 0x1.7f7d1cp-20f;
    const float xc = __builtin_amdgcn_fmed3f(x, -200.0f, 200.0f);
    const float kf = rintf(xc * kLog2e);
    float r = fmaf(-kf, kC1, xc);
    r = fmaf(-kf, kC2, r);
    float p = 0x1.a01a02p-13f;             // 1/7!
    p = fmaf(p, r, 0x1.6c16c2p-10f);       // 1/6!
    p = fmaf(p, r, 0x1.111112p-7f);        // 1/5!
    p = fmaf(p, r, 0x1.555556p-5f);        // 1/4!
    p = fmaf(p, r, 0x1.555556p-3f);        // 1/3!
    p = fmaf(p, r, 0x1.0p-1f);             // 1/2!
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    return __builtin_amdgcn_ldexpf(p, (int)kf);
}

// 1 / d for 1 <= d < 2^126, correctly rounded: the hardware reciprocal estimate refined by
// one Newton step in fused multiply-adds (Markstein's correction).  The tests check it
// against IEEE division for every d that an fp32 gate can produce here.
__device__ __forceinline__ float recip_refined(float d)
{
    const float y = __builtin_amdgcn_rcpf(d);
    const float e = fmaf(-d, y, 1.0f);
    return fmaf(e, y, y);
}

constexpr float kRecipLimit = 0x1p126f;   // d at or above: IEEE division (gate below about -87.3)

// The SwiGLU element: swish(a) * b with swish(a) = a * sigma(a), sigma(a) = 1 / (1 + E(-a)),
// every operation rounded once as written.
__device__ __forceinline__ float swiglu_exact(float a, float b)
{
    const float d = 1.0f + repro_exp_nan_free(-a);
    return (a * (1.0f / d)) * b;
}

// Same value; the refined reciprocal where it is exact, IEEE division for the lanes (a
// wave-uniform branch, practically never taken) whose denominator is 2^126 or more.
__device__ __forceinline__ float swiglu_elem(float a, float b)
{
    const float d = 1.0f + repro_exp_nan_free(-a);
    float o = (a * recip_refined(d)) * b;
    const bool far = !(d < kRecipLimit);
    if (__builtin_amdgcn_ballot_w64(far) != 0) {
        if (far) o = (a * (1.0f / d)) * b;
    }
    return o;
}

// ------------------------------------------------------------- bf16 sigma table ----

// A bf16 gate has 65536 possible values, so sigma(a) = 1 / (1 + E(-a)) can be tabulated
// once per workgroup in LDS by the definition itself (E and an IEEE division) and looked up
// per element: the product (a * sigma) * b is then evaluated exactly as defined, with the
// same sigma bits.  Outside magnitudes [2^-25, 2^7] sigma does not depend on |a|:
//   |a| <= 2^-25: E(-a) is exactly 1 (k = 0, and every Horner step rounds 1 + r back to 1
//                 for |r| <= 2^-25, ties to even at 2^-25), so sigma = 1/2;
//   a >= 128:     E(-a) = 0 (the steps underflow below -104), so sigma = 1;
//   a <= -128:    E(-a) = +inf (the steps overflow above 89), so sigma = 0;
// so the magnitude is clamped to that range, whose two ends already hold those values.
// Entry 2 (m - kSigLo) + s holds sigma of the bf16 pattern with magnitude bits m and sign s.
constexpr uint32_t kSigLo = 0x3300;      // bf16 magnitude bits of 2^-25
constexpr uint32_t kSigHi = 0x4300;      // bf16 magnitude bits of 2^7
constexpr int kSigEntries = 2 * (int)(kSigHi - kSigLo + 1);
constexpr size_t kSigTableBytes = (size_t)kSigEntries * sizeof(float);

__device__ __forceinline__ void build_sigma_table(float *tab)
{
    for (int e = threadIdx.x; e < kSigEntries; e += blockDim.x) {
        const uint32_t pattern = (kSigLo + (uint32_t)(e >> 1)) | ((uint32_t)(e & 1) << 15);
        const float a = __uint_as_float(pattern << 16);
        tab[e] = 1.0f / (1.0f + repro_exp_nan_free(-a));
    }
    __syncthreads();
}

// Table position inside the dynamic LDS (in floats), past `engine_bytes` used by the row
// engine, at a 16-byte boundary.
__device__ __forceinline__ uint32_t sigma_table_offset(size_t engine_bytes)
{
    return (uint32_t)((engine_bytes + 15) / 16 * 4);
}

__device__ __forceinline__ float *sigma_table_at(uint32_t off)
{
    extern __shared__ float lds_base[];
    return lds_base + off;
}

// sigma of the bf16 gate with 16-bit pattern p, from the table at `off`
__device__ __forceinline__ float sigma_lookup(uint32_t off, uint32_t p)
{
    extern __shared__ float lds_base[];
    const uint32_t m = min(max(p & 0x7fffu, kSigLo), kSigHi);
    return lds_base[off + (((m - kSigLo) << 1) | (p >> 15))];
}

// --------------------------------------------------------------------- loaders ----

// Activation loaders.  With kPre, the loaded (or SwiGLU) value of channel k is multiplied
// by the channel pre-scale c[k] before the rotation (one FP32 rounding), the order of an
// unfused pre-scale (ComfyUI Turing Utils README, "Load ConvRot DiT ..." bullet).
template <int DT, bool kPre>
struct ActLoader {
    // bf16/fp16 rows of 65-128 blocks are held in one pass (the wide form); fp32 rows (64
    // raw bytes a segment) would spill under its 1024-thread bound and stream twice
    static constexpr bool kLongOnePass = DT != 2;
    static constexpr bool kE2M3Fast = true;
    static constexpr bool kFetchAfterDecode = true;
    static constexpr bool kTwoPassPrefetch = true;
    static constexpr bool kSigTable = false;
    const typename Elem<DT>::T *x;
    int64_t ld;
    int64_t K;
    bool aligned;
    const float *pre;
    using Raw = RawSeg<DT>;
    using Lane = PreScaleLane<kPre>;
    __device__ __forceinline__ Lane lane(int64_t seg) const { return load_prescale<kPre>(pre, seg, K); }
    template <bool kKeep = false>
    __device__ __forceinline__ void fetch(int64_t row, int64_t seg, Raw &r) const
    {
        fetch_seg<DT, kKeep>(x + row * ld, seg * 16, K, aligned, r);
    }
    __device__ __forceinline__ void decode(const Raw &r, int64_t, const Lane &ln, float (&v)[16]) const
    {
        decode_seg<DT>(r, v);
        if constexpr (kPre) {
#pragma unroll
            for (int i = 0; i < 16; i++) v[i] = v[i] * ln.c[i];
        }
    }
};

template <int DT, bool kPre>
struct SwigluLoader {
    // rows of 65-128 blocks stream twice (fp16/fp32 gates would spill in the wide form)
    static constexpr bool kLongOnePass = false;
    // fp16/fp32 gates (the refined reciprocal, no sigma table) leave no room for the tables
    static constexpr bool kE2M3Fast = DT == 0;
    static constexpr bool kFetchAfterDecode = true;
    // fp32 segments (128 bytes a lane) leave no registers for a second buffer
    static constexpr bool kTwoPassPrefetch = DT != 2;
    static constexpr bool kSigTable = DT == 0;     // bf16 gates: sigma from the LDS table
    const typename Elem<DT>::T *h;
    int64_t ld;
    int64_t F;
    bool aligned_gate;
    bool aligned_value;
    const float *pre;
    uint32_t sig_off = 0;                          // the table's LDS position (set inside the kernel)
    struct Raw {
        RawSeg<DT> gate, value;
    };
    using Lane = PreScaleLane<kPre>;
    __device__ __forceinline__ Lane lane(int64_t seg) const { return load_prescale<kPre>(pre, seg, F); }
    template <bool kKeep = false>
    __device__ __forceinline__ void fetch(int64_t row, int64_t seg, Raw &r) const
    {
        const typename Elem<DT>::T *p = h + row * ld;
        fetch_seg<DT, kKeep>(p, seg * 16, F, aligned_gate, r.gate);
        fetch_seg<DT, kKeep>(p + F, seg * 16, F, aligned_value, r.value);
    }
    __device__ __forceinline__ void decode(const Raw &r, int64_t, const Lane &ln, float (&v)[16]) const
    {
        float b[16];
        decode_seg<DT>(r.value, b);
        if constexpr (kSigTable) {                      // zero past F: (0 * 1/2) * 0
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const uint32_t w = r.gate.w[i >> 3][(i >> 1) & 3];
                const uint32_t p = (i & 1) ? (w >> 16) : (w & 0xffffu);
                v[i] = (__uint_as_float(p << 16) * sigma_lookup(sig_off, p)) * b[i];
            }
            if constexpr (kPre) {
#pragma unroll
                for (int i = 0; i < 16; i++) v[i] = v[i] * ln.c[i];
            }
            return;
        }
        decode_seg<DT>(r.gate, v);
        bool far = false;
#pragma unroll
        for (int i = 0; i < 16; i++) {                  // zero past F: 0 * sigma * 0
            const float d = 1.0f + repro_exp_nan_free(-v[i]);
            far |= !(d < kRecipLimit);
            v[i] = (v[i] * recip_refined(d)) * b[i];
        }
        if (__builtin_amdgcn_ballot_w64(far) != 0) {   // some gate below about -87.3
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const float a = seg_elem<DT>(r.gate, i);
                const float d = 1.0f + repro_exp_nan_free(-a);
                if (!(d < kRecipLimit)) v[i] = swiglu_exact(a, seg_elem<DT>(r.value, i));
            }
        }
        if constexpr (kPre) {                           // after SwiGLU, as unfused
#pragma unroll
            for (int i = 0; i < 16; i++) v[i] = v[i] * ln.c[i];
        }
    }
};

// Unfused SwiGLU: out[m, k] = swish(h[m, k]) * h[m, F + k] in FP32 (same element function
// as the fused path: the sigma table for bf16).  One thread per element, grid-stride.
template <int DT>
__global__ void swiglu_kernel(const typename Elem<DT>::T *__restrict__ h, int64_t ld_h, int64_t M, int64_t F,
                              float *__restrict__ out, int64_t ld_out)
{
    if constexpr (DT == 0) build_sigma_table(sigma_table_at(0));
    const int64_t total = M * F;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = i / F, k = i - m * F;
        if constexpr (DT == 0) {
            const uint32_t p = h[m * ld_h + k];
            const float b = Elem<DT>::cvt(h[m * ld_h + F + k]);
            out[m * ld_out + k] = (__uint_as_float(p << 16) * sigma_lookup(0, p)) * b;
        } else {
            const float a = Elem<DT>::cvt(h[m * ld_h + k]);
            const float b = Elem<DT>::cvt(h[m * ld_h + F + k]);
            out[m * ld_out + k] = swiglu_elem(a, b);
        }
    }
}

// kBits: 8-bit codes, or packed 4-bit codes (the W4A8 weight rows)
template <class Loader, int RB, int kBits = 8>
__global__ __launch_bounds__(row_prep_max_threads<RB>()) void quant_act_kernel(Loader ld, int64_t n_rows, int nb, int8_t *__restrict__ out, int64_t ld_out,
                                 float *__restrict__ scale, int mode)
{
    if constexpr (Loader::kSigTable) {
        ld.sig_off = sigma_table_offset(row_prep_lds_bytes(blockDim.x));
        build_sigma_table(sigma_table_at(ld.sig_off));
    }
    row_prep_kernel_body<Loader, RB, kBits>(ld, n_rows, nb, out, ld_out, scale, mode);
}

// Rows of 65-128 blocks in one pass (the wide form, loaders with kLongOnePass): two blocks
// per lane group in up to 64 groups (1024 threads), so each block is loaded and rotated
// once.  With at most 128 registers a lane, two such rows fit on a CU at once.
template <class Loader, int kBits = 8>
__global__ __launch_bounds__(1024) void quant_act_wide_kernel(Loader ld, int64_t n_rows, int nb, int8_t *__restrict__ out,
                                                              int64_t ld_out, float *__restrict__ scale, int mode)
{
    row_prep_kernel_body<Loader, 2, kBits>(ld, n_rows, nb, out, ld_out, scale, mode);
}

// Several short rows per workgroup (see row_prep_multi).
template <class Loader, int kBits = 8>
__global__ __launch_bounds__(1024) void quant_act_multi_kernel(Loader ld, int64_t n_rows, int nb, int rpw,
                                                             int8_t *__restrict__ out, int64_t ld_out,
                                                             float *__restrict__ scale, int mode)
{
    if constexpr (Loader::kSigTable) {
        ld.sig_off = sigma_table_offset(row_prep_multi_lds_bytes(blockDim.x));
        build_sigma_table(sigma_table_at(ld.sig_off));
    }
    row_prep_multi<Loader, kBits>(ld, n_rows, nb, rpw, out, ld_out, scale, (mode & 2) == 0, false);
}

// --------------------------------------------------------------------- launchers ----

template <class Loader, int kBits = 8>
static hipError_t launch_rows(const Loader &L, int64_t rows, int64_t nb, int8_t *out, int64_t ld_out,
                              float *scale, bool force_two_pass, bool transposed, hipStream_t st,
                              int one_pass_groups = kMaxGroups2)
{
    const RowPrepShape s = row_prep_shape(nb, force_two_pass, one_pass_groups, Loader::kLongOnePass);
    // the sigma table sits past the engine's LDS, at a 16-byte boundary
    constexpr size_t extra = Loader::kSigTable ? kSigTableBytes + 16 : 0;
    const size_t lds = row_prep_lds_bytes(s.threads) + extra;
    const int mode = (s.two_pass ? 1 : 0) | (transposed ? 2 : 0);
    // a workgroup that builds the table works through many rows: two-pass rows then loop
    // over the resident workgroups instead of one workgroup per row
    RowPrepShape gs = s;
    if (Loader::kSigTable) gs.two_pass = false;
    const int rpw = (!s.two_pass && nb <= 32) ? row_prep_multi_rows(nb) : 1;
    if (rpw >= 2) {
        // rows whose lane groups would leave the last wave partly idle: several per workgroup
        const int threads = (int)((rpw * nb + 3) / 4 * 64);
        const size_t mlds = row_prep_multi_lds_bytes(threads) + extra;
        const RowPrepShape ms{threads, 1, false};
        const void *k = reinterpret_cast<const void *>(&quant_act_multi_kernel<Loader, kBits>);
        const dim3 grid((unsigned)row_prep_grid((rows + rpw - 1) / rpw, ms, k, mlds));
        hipLaunchKernelGGL((quant_act_multi_kernel<Loader, kBits>), grid, dim3(threads), mlds, st, L, rows, (int)nb,
                           rpw, out, ld_out, scale, mode);
        return hipGetLastError();
    }
    if constexpr (Loader::kLongOnePass) {
        if (s.wide) {
            const void *k = reinterpret_cast<const void *>(&quant_act_wide_kernel<Loader, kBits>);
            const dim3 grid((unsigned)row_prep_grid(rows, s, k, lds));
            hipLaunchKernelGGL((quant_act_wide_kernel<Loader, kBits>), grid, dim3(s.threads), lds, st,
                               L, rows, (int)nb, out, ld_out, scale, mode);
            return hipGetLastError();
        }
    }
    if (s.rb == 2) {
        const void *k = reinterpret_cast<const void *>(&quant_act_kernel<Loader, 2, kBits>);
        const dim3 grid((unsigned)row_prep_grid(rows, s, k, lds));
        hipLaunchKernelGGL((quant_act_kernel<Loader, 2, kBits>), grid, dim3(s.threads), lds, st,
                           L, rows, (int)nb, out, ld_out, scale, mode);
    } else {
        const void *k = reinterpret_cast<const void *>(&quant_act_kernel<Loader, 1, kBits>);
        const dim3 grid((unsigned)row_prep_grid(rows, gs, k, lds));
        hipLaunchKernelGGL((quant_act_kernel<Loader, 1, kBits>), grid, dim3(s.threads), lds, st,
                           L, rows, (int)nb, out, ld_out, scale, mode);
    }
    return hipGetLastError();
}

template <int DT>
static hipError_t launch_act(const void *x, int64_t ld_x, int64_t M, int64_t K, const float *pre,
                             int8_t *x_s8, int64_t ld_s8, float *x_scale, bool two_pass, bool transposed,
                             hipStream_t st)
{
    const auto *xp = static_cast<const typename Elem<DT>::T *>(x);
    const bool aligned = ((uintptr_t)x % 16 == 0) && ((ld_x * (int64_t)sizeof(typename Elem<DT>::T)) % 16 == 0);
    const int64_t nb = (K + 255) / 256;
    if (pre) return launch_rows(ActLoader<DT, true>{xp, ld_x, K, aligned, pre}, M, nb, x_s8, ld_s8, x_scale, two_pass, transposed, st);
    return launch_rows(ActLoader<DT, false>{xp, ld_x, K, aligned, nullptr}, M, nb, x_s8, ld_s8, x_scale, two_pass, transposed, st);
}

template <int DT>
static hipError_t launch_swiglu(const void *h, int64_t ld_h, int64_t M, int64_t F, const float *pre,
                                int8_t *x_s8, int64_t ld_s8, float *x_scale, bool two_pass, bool transposed,
                                hipStream_t st)
{
    const int64_t es = (int64_t)sizeof(typename Elem<DT>::T);
    const bool row_ok = ((uintptr_t)h % 16 == 0) && ((ld_h * es) % 16 == 0);
    const bool val_ok = row_ok && ((F * es) % 16 == 0);
    const auto *hp = static_cast<const typename Elem<DT>::T *>(h);
    const int64_t nb = (F + 255) / 256;
    if (pre)
        return launch_rows(SwigluLoader<DT, true>{hp, ld_h, F, row_ok, val_ok, pre}, M, nb, x_s8, ld_s8, x_scale,
                           two_pass, transposed, st, kMaxGroupsWide);
    return launch_rows(SwigluLoader<DT, false>{hp, ld_h, F, row_ok, val_ok, nullptr}, M, nb, x_s8, ld_s8, x_scale,
                       two_pass, transposed, st, kMaxGroupsWide);
}

hipError_t launch_quant_act(const void *x, int dtype, int64_t ld_x, int64_t M, int64_t K, const float *pre,
                            int8_t *x_s8, int64_t ld_s8, float *x_scale, bool two_pass, bool transposed,
                            hipStream_t st)
{
    switch (dtype) {
    case 0: return launch_act<0>(x, ld_x, M, K, pre, x_s8, ld_s8, x_scale, two_pass, transposed, st);
    case 1: return launch_act<1>(x, ld_x, M, K, pre, x_s8, ld_s8, x_scale, two_pass, transposed, st);
    case 2: return launch_act<2>(x, ld_x, M, K, pre, x_s8, ld_s8, x_scale, two_pass, transposed, st);
    default: return hipErrorInvalidValue;
    }
}

// W4A8 weight preparation from dense rows (the activation loader, no pre-scale): ConvRot256,
// 4-bit row quantization, packed codes (ComfyUI Turing Utils README: W4A8 dispatch; the
// packed format is this library's, the pages describe none)
template <int DT, int kBits>
static hipError_t launch_w4(const void *w, int64_t ld_w, int64_t N, int64_t K, uint8_t *w_s4, int64_t ld_s4,
                            float *w_scale, bool two_pass, bool transposed, hipStream_t st)
{
    const auto *wp = static_cast<const typename Elem<DT>::T *>(w);
    const bool aligned = ((uintptr_t)w % 16 == 0) && ((ld_w * (int64_t)sizeof(typename Elem<DT>::T)) % 16 == 0);
    const int64_t nb = (K + 255) / 256;
    return launch_rows<ActLoader<DT, false>, kBits>(ActLoader<DT, false>{wp, ld_w, K, aligned, nullptr}, N, nb,
                                                    reinterpret_cast<int8_t *>(w_s4), ld_s4, w_scale, two_pass,
                                                    transposed, st);
}

template <int kBits>
static hipError_t launch_weight_4bit(const void *w, int dtype, int64_t ld_w, int64_t N, int64_t K, uint8_t *out,
                                     int64_t ld_out, float *w_scale, bool two_pass, bool transposed, hipStream_t st)
{
    switch (dtype) {
    case 0: return launch_w4<0, kBits>(w, ld_w, N, K, out, ld_out, w_scale, two_pass, transposed, st);
    case 1: return launch_w4<1, kBits>(w, ld_w, N, K, out, ld_out, w_scale, two_pass, transposed, st);
    case 2: return launch_w4<2, kBits>(w, ld_w, N, K, out, ld_out, w_scale, two_pass, transposed, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_quant_weight_w4(const void *w, int dtype, int64_t ld_w, int64_t N, int64_t K, uint8_t *w_s4,
                                  int64_t ld_s4, float *w_scale, bool two_pass, bool transposed, hipStream_t st)
{
    return launch_weight_4bit<4>(w, dtype, ld_w, N, K, w_s4, ld_s4, w_scale, two_pass, transposed, st);
}

hipError_t launch_quant_weight_e2m3(const void *w, int dtype, int64_t ld_w, int64_t N, int64_t K, uint8_t *w_f6,
                                    int64_t ld_f6, float *w_scale, bool two_pass, bool transposed, hipStream_t st)
{
    return launch_weight_4bit<6>(w, dtype, ld_w, N, K, w_f6, ld_f6, w_scale, two_pass, transposed, st);
}

// W4A4 activation preparation: the activation (or SwiGLU) loader, no pre-scale, ConvRot256,
// 4-bit row quantization, packed codes or E2M3 fields (ComfyUI Turing Utils README: W4A4
// dispatch; both forms are the weight's)
template <int DT, int kBits>
static hipError_t launch_act_w4(const void *x, int64_t ld_x, bool swiglu, int64_t M, int64_t K, uint8_t *x_s4,
                                int64_t ld_s4, float *x_scale, bool two_pass, bool transposed, hipStream_t st)
{
    using T = typename Elem<DT>::T;
    const int64_t es = (int64_t)sizeof(T);
    const auto *xp = static_cast<const T *>(x);
    const int64_t nb = (K + 255) / 256;
    int8_t *out = reinterpret_cast<int8_t *>(x_s4);
    const bool row_ok = ((uintptr_t)x % 16 == 0) && ((ld_x * es) % 16 == 0);
    if (swiglu) {
        const bool val_ok = row_ok && ((K * es) % 16 == 0);
        return launch_rows<SwigluLoader<DT, false>, kBits>(
            SwigluLoader<DT, false>{xp, ld_x, K, row_ok, val_ok, nullptr}, M, nb, out, ld_s4, x_scale, two_pass,
            transposed, st, kMaxGroupsWide);
    }
    return launch_rows<ActLoader<DT, false>, kBits>(ActLoader<DT, false>{xp, ld_x, K, row_ok, nullptr}, M, nb, out,
                                                    ld_s4, x_scale, two_pass, transposed, st);
}

template <int kBits>
static hipError_t launch_act_4bit(const void *x, int dtype, int64_t ld_x, bool swiglu, int64_t M, int64_t K,
                                  uint8_t *out, int64_t ld_out, float *x_scale, bool two_pass, bool transposed,
                                  hipStream_t st)
{
    switch (dtype) {
    case 0: return launch_act_w4<0, kBits>(x, ld_x, swiglu, M, K, out, ld_out, x_scale, two_pass, transposed, st);
    case 1: return launch_act_w4<1, kBits>(x, ld_x, swiglu, M, K, out, ld_out, x_scale, two_pass, transposed, st);
    case 2: return launch_act_w4<2, kBits>(x, ld_x, swiglu, M, K, out, ld_out, x_scale, two_pass, transposed, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_quant_act_w4(const void *x, int dtype, int64_t ld_x, bool swiglu, int64_t M, int64_t K,
                               uint8_t *x_s4, int64_t ld_s4, float *x_scale, bool two_pass, bool transposed,
                               hipStream_t st)
{
    return launch_act_4bit<4>(x, dtype, ld_x, swiglu, M, K, x_s4, ld_s4, x_scale, two_pass, transposed, st);
}

hipError_t launch_quant_act_e2m3(const void *x, int dtype, int64_t ld_x, bool swiglu, int64_t M, int64_t K,
                                 uint8_t *x_f6, int64_t ld_f6, float *x_scale, bool two_pass, bool transposed,
                                 hipStream_t st)
{
    return launch_act_4bit<6>(x, dtype, ld_x, swiglu, M, K, x_f6, ld_f6, x_scale, two_pass, transposed, st);
}

// Nibble form -> E2M3 fields (W4A4 weights prepared once in the packed form): one thread per
// 16-code group of a row.  The group's 8 bytes (byte j: codes j and 4 + j, byte 4 + j: codes
// 8 + j and 12 + j, low nibble first) become 16 six-bit fields, stored where the E2M3 form
// keeps that half of that quarter (rows in quads, store_codes' layout).  Codes are copied, not
// recomputed: the results equal the E2M3 preparation of the same rows bit for bit.
__global__ __launch_bounds__(256) void repack_w4_e2m3_kernel(const uint8_t *__restrict__ src, int64_t ld_s4,
                                                             int64_t n_rows, int groups, uint8_t *__restrict__ dst,
                                                             int64_t ld_f6)
{
    const int64_t total = n_rows * groups;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = i / groups;
        const int G = (int)(i - row * groups);
        // the group's bytes: 64-code unit G / 4, groups stored in the order G0 G2 G1 G3
        const int p = G & 3, pslot = ((p & 1) << 1) | (p >> 1);
        const uint2 d = *reinterpret_cast<const uint2 *>(src + row * ld_s4 + (G >> 2) * 32 + pslot * 8);
        uint32_t w[3] = {0u, 0u, 0u};
#pragma unroll
        for (int c = 0; c < 16; c++) {
            // code c: byte (c & 3) of the low (c < 8) or high word, high nibble when (c >> 2) is odd
            const uint32_t word = (c < 8) ? d.x : d.y;
            const uint32_t nib = (word >> (8 * (c & 3) + 4 * ((c >> 2) & 1))) & 15u;
            const int q = (int)nib - (nib >= 8u ? 16 : 0);
            const int m = (q < 0 ? -q : q) & 7;          // codes are -7..7 (nibble 8 is no code)
            // E2M3 magnitude codes of 0..7 and the sign bit
            const uint32_t mag = (uint32_t)((0x1E1C1A1814100800ull >> (8 * m)) & 0xFFu);
            const uint32_t code = mag | (q < 0 ? 0x20u : 0u);
            const int bit = 6 * c;
            w[bit / 32] |= code << (bit % 32);
            if (bit % 32 > 26) w[bit / 32 + 1] |= code >> (32 - bit % 32);
        }
        // quarter (G >> 1) & 3 of 128-code unit G >> 3, half G & 1
        const int g = (G >> 1) & 3, slot = ((g & 1) << 1) | (g >> 1), h = G & 1;
        uint8_t *base = dst + (row >> 2) * ld_f6 + (row & 3) * 96 + (int64_t)(G >> 3) * 384;
        const int o0 = 16 * slot + 12 * h;
        const int o1 = h ? 64 + 8 * slot : o0 + 4;
        *reinterpret_cast<uint32_t *>(base + o0) = w[0];
        *reinterpret_cast<uint2 *>(base + o1) = make_uint2(w[1], w[2]);
    }
}

hipError_t launch_repack_w4_e2m3(const uint8_t *w_s4, int64_t ld_s4, int64_t N, int64_t K_pad, uint8_t *w_f6,
                                 int64_t ld_f6, hipStream_t st)
{
    const int groups = (int)(K_pad / 16);
    const int64_t total = N * groups;
    const int64_t blocks = (total + 255) / 256;
    const dim3 grid((unsigned)(blocks < 65536 ? blocks : 65536));
    hipLaunchKernelGGL(repack_w4_e2m3_kernel, grid, dim3(256), 0, st, w_s4, ld_s4, N, groups, w_f6, ld_f6);
    return hipGetLastError();
}

hipError_t launch_swiglu(const void *h, int dtype, int64_t ld_h, int64_t M, int64_t F, float *out,
                         int64_t ld_out, hipStream_t st)
{
    const int64_t total = M * F;
    const int threads = 256;
    const int64_t want = (total + threads - 1) / threads;
    const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
    switch (dtype) {
    case 0: {
        // every workgroup tabulates sigma first: larger workgroups, fewer of them
        const int64_t want16 = (total + 1023) / 1024;
        hipLaunchKernelGGL(swiglu_kernel<0>, dim3((unsigned)(want16 < 2048 ? want16 : 2048)), dim3(1024),
                           kSigTableBytes, st, static_cast<const uint16_t *>(h), ld_h, M, F, out, ld_out);
        break;
    }
    case 1: hipLaunchKernelGGL(swiglu_kernel<1>, dim3(blocks), dim3(threads), 0, st,
                               static_cast<const uint16_t *>(h), ld_h, M, F, out, ld_out); break;
    case 2: hipLaunchKernelGGL(swiglu_kernel<2>, dim3(blocks), dim3(threads), 0, st,
                               static_cast<const float *>(h), ld_h, M, F, out, ld_out); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_quant_act_swiglu(const void *h, int dtype, int64_t ld_h, int64_t M, int64_t F,
                                   const float *pre, int8_t *x_s8, int64_t ld_s8, float *x_scale,
                                   bool two_pass, bool transposed, hipStream_t st)
{
    switch (dtype) {
    case 0: return launch_swiglu<0>(h, ld_h, M, F, pre, x_s8, ld_s8, x_scale, two_pass, transposed, st);
    case 1: return launch_swiglu<1>(h, ld_h, M, F, pre, x_s8, ld_s8, x_scale, two_pass, transposed, st);
    case 2: return launch_swiglu<2>(h, ld_h, M, F, pre, x_s8, ld_s8, x_scale, two_pass, transposed, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace convrot
