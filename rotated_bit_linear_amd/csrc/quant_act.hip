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

// 16 consecutive elements starting at p (16-byte aligned) as fp32.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// The activation is read exactly once: non-temporal loads keep it from displacing the
// GEMM operands in L2.
template <int DT>
__device__ __forceinline__ void load16_vec(const typename Elem<DT>::T *p, float (&v)[16])
{
    if constexpr (DT == 2) {
#pragma unroll
        for (int c = 0; c < 4; c++) {
            f32x4 q = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p) + c);
            v[4 * c] = q.x; v[4 * c + 1] = q.y; v[4 * c + 2] = q.z; v[4 * c + 3] = q.w;
        }
    } else {
#pragma unroll
        for (int c = 0; c < 2; c++) {
            u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p) + c);
            uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                v[8 * c + 2 * i] = Elem<DT>::cvt((uint16_t)(w[i] & 0xffffu));
                v[8 * c + 2 * i + 1] = Elem<DT>::cvt((uint16_t)(w[i] >> 16));
            }
        }
    }
}

// Elements [k0, k0+16) of a row with logical length K (zero past K); `aligned` says the
// row base permits 16-byte vector loads.
template <int DT>
__device__ __forceinline__ void load16_row(const typename Elem<DT>::T *row, int64_t k0, int64_t K,
                                           bool aligned, float (&v)[16])
{
    if (aligned && k0 + 16 <= K) {
        load16_vec<DT>(row + k0, v);
        return;
    }
    if (k0 >= K) {                     // pure padding: nothing is read
#pragma unroll
        for (int i = 0; i < 16; i++) v[i] = 0.0f;
        return;
    }
#pragma unroll
    for (int i = 0; i < 16; i++) v[i] = (k0 + i < K) ? Elem<DT>::cvt(row[k0 + i]) : 0.0f;
}

// ------------------------------------------------------ reproducible exponential ----

// E(x) ~ exp(x) from IEEE basic operations only: Cody & Waite (1980) reduction
// x = k ln2 + r, k = rint(x log2 e), ln2 = C1 + C2 with C1 holding 15 significant bits,
// then the degree-7 Taylor polynomial of exp(r) in Horner form with fused multiply-adds,
// then the exact scaling by 2^k.  Coefficients: RN(1/n!).
__device__ __forceinline__ float repro_exp(float x)
{
    const float kLog2e = 0x1.715476p+0f;
    const float kC1 = 0x1.62e4p-1f;
    const float kC2 = 0x1.7f7d1cp-20f;
    if (x != x) return x;
    if (x > 89.0f) return __builtin_inff();
    if (x < -104.0f) return 0.0f;
    const float kf = rintf(x * kLog2e);
    float r = fmaf(-kf, kC1, x);
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

// swish(gate) * value with swish(a) = a / (1 + E(-a)) evaluated as a * (1 / (1 + E(-a))).
__device__ __forceinline__ float swiglu_elem(float gate, float value)
{
    const float t = repro_exp(-gate);
    const float sig = 1.0f / (1.0f + t);
    const float sw = gate * sig;
    return sw * value;
}

// --------------------------------------------------------------------- loaders ----

template <int DT>
struct ActLoader {
    const typename Elem<DT>::T *x;
    int64_t ld;
    int64_t K;
    bool aligned;
    __device__ __forceinline__ void load16(int64_t row, int64_t seg, float (&v)[16]) const
    {
        load16_row<DT>(x + row * ld, seg * 16, K, aligned, v);
    }
};

template <int DT>
struct SwigluLoader {
    const typename Elem<DT>::T *h;
    int64_t ld;
    int64_t F;
    bool aligned_gate;
    bool aligned_value;
    __device__ __forceinline__ void load16(int64_t row, int64_t seg, float (&v)[16]) const
    {
        const typename Elem<DT>::T *r = h + row * ld;
        float b[16];
        load16_row<DT>(r, seg * 16, F, aligned_gate, v);
        load16_row<DT>(r + F, seg * 16, F, aligned_value, b);
#pragma unroll
        for (int i = 0; i < 16; i++) v[i] = swiglu_elem(v[i], b[i]);   // zero past F: 0 * sig * 0
    }
};

// Unfused SwiGLU: out[m, k] = swish(h[m, k]) * h[m, F + k] in FP32 (same element function
// as the fused path).  One thread per element, grid-stride over rows.
template <int DT>
__global__ void swiglu_kernel(const typename Elem<DT>::T *__restrict__ h, int64_t ld_h, int64_t M, int64_t F,
                              float *__restrict__ out, int64_t ld_out)
{
    const int64_t total = M * F;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = i / F, k = i - m * F;
        const float a = Elem<DT>::cvt(h[m * ld_h + k]);
        const float b = Elem<DT>::cvt(h[m * ld_h + F + k]);
        out[m * ld_out + k] = swiglu_elem(a, b);
    }
}

template <class Loader, int RB>
__global__ void quant_act_kernel(Loader ld, int nb, int8_t *__restrict__ out, int64_t ld_out,
                                 float *__restrict__ scale, int two_pass)
{
    row_prep<Loader, RB>(ld, (int64_t)blockIdx.x, nb, out, ld_out, scale, two_pass != 0);
}

// --------------------------------------------------------------------- launchers ----

template <class Loader>
static hipError_t launch_rows(const Loader &L, int64_t rows, int64_t nb, int8_t *out, int64_t ld_out,
                              float *scale, bool force_two_pass, hipStream_t st)
{
    const RowPrepShape s = row_prep_shape(nb, force_two_pass);
    const size_t lds = row_prep_lds_bytes(s.threads);
    if (s.rb == 2)
        hipLaunchKernelGGL((quant_act_kernel<Loader, 2>), dim3((unsigned)rows), dim3(s.threads), lds, st,
                           L, (int)nb, out, ld_out, scale, 0);
    else
        hipLaunchKernelGGL((quant_act_kernel<Loader, 1>), dim3((unsigned)rows), dim3(s.threads), lds, st,
                           L, (int)nb, out, ld_out, scale, s.two_pass ? 1 : 0);
    return hipGetLastError();
}

template <int DT>
static hipError_t launch_act(const void *x, int64_t ld_x, int64_t M, int64_t K, int8_t *x_s8,
                             int64_t ld_s8, float *x_scale, bool two_pass, hipStream_t st)
{
    ActLoader<DT> L{static_cast<const typename Elem<DT>::T *>(x), ld_x, K,
                    ((uintptr_t)x % 16 == 0) && ((ld_x * (int64_t)sizeof(typename Elem<DT>::T)) % 16 == 0)};
    return launch_rows(L, M, (K + 255) / 256, x_s8, ld_s8, x_scale, two_pass, st);
}

template <int DT>
static hipError_t launch_swiglu(const void *h, int64_t ld_h, int64_t M, int64_t F, int8_t *x_s8,
                                int64_t ld_s8, float *x_scale, bool two_pass, hipStream_t st)
{
    const int64_t es = (int64_t)sizeof(typename Elem<DT>::T);
    const bool row_ok = ((uintptr_t)h % 16 == 0) && ((ld_h * es) % 16 == 0);
    SwigluLoader<DT> L{static_cast<const typename Elem<DT>::T *>(h), ld_h, F, row_ok,
                       row_ok && ((F * es) % 16 == 0)};
    return launch_rows(L, M, (F + 255) / 256, x_s8, ld_s8, x_scale, two_pass, st);
}

hipError_t launch_quant_act(const void *x, int dtype, int64_t ld_x, int64_t M, int64_t K,
                            int8_t *x_s8, int64_t ld_s8, float *x_scale, bool two_pass,
                            hipStream_t st)
{
    switch (dtype) {
    case 0: return launch_act<0>(x, ld_x, M, K, x_s8, ld_s8, x_scale, two_pass, st);
    case 1: return launch_act<1>(x, ld_x, M, K, x_s8, ld_s8, x_scale, two_pass, st);
    case 2: return launch_act<2>(x, ld_x, M, K, x_s8, ld_s8, x_scale, two_pass, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_swiglu(const void *h, int dtype, int64_t ld_h, int64_t M, int64_t F, float *out,
                         int64_t ld_out, hipStream_t st)
{
    const int64_t total = M * F;
    const int threads = 256;
    const int64_t want = (total + threads - 1) / threads;
    const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
    switch (dtype) {
    case 0: hipLaunchKernelGGL(swiglu_kernel<0>, dim3(blocks), dim3(threads), 0, st,
                               static_cast<const uint16_t *>(h), ld_h, M, F, out, ld_out); break;
    case 1: hipLaunchKernelGGL(swiglu_kernel<1>, dim3(blocks), dim3(threads), 0, st,
                               static_cast<const uint16_t *>(h), ld_h, M, F, out, ld_out); break;
    case 2: hipLaunchKernelGGL(swiglu_kernel<2>, dim3(blocks), dim3(threads), 0, st,
                               static_cast<const float *>(h), ld_h, M, F, out, ld_out); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_quant_act_swiglu(const void *h, int dtype, int64_t ld_h, int64_t M, int64_t F,
                                   int8_t *x_s8, int64_t ld_s8, float *x_scale, bool two_pass,
                                   hipStream_t st)
{
    switch (dtype) {
    case 0: return launch_swiglu<0>(h, ld_h, M, F, x_s8, ld_s8, x_scale, two_pass, st);
    case 1: return launch_swiglu<1>(h, ld_h, M, F, x_s8, ld_s8, x_scale, two_pass, st);
    case 2: return launch_swiglu<2>(h, ld_h, M, F, x_s8, ld_s8, x_scale, two_pass, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace convrot
