// Weight preparation kernel: NVFP4 decode + ConvRot256 + per-row S8 quantization, fused.
//
// ComfyUI Turing Utils README, "Load ConvRot DiT ..." bullet: packed NVFP4 weights stay
// unchanged in memory; for each call a bounded tile of rows is decoded, rotated in FP32
// with the same block rotation as the activations, and quantized to S8 with an FP32 row
// scale; logical K is zero-padded to a multiple of 256 and serialized padding is ignored.
// The same kernel in "row maximum" mode writes only a[n] = max |rotated row| (no codes),
// which a GEMM that quantizes weight blocks on the fly needs before it starts.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"
#include "row_prep.hpp"
#include "nvfp4.hpp"

namespace convrot {

template <int RB>
__global__ __launch_bounds__(row_prep_max_threads<RB>()) void prep_weight_kernel(NVFP4Loader ld, int64_t n_rows, int nb, int8_t *__restrict__ out,
                                   int64_t ld_out, float *__restrict__ scale, int mode)
{
    ld.gs = *ld.g;
    row_prep_kernel_body<NVFP4Loader, RB>(ld, n_rows, nb, out, ld_out, scale, mode);
}

// Rows of 65-128 blocks in one pass (the wide form): two blocks per lane group in up to 64
// groups, 1024 threads at most.
__global__ __launch_bounds__(1024) void prep_weight_wide_kernel(NVFP4Loader ld, int64_t n_rows, int nb, int8_t *__restrict__ out,
                                                                int64_t ld_out, float *__restrict__ scale, int mode)
{
    ld.gs = *ld.g;
    row_prep_kernel_body<NVFP4Loader, 2>(ld, n_rows, nb, out, ld_out, scale, mode);
}

// Several short rows per workgroup (see row_prep_multi): rows of up to 32 blocks whose
// lane groups would not fill the workgroup's last wave.
__global__ __launch_bounds__(1024) void prep_weight_multi_kernel(NVFP4Loader ld, int64_t n_rows, int nb, int rpw,
                                                               int8_t *__restrict__ out, int64_t ld_out,
                                                               float *__restrict__ scale, int mode)
{
    ld.gs = *ld.g;
    row_prep_multi(ld, n_rows, nb, rpw, out, ld_out, scale, (mode & 2) == 0, (mode & 4) != 0);
}

// the multi-row launch when it leaves fewer lanes idle than one row per workgroup
static bool launch_multi(const NVFP4Loader &L, int64_t n_rows, int64_t nb, bool two_pass, int8_t *out,
                         int64_t ld_out, float *scale, int mode, hipStream_t st)
{
    if (two_pass || nb > 32) return false;
    const int rpw = row_prep_multi_rows(nb);
    if (rpw < 2) return false;
    const int threads = (int)((rpw * nb + 3) / 4 * 64);
    const size_t lds = row_prep_multi_lds_bytes(threads);
    const RowPrepShape s{threads, 1, false};
    const void *k = reinterpret_cast<const void *>(&prep_weight_multi_kernel);
    const dim3 grid((unsigned)row_prep_grid((n_rows + rpw - 1) / rpw, s, k, lds));
    hipLaunchKernelGGL(prep_weight_multi_kernel, grid, dim3(threads), lds, st, L, n_rows, (int)nb, rpw, out, ld_out,
                       scale, mode);
    return true;
}

hipError_t launch_prep_weight(const uint8_t *codes, int64_t ld_codes, const uint8_t *sf, int64_t ld_sf,
                              const float *g, int64_t n_rows, int64_t K, int8_t *w_s8, int64_t ld_s8,
                              float *w_scale, bool two_pass, bool transposed, hipStream_t st)
{
    const int64_t nb = (K + 255) / 256;
    const RowPrepShape s = row_prep_shape(nb, two_pass);
    const size_t lds = row_prep_lds_bytes(s.threads);
    const int mode = (s.two_pass ? 1 : 0) | (transposed ? 2 : 0);
    NVFP4Loader L{codes, ld_codes, sf, ld_sf, g, K, 0.0f};
    if (launch_multi(L, n_rows, nb, s.two_pass, w_s8, ld_s8, w_scale, mode, st)) return hipGetLastError();
    if (s.wide) {
        const void *k = reinterpret_cast<const void *>(&prep_weight_wide_kernel);
        const dim3 grid((unsigned)row_prep_grid(n_rows, s, k, lds));
        hipLaunchKernelGGL(prep_weight_wide_kernel, grid, dim3(s.threads), lds, st,
                           L, n_rows, (int)nb, w_s8, ld_s8, w_scale, mode);
    } else if (s.rb == 2) {
        const void *k = reinterpret_cast<const void *>(&prep_weight_kernel<2>);
        const dim3 grid((unsigned)row_prep_grid(n_rows, s, k, lds));
        hipLaunchKernelGGL(prep_weight_kernel<2>, grid, dim3(s.threads), lds, st,
                           L, n_rows, (int)nb, w_s8, ld_s8, w_scale, mode);
    } else {
        const void *k = reinterpret_cast<const void *>(&prep_weight_kernel<1>);
        const dim3 grid((unsigned)row_prep_grid(n_rows, s, k, lds));
        hipLaunchKernelGGL(prep_weight_kernel<1>, grid, dim3(s.threads), lds, st,
                           L, n_rows, (int)nb, w_s8, ld_s8, w_scale, mode);
    }
    return hipGetLastError();
}

hipError_t launch_weight_amax(const uint8_t *codes, int64_t ld_codes, const uint8_t *sf, int64_t ld_sf,
                              const float *g, int64_t n_rows, int64_t K, float *amax, bool two_pass,
                              hipStream_t st)
{
    const int64_t nb = (K + 255) / 256;
    const RowPrepShape s = row_prep_shape(nb, two_pass);
    const size_t lds = row_prep_lds_bytes(s.threads);
    const int mode = (s.two_pass ? 1 : 0) | 2 | 4;     // the order of z does not matter for the maximum
    NVFP4Loader L{codes, ld_codes, sf, ld_sf, g, K, 0.0f};
    if (launch_multi(L, n_rows, nb, s.two_pass, nullptr, 0, amax, mode, st)) return hipGetLastError();
    if (s.wide) {
        const void *k = reinterpret_cast<const void *>(&prep_weight_wide_kernel);
        const dim3 grid((unsigned)row_prep_grid(n_rows, s, k, lds));
        hipLaunchKernelGGL(prep_weight_wide_kernel, grid, dim3(s.threads), lds, st,
                           L, n_rows, (int)nb, nullptr, (int64_t)0, amax, mode);
    } else if (s.rb == 2) {
        const void *k = reinterpret_cast<const void *>(&prep_weight_kernel<2>);
        const dim3 grid((unsigned)row_prep_grid(n_rows, s, k, lds));
        hipLaunchKernelGGL(prep_weight_kernel<2>, grid, dim3(s.threads), lds, st,
                           L, n_rows, (int)nb, nullptr, (int64_t)0, amax, mode);
    } else {
        const void *k = reinterpret_cast<const void *>(&prep_weight_kernel<1>);
        const dim3 grid((unsigned)row_prep_grid(n_rows, s, k, lds));
        hipLaunchKernelGGL(prep_weight_kernel<1>, grid, dim3(s.threads), lds, st,
                           L, n_rows, (int)nb, nullptr, (int64_t)0, amax, mode);
    }
    return hipGetLastError();
}

}  // namespace convrot
