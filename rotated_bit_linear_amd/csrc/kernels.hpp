// Internal launchers of the gfx950 kernels (argument checking happens in api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convrot {

// output tile of one GEMM workgroup (rows of A = activation rows, rows of B = weight rows)
constexpr int64_t kGemmTileCols = 256;   // M direction
constexpr int64_t kGemmTileRows = 256;   // N direction (weight rows)

// dtype codes follow cr_dtype: 0 bf16, 1 fp16, 2 fp32, 3 int32 (GEMM output only)
// pre: optional [K] (or [F]) channel pre-scale, nullptr for none; transposed: codes in the
// block-transposed column order (see row_prep.hpp)
hipError_t launch_quant_act(const void *x, int dtype, int64_t ld_x, int64_t M, int64_t K, const float *pre,
                            int8_t *x_s8, int64_t ld_s8, float *x_scale, bool two_pass, bool transposed,
                            hipStream_t st);

hipError_t launch_quant_act_swiglu(const void *h, int dtype, int64_t ld_h, int64_t M, int64_t F,
                                   const float *pre, int8_t *x_s8, int64_t ld_s8, float *x_scale,
                                   bool two_pass, bool transposed, hipStream_t st);

hipError_t launch_swiglu(const void *h, int dtype, int64_t ld_h, int64_t M, int64_t F, float *out,
                         int64_t ld_out, hipStream_t st);

// W4A8: dense weight rows -> ConvRot256 -> packed 4-bit codes [N, ld_s4 bytes] + scales
hipError_t launch_quant_weight_w4(const void *w, int dtype, int64_t ld_w, int64_t N, int64_t K, uint8_t *w_s4,
                                  int64_t ld_s4, float *w_scale, bool two_pass, bool transposed, hipStream_t st);

// The same 4-bit weight rows as E2M3 fields [N, ld_f6 bytes] (ld_f6 >= 3 K_pad / 4)
hipError_t launch_quant_weight_e2m3(const void *w, int dtype, int64_t ld_w, int64_t N, int64_t K, uint8_t *w_f6,
                                    int64_t ld_f6, float *w_scale, bool two_pass, bool transposed, hipStream_t st);

// nibble-form 4-bit rows [N, ld_s4] -> the same codes as E2M3 fields (quads of ld_f6 bytes)
hipError_t launch_repack_w4_e2m3(const uint8_t *w_s4, int64_t ld_s4, int64_t N, int64_t K_pad, uint8_t *w_f6,
                                 int64_t ld_f6, hipStream_t st);

// W4A4: activation rows (swiglu: H [M, 2K], SwiGLU first) -> ConvRot256 -> packed 4-bit
// codes [M, ld_s4 bytes] + scales, the format of launch_quant_weight_w4
hipError_t launch_quant_act_w4(const void *x, int dtype, int64_t ld_x, bool swiglu, int64_t M, int64_t K,
                               uint8_t *x_s4, int64_t ld_s4, float *x_scale, bool two_pass, bool transposed,
                               hipStream_t st);
hipError_t launch_quant_act_e2m3(const void *x, int dtype, int64_t ld_x, bool swiglu, int64_t M, int64_t K,
                                 uint8_t *x_f6, int64_t ld_f6, float *x_scale, bool two_pass, bool transposed,
                                 hipStream_t st);

hipError_t launch_prep_weight(const uint8_t *codes, int64_t ld_codes, const uint8_t *sf, int64_t ld_sf,
                              const float *g, int64_t n_rows, int64_t K, int8_t *w_s8, int64_t ld_s8,
                              float *w_scale, bool two_pass, bool transposed, hipStream_t st);

// bias: optional [N] FP32 bias added in the epilogue, nullptr for none (not with int32 out)
hipError_t launch_gemm_s8(const int8_t *A, int64_t lda, const float *sa, const int8_t *B, int64_t ldb,
                          const float *sb, const float *bias, int64_t M, int64_t N, int64_t K_pad, void *C,
                          int out_dtype, int64_t ldc, hipStream_t st);

// W4A8: S8 activation x packed 4-bit weight (the layout of launch_quant_weight_w4), same
// epilogue as launch_gemm_s8; ldb in bytes
hipError_t launch_gemm_s8s4(const int8_t *A, int64_t lda, const float *sa, const uint8_t *B, int64_t ldb,
                            const float *sb, const float *bias, int64_t M, int64_t N, int64_t K_pad, void *C,
                            int out_dtype, int64_t ldc, hipStream_t st);

// W4A4: packed 4-bit activation x packed 4-bit weight, same epilogue; lda, ldb in bytes
hipError_t launch_gemm_s4s4(const uint8_t *A, int64_t lda, const float *sa, const uint8_t *B, int64_t ldb,
                            const float *sb, const float *bias, int64_t M, int64_t N, int64_t K_pad, void *C,
                            int out_dtype, int64_t ldc, hipStream_t st);

// W4A4 on the 6-bit matrix cores: two E2M3-field operands (lda, ldb in bytes), same epilogue
hipError_t launch_gemm_e2m3(const uint8_t *A, int64_t lda, const float *sa, const uint8_t *B, int64_t ldb,
                            const float *sb, const float *bias, int64_t M, int64_t N, int64_t K_pad, void *C,
                            int out_dtype, int64_t ldc, hipStream_t st);

// row maximum a = max |rotated row| of NVFP4 weight rows (no codes)
hipError_t launch_weight_amax(const uint8_t *codes, int64_t ld_codes, const uint8_t *sf, int64_t ld_sf,
                              const float *g, int64_t n_rows, int64_t K, float *amax, bool two_pass,
                              hipStream_t st);

// decode-inside-GEMM over NVFP4 weights with given row maxima (transposed: order of A)
hipError_t launch_gemm_nvfp4_fused(const int8_t *A, int64_t lda, const float *sa, const uint8_t *codes,
                                   int64_t ld_codes, const uint8_t *sf, int64_t ld_sf, const float *g,
                                   const float *amax, const float *bias, int64_t M, int64_t N, int64_t K,
                                   void *C, int out_dtype, int64_t ldc, bool transposed, hipStream_t st);


}  // namespace convrot
