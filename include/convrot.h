/*
 * convrot.h — C ABI of the MI355X (gfx950) rotated W8A8 linear layer over NVFP4 weights.
 *
 * What the layer computes (ComfyUI Turing Utils README on comfy.icu, section "Nodes",
 * bullet "Load ConvRot DiT and Load ConvRot CLIP"; MiniMax H3 explainer on modelpad.app,
 * "Foundations" and the MLP and "convrot" paragraphs):
 *   y = x W^T for a linear layer whose weight W [N, K] is stored packed as NVFP4.
 *   Both operands are zero-padded along K to K_pad = 256 * ceil(K / 256), rotated by the
 *   same 256-wide block rotation R = H/16 (H the Sylvester-ordered Walsh-Hadamard matrix
 *   of order 256, applied to each 256-column block), quantized per row to symmetric S8
 *   with an FP32 scale, multiplied in an INT8 GEMM with int32 accumulation, and the
 *   accumulator is dequantized by the two row scales.  Because R R^T = I the rotation
 *   cancels in the product; it only spreads outlier channels before quantization.
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers unless stated otherwise.  The caller owns every buffer;
 *     outputs must not alias inputs.  Calls are asynchronous on `stream`; nothing is
 *     synchronised and no device memory is allocated.
 *   - Arguments are validated on the host before anything is enqueued; a non-CR_OK status
 *     means nothing was launched.  Faults inside a launched kernel surface at the caller's
 *     next synchronisation.  There is no fallback path: an unsupported device (anything
 *     but gfx950) yields CR_ERR_NO_DEVICE.
 *   - Strides (ld_*) are in elements of the pointed-to type.  Every base pointer must be
 *     16-byte aligned and every row stride a multiple of 16 bytes, except the NVFP4 block
 *     scales (any stride) and the output of the GEMM (element-aligned).  Violations return
 *     CR_ERR_MISALIGNED.
 *   - K_pad may not exceed CR_MAX_K_PAD, so that 127 * 127 * K_pad fits in an int32.
 *   - A GEMM may have at most 8388607 output tiles of 256 x 256 (ceil(M/256) * ceil(N/256)),
 *     and cr_gemm_nvfp4_fused at most 536870880 weight rows: a dispatch counts its work-items
 *     in 32 bits.  Larger shapes return CR_ERR_TOO_LARGE; split them along M or N.
 *   - Empty extents: a row count M (or n_rows) or an output width N of 0 is a valid call
 *     that enqueues nothing and returns CR_OK once the other arguments pass the checks
 *     that do not depend on the empty extent (dtypes, flags, K >= 1, strides); buffers of
 *     zero size may be NULL.  K (or F) must be at least 1: the layer has at least one
 *     input column.  Negative sizes are CR_ERR_INVALID_ARG.
 *   - Rows are independent.  A row whose maximum |value| after rotation is 0 gets scale 0
 *     and all-zero codes.
 *   - Inputs are assumed finite.  A NaN or an infinity in an activation row, or a NaN E4M3
 *     block scale in a weight row, leaves that row's codes, scale and outputs unspecified;
 *     every other row is unaffected (bit for bit), and the call still completes.
 *
 * Arithmetic (binary32, round to nearest even; each step evaluated exactly as written):
 *   NVFP4 element k of weight row n: code = nibble k of the row (low nibble of byte k/2
 *     for even k, high nibble for odd k), block scale = E4M3 byte k/16 of the row,
 *     value = fp32(E2M1(code) * E4M3(scale)) * g, g the FP32 global scale; columns
 *     k >= K are 0 whatever bytes the row padding holds.
 *   SwiGLU element (MiniMax H3 explainer, MLP paragraph): gate a = h[m, k], value
 *     b = h[m, F + k]; sigma = 1 / (1 + E(-a)) with E a fixed exp built from IEEE basic
 *     operations (Cody-Waite reduction, degree-7 Taylor polynomial, scaling by 2^k);
 *     result (a * sigma) * b, kept in FP32.
 *   Rotation: per 256-block, butterfly stages h = 1, 2, ..., 128 ((u, v) -> (u+v, u-v)
 *     on the pair j, j+h), then * 0.0625.
 *   Row quantization: a = max |y|; scale = a / 127; r = 127 / a; q = clamp(rint(y * r),
 *     -127, 127).  A row whose 127 / a overflows FP32 (a below about 3.7e-37) is quantized
 *     as its exact copy multiplied by 2^64 (the codes of a row do not change under exact
 *     power-of-two scaling wherever r is finite); its scale is still a / 127.
 *   Epilogue: out = ((float)acc * a_scale[m]) * b_scale[n], rounded once to the output type.
 */
#ifndef CONVROT_H
#define CONVROT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CR_ABI_VERSION 3
#define CR_MAX_K_PAD 133120       /* largest multiple of 256 with 127*127*K_pad < 2^31 */
#define CR_TWO_PASS_K_PAD 16384   /* SwiGLU and fp32 activation rows (and dense fp32 4-bit weight
                                     rows) with K_pad above this stream twice */
#define CR_W_TWO_PASS_K_PAD 32768 /* NVFP4 weight rows, and bf16/fp16 plain activation rows and
                                     dense 4-bit weight rows, with K_pad above this stream twice */
#define CR_DEFAULT_MAX_TILE_BYTES ((size_t)128 << 20)

typedef enum {
    CR_OK = 0,
    CR_ERR_INVALID_ARG = 1,       /* null pointer, negative size, K < 1, stride too small, bad flag */
    CR_ERR_UNSUPPORTED_DTYPE = 2, /* dtype not accepted by this entry point */
    CR_ERR_MISALIGNED = 3,        /* base pointer or row stride alignment violated */
    CR_ERR_TOO_LARGE = 4,         /* K_pad > CR_MAX_K_PAD, or workspace too small */
    CR_ERR_NO_DEVICE = 5,         /* no current HIP device, or it is not gfx950 */
    CR_ERR_LAUNCH = 6,            /* the HIP runtime rejected a launch or an event call */
    /* not statuses: they give the type the whole range of int, so that any int a C caller
     * passes is a value of the type (the library reads it; unknown values are rejected) */
    CR_STATUS_RANGE_MIN_ = -0x7fffffff - 1,
    CR_STATUS_RANGE_MAX_ = 0x7fffffff
} cr_status;

typedef enum {
    CR_BF16 = 0, CR_FP16 = 1, CR_FP32 = 2, CR_I32 = 3,
    /* not dtypes: the whole range of int, as for cr_status (unknown values are
     * CR_ERR_UNSUPPORTED_DTYPE) */
    CR_DTYPE_RANGE_MIN_ = -0x7fffffff - 1,
    CR_DTYPE_RANGE_MAX_ = 0x7fffffff
} cr_dtype;

enum {
    CR_FLAG_NONE = 0,
    CR_FLAG_FORCE_TWO_PASS = 1,   /* stream rows twice whatever their length */
    CR_FLAG_BLOCK_TRANSPOSED = 2  /* S8 codes in block-transposed column order (below) */
};

/* Column order of the S8 outputs of the preparation calls.  Default (natural): column k
 * holds the code of rotated element k.  With CR_FLAG_BLOCK_TRANSPOSED, inside every
 * 256-column block, column 16 t + j holds the code of rotated element 16 j + t (t, j in
 * 0..15): the same codes and row scales, in an order the kernels can write without their
 * last LDS transposition.  The GEMM sums over K, so cr_gemm_s8_rowscale gives the same
 * int32 sums when both of its operands use the same order; mixing orders is an error the
 * library cannot detect.  cr_linear_nvfp4 uses the transposed order for its workspace. */

/* ABI version of the loaded library (CR_ABI_VERSION when header and library match). */
int cr_abi_version(void);

/* Static, human-readable name of a status. */
const char *cr_status_string(cr_status s);

/* 256 * ceil(k / 256) for k >= 1; 0 for k < 1. */
int64_t cr_padded_k(int64_t k);

/*
 * Weight preparation: NVFP4 decode, ConvRot256, row quantization (the three are fused;
 * ComfyUI Turing Utils README, "Load ConvRot DiT ..." bullet: decode, FP32 rotation and
 * S8 quantization of the weight are one step, and only a bounded call-local S8 tile is
 * expanded while the packed NVFP4 bytes stay untouched).
 *   w_fp4        [n_rows, ld_fp4] uint8, element k in byte k/2 (low nibble = even k);
 *                ld_fp4 >= ceil(K/2), a multiple of 16.
 *   w_sf         [n_rows, ld_sf] uint8 E4M3 block scales, ld_sf >= ceil(K/16), any stride.
 *   global_scale device pointer to one float g.
 *   n_rows, K    rows to prepare and the logical K (1 <= K, K_pad <= CR_MAX_K_PAD).
 *   w_s8         [n_rows, ld_s8] int8 out, ld_s8 >= K_pad, a multiple of 16.
 *   w_scale      [n_rows] float out.
 *   flags        CR_FLAG_NONE, CR_FLAG_FORCE_TWO_PASS and/or CR_FLAG_BLOCK_TRANSPOSED.
 */
cr_status cr_prep_weight_nvfp4(const uint8_t *w_fp4, int64_t ld_fp4,
                               const uint8_t *w_sf, int64_t ld_sf,
                               const float *global_scale, int64_t n_rows, int64_t K,
                               int8_t *w_s8, int64_t ld_s8, float *w_scale,
                               uint32_t flags, hipStream_t stream);

/*
 * Activation preparation: ConvRot256 and row quantization of X [M, K] (same bullet:
 * the rotation is paired, identical for activations and weights).
 *   x        [M, ld_x] of x_dtype (CR_BF16, CR_FP16 or CR_FP32); ld_x >= K.
 *   x_s8     [M, ld_s8] int8 out, ld_s8 >= K_pad.   x_scale [M] float out.
 */
cr_status cr_quant_act(const void *x, cr_dtype x_dtype, int64_t ld_x, int64_t M, int64_t K,
                       int8_t *x_s8, int64_t ld_s8, float *x_scale,
                       uint32_t flags, hipStream_t stream);

/*
 * Fused SwiGLU + activation preparation (same bullet: SwiGLU runs before the rotation;
 * MiniMax H3 explainer, MLP paragraph: the first half of fc1's output is the gate).
 *   h        [M, ld_h] of h_dtype; gate = h[:, 0:F], value = h[:, F:2F]; ld_h >= 2F.
 *   F        logical width of the SwiGLU output (the GEMM's K).
 *   x_s8     [M, ld_s8] int8 out with ld_s8 >= 256 * ceil(F/256); x_scale [M] float out.
 */
cr_status cr_quant_act_swiglu(const void *h, cr_dtype h_dtype, int64_t ld_h, int64_t M, int64_t F,
                              int8_t *x_s8, int64_t ld_s8, float *x_scale,
                              uint32_t flags, hipStream_t stream);

/*
 * Activation preparation with an optional channel pre-scale (ComfyUI Turing Utils README,
 * "Load ConvRot DiT ..." bullet: pre-scales and SwiGLU run before the rotation, and channel
 * pre-scales keep the unfused order).  The loaded value of channel k (for swiglu != 0 the
 * SwiGLU value) is multiplied by pre_scale[k] in FP32, then rotated and quantized as in
 * cr_quant_act / cr_quant_act_swiglu.
 *   x, x_dtype, ld_x   X [M, K], or H [M, 2K] when swiglu != 0 (K is then F).
 *   pre_scale          [K] float, 4-byte aligned, or NULL (then identical to the calls
 *                      above).  Channels k >= K are padding and stay 0.
 *   x_s8, ld_s8, x_scale, flags as above.
 */
cr_status cr_quant_act_ex(const void *x, cr_dtype x_dtype, int64_t ld_x, int swiglu, int64_t M, int64_t K,
                          const float *pre_scale, int8_t *x_s8, int64_t ld_s8, float *x_scale,
                          uint32_t flags, hipStream_t stream);

/*
 * Unfused SwiGLU to FP32 (the ComfyUI Turing Utils README compares the fused
 * SwiGLU + rotation + A8 path against an unfused activation): out[m, k] =
 * swish(h[m, k]) * h[m, F + k] with the same element arithmetic as cr_quant_act_swiglu.
 *   h [M, ld_h] of h_dtype (element-aligned), ld_h >= 2F; out [M, ld_out] float, ld_out >= F.
 */
cr_status cr_swiglu(const void *h, cr_dtype h_dtype, int64_t ld_h, int64_t M, int64_t F,
                    float *out, int64_t ld_out, hipStream_t stream);

/*
 * Row-scaled INT8 GEMM with the dequantizing epilogue fused (the int32 accumulator never
 * reaches memory unless c_dtype is CR_I32; MiniMax H3 explainer, fused-kernel paragraph).
 *   a_s8 [M, lda] int8 and b_s8 [N, ldb] int8, both K-contiguous; K_pad a multiple of 256.
 *   a_scale [M], b_scale [N] float; may be NULL only when c_dtype == CR_I32.
 *   c [M, ldc] of c_dtype (CR_BF16, CR_FP16, CR_FP32 or CR_I32 for the raw accumulator);
 *   ldc >= N; columns n >= N of each output row are never written.
 */
cr_status cr_gemm_s8_rowscale(const int8_t *a_s8, int64_t lda, const float *a_scale,
                              const int8_t *b_s8, int64_t ldb, const float *b_scale,
                              int64_t M, int64_t N, int64_t K_pad,
                              void *c, cr_dtype c_dtype, int64_t ldc, hipStream_t stream);

/*
 * The same GEMM with a bias added in the epilogue (MiniMax H3 explainer, "Foundations":
 * a linear layer is y = x W^T + b; glossary entry "Epilogue": scaling and bias fused onto
 * the end of the GEMM):
 *   out = (((float)acc * a_scale[m]) * b_scale[n]) + bias[n], each operation rounded in
 *   FP32, then one rounding to c_dtype.
 *   bias  [N] float, 4-byte aligned, or NULL (then identical to cr_gemm_s8_rowscale).
 *         Not accepted with CR_I32 (CR_ERR_INVALID_ARG).
 */
cr_status cr_gemm_s8_rowscale_bias(const int8_t *a_s8, int64_t lda, const float *a_scale,
                                   const int8_t *b_s8, int64_t ldb, const float *b_scale,
                                   const float *bias, int64_t M, int64_t N, int64_t K_pad,
                                   void *c, cr_dtype c_dtype, int64_t ldc, hipStream_t stream);

/*
 * The whole layer with bounded call-local staging (ComfyUI Turing Utils README, same
 * bullet: weights stay packed, S8 weight tiles of bounded size are prepared per chunk of
 * output columns, optionally on a second stream with producer/consumer events; serial and
 * pipelined results are identical).
 *   x          [M, ld_x] X (or H [M, ld_h] with 2K columns used when swiglu != 0).
 *   K          logical K of the GEMM (F when swiglu != 0).
 *   w_fp4, ld_fp4, w_sf, ld_sf, global_scale   the NVFP4 weight [N, K] as above.
 *   out [M, ldc] of out_dtype (not CR_I32).
 *   workspace  device buffer of at least cr_linear_nvfp4_workspace_bytes(...) bytes,
 *              256-byte aligned; holds the S8 activation, its scales and the S8 weight
 *              tiles (two when the weight is chunked).  An empty layer (M or N = 0)
 *              needs none: the size is 0 and workspace, x and out may be NULL.
 *   max_tile_bytes  bound of one S8 weight tile (0 selects CR_DEFAULT_MAX_TILE_BYTES);
 *              tiles hold a multiple of 256 rows (at least 256).
 *   s_main     stream of the activation preparation and the GEMMs.
 *   s_aux      NULL: weight tiles are prepared on s_main (serial staging); otherwise,
 *              when the weight takes more than one chunk, they are prepared on s_aux,
 *              ordered against s_main by events (a single chunk is staged on s_main).
 *              On MI355X serial staging measured faster (1-3.5 % per layer at 19989
 *              rows): a preparation kernel beside a running GEMM competes for its CUs.
 *              On return all work is ordered before any later work on s_main.
 * Short batches (M <= 64) take the decode-inside-GEMM path instead: the activation
 * preparation, then cr_gemm_nvfp4_fused with w_amax NULL (the row maxima from its own
 * first pass), both on s_main (s_aux is not used); the workspace then holds the S8
 * activation and its scales, and max_tile_bytes is not used.  Both paths give the same
 * bits.
 */
size_t cr_linear_nvfp4_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t max_tile_bytes);

/* The chunking cr_linear_nvfp4 uses on the current device: rows per weight chunk (a
 * multiple of 256) and the number of chunks.  The bound max_tile_bytes caps a chunk.  A
 * weight the bound splits gets the chunk height, within the bound, whose GEMMs need the
 * fewest workgroup rounds over the device's compute units in total (the tallest such
 * height).  A weight that fits one chunk is still split in two when the two GEMMs need no
 * more rounds than one: with a second stream the second chunk is then prepared while the
 * first multiplies, and staged serially the split costs nothing.  Both are 0 for short
 * batches (M <= 64), which decode the weight inside the GEMM, and for an empty layer (M or
 * N = 0, which needs no workspace and launches nothing).  Host pointers; CR_OK or an
 * argument status. */
cr_status cr_linear_nvfp4_plan(int64_t M, int64_t N, int64_t K, size_t max_tile_bytes,
                               int64_t *rows_per_chunk, int64_t *nchunks);

cr_status cr_linear_nvfp4(const void *x, cr_dtype x_dtype, int64_t ld_x, int swiglu,
                          int64_t M, int64_t K,
                          const uint8_t *w_fp4, int64_t ld_fp4,
                          const uint8_t *w_sf, int64_t ld_sf, const float *global_scale,
                          int64_t N, void *out, cr_dtype out_dtype, int64_t ldc,
                          void *workspace, size_t ws_bytes, size_t max_tile_bytes,
                          uint32_t flags, hipStream_t s_main, hipStream_t s_aux);

/* The layer with an optional channel pre-scale of its input (pre_scale [K] or NULL, as in
 * cr_quant_act_ex) and an optional bias (bias [N] or NULL, as in cr_gemm_s8_rowscale_bias);
 * the other arguments as in cr_linear_nvfp4, which is this call with both NULL. */
cr_status cr_linear_nvfp4_ex(const void *x, cr_dtype x_dtype, int64_t ld_x, int swiglu,
                             int64_t M, int64_t K, const float *pre_scale,
                             const uint8_t *w_fp4, int64_t ld_fp4,
                             const uint8_t *w_sf, int64_t ld_sf, const float *global_scale,
                             int64_t N, const float *bias, void *out, cr_dtype out_dtype, int64_t ldc,
                             void *workspace, size_t ws_bytes, size_t max_tile_bytes,
                             uint32_t flags, hipStream_t s_main, hipStream_t s_aux);

/*
 * W4A8 variant: 4-bit weights, 8-bit activations (ComfyUI Turing Utils README, opening
 * paragraph and section "Nodes", bullet "Load ConvRot DiT": the ConvRot path dispatches
 * W8A8, W4A8 and W4A4 layers; section "Turing behavior": a packed W4A8 kernel).  The pages
 * name the format but do not describe it; this library reads it as the W8A8 method with
 * 4-bit weight rows: ConvRot256 as above, then per weight row a = max |y|, scale = a / 7,
 * r = 7 / a (rounded to FP32), q = clamp(rint(y * r), -7, 7), the 2^64 extension for rows
 * whose 7 / a overflows; activations as for W8A8; int32 accumulation; the same epilogue.
 *
 * Packed 4-bit codes (this library's format): a row of K_pad codes takes K_pad / 2 bytes
 * in units of 32 bytes per 64 codes.  A unit's groups of 16 codes G0 (codes 0..15), G1,
 * G2, G3 are stored in the order G0, G2, G1, G3, 8 bytes each; a group's codes c[0..15]
 * are two's complement nibbles, byte j (j = 0..3) holding c[j] (low nibble) and c[4 + j]
 * (high nibble), byte 4 + j holding c[8 + j] and c[12 + j].  The codes follow the column
 * order of the flags (natural, or block-transposed with CR_FLAG_BLOCK_TRANSPOSED).
 *
 * Weight preparation (done once, offline: the packed codes and scales are what a W4A8
 * checkpoint stores):
 *   w          [N, ld_w] of w_dtype (CR_BF16, CR_FP16 or CR_FP32), the dense weight;
 *              ld_w >= K, rows of 16-byte multiples, 16-byte aligned.
 *   w_s4       [N, ld_s4] bytes out, ld_s4 >= K_pad / 2, a multiple of 16.
 *   w_scale    [N] float out (a / 7).
 *   flags      CR_FLAG_NONE, CR_FLAG_FORCE_TWO_PASS and/or CR_FLAG_BLOCK_TRANSPOSED.
 */
cr_status cr_quant_weight_w4(const void *w, cr_dtype w_dtype, int64_t ld_w, int64_t N, int64_t K,
                             uint8_t *w_s4, int64_t ld_s4, float *w_scale, uint32_t flags, hipStream_t stream);

/*
 * W4A8 GEMM: out = ((float)sum_k a_s8[m, k] q[n, k] * a_scale[m]) * b_scale[n] (+ bias[n]),
 * q the codes of the packed weight b_s4 [N, ldb bytes] (ldb >= K_pad / 2, a multiple of
 * 16).  The other arguments, the limits and CR_I32 as in cr_gemm_s8_rowscale_bias; both
 * operands must use the same column order.
 */
cr_status cr_gemm_s8s4_rowscale(const int8_t *a_s8, int64_t lda, const float *a_scale,
                                const uint8_t *b_s4, int64_t ldb, const float *b_scale, const float *bias,
                                int64_t M, int64_t N, int64_t K_pad, void *c, cr_dtype c_dtype, int64_t ldc,
                                hipStream_t stream);

/*
 * The W4A8 layer: activation preparation of X [M, K] (or of SwiGLU(H [M, 2K]) when swiglu
 * != 0) into the workspace, then cr_gemm_s8s4_rowscale against the prepared weight, both on
 * `stream`.  flags: CR_FLAG_BLOCK_TRANSPOSED when the weight's codes are in that order (the
 * activation is then prepared in the same order), CR_FLAG_FORCE_TWO_PASS.  workspace:
 * cr_linear_w4a8_workspace_bytes(M, K) bytes, 256-byte aligned (S8 activation and its
 * scales); an empty layer (M or N = 0) needs none.  out [M, ldc] of out_dtype (not CR_I32).
 */
size_t cr_linear_w4a8_workspace_bytes(int64_t M, int64_t K);
cr_status cr_linear_w4a8(const void *x, cr_dtype x_dtype, int64_t ld_x, int swiglu, int64_t M, int64_t K,
                         const uint8_t *w_s4, int64_t ld_s4, const float *w_scale, int64_t N, const float *bias,
                         void *out, cr_dtype out_dtype, int64_t ldc, void *workspace, size_t ws_bytes,
                         uint32_t flags, hipStream_t stream);

/*
 * W4A4 variant: 4-bit weights and 4-bit activations (ComfyUI Turing Utils README, opening
 * paragraph and section "Nodes", bullet "Load ConvRot DiT": W4A4 dispatch; the packed
 * layout is named there, not described).  This library reads it as the W4A8 reading on
 * both operands: the activation row (SwiGLU first when swiglu != 0) goes through ConvRot256
 * and the 4-bit per-row rule above (a = max |y|, scale a / 7, codes -7..7) and is packed in
 * the format above; the weight is the one cr_quant_weight_w4 prepares; int32 sums of the
 * 4-bit products; the same epilogue.
 *
 * Activation preparation: X [M, ld_x] (ld_x >= K; swiglu: H [M, ld_x], ld_x >= 2K, gate
 * H[:, :K], value H[:, K:2K]) of x_dtype (CR_BF16, CR_FP16, CR_FP32), rows of 16-byte
 * multiples, 16-byte aligned -> x_s4 [M, ld_s4] bytes (ld_s4 >= K_pad / 2, a multiple of
 * 16) and x_scale [M] float.  flags as for cr_quant_weight_w4.
 */
cr_status cr_quant_act_w4(const void *x, cr_dtype x_dtype, int64_t ld_x, int swiglu, int64_t M, int64_t K,
                          uint8_t *x_s4, int64_t ld_s4, float *x_scale, uint32_t flags, hipStream_t stream);

/*
 * W4A4 GEMM: out = ((float)sum_k p[m, k] q[n, k] * a_scale[m]) * b_scale[n] (+ bias[n]), p and
 * q the codes of the packed rows a_s4 [M, lda bytes] and b_s4 [N, ldb bytes] (lda, ldb >=
 * K_pad / 2, multiples of 16).  The other arguments, the limits and CR_I32 as in
 * cr_gemm_s8_rowscale_bias; both operands must use the same column order.
 */
cr_status cr_gemm_s4s4_rowscale(const uint8_t *a_s4, int64_t lda, const float *a_scale,
                                const uint8_t *b_s4, int64_t ldb, const float *b_scale, const float *bias,
                                int64_t M, int64_t N, int64_t K_pad, void *c, cr_dtype c_dtype, int64_t ldc,
                                hipStream_t stream);

/*
 * The W4A4 layer: cr_quant_act_w4 into the workspace, then cr_gemm_s4s4_rowscale against the
 * prepared weight, both on `stream`.  Arguments, flags and errors as for cr_linear_w4a8;
 * workspace: cr_linear_w4a4_workspace_bytes(M, K) bytes, 256-byte aligned (the packed
 * activation and its scales); an empty layer (M or N = 0) needs none.
 */
size_t cr_linear_w4a4_workspace_bytes(int64_t M, int64_t K);
cr_status cr_linear_w4a4(const void *x, cr_dtype x_dtype, int64_t ld_x, int swiglu, int64_t M, int64_t K,
                         const uint8_t *w_s4, int64_t ld_s4, const float *w_scale, int64_t N, const float *bias,
                         void *out, cr_dtype out_dtype, int64_t ldc, void *workspace, size_t ws_bytes,
                         uint32_t flags, hipStream_t stream);

/*
 * W4A4 on the 6-bit matrix cores.  The same 4-bit codes in a second storage form (this
 * library's; the pages describe none): each code -7..7 stored as the E2M3 number of equal
 * value (1 sign, 2 exponent bits with bias 1, 3 mantissa bits), so that gfx950's 6-bit
 * floating-point matrix instructions multiply the codes exactly; the sums are those of the
 * nibble form, bit for bit.  A row's 128-code unit takes 96 bytes: each quarter of 32 codes
 * is a 192-bit field with code e in bits 6e .. 6e+5 (little-endian); a unit holds the first
 * 16 bytes of the fields of quarters Q0, Q2, Q1, Q3, then their last 8 bytes in the same
 * order.  Rows are stored in quads: rows 4q .. 4q+3 occupy the ld_f6 bytes from q * ld_f6
 * (ld_f6 >= 3 K_pad, a multiple of 16; a multiple of 128 keeps every step of the GEMM on
 * whole cache lines), and unit u of row 4q + i starts at byte u * 384 + i * 96 of its quad.
 * A buffer of `rows` rows holds ceil(rows / 4) quads; the bytes of rows past `rows` in the
 * last quad are neither written nor read.  Column order as for the nibble form (flags).
 *
 * cr_quant_weight_w4_e2m3 and cr_quant_act_w4_e2m3 are cr_quant_weight_w4 and
 * cr_quant_act_w4 with that output form: w_f6 / x_f6 [ceil(rows / 4), ld_f6] bytes.
 * cr_gemm_e2m3_rowscale is cr_gemm_s4s4_rowscale on two such operands (lda, ldb: bytes per
 * quad, >= 3 K_pad, multiples of 16).  cr_linear_w4a4_e2m3 is cr_linear_w4a4 with the weight
 * in that form and cr_linear_w4a4_e2m3_workspace_bytes(M, K) bytes of workspace.
 */
cr_status cr_quant_weight_w4_e2m3(const void *w, cr_dtype w_dtype, int64_t ld_w, int64_t N, int64_t K,
                                  uint8_t *w_f6, int64_t ld_f6, float *w_scale, uint32_t flags, hipStream_t stream);
/*
 * The same weight codes moved from the nibble form (w_s4 [N, ld_s4 bytes], as written by
 * cr_quant_weight_w4; ld_s4 >= K_pad / 2, a multiple of 16) to the E2M3 form (w_f6
 * [ceil(N / 4), ld_f6 bytes], ld_f6 >= 3 K_pad, a multiple of 16), for a 4-bit weight kept in
 * the compact form; the row scales stay as they are.  The codes must be -7..7 (nibble 8 is
 * not a code of the form and gives an unspecified field).  The codes are copied, so the result
 * equals cr_quant_weight_w4_e2m3 of the same dense weight bit for bit.  K_pad a multiple of
 * 256, at most CR_MAX_K_PAD.
 */
cr_status cr_repack_w4_e2m3(const uint8_t *w_s4, int64_t ld_s4, int64_t N, int64_t K_pad, uint8_t *w_f6,
                            int64_t ld_f6, hipStream_t stream);
cr_status cr_quant_act_w4_e2m3(const void *x, cr_dtype x_dtype, int64_t ld_x, int swiglu, int64_t M, int64_t K,
                               uint8_t *x_f6, int64_t ld_f6, float *x_scale, uint32_t flags, hipStream_t stream);
cr_status cr_gemm_e2m3_rowscale(const uint8_t *a_f6, int64_t lda, const float *a_scale,
                                const uint8_t *b_f6, int64_t ldb, const float *b_scale, const float *bias,
                                int64_t M, int64_t N, int64_t K_pad, void *c, cr_dtype c_dtype, int64_t ldc,
                                hipStream_t stream);
size_t cr_linear_w4a4_e2m3_workspace_bytes(int64_t M, int64_t K);
cr_status cr_linear_w4a4_e2m3(const void *x, cr_dtype x_dtype, int64_t ld_x, int swiglu, int64_t M, int64_t K,
                              const uint8_t *w_f6, int64_t ld_f6, const float *w_scale, int64_t N,
                              const float *bias, void *out, cr_dtype out_dtype, int64_t ldc, void *workspace,
                              size_t ws_bytes, uint32_t flags, hipStream_t stream);

/*
 * The layer for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): cr_linear_nvfp4_ex with serial
 * staging on `stream` and, as its workspace, a device array of CR_NOALLOC_SCRATCH_BYTES
 * inside the library (one per GPU, created when the library's code is loaded on that GPU
 * and kept until the process ends).  Nothing is allocated: no hipMalloc, no hipFree, no
 * event creation.  The results are those of cr_linear_nvfp4_ex, bit for bit.
 *   x ... ldc        as in cr_linear_nvfp4_ex (the caller still owns inputs and outputs).
 *   max_tile_bytes   bound of one S8 weight tile; 0 selects the largest bound for which
 *                    the S8 activation, its scales and two weight tiles fit the array.
 *   stream           every launch goes to this stream.
 * Returns CR_ERR_TOO_LARGE, with nothing enqueued, when the layer's workspace (see
 * cr_linear_nvfp4_workspace_bytes) would exceed CR_NOALLOC_SCRATCH_BYTES: the S8 activation
 * alone takes M * K_pad bytes, so M * K_pad must stay well below 64 MiB (for example
 * M <= 11000 at K = 5376).  All calls on one GPU share its array, and nothing in it needs
 * to start at zero: calls that overlap in time on one GPU (two streams, or two host
 * threads) race on it and must be ordered by the caller.
 */
#define CR_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
cr_status cr_linear_nvfp4_noalloc(const void *x, cr_dtype x_dtype, int64_t ld_x, int swiglu,
                                  int64_t M, int64_t K, const float *pre_scale,
                                  const uint8_t *w_fp4, int64_t ld_fp4,
                                  const uint8_t *w_sf, int64_t ld_sf, const float *global_scale,
                                  int64_t N, const float *bias, void *out, cr_dtype out_dtype, int64_t ldc,
                                  size_t max_tile_bytes, uint32_t flags, hipStream_t stream);

/*
 * Row maxima of the rotated weight, without the codes: w_amax[n] = a = max_k |y[n, k]|,
 * y the NVFP4 decode of row n followed by ConvRot256 (the a of the row quantization; the
 * weight scale is a / 127).  It is what cr_gemm_nvfp4_fused needs before it can quantize a
 * weight block on the fly (ComfyUI Turing Utils README, "Load ConvRot DiT ..." bullet: the
 * row scale covers the whole padded row).  For a fixed weight it can be computed once and
 * kept ([N] floats).
 *   w_fp4, ld_fp4, w_sf, ld_sf, global_scale, n_rows, K   as in cr_prep_weight_nvfp4.
 *   w_amax   [n_rows] float out, 4-byte aligned.
 *   flags    CR_FLAG_NONE or CR_FLAG_FORCE_TWO_PASS (CR_FLAG_BLOCK_TRANSPOSED is accepted
 *            and changes nothing).
 */
cr_status cr_weight_amax_nvfp4(const uint8_t *w_fp4, int64_t ld_fp4,
                               const uint8_t *w_sf, int64_t ld_sf,
                               const float *global_scale, int64_t n_rows, int64_t K,
                               float *w_amax, uint32_t flags, hipStream_t stream);

/*
 * Decode-inside-GEMM (the weight's S8 codes and scales are never stored): the result of
 * cr_gemm_s8_rowscale_bias on b_s8, b_scale = cr_prep_weight_nvfp4(W), bit for bit, computed
 * by decoding, rotating and quantizing each 256-column block of the NVFP4 weight inside the
 * GEMM (same bullet: the weight is decoded, rotated and quantized per call).  Every
 * workgroup repeats the decode for its 32 weight rows once per 128 activation rows, so this
 * is the path for short batches (M up to a few hundred); for long ones, prepare the weight
 * once and use cr_gemm_s8_rowscale.
 *   a_s8 [M, lda], a_scale [M]   the prepared activation (cr_quant_act and variants), in
 *                natural column order, or block-transposed with CR_FLAG_BLOCK_TRANSPOSED.
 *   w_fp4, ld_fp4, w_sf, ld_sf, global_scale, K   the NVFP4 weight [N, K] as above.
 *   w_amax       [N] float from cr_weight_amax_nvfp4 on the same weight, or NULL: then the
 *                kernel finds the row maxima itself in a first pass over the weight (decode
 *                and rotation only; every workgroup for its own 32 rows).
 *   bias         [N] float or NULL, as in cr_gemm_s8_rowscale_bias.
 *   c [M, ldc] of c_dtype (CR_I32: the raw accumulator, a_scale may be NULL, no bias).
 *   flags        CR_FLAG_NONE or CR_FLAG_BLOCK_TRANSPOSED (the order of a_s8);
 *                CR_FLAG_FORCE_TWO_PASS is accepted and changes nothing.
 * M is at most 8388480 (65535 workgroup rows of 128).
 */
cr_status cr_gemm_nvfp4_fused(const int8_t *a_s8, int64_t lda, const float *a_scale,
                              const uint8_t *w_fp4, int64_t ld_fp4,
                              const uint8_t *w_sf, int64_t ld_sf, const float *global_scale,
                              const float *w_amax, const float *bias, int64_t M, int64_t N, int64_t K,
                              void *c, cr_dtype c_dtype, int64_t ldc, uint32_t flags, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CONVROT_H */
