/*
 * Plain CPU oracle for the rotated W8A8 linear layer over NVFP4 weights.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load this
 * file: only the test suite, the smoke check and the benchmark's CPU-baseline leg do.
 * It shares no code, header, table or constant with the GPU library.
 *
 * It is written to be read against the pages, step by step, with no blocking or fusion:
 *   - "ComfyUI Turing Utils" README (comfy.icu page for comfyui-svdint4), section
 *     "Nodes", bullet "Load ConvRot DiT and Load ConvRot CLIP": the NVFP4 runtime path
 *     applies one 256-wide block rotation (paired ConvRot256) to activations and to
 *     decoded NVFP4 weights, quantizes rows to S8 with an FP32 scale, runs a row-scaled
 *     INT8 GEMM; logical K is zero-padded to a multiple of 256 before rotation and the
 *     serialized padding is ignored; N tails and FP16/BF16/FP32 outputs are supported;
 *     K above 16384 uses a two-pass form of the same algorithm; SwiGLU runs before the
 *     rotation.
 *   - modelpad.app explainer of the MiniMax H3 DiT, "Foundations" (a linear layer is
 *     y = x W^T with W stored [out, in]), the MLP paragraph (fc1's output is split into
 *     two halves; swish of the first half gates the second half by an elementwise
 *     product) and the "convrot" paragraph before the glossary (activations are
 *     multiplied by a Hadamard matrix before quantization; being orthogonal, its inverse
 *     is absorbed by the weights).
 *
 * Floating point: IEEE binary32, round to nearest even, subnormals kept.  Build with
 * -ffp-contract=off and without -ffast-math so every expression below is evaluated
 * exactly as written (one rounding per operation).
 *
 * Readings taken where the pages are silent (each is listed in the design notes):
 *   rotation matrix  R = H/16 with H[i][j] = (-1)^popcount(i&j) (Sylvester, natural
 *                    order), evaluated as the iterative transform with stages
 *                    h = 1, 2, ..., 128 and butterflies (u+v, u-v), then *0.0625;
 *   quantizer        a = max|y|; s = a/127; r = 127/a, itself rounded to FP32 and reused
 *                    for the whole row; q = clamp(rint(y*r), -127, 127); a zero row
 *                    gives s = 0 and q = 0; a row whose 127/a overflows (a < ~3.7e-37)
 *                    is quantized as its exact copy scaled by 2^64;
 *   NVFP4 layout     element k of row n is the nibble of byte n*ld + k/2 (low nibble for
 *                    even k); block scale of k is the E4M3 byte n*ld_sf + k/16; decoded
 *                    value = fp32(E2M1 * E4M3) * g (the first product is exact);
 *   swish            swish(a) = a * sigma(a), sigma(a) = 1/(1 + E(-a)) with E the
 *                    reproducible exponential below; the gate is the first half;
 *                    the SwiGLU product stays fp32;
 *   epilogue         out = ((float)acc * s_x[m]) * s_w[n], rounded once to the output type.
 * Parity against the pages' own implementation is unpinned: they print no vectors.
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <stdlib.h>
#include <math.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the row loops below run on (OpenMP over independent rows only). */
int or_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

#define OR_DT_BF16 0
#define OR_DT_FP16 1
#define OR_DT_FP32 2
#define OR_DT_I32 3

/* ---------------------------------------------------------------- padding ---- */

/* Logical K is zero-padded up to a multiple of the 256-wide rotation block. */
int64_t or_padded_k(int64_t k) { return ((k + 255) / 256) * 256; }

/* ------------------------------------------------------ number formats ---- */

static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* E2M1 (4-bit float: 1 sign, 2 exponent bits with bias 1, 1 mantissa bit, no inf/NaN).
 * Exponent field 0 is subnormal: value = m * 0.5.  Otherwise (1 + m/2) * 2^(e-1). */
float or_e2m1(uint8_t code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    float mag = (e == 0) ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, e - 1);
    return s ? -mag : mag;
}

/* E4M3 (the "fn" variant: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no inf;
 * S.1111.111 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448). */
float or_e4m3(uint8_t b)
{
    int s = (b >> 7) & 1, e = (b >> 3) & 15, m = b & 7;
    float mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexpf((float)m / 8.0f, -6);
    else mag = ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return s ? -mag : mag;
}

/* E2M3 (6-bit float: 1 sign, 2 exponent bits with bias 1, 3 mantissa bits, no inf/NaN).
 * Exponent field 0 is subnormal: value = m / 8.  Otherwise (1 + m/8) * 2^(e-1); the
 * integers 0..7 are all exact (largest magnitude 7.5). */
float or_e2m3(uint8_t code)
{
    int s = (code >> 5) & 1, e = (code >> 3) & 3, m = code & 7;
    float mag = (e == 0) ? (float)m / 8.0f : ldexpf(1.0f + (float)m / 8.0f, e - 1);
    return s ? -mag : mag;
}

/* bfloat16 is the top half of a binary32: widening is exact. */
float or_bf16_to_f32(uint16_t h) { return bits_to_f32((uint32_t)h << 16); }

/* binary16: 1 sign, 5 exponent bits (bias 15), 10 mantissa bits.  Widening is exact. */
float or_fp16_to_f32(uint16_t h)
{
    int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    float mag;
    if (e == 0) mag = ldexpf((float)m, -24);
    else if (e == 31) mag = m ? NAN : INFINITY;
    else mag = ldexpf((float)(1024 + m), e - 25);
    return s ? -mag : mag;
}

/* binary32 -> bfloat16, round to nearest even (NaN stays a quiet NaN). */
uint16_t or_f32_to_bf16(float f)
{
    uint32_t u = f32_to_bits(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
    uint32_t lsb = (u >> 16) & 1;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

/* binary32 -> binary16, round to nearest even, overflow to inf, subnormals kept. */
uint16_t or_f32_to_fp16(float f)
{
    uint32_t u = f32_to_bits(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000);
    uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return sign | 0x7e00;             /* NaN */
    if (a >= 0x477ff000u) return sign | 0x7c00;            /* >= 65520 rounds to inf */
    if (a < 0x38800000u) {                                 /* below 2^-14: subnormal */
        /* value = a_f * 2^24 units of 2^-24, round to nearest even integer */
        float mag = bits_to_f32(a);
        float scaled = ldexpf(mag, 24);                    /* exact: power-of-two scaling */
        float r = rintf(scaled);                           /* half to even */
        return sign | (uint16_t)r;
    }
    /* normal: keep 10 mantissa bits, round the 13 dropped bits to nearest even */
    uint32_t e = (a >> 23) - 127 + 15;
    uint32_t m = a & 0x7fffffu;
    uint32_t h = (e << 10) | (m >> 13);
    uint32_t rest = m & 0x1fffu;
    if (rest > 0x1000u || (rest == 0x1000u && (h & 1))) h += 1;  /* carries into exponent */
    return sign | (uint16_t)h;
}

/* ------------------------------------------------ reproducible exponential ---- */

/* E(x) ~ exp(x) from basic IEEE binary32 operations only, so that two independent
 * implementations agree bit for bit.  Method: Cody & Waite (1980) argument reduction
 * x = k*ln2 + r with k = rint(x*log2 e) and ln2 split as L1 + L2 (L1 carries 15
 * significant bits so k*L1 is exact for |k| < 512), then the degree-7 Taylor polynomial
 * of exp(r) in Horner form with fused multiply-adds, then scaling by 2^k.
 * Constants: LOG2E = RN(log2 e); L1 = ln2 truncated to 15 significant bits;
 * L2 = RN(ln2 - L1); C_n = RN(1/n!).  For |r| <= ln2/2 the truncation error of the
 * polynomial is below 1e-8 relative. */
static const float OR_LOG2E = 0x1.715476p+0f;
static const float OR_L1 = 0x1.62e4p-1f;
static const float OR_L2 = 0x1.7f7d1cp-20f;
static const float OR_C2 = 0x1.0p-1f;
static const float OR_C3 = 0x1.555556p-3f;
static const float OR_C4 = 0x1.555556p-5f;
static const float OR_C5 = 0x1.111112p-7f;
static const float OR_C6 = 0x1.6c16c2p-10f;
static const float OR_C7 = 0x1.a01a02p-13f;

float or_exp(float x)
{
    if (x != x) return x;                 /* NaN in, NaN out */
    if (x > 89.0f) return INFINITY;       /* exp(89) > FLT_MAX */
    if (x < -104.0f) return 0.0f;         /* exp(-104) rounds to the smallest subnormal; below that, 0 */
    float kf = rintf(x * OR_LOG2E);
    float r = fmaf(-kf, OR_L1, x);
    r = fmaf(-kf, OR_L2, r);
    float p = OR_C7;
    p = fmaf(p, r, OR_C6);
    p = fmaf(p, r, OR_C5);
    p = fmaf(p, r, OR_C4);
    p = fmaf(p, r, OR_C3);
    p = fmaf(p, r, OR_C2);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    return ldexpf(p, (int)kf);
}

/* logistic sigma(a) = 1 / (1 + exp(-a)), one correctly rounded division */
float or_sigmoid(float a)
{
    float t = or_exp(-a);
    return 1.0f / (1.0f + t);
}

/* SwiGLU element: swish(gate) * value with swish(a) = a * sigma(a) (MLP paragraph). */
float or_swiglu(float gate, float value)
{
    float sig = or_sigmoid(gate);
    float sw = gate * sig;
    return sw * value;
}

/* ---------------------------------------------------------- NVFP4 decode ---- */

/* Decode rows [0, n_rows) of a packed NVFP4 matrix into fp32 rows of length K_pad.
 * codes: byte n*ld_codes + k/2 holds element k (low nibble for even k).
 * sf:    byte n*ld_sf + k/16 is the E4M3 scale of the 16-element block holding k.
 * Decoded value = fp32(E2M1 * E4M3) * g; k >= K (padding, serialized or not) gives 0. */
void or_nvfp4_decode(const uint8_t *codes, int64_t ld_codes, const uint8_t *sf, int64_t ld_sf,
                     float g, int64_t n_rows, int64_t K, float *w, int64_t ld_w)
{
    int64_t kp = or_padded_k(K);
#pragma omp parallel for
    for (int64_t n = 0; n < n_rows; n++) {
        for (int64_t k = 0; k < kp; k++) {
            float v = 0.0f;
            if (k < K) {
                uint8_t byte = codes[n * ld_codes + k / 2];
                uint8_t code = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
                float e2m1 = or_e2m1(code);
                float e4m3 = or_e4m3(sf[n * ld_sf + k / 16]);
                float prod = e2m1 * e4m3;     /* exact: at most 2 + 4 significant bits */
                v = prod * g;
            }
            w[n * ld_w + k] = v;
        }
    }
}

/* ------------------------------------------------------------- rotation ---- */

/* One 256-wide block: y <- y * (H/16), H Sylvester/natural order.  The iterative
 * transform visits stages h = 1, 2, 4, ..., 128; at stage h every index j whose bit h
 * is clear is paired with j + h and replaced by (u + v, u - v). */
void or_fwht256(float *y)
{
    for (int h = 1; h < 256; h *= 2) {
        for (int j = 0; j < 256; j++) {
            if (j & h) continue;
            float u = y[j], v = y[j + h];
            y[j] = u + v;
            y[j + h] = u - v;
        }
    }
    for (int i = 0; i < 256; i++) y[i] = y[i] * 0.0625f;
}

/* ConvRot256 on every 256-block of every row (rows of length K_pad, stride ld). */
void or_convrot256(float *y, int64_t n_rows, int64_t K_pad, int64_t ld)
{
#pragma omp parallel for
    for (int64_t n = 0; n < n_rows; n++)
        for (int64_t b = 0; b < K_pad; b += 256)
            or_fwht256(y + n * ld + b);
}

/* --------------------------------------------------------- quantization ---- */

/* Symmetric per-row INT8 quantization with an FP32 scale:
 * a = max_k |y_k| over all K_pad columns; a == 0 -> s = 0, every q = 0;
 * else s = a/127, r = 127/a (one FP32 reciprocal per row), q = clamp(rint(y*r), -127, 127).
 * For a below about 3.7e-37, 127/a overflows FP32 and y*r would be +-inf or NaN (0*inf);
 * wherever r is finite the codes do not change when the whole row is multiplied by a power
 * of two (every product involved scales exactly), so such a row is quantized as its copy
 * multiplied by 2^64, which is exact and brings r back into range.  s stays a/127 of the row
 * as given. */
void or_row_quant(const float *y, int64_t n_rows, int64_t K_pad, int64_t ld_y,
                  int8_t *q, int64_t ld_q, float *s)
{
#pragma omp parallel for
    for (int64_t n = 0; n < n_rows; n++) {
        const float *row = y + n * ld_y;
        float a = 0.0f;
        for (int64_t k = 0; k < K_pad; k++) {
            float m = fabsf(row[k]);
            if (m > a) a = m;
        }
        if (a == 0.0f) {
            s[n] = 0.0f;
            for (int64_t k = 0; k < K_pad; k++) q[n * ld_q + k] = 0;
            continue;
        }
        s[n] = a / 127.0f;
        const float up = isinf(127.0f / a) ? 0x1p64f : 1.0f;
        float r = 127.0f / (a * up);
        for (int64_t k = 0; k < K_pad; k++) {
            float t = rintf((row[k] * up) * r);
            if (t > 127.0f) t = 127.0f;
            if (t < -127.0f) t = -127.0f;
            q[n * ld_q + k] = (int8_t)t;
        }
    }
}

/* -------------------------------------------------------- activations ---- */

static float load_elem(const void *x, int dtype, int64_t idx)
{
    if (dtype == OR_DT_BF16) return or_bf16_to_f32(((const uint16_t *)x)[idx]);
    if (dtype == OR_DT_FP16) return or_fp16_to_f32(((const uint16_t *)x)[idx]);
    return ((const float *)x)[idx];
}

/* X[M, K] (row stride ld_x elements) -> fp32 [M, K_pad] with zeros for k >= K. */
void or_act_load(const void *x, int dtype, int64_t ld_x, int64_t M, int64_t K,
                 float *out, int64_t ld_out)
{
    int64_t kp = or_padded_k(K);
#pragma omp parallel for
    for (int64_t m = 0; m < M; m++)
        for (int64_t k = 0; k < kp; k++)
            out[m * ld_out + k] = (k < K) ? load_elem(x, dtype, m * ld_x + k) : 0.0f;
}

/* H[M, 2F]: gate = H[:, :F], value = H[:, F:2F] -> fp32 swish(gate)*value [M, F_pad]. */
void or_act_load_swiglu(const void *h, int dtype, int64_t ld_h, int64_t M, int64_t F,
                        float *out, int64_t ld_out)
{
    int64_t kp = or_padded_k(F);
#pragma omp parallel for
    for (int64_t m = 0; m < M; m++)
        for (int64_t k = 0; k < kp; k++) {
            float v = 0.0f;
            if (k < F) {
                float gate = load_elem(h, dtype, m * ld_h + k);
                float value = load_elem(h, dtype, m * ld_h + F + k);
                v = or_swiglu(gate, value);
            }
            out[m * ld_out + k] = v;
        }
}

/* Channel pre-scale of the layer input (ComfyUI Turing Utils README, "Load ConvRot DiT
 * ..." bullet: pre-scales and SwiGLU run before the rotation, and channel pre-scales keep
 * the unfused order): buf[m, k] = buf[m, k] * c[k] for k < K, one FP32 rounding, applied
 * to the loaded (or SwiGLU) value.  Padding columns stay 0. */
void or_act_prescale(float *buf, int64_t M, int64_t K, int64_t ld, const float *c)
{
#pragma omp parallel for
    for (int64_t m = 0; m < M; m++)
        for (int64_t k = 0; k < K; k++)
            buf[m * ld + k] = buf[m * ld + k] * c[k];
}

/* Activation preparation: load (+SwiGLU), optional channel pre-scale (pre_scale [K] or
 * NULL), ConvRot256, row quantization.  x_s8 [M, K_pad] with stride ld_s8, x_scale [M].
 * Returns 0, or -1 on allocation failure. */
int or_quant_act_ex(const void *x, int dtype, int64_t ld_x, int swiglu, int64_t M, int64_t K,
                    const float *pre_scale, int8_t *x_s8, int64_t ld_s8, float *x_scale)
{
    int64_t kp = or_padded_k(K);
    float *buf = (float *)malloc(sizeof(float) * (size_t)(M > 0 ? M : 1) * (size_t)kp);
    if (!buf) return -1;
    if (swiglu) or_act_load_swiglu(x, dtype, ld_x, M, K, buf, kp);
    else or_act_load(x, dtype, ld_x, M, K, buf, kp);
    if (pre_scale) or_act_prescale(buf, M, K, kp, pre_scale);
    or_convrot256(buf, M, kp, kp);
    or_row_quant(buf, M, kp, kp, x_s8, ld_s8, x_scale);
    free(buf);
    return 0;
}

int or_quant_act(const void *x, int dtype, int64_t ld_x, int swiglu, int64_t M, int64_t K,
                 int8_t *x_s8, int64_t ld_s8, float *x_scale)
{
    return or_quant_act_ex(x, dtype, ld_x, swiglu, M, K, NULL, x_s8, ld_s8, x_scale);
}

/* Weight preparation: NVFP4 decode, ConvRot256, row quantization. */
int or_prep_weight_nvfp4(const uint8_t *codes, int64_t ld_codes, const uint8_t *sf, int64_t ld_sf,
                         float g, int64_t n_rows, int64_t K, int8_t *w_s8, int64_t ld_s8,
                         float *w_scale)
{
    int64_t kp = or_padded_k(K);
    float *buf = (float *)malloc(sizeof(float) * (size_t)(n_rows > 0 ? n_rows : 1) * (size_t)kp);
    if (!buf) return -1;
    or_nvfp4_decode(codes, ld_codes, sf, ld_sf, g, n_rows, K, buf, kp);
    or_convrot256(buf, n_rows, kp, kp);
    or_row_quant(buf, n_rows, kp, kp, w_s8, ld_s8, w_scale);
    free(buf);
    return 0;
}

/* Row maxima of the rotated weight: a[n] = max_k |y[n, k]| over all K_pad columns, where y
 * is the NVFP4 decode followed by ConvRot256 (the quantity the row quantizer above starts
 * from; s = a/127 and r = 127/a follow from it).  A GEMM that quantizes weight blocks on
 * the fly needs a before it sees the whole row (ComfyUI Turing Utils README, "Load ConvRot
 * DiT ..." bullet: the row scale covers the whole padded row, which is why long rows take
 * two passes). */
int or_weight_amax_nvfp4(const uint8_t *codes, int64_t ld_codes, const uint8_t *sf, int64_t ld_sf,
                         float g, int64_t n_rows, int64_t K, float *amax)
{
    int64_t kp = or_padded_k(K);
    float *buf = (float *)malloc(sizeof(float) * (size_t)(n_rows > 0 ? n_rows : 1) * (size_t)kp);
    if (!buf) return -1;
    or_nvfp4_decode(codes, ld_codes, sf, ld_sf, g, n_rows, K, buf, kp);
    or_convrot256(buf, n_rows, kp, kp);
#pragma omp parallel for
    for (int64_t n = 0; n < n_rows; n++) {
        float a = 0.0f;
        for (int64_t k = 0; k < kp; k++) {
            float m = fabsf(buf[n * kp + k]);
            if (m > a) a = m;
        }
        amax[n] = a;
    }
    free(buf);
    return 0;
}

/* ----------------------------------------------------------------- GEMM ---- */

/* acc[m, n] = sum_k A[m, k] * B[n, k] (both operands K-contiguous, y = x W^T). */
void or_gemm_s8(const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb,
                int64_t M, int64_t N, int64_t K_pad, int32_t *acc, int64_t ldc)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; m++) {
        for (int64_t n = 0; n < N; n++) {
            int32_t sum = 0;
            for (int64_t k = 0; k < K_pad; k++)
                sum += (int32_t)A[m * lda + k] * (int32_t)B[n * ldb + k];
            acc[m * ldc + n] = sum;
        }
    }
}

/* ------------------------------------------------------------- epilogue ---- */

/* out[m, n] = ((float)acc[m, n] * s_x[m]) * s_w[n] (+ bias[n] when bias is not NULL:
 * the linear layer's y = x W^T + b, MiniMax H3 explainer, "Foundations"; the bias is added
 * in the epilogue, glossary entry "Epilogue"), each operation rounded in FP32, then one
 * rounding to out_dtype.  OR_DT_I32 copies acc (no bias).  Only columns n < N are written. */
void or_epilogue_ex(const int32_t *acc, int64_t ld_acc, const float *s_x, const float *s_w,
                    const float *bias, int64_t M, int64_t N, int out_dtype, void *out, int64_t ldc)
{
#pragma omp parallel for
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            int32_t a = acc[m * ld_acc + n];
            if (out_dtype == OR_DT_I32) { ((int32_t *)out)[m * ldc + n] = a; continue; }
            float v = ((float)a * s_x[m]) * s_w[n];
            if (bias) v = v + bias[n];
            if (out_dtype == OR_DT_BF16) ((uint16_t *)out)[m * ldc + n] = or_f32_to_bf16(v);
            else if (out_dtype == OR_DT_FP16) ((uint16_t *)out)[m * ldc + n] = or_f32_to_fp16(v);
            else ((float *)out)[m * ldc + n] = v;
        }
}

void or_epilogue(const int32_t *acc, int64_t ld_acc, const float *s_x, const float *s_w,
                 int64_t M, int64_t N, int out_dtype, void *out, int64_t ldc)
{
    or_epilogue_ex(acc, ld_acc, s_x, s_w, NULL, M, N, out_dtype, out, ldc);
}

/* -------------------------------------------------------------- layer ---- */

/* The whole layer: activation preparation once, weight preparation, GEMM, epilogue.
 * (The pages' chunking over N and two-stream staging change no value, so the oracle
 * prepares the whole weight at once.)  Returns 0, or -1 on allocation failure. */
int or_linear_nvfp4_ex(const void *x, int x_dtype, int64_t ld_x, int swiglu, int64_t M, int64_t K,
                       const float *pre_scale,
                       const uint8_t *codes, int64_t ld_codes, const uint8_t *sf, int64_t ld_sf,
                       float g, int64_t N, const float *bias, void *out, int out_dtype, int64_t ldc)
{
    int64_t kp = or_padded_k(K);
    int8_t *xq = (int8_t *)malloc((size_t)(M > 0 ? M : 1) * (size_t)kp);
    float *xs = (float *)malloc(sizeof(float) * (size_t)(M > 0 ? M : 1));
    int8_t *wq = (int8_t *)malloc((size_t)(N > 0 ? N : 1) * (size_t)kp);
    float *ws = (float *)malloc(sizeof(float) * (size_t)(N > 0 ? N : 1));
    int32_t *acc = (int32_t *)malloc(sizeof(int32_t) * (size_t)(M > 0 ? M : 1) * (size_t)(N > 0 ? N : 1));
    int rc = -1;
    if (xq && xs && wq && ws && acc &&
        or_quant_act_ex(x, x_dtype, ld_x, swiglu, M, K, pre_scale, xq, kp, xs) == 0 &&
        or_prep_weight_nvfp4(codes, ld_codes, sf, ld_sf, g, N, K, wq, kp, ws) == 0) {
        or_gemm_s8(xq, kp, wq, kp, M, N, kp, acc, N);
        or_epilogue_ex(acc, N, xs, ws, bias, M, N, out_dtype, out, ldc);
        rc = 0;
    }
    free(xq); free(xs); free(wq); free(ws); free(acc);
    return rc;
}

int or_linear_nvfp4(const void *x, int x_dtype, int64_t ld_x, int swiglu, int64_t M, int64_t K,
                    const uint8_t *codes, int64_t ld_codes, const uint8_t *sf, int64_t ld_sf,
                    float g, int64_t N, void *out, int out_dtype, int64_t ldc)
{
    return or_linear_nvfp4_ex(x, x_dtype, ld_x, swiglu, M, K, NULL, codes, ld_codes, sf, ld_sf,
                              g, N, NULL, out, out_dtype, ldc);
}

/* ------------------------------------------------ W4A8 variant (4-bit weights) ---- */

/* ComfyUI Turing Utils README: the ConvRot path supports W8A8, W4A8 and W4A4 dispatch and
 * ships a packed W4A8 kernel (opening paragraph; section "Nodes", bullet "Load ConvRot
 * DiT"; section "Turing behavior").  The pages name these formats but do not describe
 * them.  Reading taken: the W8A8 method with 4-bit weights.  The weight is rotated by the
 * same ConvRot256 and each row is quantized symmetrically to the 15 levels -7..7 with one
 * FP32 scale (a = max|y|, s = a/7, r = 7/a rounded to FP32, q = clamp(rint(y*r), -7, 7));
 * activations are prepared exactly as for W8A8; the GEMM accumulates int8 x int4 products
 * in int32; the epilogue is the W8A8 one. */

/* 4-bit row quantization: the rule of or_row_quant with 7 levels.  A row whose 7/a
 * overflows FP32 (a below about 2e-38) is quantized as its copy multiplied by 2^64, as
 * for the 8-bit codes. */
void or_row_quant_s4(const float *y, int64_t n_rows, int64_t K_pad, int64_t ld_y,
                     int8_t *q, int64_t ld_q, float *s)
{
#pragma omp parallel for
    for (int64_t n = 0; n < n_rows; n++) {
        const float *row = y + n * ld_y;
        float a = 0.0f;
        for (int64_t k = 0; k < K_pad; k++) {
            float m = fabsf(row[k]);
            if (m > a) a = m;
        }
        if (a == 0.0f) {
            s[n] = 0.0f;
            for (int64_t k = 0; k < K_pad; k++) q[n * ld_q + k] = 0;
            continue;
        }
        s[n] = a / 7.0f;
        const float up = isinf(7.0f / a) ? 0x1p64f : 1.0f;
        float r = 7.0f / (a * up);
        for (int64_t k = 0; k < K_pad; k++) {
            float t = rintf((row[k] * up) * r);
            if (t > 7.0f) t = 7.0f;
            if (t < -7.0f) t = -7.0f;
            q[n * ld_q + k] = (int8_t)t;
        }
    }
}

/* The packed int4 format (this library's own; the pages print none): two's complement
 * nibbles, 32 bytes per unit of 64 consecutive codes of a row.  The unit's four groups of
 * 16 codes, G0 (codes 0..15), G1, G2, G3, are stored in the order G0, G2, G1, G3, 8 bytes
 * each.  A group of codes c[0..15] takes 8 bytes: byte j (j = 0..3) holds c[j] in its low
 * nibble and c[4 + j] in its high nibble; byte 4 + j holds c[8 + j] and c[12 + j].  Row n
 * starts at byte n * ld_p; a row of K_pad codes (a multiple of 64) takes K_pad / 2 bytes. */
static int64_t s4_group_offset(int64_t g)     /* byte offset of group g (16 codes) in a row */
{
    static const int slot[4] = {0, 2, 1, 3};
    return 32 * (g / 4) + 8 * slot[g % 4];
}

void or_pack_s4(const int8_t *q, int64_t n_rows, int64_t K_pad, int64_t ld_q, uint8_t *p, int64_t ld_p)
{
    for (int64_t n = 0; n < n_rows; n++)
        for (int64_t g = 0; g < K_pad / 16; g++) {
            const int8_t *c = q + n * ld_q + 16 * g;
            uint8_t *b = p + n * ld_p + s4_group_offset(g);
            for (int j = 0; j < 4; j++) {
                b[j] = (uint8_t)((c[j] & 15) | ((c[4 + j] & 15) << 4));
                b[4 + j] = (uint8_t)((c[8 + j] & 15) | ((c[12 + j] & 15) << 4));
            }
        }
}

static int8_t nibble_value(uint8_t u) { return (int8_t)(u < 8 ? u : (int)u - 16); }

/* The inverse of or_pack_s4: codes -8..7 from the nibbles. */
void or_unpack_s4(const uint8_t *p, int64_t n_rows, int64_t K_pad, int64_t ld_p, int8_t *q, int64_t ld_q)
{
    for (int64_t n = 0; n < n_rows; n++)
        for (int64_t g = 0; g < K_pad / 16; g++) {
            const uint8_t *b = p + n * ld_p + s4_group_offset(g);
            int8_t *c = q + n * ld_q + 16 * g;
            for (int j = 0; j < 4; j++) {
                c[j] = nibble_value(b[j] & 15);
                c[4 + j] = nibble_value(b[j] >> 4);
                c[8 + j] = nibble_value(b[4 + j] & 15);
                c[12 + j] = nibble_value(b[4 + j] >> 4);
            }
        }
}

/* W4A8 weight preparation from a dense weight W [N, K] (bf16/fp16/fp32, row stride ld_w):
 * zero padding to K_pad, ConvRot256, 4-bit row quantization, packing.  Out: w_s4
 * [N, ld_s4 bytes] (ld_s4 >= K_pad / 2), w_scale [N].  Returns 0, or -1 on allocation
 * failure. */
int or_quant_weight_w4(const void *w, int dtype, int64_t ld_w, int64_t N, int64_t K,
                       uint8_t *w_s4, int64_t ld_s4, float *w_scale)
{
    int64_t kp = or_padded_k(K);
    float *buf = (float *)malloc(sizeof(float) * (size_t)(N > 0 ? N : 1) * (size_t)kp);
    int8_t *q = (int8_t *)malloc((size_t)(N > 0 ? N : 1) * (size_t)kp);
    int rc = -1;
    if (buf && q) {
        or_act_load(w, dtype, ld_w, N, K, buf, kp);
        or_convrot256(buf, N, kp, kp);
        or_row_quant_s4(buf, N, kp, kp, q, kp, w_scale);
        or_pack_s4(q, N, kp, kp, w_s4, ld_s4);
        rc = 0;
    }
    free(buf);
    free(q);
    return rc;
}

/* acc[m, n] = sum_k A[m, k] * Wq[n, k], Wq the unpacked 4-bit codes of B [N, ldb bytes]. */
int or_gemm_s8s4(const int8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                 int64_t M, int64_t N, int64_t K_pad, int32_t *acc, int64_t ldc)
{
    int8_t *bq = (int8_t *)malloc((size_t)(N > 0 ? N : 1) * (size_t)K_pad);
    if (!bq) return -1;
    or_unpack_s4(B, N, K_pad, ldb, bq, K_pad);
    or_gemm_s8(A, lda, bq, K_pad, M, N, K_pad, acc, ldc);
    free(bq);
    return 0;
}

/* The W4A8 layer: activation preparation (as for W8A8, optional SwiGLU), the int8 x int4
 * GEMM against the prepared weight, the row-scale epilogue (+ optional bias [N]).
 * Returns 0, or -1 on allocation failure. */
int or_linear_w4a8(const void *x, int x_dtype, int64_t ld_x, int swiglu, int64_t M, int64_t K,
                   const uint8_t *w_s4, int64_t ld_s4, const float *w_scale, int64_t N,
                   const float *bias, void *out, int out_dtype, int64_t ldc)
{
    int64_t kp = or_padded_k(K);
    int8_t *xq = (int8_t *)malloc((size_t)(M > 0 ? M : 1) * (size_t)kp);
    float *xs = (float *)malloc(sizeof(float) * (size_t)(M > 0 ? M : 1));
    int32_t *acc = (int32_t *)malloc(sizeof(int32_t) * (size_t)(M > 0 ? M : 1) * (size_t)(N > 0 ? N : 1));
    int rc = -1;
    if (xq && xs && acc && or_quant_act_ex(x, x_dtype, ld_x, swiglu, M, K, NULL, xq, kp, xs) == 0 &&
        or_gemm_s8s4(xq, kp, w_s4, ld_s4, M, N, kp, acc, N) == 0) {
        or_epilogue_ex(acc, N, xs, w_scale, bias, M, N, out_dtype, out, ldc);
        rc = 0;
    }
    free(xq); free(xs); free(acc);
    return rc;
}

/* --------------------------------------- 4-bit codes in E2M3 fields (execution form) ---- */

/* This library's second storage form of 4-bit code rows (the pages describe none): every
 * code -7..7 is stored as the E2M3 number of the same value, so that matrix cores with
 * 6-bit floating-point inputs multiply the codes directly and exactly.  A row's 128-code
 * unit takes 96 bytes: its quarters of 32 codes Q0 (codes 0..31), Q1, Q2, Q3 each form a
 * 192-bit field, code e in bits 6e .. 6e+5; the unit holds the first 16 bytes of the fields
 * of Q0, Q2, Q1, Q3 (bits 0..127, little-endian), then their last 8 bytes in the same order.
 * Rows are stored in quads: rows 4q .. 4q+3 occupy the ld_p bytes from q * ld_p (ld_p >=
 * 3 K_pad / 4 * 4), and unit u of row 4q + i sits at u * 384 + i * 96 inside them, so the four
 * rows' units u are contiguous.  Bytes of rows past n_rows in the last quad are unused (the
 * packing here writes zeros).  The codes follow the column order of the flags, as in the
 * nibble form. */

/* the code whose E2M3 value is q (+0 for 0), found by search over the 64 codes */
static uint8_t e2m3_code_of(int q)
{
    for (int c = 0; c < 64; c++)
        if (or_e2m3((uint8_t)c) == (float)q && !(q == 0 && c != 0)) return (uint8_t)c;
    return 0xFF;
}

/* byte of bit `bit` (0..191) of quarter g's field of row n, from the start of the buffer */
static int64_t e2m3_field_byte(int64_t n, int64_t ld_p, int64_t g, int bit)
{
    static const int slot[4] = {0, 2, 1, 3};
    const int64_t unit = (n / 4) * ld_p + 384 * (g / 4) + 96 * (n % 4), k = slot[g % 4];
    const int byte = bit / 8;
    return byte < 16 ? unit + 16 * k + byte : unit + 64 + 8 * k + (byte - 16);
}

/* Codes q [n_rows, ld_q] (each -7..7) -> E2M3 fields p [ceil(n_rows / 4) quads of ld_p
 * bytes]; returns 0, or -1 if a code is out of range. */
int or_pack_e2m3(const int8_t *q, int64_t n_rows, int64_t K_pad, int64_t ld_q, uint8_t *p, int64_t ld_p)
{
    uint8_t table[15];
    for (int v = -7; v <= 7; v++) table[v + 7] = e2m3_code_of(v);
    memset(p, 0, (size_t)(((n_rows + 3) / 4) * ld_p));
    for (int64_t n = 0; n < n_rows; n++)
        for (int64_t g = 0; g < K_pad / 32; g++)
            for (int e = 0; e < 32; e++) {
                const int v = q[n * ld_q + 32 * g + e];
                if (v < -7 || v > 7) return -1;
                const uint32_t c = table[v + 7];
                for (int b = 0; b < 6; b++)
                    if ((c >> b) & 1) p[e2m3_field_byte(n, ld_p, g, 6 * e + b)] |= (uint8_t)(1u << ((6 * e + b) % 8));
            }
    return 0;
}

/* The inverse: every field decoded as E2M3; returns 0, or -1 if a value is not an integer
 * in -7..7. */
int or_unpack_e2m3(const uint8_t *p, int64_t n_rows, int64_t K_pad, int64_t ld_p, int8_t *q, int64_t ld_q)
{
    for (int64_t n = 0; n < n_rows; n++)
        for (int64_t g = 0; g < K_pad / 32; g++)
            for (int e = 0; e < 32; e++) {
                uint8_t c = 0;
                for (int b = 0; b < 6; b++)
                    if ((p[e2m3_field_byte(n, ld_p, g, 6 * e + b)] >> ((6 * e + b) % 8)) & 1) c |= (uint8_t)(1u << b);
                const float v = or_e2m3(c);
                if (v != floorf(v) || v < -7.0f || v > 7.0f) return -1;
                q[n * ld_q + 32 * g + e] = (int8_t)v;
            }
    return 0;
}

/* acc[m, n] = sum_k A[m, k] B[n, k] over the codes of two E2M3-field operands (quads of
 * lda and ldb bytes). */
int or_gemm_e2m3(const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb, int64_t M, int64_t N,
                 int64_t K_pad, int32_t *acc, int64_t ldc)
{
    int8_t *aq = (int8_t *)malloc((size_t)(M > 0 ? M : 1) * (size_t)K_pad);
    int8_t *bq = (int8_t *)malloc((size_t)(N > 0 ? N : 1) * (size_t)K_pad);
    int rc = -1;
    if (aq && bq && or_unpack_e2m3(A, M, K_pad, lda, aq, K_pad) == 0 &&
        or_unpack_e2m3(B, N, K_pad, ldb, bq, K_pad) == 0) {
        or_gemm_s8(aq, K_pad, bq, K_pad, M, N, K_pad, acc, ldc);
        rc = 0;
    }
    free(aq);
    free(bq);
    return rc;
}

/* ------------------------------------------------ W4A4 variant (4-bit both sides) ---- */

/* ComfyUI Turing Utils README: W4A4 is the third ConvRot format it dispatches (opening
 * paragraph; section "Nodes", bullet "Load ConvRot DiT"), again without a description.
 * Reading taken, as for W4A8: the W8A8 method with 4-bit rows on both sides; the
 * activation row (after SwiGLU when fused) is rotated and quantized by the 4-bit rule
 * above and packed like the weight; int32 accumulation of the 4-bit products; the W8A8
 * epilogue. */

/* Activation preparation to packed 4-bit rows: load (+SwiGLU), ConvRot256, 4-bit row
 * quantization, packing.  x_s4 [M, ld_s4 bytes] (ld_s4 >= K_pad / 2), x_scale [M].
 * Returns 0, or -1 on allocation failure. */
int or_quant_act_w4(const void *x, int dtype, int64_t ld_x, int swiglu, int64_t M, int64_t K,
                    uint8_t *x_s4, int64_t ld_s4, float *x_scale)
{
    int64_t kp = or_padded_k(K);
    float *buf = (float *)malloc(sizeof(float) * (size_t)(M > 0 ? M : 1) * (size_t)kp);
    int8_t *q = (int8_t *)malloc((size_t)(M > 0 ? M : 1) * (size_t)kp);
    int rc = -1;
    if (buf && q) {
        if (swiglu) or_act_load_swiglu(x, dtype, ld_x, M, K, buf, kp);
        else or_act_load(x, dtype, ld_x, M, K, buf, kp);
        or_convrot256(buf, M, kp, kp);
        or_row_quant_s4(buf, M, kp, kp, q, kp, x_scale);
        or_pack_s4(q, M, kp, kp, x_s4, ld_s4);
        rc = 0;
    }
    free(buf);
    free(q);
    return rc;
}

/* acc[m, n] = sum_k Aq[m, k] * Wq[n, k], both the unpacked 4-bit codes of packed rows. */
int or_gemm_s4s4(const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                 int64_t M, int64_t N, int64_t K_pad, int32_t *acc, int64_t ldc)
{
    int8_t *aq = (int8_t *)malloc((size_t)(M > 0 ? M : 1) * (size_t)K_pad);
    int rc = -1;
    if (aq) {
        or_unpack_s4(A, M, K_pad, lda, aq, K_pad);
        rc = or_gemm_s8s4(aq, K_pad, B, ldb, M, N, K_pad, acc, ldc);
    }
    free(aq);
    return rc;
}

/* The W4A4 layer: 4-bit activation preparation, the 4-bit x 4-bit GEMM against the
 * prepared weight, the row-scale epilogue (+ optional bias [N]).  Returns 0 or -1. */
int or_linear_w4a4(const void *x, int x_dtype, int64_t ld_x, int swiglu, int64_t M, int64_t K,
                   const uint8_t *w_s4, int64_t ld_s4, const float *w_scale, int64_t N,
                   const float *bias, void *out, int out_dtype, int64_t ldc)
{
    int64_t kp = or_padded_k(K);
    uint8_t *xq = (uint8_t *)malloc((size_t)(M > 0 ? M : 1) * (size_t)(kp / 2));
    float *xs = (float *)malloc(sizeof(float) * (size_t)(M > 0 ? M : 1));
    int32_t *acc = (int32_t *)malloc(sizeof(int32_t) * (size_t)(M > 0 ? M : 1) * (size_t)(N > 0 ? N : 1));
    int rc = -1;
    if (xq && xs && acc && or_quant_act_w4(x, x_dtype, ld_x, swiglu, M, K, xq, kp / 2, xs) == 0 &&
        or_gemm_s4s4(xq, kp / 2, w_s4, ld_s4, M, N, kp, acc, N) == 0) {
        or_epilogue_ex(acc, N, xs, w_scale, bias, M, N, out_dtype, out, ldc);
        rc = 0;
    }
    free(xq); free(xs); free(acc);
    return rc;
}

/* ----------------------------------------------- elementwise array helpers ---- */
/* Thin loops so the tests can sweep whole code spaces without one foreign call per value. */

void or_exp_array(const float *x, float *y, int64_t n)
{
    for (int64_t i = 0; i < n; i++) y[i] = or_exp(x[i]);
}

void or_sigmoid_array(const float *x, float *y, int64_t n)
{
    for (int64_t i = 0; i < n; i++) y[i] = or_sigmoid(x[i]);
}

void or_swiglu_array(const float *gate, const float *value, float *y, int64_t n)
{
    for (int64_t i = 0; i < n; i++) y[i] = or_swiglu(gate[i], value[i]);
}

void or_bf16_to_f32_array(const uint16_t *h, float *y, int64_t n)
{
    for (int64_t i = 0; i < n; i++) y[i] = or_bf16_to_f32(h[i]);
}

void or_fp16_to_f32_array(const uint16_t *h, float *y, int64_t n)
{
    for (int64_t i = 0; i < n; i++) y[i] = or_fp16_to_f32(h[i]);
}

void or_f32_to_bf16_array(const float *x, uint16_t *h, int64_t n)
{
    for (int64_t i = 0; i < n; i++) h[i] = or_f32_to_bf16(x[i]);
}

void or_f32_to_fp16_array(const float *x, uint16_t *h, int64_t n)
{
    for (int64_t i = 0; i < n; i++) h[i] = or_f32_to_fp16(x[i]);
}
