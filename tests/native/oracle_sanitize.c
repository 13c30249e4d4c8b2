/*
 * Sanitizer driver for the CPU oracle (oracle/oracle.c), built by the test suite with
 * gcc -fsanitize=address,undefined,float-cast-overflow,float-divide-by-zero and run on the
 * CPU.  Every oracle entry point is called on small inputs held in buffers of exactly the
 * size the call may touch (logical K not a multiple of 16 or 256, tight row strides, zero
 * rows, rows near the bottom of the binary32 range, every dtype), so an out-of-bounds
 * access, an uninitialised read path or undefined arithmetic aborts the run.  A few cheap
 * identities are checked on the way (exit status 1 names the first that fails); the value
 * pins themselves live in the Python tests.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* the oracle's exported functions (declared here: the oracle has no header) */
int64_t or_padded_k(int64_t k);
float or_e2m1(uint8_t code);
float or_e4m3(uint8_t b);
float or_exp(float x);
float or_sigmoid(float a);
float or_swiglu(float gate, float value);
void or_bf16_to_f32_array(const uint16_t *h, float *y, int64_t n);
void or_fp16_to_f32_array(const uint16_t *h, float *y, int64_t n);
void or_f32_to_bf16_array(const float *x, uint16_t *h, int64_t n);
void or_f32_to_fp16_array(const float *x, uint16_t *h, int64_t n);
void or_nvfp4_decode(const uint8_t *codes, int64_t ld_codes, const uint8_t *sf, int64_t ld_sf, float g,
                     int64_t n_rows, int64_t K, float *w, int64_t ld_w);
void or_fwht256(float *y);
void or_convrot256(float *y, int64_t n_rows, int64_t K_pad, int64_t ld);
void or_row_quant(const float *y, int64_t n_rows, int64_t K_pad, int64_t ld_y, int8_t *q, int64_t ld_q, float *s);
int or_quant_act_ex(const void *x, int dtype, int64_t ld_x, int swiglu, int64_t M, int64_t K,
                    const float *pre_scale, int8_t *x_s8, int64_t ld_s8, float *x_scale);
int or_prep_weight_nvfp4(const uint8_t *codes, int64_t ld_codes, const uint8_t *sf, int64_t ld_sf, float g,
                         int64_t n_rows, int64_t K, int8_t *w_s8, int64_t ld_s8, float *w_scale);
int or_weight_amax_nvfp4(const uint8_t *codes, int64_t ld_codes, const uint8_t *sf, int64_t ld_sf, float g,
                         int64_t n_rows, int64_t K, float *amax);
void or_gemm_s8(const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb, int64_t M, int64_t N,
                int64_t K_pad, int32_t *acc, int64_t ldc);
void or_epilogue_ex(const int32_t *acc, int64_t ld_acc, const float *s_x, const float *s_w, const float *bias,
                    int64_t M, int64_t N, int out_dtype, void *out, int64_t ldc);
int or_linear_nvfp4_ex(const void *x, int x_dtype, int64_t ld_x, int swiglu, int64_t M, int64_t K,
                       const float *pre_scale, const uint8_t *codes, int64_t ld_codes, const uint8_t *sf,
                       int64_t ld_sf, float g, int64_t N, const float *bias, void *out, int out_dtype, int64_t ldc);
void or_row_quant_s4(const float *y, int64_t n_rows, int64_t K_pad, int64_t ld_y, int8_t *q, int64_t ld_q, float *s);
void or_pack_s4(const int8_t *q, int64_t n_rows, int64_t K_pad, int64_t ld_q, uint8_t *p, int64_t ld_p);
void or_unpack_s4(const uint8_t *p, int64_t n_rows, int64_t K_pad, int64_t ld_p, int8_t *q, int64_t ld_q);
int or_quant_weight_w4(const void *w, int dtype, int64_t ld_w, int64_t N, int64_t K, uint8_t *w_s4, int64_t ld_s4,
                       float *w_scale);
int or_gemm_s8s4(const int8_t *A, int64_t lda, const uint8_t *B, int64_t ldb, int64_t M, int64_t N, int64_t K_pad,
                 int32_t *acc, int64_t ldc);
int or_linear_w4a8(const void *x, int x_dtype, int64_t ld_x, int swiglu, int64_t M, int64_t K, const uint8_t *w_s4,
                   int64_t ld_s4, const float *w_scale, int64_t N, const float *bias, void *out, int out_dtype,
                   int64_t ldc);
float or_e2m3(uint8_t code);
int or_pack_e2m3(const int8_t *q, int64_t n_rows, int64_t K_pad, int64_t ld_q, uint8_t *p, int64_t ld_p);
int or_unpack_e2m3(const uint8_t *p, int64_t n_rows, int64_t K_pad, int64_t ld_p, int8_t *q, int64_t ld_q);
int or_gemm_e2m3(const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb, int64_t M, int64_t N, int64_t K_pad,
                 int32_t *acc, int64_t ldc);
int or_quant_act_w4(const void *x, int dtype, int64_t ld_x, int swiglu, int64_t M, int64_t K, uint8_t *x_s4,
                    int64_t ld_s4, float *x_scale);
int or_gemm_s4s4(const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb, int64_t M, int64_t N, int64_t K_pad,
                 int32_t *acc, int64_t ldc);
int or_linear_w4a4(const void *x, int x_dtype, int64_t ld_x, int swiglu, int64_t M, int64_t K, const uint8_t *w_s4,
                   int64_t ld_s4, const float *w_scale, int64_t N, const float *bias, void *out, int out_dtype,
                   int64_t ldc);

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static uint32_t next_u32(void)
{
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (uint32_t)(rng >> 16);
}
static float next_normal(void)   /* sum of four uniforms, centred: enough spread for a driver */
{
    float s = 0.0f;
    for (int i = 0; i < 4; i++) s += (float)(next_u32() & 0xffff) / 65536.0f;
    return (s - 2.0f) * 1.7f;
}

#define CHECK(c, what) do { if (!(c)) { fprintf(stderr, "check failed: %s\n", what); exit(1); } } while (0)

static void *xmalloc(size_t n) { void *p = malloc(n ? n : 1); CHECK(p != NULL, "malloc"); return p; }

static void formats(void)
{
    for (int c = 0; c < 16; c++) CHECK(isfinite(or_e2m1((uint8_t)c)), "e2m1 finite");
    int nan = 0;
    for (int b = 0; b < 256; b++) nan += isnan(or_e4m3((uint8_t)b));
    CHECK(nan == 2, "two E4M3 NaN bytes");
    uint16_t *h = xmalloc(65536 * sizeof(uint16_t));
    float *f = xmalloc(65536 * sizeof(float));
    uint16_t *back = xmalloc(65536 * sizeof(uint16_t));
    for (int i = 0; i < 65536; i++) h[i] = (uint16_t)i;
    or_bf16_to_f32_array(h, f, 65536);
    or_f32_to_bf16_array(f, back, 65536);
    for (int i = 0; i < 65536; i++)
        if (!isnan(f[i])) CHECK(back[i] == h[i], "bf16 round trip");
    or_fp16_to_f32_array(h, f, 65536);
    or_f32_to_fp16_array(f, back, 65536);
    for (int i = 0; i < 65536; i++)
        if (!isnan(f[i])) CHECK(back[i] == h[i], "fp16 round trip");
    free(h); free(f); free(back);
}

static void swish(void)
{
    const float xs[] = {0.0f, -0.0f, 1e-30f, -1e-30f, 0.5f, -3.0f, 88.0f, 89.5f, -103.0f, -104.5f, -200.0f,
                        200.0f, INFINITY, -INFINITY, NAN, 3.4e38f, -3.4e38f, 1.4e-45f};
    for (size_t i = 0; i < sizeof xs / sizeof xs[0]; i++) {
        (void)or_exp(xs[i]);
        (void)or_sigmoid(xs[i]);
        (void)or_swiglu(xs[i], 2.0f);
    }
    CHECK(or_exp(0.0f) == 1.0f, "E(0) = 1");
}

/* one NVFP4 weight with exactly-sized arrays: codes [N, ceil(K/2)], scales [N, ceil(K/16)] */
static void nvfp4_case(int64_t N, int64_t K, float g)
{
    const int64_t ldc = (K + 1) / 2, lds = (K + 15) / 16, kp = or_padded_k(K);
    uint8_t *codes = xmalloc((size_t)(N * ldc));
    uint8_t *sf = xmalloc((size_t)(N * lds));
    for (int64_t i = 0; i < N * ldc; i++) codes[i] = (uint8_t)next_u32();
    for (int64_t i = 0; i < N * lds; i++) {
        uint8_t b = (uint8_t)next_u32();
        sf[i] = ((b & 0x7f) == 0x7f) ? 0x38 : b;      /* finite scales only */
    }
    for (int64_t k = 0; k < lds && N > 1; k++) sf[lds + k] = 0;   /* row 1: a zero row */
    float *w = xmalloc(sizeof(float) * (size_t)(N * kp));
    or_nvfp4_decode(codes, ldc, sf, lds, g, N, K, w, kp);
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = K; k < kp; k++) CHECK(w[n * kp + k] == 0.0f, "decode pads with zeros");
    int8_t *q = xmalloc((size_t)(N * kp));
    float *s = xmalloc(sizeof(float) * (size_t)N);
    float *a = xmalloc(sizeof(float) * (size_t)N);
    CHECK(or_prep_weight_nvfp4(codes, ldc, sf, lds, g, N, K, q, kp, s) == 0, "prep_weight");
    CHECK(or_weight_amax_nvfp4(codes, ldc, sf, lds, g, N, K, a) == 0, "weight_amax");
    for (int64_t n = 0; n < N; n++) {
        int mx = 0;
        for (int64_t k = 0; k < kp; k++) mx = abs(q[n * kp + k]) > mx ? abs(q[n * kp + k]) : mx;
        CHECK((s[n] == 0.0f && mx == 0) || mx == 127, "every nonzero row reaches 127");
        CHECK(s[n] == a[n] / 127.0f, "scale = a / 127");
    }
    free(codes); free(sf); free(w); free(q); free(s); free(a);
}

static void rotation_and_quant(void)
{
    float blk[256];
    for (int i = 0; i < 256; i++) blk[i] = (float)(int)(next_u32() % 17) - 8.0f;   /* small: both transforms stay exact */
    float orig[256];
    memcpy(orig, blk, sizeof blk);
    or_fwht256(blk);
    or_fwht256(blk);
    for (int i = 0; i < 256; i++) CHECK(blk[i] == orig[i], "rotation is an involution on integers");
    const int64_t rows = 4, kp = 512;
    float *y = xmalloc(sizeof(float) * rows * kp);
    for (int64_t i = 0; i < rows * kp; i++) y[i] = next_normal();
    for (int64_t k = 0; k < kp; k++) { y[kp + k] = 0.0f; y[2 * kp + k] *= 1e-38f; y[3 * kp + k] *= 1e-44f; }
    or_convrot256(y, rows, kp, kp);
    int8_t *q = xmalloc((size_t)(rows * kp));
    float *s = xmalloc(sizeof(float) * rows);
    or_row_quant(y, rows, kp, kp, q, kp, s);
    CHECK(s[1] == 0.0f, "zero row scale");
    free(y); free(q); free(s);
}

/* activation rows of every dtype, held with row stride exactly the used width */
static void act_case(int dtype, int swiglu, int64_t M, int64_t K, int pre)
{
    const int64_t cols = swiglu ? 2 * K : K, kp = or_padded_k(K);
    const size_t es = dtype == 2 ? 4 : 2;
    void *x = xmalloc(es * (size_t)(M * cols));
    for (int64_t i = 0; i < M * cols; i++) {
        float v = next_normal();
        if (dtype == 2) ((float *)x)[i] = v;
        else or_f32_to_bf16_array(&v, (uint16_t *)x + i, 1);   /* bf16 bits also read as fp16: any finite */
    }
    if (dtype == 1)
        for (int64_t i = 0; i < M * cols; i++) {
            uint16_t *h = (uint16_t *)x + i;
            if ((*h & 0x7c00) == 0x7c00) *h &= 0x83ff;           /* keep fp16 values finite */
        }
    float *c = NULL;
    if (pre) {
        c = xmalloc(sizeof(float) * (size_t)K);
        for (int64_t k = 0; k < K; k++) c[k] = 0.5f + (float)(next_u32() % 1000) / 1000.0f;
    }
    int8_t *q = xmalloc((size_t)(M * kp));
    float *s = xmalloc(sizeof(float) * (size_t)M);
    CHECK(or_quant_act_ex(x, dtype, cols, swiglu, M, K, c, q, kp, s) == 0, "quant_act");
    free(x); free(q); free(s); free(c);
}

static void gemm_epilogue_layer(void)
{
    const int64_t M = 5, N = 7, K = 300, kp = or_padded_k(K);
    int8_t *a = xmalloc((size_t)(M * kp)), *b = xmalloc((size_t)(N * kp));
    for (int64_t i = 0; i < M * kp; i++) a[i] = (int8_t)((int)(next_u32() % 255) - 127);
    for (int64_t i = 0; i < N * kp; i++) b[i] = (int8_t)((int)(next_u32() % 255) - 127);
    int32_t *acc = xmalloc(sizeof(int32_t) * M * N);
    or_gemm_s8(a, kp, b, kp, M, N, kp, acc, N);
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            int64_t t = 0;
            for (int64_t k = 0; k < kp; k++) t += (int64_t)a[m * kp + k] * b[n * kp + k];
            CHECK(t == acc[m * N + n], "int32 GEMM = int64 sum");
        }
    float sx[5], sw[7], bias[7];
    for (int i = 0; i < 5; i++) sx[i] = 1e-3f * (float)(i + 1);
    for (int i = 0; i < 7; i++) { sw[i] = 2e-4f * (float)(i + 1); bias[i] = (float)i - 3.0f; }
    void *out = xmalloc(4 * M * N);
    for (int dt = 0; dt < 4; dt++) {
        or_epilogue_ex(acc, N, sx, sw, NULL, M, N, dt, out, N);
        if (dt != 3) or_epilogue_ex(acc, N, sx, sw, bias, M, N, dt, out, N);
    }
    free(a); free(b); free(acc); free(out);

    /* the whole layer, tight strides, with and without pre-scale and bias */
    const int64_t ldc = (K + 1) / 2, lds = (K + 15) / 16;
    uint8_t *codes = xmalloc((size_t)(N * ldc)), *sf = xmalloc((size_t)(N * lds));
    for (int64_t i = 0; i < N * ldc; i++) codes[i] = (uint8_t)next_u32();
    for (int64_t i = 0; i < N * lds; i++) sf[i] = (uint8_t)(0x30 + next_u32() % 16);
    uint16_t *x = xmalloc(2 * (size_t)(M * 2 * K));
    for (int64_t i = 0; i < M * 2 * K; i++) { float v = next_normal(); or_f32_to_bf16_array(&v, x + i, 1); }
    float *pre = xmalloc(sizeof(float) * K);
    for (int64_t k = 0; k < K; k++) pre[k] = 1.0f + (float)k / (float)K;
    void *y = xmalloc(4 * M * N);
    for (int sw_ = 0; sw_ < 2; sw_++)
        for (int dt = 0; dt < 3; dt++) {
            CHECK(or_linear_nvfp4_ex(x, 0, sw_ ? 2 * K : K, sw_, M, K, NULL, codes, ldc, sf, lds, 0.0137f, N,
                                     NULL, y, dt, N) == 0, "layer");
            CHECK(or_linear_nvfp4_ex(x, 0, sw_ ? 2 * K : K, sw_, M, K, pre, codes, ldc, sf, lds, 0.0137f, N,
                                     bias, y, dt, N) == 0, "layer with pre-scale and bias");
        }
    free(codes); free(sf); free(x); free(pre); free(y);
}

/* the W4A8 functions on exactly-sized buffers: packed rows of K_pad / 2 bytes */
static void w4a8_case(int64_t M, int64_t N, int64_t K)
{
    const int64_t kp = or_padded_k(K), lp = kp / 2;
    float *w = xmalloc(sizeof(float) * (size_t)(N * K));
    for (int64_t i = 0; i < N * K; i++) w[i] = next_normal() * 0.02f;
    for (int64_t k = 0; k < K && N > 1; k++) w[K + k] = 0.0f;          /* row 1: a zero row */
    uint8_t *p = xmalloc((size_t)(N * lp));
    float *s = xmalloc(sizeof(float) * (size_t)N);
    CHECK(or_quant_weight_w4(w, 2, K, N, K, p, lp, s) == 0, "quant_weight_w4");
    int8_t *q = xmalloc((size_t)(N * kp));
    or_unpack_s4(p, N, kp, lp, q, kp);
    uint8_t *p2 = xmalloc((size_t)(N * lp));
    or_pack_s4(q, N, kp, kp, p2, lp);
    CHECK(memcmp(p, p2, (size_t)(N * lp)) == 0, "pack(unpack(p)) == p");
    for (int64_t n = 0; n < N; n++) {
        int mx = 0;
        for (int64_t k = 0; k < kp; k++) mx = abs(q[n * kp + k]) > mx ? abs(q[n * kp + k]) : mx;
        CHECK((s[n] == 0.0f && mx == 0) || mx == 7, "every nonzero 4-bit row reaches 7");
    }
    uint16_t *x = xmalloc(2 * (size_t)(M * K));
    for (int64_t i = 0; i < M * K; i++) { float v = next_normal(); or_f32_to_bf16_array(&v, x + i, 1); }
    int8_t *a = xmalloc((size_t)(M * kp));
    for (int64_t i = 0; i < M * kp; i++) a[i] = (int8_t)((int)(next_u32() % 255) - 127);
    int32_t *acc = xmalloc(sizeof(int32_t) * (size_t)(M * N));
    CHECK(or_gemm_s8s4(a, kp, p, lp, M, N, kp, acc, N) == 0, "gemm_s8s4");
    void *y = xmalloc(4 * (size_t)(M * N));
    for (int dt = 0; dt < 3; dt++) CHECK(or_linear_w4a8(x, 0, K, 0, M, K, p, lp, s, N, NULL, y, dt, N) == 0, "w4a8");
    /* W4A4: 4-bit activation rows (plain and SwiGLU over the first K/2 pairs), the 4x4 GEMM */
    uint8_t *xp = xmalloc((size_t)(M * lp));
    float *xs = xmalloc(sizeof(float) * (size_t)M);
    CHECK(or_quant_act_w4(x, 0, K, 0, M, K, xp, lp, xs) == 0, "quant_act_w4");
    CHECK(or_gemm_s4s4(xp, lp, p, lp, M, N, kp, acc, N) == 0, "gemm_s4s4");
    if (K >= 2) {
        const int64_t kh = K / 2, lph = or_padded_k(kh) / 2;
        uint8_t *hp = xmalloc((size_t)(M * lph));
        CHECK(or_quant_act_w4(x, 0, K, 1, M, kh, hp, lph, xs) == 0, "quant_act_w4 swiglu");
        free(hp);
    }
    for (int dt = 0; dt < 3; dt++) CHECK(or_linear_w4a4(x, 0, K, 0, M, K, p, lp, s, N, s, y, dt, N) == 0, "w4a4");
    /* the E2M3 field form of the same codes: quads of rows, exactly 3 K_pad bytes each */
    {
        const int64_t l6 = 3 * kp;                              /* one quad of rows */
        uint8_t *f = xmalloc((size_t)((N + 3) / 4 * l6));
        int8_t *q2 = xmalloc((size_t)(N * kp));
        CHECK(or_pack_e2m3(q, N, kp, kp, f, l6) == 0, "pack_e2m3");
        CHECK(or_unpack_e2m3(f, N, kp, l6, q2, kp) == 0 && memcmp(q, q2, (size_t)(N * kp)) == 0, "unpack_e2m3");
        int32_t *acc2 = xmalloc(sizeof(int32_t) * (size_t)(N * N));
        CHECK(or_gemm_e2m3(f, l6, f, l6, N, N, kp, acc2, N) == 0, "gemm_e2m3");
        for (int c = 0; c < 64; c++) (void)or_e2m3((uint8_t)c);
        free(f); free(q2); free(acc2);
    }
    free(xp); free(xs);
    float y4[256];
    for (int i = 0; i < 256; i++) y4[i] = (float)(int)(next_u32() % 15) - 7.0f;
    int8_t q4[256];
    float s4;
    or_row_quant_s4(y4, 1, 256, 256, q4, 256, &s4);
    free(w); free(p); free(s); free(q); free(p2); free(x); free(a); free(acc); free(y);
}

int main(void)
{
    formats();
    swish();
    rotation_and_quant();
    const int64_t Ks[] = {1, 15, 16, 17, 255, 256, 257, 300, 1000};
    for (size_t i = 0; i < sizeof Ks / sizeof Ks[0]; i++) {
        nvfp4_case(3, Ks[i], 0.0137f);
        nvfp4_case(2, Ks[i], 7.1e-37f);
        for (int dt = 0; dt < 3; dt++) {
            act_case(dt, 0, 3, Ks[i], 0);
            act_case(dt, 1, 2, Ks[i], (int)(i & 1));
        }
    }
    nvfp4_case(2, 16385, 0.25f);          /* a row past the two-pass width */
    act_case(1, 0, 2, 20000, 1);
    gemm_epilogue_layer();
    w4a8_case(3, 5, 300);
    w4a8_case(2, 3, 17);
    w4a8_case(1, 2, 16385);
    printf("oracle sanitizer driver: ok\n");
    return 0;
}
