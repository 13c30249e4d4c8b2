// Native consumer of the C ABI: no Python, no torch.  Device memory from hipMalloc, inputs
// from a fixed-seed generator on the host.  Runs the layer through the component calls and
// through cr_linear_nvfp4 (staged and short-batch paths, one and two streams), and the
// W4A8 / W4A4 variants through theirs, and checks that every route gives the same bits;
// also checks argument errors come back as statuses.
// Exit status 0 on success.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "convrot.h"

#define HIP_OK(x)                                                                   \
    do {                                                                            \
        hipError_t e_ = (x);                                                        \
        if (e_ != hipSuccess) {                                                     \
            std::fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
            return 1;                                                               \
        }                                                                           \
    } while (0)
#define CR_OK_(x)                                                                   \
    do {                                                                            \
        cr_status s_ = (x);                                                         \
        if (s_ != CR_OK) {                                                          \
            std::fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, cr_status_string(s_)); \
            return 1;                                                               \
        }                                                                           \
    } while (0)

namespace {

uint32_t lcg(uint64_t &s)
{
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(s >> 33);
}

uint16_t bf16_of(float f)      // truncation is fine for making inputs
{
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

int run_case(int64_t M, int64_t N, int64_t K, hipStream_t s_main, hipStream_t s_aux)
{
    const int64_t kp = cr_padded_k(K), ld_fp4 = ((K + 1) / 2 + 15) / 16 * 16, ld_sf = (K + 15) / 16;
    uint64_t seed = (uint64_t)(M * 1000003 + N * 1009 + K);
    std::vector<uint16_t> hx((size_t)(M * kp));
    for (auto &v : hx) v = bf16_of(((float)(lcg(seed) % 2001) - 1000.0f) / 400.0f);
    std::vector<uint8_t> hc((size_t)(N * ld_fp4)), hs((size_t)(N * ld_sf));
    for (auto &v : hc) v = (uint8_t)lcg(seed);
    for (auto &v : hs) v = (uint8_t)(0x30 + lcg(seed) % 16);     // E4M3 scales 0.5 .. 1.875
    const float g = 0.01f;

    void *x, *out_a, *out_b, *ws;
    uint8_t *codes, *sf;
    int8_t *qx, *qw;
    float *sx, *sw, *gd;
    HIP_OK(hipMalloc(&x, hx.size() * 2));
    HIP_OK(hipMalloc((void **)&codes, hc.size()));
    HIP_OK(hipMalloc((void **)&sf, hs.size()));
    HIP_OK(hipMalloc((void **)&gd, 4));
    HIP_OK(hipMalloc((void **)&qx, (size_t)(M * kp)));
    HIP_OK(hipMalloc((void **)&qw, (size_t)(N * kp)));
    HIP_OK(hipMalloc((void **)&sx, (size_t)M * 4));
    HIP_OK(hipMalloc((void **)&sw, (size_t)N * 4));
    HIP_OK(hipMalloc(&out_a, (size_t)(M * N * 2)));
    HIP_OK(hipMalloc(&out_b, (size_t)(M * N * 2)));
    const size_t wsb = cr_linear_nvfp4_workspace_bytes(M, N, K, 0);
    HIP_OK(hipMalloc(&ws, wsb));
    HIP_OK(hipMemcpy(x, hx.data(), hx.size() * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(codes, hc.data(), hc.size(), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(sf, hs.data(), hs.size(), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(gd, &g, 4, hipMemcpyHostToDevice));

    // components: natural column order
    CR_OK_(cr_quant_act(x, CR_BF16, kp, M, K, qx, kp, sx, CR_FLAG_NONE, s_main));
    CR_OK_(cr_prep_weight_nvfp4(codes, ld_fp4, sf, ld_sf, gd, N, K, qw, kp, sw, CR_FLAG_NONE, s_main));
    CR_OK_(cr_gemm_s8_rowscale(qx, kp, sx, qw, kp, sw, M, N, kp, out_a, CR_BF16, N, s_main));
    HIP_OK(hipStreamSynchronize(s_main));
    std::vector<uint16_t> ra((size_t)(M * N)), rb((size_t)(M * N));
    HIP_OK(hipMemcpy(ra.data(), out_a, ra.size() * 2, hipMemcpyDeviceToHost));

    for (int two = 0; two < 2; two++) {
        HIP_OK(hipMemset(out_b, 0xFF, (size_t)(M * N * 2)));
        CR_OK_(cr_linear_nvfp4(x, CR_BF16, kp, 0, M, K, codes, ld_fp4, sf, ld_sf, gd, N, out_b, CR_BF16, N, ws, wsb,
                               0, CR_FLAG_NONE, s_main, two ? s_aux : nullptr));
        HIP_OK(hipStreamSynchronize(s_main));
        HIP_OK(hipMemcpy(rb.data(), out_b, rb.size() * 2, hipMemcpyDeviceToHost));
        if (std::memcmp(ra.data(), rb.data(), ra.size() * 2) != 0) {
            std::fprintf(stderr, "M=%lld N=%lld K=%lld: layer (streams=%d) differs from the components\n",
                         (long long)M, (long long)N, (long long)K, 1 + two);
            return 1;
        }
    }
    int64_t rows = 0, chunks = 0;
    CR_OK_(cr_linear_nvfp4_plan(M, N, K, 0, &rows, &chunks));
    std::printf("M=%lld N=%lld K=%lld: components == layer (%s path), ok\n", (long long)M, (long long)N,
                (long long)K, chunks == 0 ? "decode-inside-GEMM" : "staged");

    // argument errors are statuses, nothing launched; empty extents are valid no-ops
    if (cr_gemm_s8_rowscale(qx, kp, sx, qw, kp, sw, M, N, kp + 1, out_a, CR_BF16, N, s_main) != CR_ERR_INVALID_ARG ||
        cr_quant_act(x, CR_BF16, kp, -1, K, qx, kp, sx, CR_FLAG_NONE, s_main) != CR_ERR_INVALID_ARG ||
        cr_quant_act(nullptr, CR_BF16, kp, 0, K, nullptr, kp, nullptr, CR_FLAG_NONE, s_main) != CR_OK ||
        cr_linear_nvfp4(nullptr, CR_BF16, kp, 0, 0, K, codes, ld_fp4, sf, ld_sf, gd, N, nullptr, CR_BF16, N,
                        nullptr, 0, 0, CR_FLAG_NONE, s_main, nullptr) != CR_OK ||
        cr_linear_nvfp4(x, CR_BF16, kp, 0, M, K, codes, ld_fp4, sf, ld_sf, gd, N, out_b, CR_BF16, N, ws, wsb - 1, 0,
                        CR_FLAG_NONE, s_main, nullptr) != CR_ERR_TOO_LARGE) {
        std::fprintf(stderr, "argument checks did not return the documented statuses\n");
        return 1;
    }
    for (void *p : {(void *)x, (void *)codes, (void *)sf, (void *)gd, (void *)qx, (void *)qw, (void *)sx, (void *)sw,
                    out_a, out_b, ws})
        HIP_OK(hipFree(p));
    return 0;
}

// The 4-bit variants through their C calls: W4A8 and W4A4 (nibble and E2M3 forms) each as
// components and as the layer call, the E2M3 weight both prepared directly and repacked
// from the nibble form; all routes of one variant give the same bits, and the two W4A4
// forms give the same bits.
int run_w4_case(int64_t M, int64_t N, int64_t K, hipStream_t s)
{
    const int64_t kp = cr_padded_k(K), ldx = (K + 7) / 8 * 8, l4 = kp / 2, l6 = 3 * kp;
    const int64_t q_m = (M + 3) / 4, q_n = (N + 3) / 4;
    uint64_t seed = (uint64_t)(M * 7919 + N * 31 + K);
    std::vector<uint16_t> hx((size_t)(M * ldx)), hw((size_t)(N * ldx));
    for (auto &v : hx) v = bf16_of(((float)(lcg(seed) % 2001) - 1000.0f) / 400.0f);
    for (auto &v : hw) v = bf16_of(((float)(lcg(seed) % 2001) - 1000.0f) / 50000.0f);

    void *x, *w, *out_a, *out_b, *ws;
    int8_t *qx8;
    uint8_t *p4, *p6, *p6r, *qx4, *qx6;
    float *sx8, *sx4, *sx6, *sw4, *sw6;
    const size_t ob = (size_t)(M * N * 2);
    const size_t wsb = cr_linear_w4a8_workspace_bytes(M, K) > cr_linear_w4a4_e2m3_workspace_bytes(M, K)
                           ? cr_linear_w4a8_workspace_bytes(M, K) : cr_linear_w4a4_e2m3_workspace_bytes(M, K);
    HIP_OK(hipMalloc(&x, hx.size() * 2));
    HIP_OK(hipMalloc(&w, hw.size() * 2));
    HIP_OK(hipMalloc((void **)&qx8, (size_t)(M * kp)));
    HIP_OK(hipMalloc((void **)&qx4, (size_t)(M * l4)));
    HIP_OK(hipMalloc((void **)&qx6, (size_t)(q_m * l6)));
    HIP_OK(hipMalloc((void **)&p4, (size_t)(N * l4)));
    HIP_OK(hipMalloc((void **)&p6, (size_t)(q_n * l6)));
    HIP_OK(hipMalloc((void **)&p6r, (size_t)(q_n * l6)));
    for (float **f : {&sx8, &sx4, &sx6}) HIP_OK(hipMalloc((void **)f, (size_t)M * 4));
    for (float **f : {&sw4, &sw6}) HIP_OK(hipMalloc((void **)f, (size_t)N * 4));
    HIP_OK(hipMalloc(&out_a, ob));
    HIP_OK(hipMalloc(&out_b, ob));
    HIP_OK(hipMalloc(&ws, wsb));
    HIP_OK(hipMemcpy(x, hx.data(), hx.size() * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(w, hw.data(), hw.size() * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemset(p6, 0, (size_t)(q_n * l6)));       // rows past N in the last quad
    HIP_OK(hipMemset(p6r, 0, (size_t)(q_n * l6)));

    const uint32_t bt = CR_FLAG_BLOCK_TRANSPOSED;
    CR_OK_(cr_quant_weight_w4(w, CR_BF16, ldx, N, K, p4, l4, sw4, bt, s));
    CR_OK_(cr_quant_weight_w4_e2m3(w, CR_BF16, ldx, N, K, p6, l6, sw6, bt, s));
    CR_OK_(cr_repack_w4_e2m3(p4, l4, N, kp, p6r, l6, s));
    HIP_OK(hipStreamSynchronize(s));
    std::vector<uint8_t> f6a((size_t)(q_n * l6)), f6b((size_t)(q_n * l6));
    std::vector<float> sa((size_t)N), sb((size_t)N);
    HIP_OK(hipMemcpy(f6a.data(), p6, f6a.size(), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(f6b.data(), p6r, f6b.size(), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(sa.data(), sw4, (size_t)N * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(sb.data(), sw6, (size_t)N * 4, hipMemcpyDeviceToHost));
    if (f6a != f6b || std::memcmp(sa.data(), sb.data(), sa.size() * 4) != 0) {
        std::fprintf(stderr, "M=%lld N=%lld K=%lld: repacked E2M3 weight differs from the direct one\n",
                     (long long)M, (long long)N, (long long)K);
        return 1;
    }

    std::vector<uint16_t> ra((size_t)(M * N)), rb((size_t)(M * N)), r4((size_t)(M * N));
    auto same = [&](const char *what, const std::vector<uint16_t> &want) -> bool {
        if (hipStreamSynchronize(s) != hipSuccess || hipMemcpy(rb.data(), out_b, ob, hipMemcpyDeviceToHost) != hipSuccess)
            return false;
        if (std::memcmp(want.data(), rb.data(), ob) != 0) {
            std::fprintf(stderr, "M=%lld N=%lld K=%lld: %s differs\n", (long long)M, (long long)N, (long long)K, what);
            return false;
        }
        return true;
    };
    // W4A8: components == layer
    CR_OK_(cr_quant_act(x, CR_BF16, ldx, M, K, qx8, kp, sx8, bt, s));
    CR_OK_(cr_gemm_s8s4_rowscale(qx8, kp, sx8, p4, l4, sw4, nullptr, M, N, kp, out_a, CR_BF16, N, s));
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(ra.data(), out_a, ob, hipMemcpyDeviceToHost));
    HIP_OK(hipMemset(out_b, 0xFF, ob));
    CR_OK_(cr_linear_w4a8(x, CR_BF16, ldx, 0, M, K, p4, l4, sw4, N, nullptr, out_b, CR_BF16, N, ws, wsb, bt, s));
    if (!same("cr_linear_w4a8 vs its components", ra)) return 1;
    // W4A4, nibble form: components == layer
    CR_OK_(cr_quant_act_w4(x, CR_BF16, ldx, 0, M, K, qx4, l4, sx4, bt, s));
    CR_OK_(cr_gemm_s4s4_rowscale(qx4, l4, sx4, p4, l4, sw4, nullptr, M, N, kp, out_a, CR_BF16, N, s));
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(r4.data(), out_a, ob, hipMemcpyDeviceToHost));
    HIP_OK(hipMemset(out_b, 0xFF, ob));
    CR_OK_(cr_linear_w4a4(x, CR_BF16, ldx, 0, M, K, p4, l4, sw4, N, nullptr, out_b, CR_BF16, N, ws, wsb, bt, s));
    if (!same("cr_linear_w4a4 vs its components", r4)) return 1;
    // W4A4, E2M3 form: components and layer == the nibble form
    CR_OK_(cr_quant_act_w4_e2m3(x, CR_BF16, ldx, 0, M, K, qx6, l6, sx6, bt, s));
    HIP_OK(hipMemset(out_b, 0xFF, ob));
    CR_OK_(cr_gemm_e2m3_rowscale(qx6, l6, sx6, p6r, l6, sw6, nullptr, M, N, kp, out_b, CR_BF16, N, s));
    if (!same("E2M3 GEMM vs the nibble-form layer", r4)) return 1;
    HIP_OK(hipMemset(out_b, 0xFF, ob));
    CR_OK_(cr_linear_w4a4_e2m3(x, CR_BF16, ldx, 0, M, K, p6, l6, sw6, N, nullptr, out_b, CR_BF16, N, ws, wsb, bt, s));
    if (!same("cr_linear_w4a4_e2m3 vs the nibble-form layer", r4)) return 1;
    std::printf("M=%lld N=%lld K=%lld: W4A8 and W4A4 (both forms) components == layers, repack == direct, ok\n",
                (long long)M, (long long)N, (long long)K);

    // argument errors come back as statuses
    if (cr_gemm_e2m3_rowscale(qx6, l6 - 16, sx6, p6, l6, sw6, nullptr, M, N, kp, out_b, CR_BF16, N, s) != CR_ERR_INVALID_ARG ||
        cr_repack_w4_e2m3(p4, l4, N, kp + 128, p6r, l6 + 384, s) != CR_ERR_INVALID_ARG ||
        cr_quant_act_w4(x, CR_BF16, ldx, 0, M, K, qx4 + 1, l4, sx4, bt, s) != CR_ERR_MISALIGNED ||
        cr_linear_w4a4_e2m3(x, CR_BF16, ldx, 0, M, K, p6, l6, sw6, N, nullptr, out_b, CR_BF16, N, ws,
                            cr_linear_w4a4_e2m3_workspace_bytes(M, K) - 1, bt, s) != CR_ERR_TOO_LARGE ||
        cr_linear_w4a8(x, CR_BF16, ldx, 0, 0, K, p4, l4, sw4, N, nullptr, nullptr, CR_BF16, N, nullptr, 0, bt, s) != CR_OK) {
        std::fprintf(stderr, "4-bit argument checks did not return the documented statuses\n");
        return 1;
    }
    for (void *p : {(void *)x, (void *)w, (void *)qx8, (void *)qx4, (void *)qx6, (void *)p4, (void *)p6, (void *)p6r,
                    (void *)sx8, (void *)sx4, (void *)sx6, (void *)sw4, (void *)sw6, out_a, out_b, ws})
        HIP_OK(hipFree(p));
    return 0;
}

}  // namespace

int main()
{
    if (cr_abi_version() != CR_ABI_VERSION) {
        std::fprintf(stderr, "ABI version mismatch\n");
        return 1;
    }
    hipStream_t s_main, s_aux;
    HIP_OK(hipStreamCreate(&s_main));
    HIP_OK(hipStreamCreate(&s_aux));
    const int64_t cases[][3] = {{300, 520, 1000}, {8, 300, 5376}, {70, 1000, 20000}};
    for (const auto &c : cases)
        if (run_case(c[0], c[1], c[2], s_main, s_aux) != 0) return 1;
    const int64_t w4_cases[][3] = {{300, 517, 1000}, {33, 256, 5376}, {70, 90, 20000}};
    for (const auto &c : w4_cases)
        if (run_w4_case(c[0], c[1], c[2], s_main) != 0) return 1;
    HIP_OK(hipStreamDestroy(s_main));
    HIP_OK(hipStreamDestroy(s_aux));
    std::printf("abi_smoke: all cases ok\n");
    return 0;
}
