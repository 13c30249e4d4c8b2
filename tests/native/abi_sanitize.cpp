// Sanitizer driver for the host side of the C ABI (argument validation, the chunk planner,
// workspace sizes, the allocation-free entry point's refusals).  The test suite builds
// api.cpp with AddressSanitizer and UndefinedBehaviorSanitizer on its host side, links it
// with the library's kernel objects and this program, and runs it on the CPU.  Every call
// below either fails validation or has an empty extent, so no kernel is ever launched: the
// pointers are aligned host addresses that no call may dereference.  Calls with fully valid
// arguments are made only when no GPU is visible, where they must return CR_ERR_NO_DEVICE.
// Exit status 1 names the first unexpected status.
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "convrot.h"

namespace {

int failures = 0;

void expect(const char *what, cr_status got, cr_status want)
{
    if (got != want) {
        std::fprintf(stderr, "%s: got %s, want %s\n", what, cr_status_string(got), cr_status_string(want));
        failures++;
    }
}

alignas(256) unsigned char arena[1 << 16];
void *P(size_t off = 0) { return arena + 256 + off; }
template <class T> T *Q(size_t off = 0) { return reinterpret_cast<T *>(arena + 256 + off); }

}  // namespace

int main()
{
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess) ndev = 0;
    (void)hipGetLastError();
    const int64_t BIG = CR_MAX_K_PAD + 1;

    expect("abi version", cr_abi_version() == CR_ABI_VERSION ? CR_OK : CR_ERR_INVALID_ARG, CR_OK);
    for (int s = -1; s < 9; s++) (void)cr_status_string((cr_status)s);   // -1, 7, 8: not statuses
    if (cr_padded_k(0) != 0 || cr_padded_k(1) != 256 || cr_padded_k(20000) != 20224) failures++;

    // activation preparation
    auto qa = [&](const void *x, int dt, int64_t ldx, int64_t M, int64_t K, void *q, int64_t ldq, void *s,
                  uint32_t fl) {
        return cr_quant_act(x, (cr_dtype)dt, ldx, M, K, (int8_t *)q, ldq, (float *)s, fl, nullptr);
    };
    expect("qa null x", qa(nullptr, 0, 512, 4, 512, P(), 512, P(), 0), CR_ERR_INVALID_ARG);
    expect("qa M<0", qa(P(), 0, 512, -1, 512, P(), 512, P(), 0), CR_ERR_INVALID_ARG);
    expect("qa K=0", qa(P(), 0, 512, 4, 0, P(), 512, P(), 0), CR_ERR_INVALID_ARG);
    expect("qa dtype", qa(P(), 3, 512, 4, 512, P(), 512, P(), 0), CR_ERR_UNSUPPORTED_DTYPE);
    expect("qa ld_x<K", qa(P(), 0, 500, 4, 512, P(), 512, P(), 0), CR_ERR_INVALID_ARG);
    expect("qa ld_s8<K_pad", qa(P(), 0, 512, 4, 512, P(), 256, P(), 0), CR_ERR_INVALID_ARG);
    expect("qa misaligned x", qa(P(2), 0, 512, 4, 512, P(), 512, P(), 0), CR_ERR_MISALIGNED);
    expect("qa odd row bytes", qa(P(), 0, 513, 4, 512, P(), 512, P(), 0), CR_ERR_MISALIGNED);
    expect("qa K too large", qa(P(), 0, BIG + 16, 4, BIG, P(), BIG + 256, P(), 0), CR_ERR_TOO_LARGE);
    expect("qa bad flag", qa(P(), 0, 512, 4, 512, P(), 512, P(), 8), CR_ERR_INVALID_ARG);
    expect("qa empty batch", qa(nullptr, 0, 512, 0, 512, nullptr, 512, nullptr, 0), CR_OK);
    expect("swiglu ld_h<2F", cr_quant_act_swiglu(P(), CR_BF16, 1000, 4, 512, Q<int8_t>(), 512, Q<float>(), 0,
                                                 nullptr), CR_ERR_INVALID_ARG);
    expect("swiglu huge F", cr_quant_act_swiglu(P(), CR_BF16, 1024, 4, (int64_t)1 << 41, Q<int8_t>(), 512,
                                                Q<float>(), 0, nullptr), CR_ERR_TOO_LARGE);
    expect("ex pre misaligned", cr_quant_act_ex(P(), CR_BF16, 512, 0, 4, 512, Q<float>(2), Q<int8_t>(), 512,
                                                Q<float>(), 0, nullptr), CR_ERR_MISALIGNED);
    expect("cr_swiglu F=0", cr_swiglu(P(), CR_BF16, 16, 4, 0, Q<float>(), 16, nullptr), CR_ERR_INVALID_ARG);
    expect("cr_swiglu overflowing size", cr_swiglu(P(), CR_BF16, (int64_t)1 << 41, (int64_t)1 << 30,
                                                   (int64_t)1 << 20, Q<float>(), (int64_t)1 << 20, nullptr),
           CR_ERR_INVALID_ARG);

    // weight preparation and row maxima
    auto pw = [&](int64_t ld, int64_t ldsf, const void *g, int64_t n, int64_t K, int64_t ldq, uint32_t fl,
                  size_t off = 0) {
        return cr_prep_weight_nvfp4(Q<uint8_t>(off), ld, Q<uint8_t>(), ldsf, (const float *)g, n, K,
                                    Q<int8_t>(), ldq, Q<float>(), fl, nullptr);
    };
    expect("pw null g", pw(256, 32, nullptr, 8, 512, 512, 0), CR_ERR_INVALID_ARG);
    expect("pw n<0", pw(256, 32, P(), -1, 512, 512, 0), CR_ERR_INVALID_ARG);
    expect("pw ld<K/2", pw(200, 32, P(), 8, 512, 512, 0), CR_ERR_INVALID_ARG);
    expect("pw ld_sf<K/16", pw(256, 31, P(), 8, 512, 512, 0), CR_ERR_INVALID_ARG);
    expect("pw ld%16", pw(264, 32, P(), 8, 512, 512, 0), CR_ERR_MISALIGNED);
    expect("pw codes misaligned", pw(256, 32, P(), 8, 512, 512, 0, 4), CR_ERR_MISALIGNED);
    expect("pw K too large", pw(BIG, BIG, P(), 8, BIG, BIG + 256, 0), CR_ERR_TOO_LARGE);
    expect("pw bad flag", pw(256, 32, P(), 8, 512, 512, 4), CR_ERR_INVALID_ARG);
    expect("pw empty", cr_prep_weight_nvfp4(nullptr, 256, nullptr, 32, nullptr, 0, 512, nullptr, 512, nullptr, 0,
                                            nullptr), CR_OK);
    expect("amax ld_sf", cr_weight_amax_nvfp4(Q<uint8_t>(), 256, Q<uint8_t>(), 31, Q<float>(), 8, 512,
                                              Q<float>(), 0, nullptr), CR_ERR_INVALID_ARG);
    expect("amax misaligned out", cr_weight_amax_nvfp4(Q<uint8_t>(), 256, Q<uint8_t>(), 32, Q<float>(), 8, 512,
                                                       Q<float>(2), 0, nullptr), CR_ERR_MISALIGNED);

    // GEMM
    auto gm = [&](int64_t lda, const void *sa, int64_t M, int64_t N, int64_t K, int dt, int64_t ldc,
                  size_t aoff = 0) {
        return cr_gemm_s8_rowscale(Q<int8_t>(aoff), lda, (const float *)sa, Q<int8_t>(), 512, Q<float>(), M, N, K,
                                   P(), (cr_dtype)dt, ldc, nullptr);
    };
    expect("gemm K%256", gm(512, P(), 8, 8, 500, 0, 8), CR_ERR_INVALID_ARG);
    expect("gemm null sa", gm(512, nullptr, 8, 8, 512, 0, 8), CR_ERR_INVALID_ARG);
    expect("gemm ldc<N", gm(512, P(), 8, 8, 512, 0, 7), CR_ERR_INVALID_ARG);
    expect("gemm dtype", gm(512, P(), 8, 8, 512, 7, 8), CR_ERR_UNSUPPORTED_DTYPE);
    expect("gemm misaligned a", gm(512, P(), 8, 8, 512, 0, 8, 1), CR_ERR_MISALIGNED);
    expect("gemm lda%16", gm(520, P(), 8, 8, 512, 0, 8), CR_ERR_MISALIGNED);
    expect("gemm too many tiles", gm(512, P(), (int64_t)1 << 30, (int64_t)1 << 30, 512, 0, (int64_t)1 << 30),
           CR_ERR_TOO_LARGE);
    expect("gemm empty", gm(512, P(), 0, 8, 512, 0, 8), CR_OK);
    expect("gemm bias on i32", cr_gemm_s8_rowscale_bias(Q<int8_t>(), 512, Q<float>(), Q<int8_t>(), 512, Q<float>(),
                                                        Q<float>(), 8, 8, 512, P(), CR_I32, 8, nullptr),
           CR_ERR_INVALID_ARG);
    expect("fused M too large", cr_gemm_nvfp4_fused(Q<int8_t>(), 512, Q<float>(), Q<uint8_t>(), 256, Q<uint8_t>(),
                                                    32, Q<float>(), nullptr, nullptr, (int64_t)1 << 24, 8, 512, P(),
                                                    CR_BF16, 8, 0, nullptr), CR_ERR_TOO_LARGE);

    // the layer: plan, workspace sizes and validation
    for (int64_t M : {1, 64, 65, 300, 19989})
        for (int64_t N : {1, 255, 256, 1000, 21504})
            for (int64_t K : {1, 300, 5376, 14336, 20000})
                for (size_t mt : {(size_t)0, (size_t)256 << 10, (size_t)16 << 20}) {
                    int64_t R = -1, nc = -1;
                    expect("plan", cr_linear_nvfp4_plan(M, N, K, mt, &R, &nc), CR_OK);
                    const size_t ws = cr_linear_nvfp4_workspace_bytes(M, N, K, mt);
                    if (M <= 64 ? (R != 0 || nc != 0) : (R < 256 || R % 256 != 0 || nc * R < N || (nc - 1) * R >= N))
                        expect("plan shape", CR_ERR_INVALID_ARG, CR_OK);
                    if (ws < (size_t)M * (size_t)cr_padded_k(K)) expect("workspace size", CR_ERR_INVALID_ARG, CR_OK);
                }
    expect("plan null out", cr_linear_nvfp4_plan(8, 8, 8, 0, nullptr, nullptr), CR_ERR_INVALID_ARG);
    auto lin = [&](int64_t M, int64_t N, int64_t K, int odt, size_t ws, void *wsp) {
        return cr_linear_nvfp4(P(), CR_BF16, 5376, 0, M, K, Q<uint8_t>(), 2688, Q<uint8_t>(), 336, Q<float>(), N,
                               P(), (cr_dtype)odt, 21504, wsp, ws, 0, 0, nullptr, nullptr);
    };
    const size_t need = cr_linear_nvfp4_workspace_bytes(300, 1000, 5376, 0);
    expect("layer i32 out", lin(300, 1000, 5376, CR_I32, need, P()), CR_ERR_UNSUPPORTED_DTYPE);
    expect("layer small workspace", lin(300, 1000, 5376, CR_BF16, need - 1, P()), CR_ERR_TOO_LARGE);
    expect("layer misaligned workspace", lin(300, 1000, 5376, CR_BF16, need, P(16)), CR_ERR_MISALIGNED);
    expect("layer null workspace", lin(300, 1000, 5376, CR_BF16, need, nullptr), CR_ERR_INVALID_ARG);
    expect("layer empty", lin(0, 1000, 5376, CR_BF16, 0, nullptr), CR_OK);
    expect("layer K too large", lin(300, 1000, BIG, CR_BF16, need, P()), CR_ERR_TOO_LARGE);
    // W4A8
    expect("w4 ld_s4 < K_pad/2", cr_quant_weight_w4(P(), CR_FP32, 512, 8, 512, Q<uint8_t>(), 255, Q<float>(), 0,
                                                    nullptr), CR_ERR_INVALID_ARG);
    expect("w4 dtype", cr_quant_weight_w4(P(), CR_I32, 512, 8, 512, Q<uint8_t>(), 256, Q<float>(), 0, nullptr),
           CR_ERR_UNSUPPORTED_DTYPE);
    expect("w4 empty", cr_quant_weight_w4(nullptr, CR_FP32, 512, 0, 512, nullptr, 256, nullptr, 0, nullptr), CR_OK);
    expect("s8s4 ldb < K_pad/2", cr_gemm_s8s4_rowscale(Q<int8_t>(), 512, Q<float>(), Q<uint8_t>(), 240, Q<float>(),
                                                       nullptr, 8, 8, 512, P(), CR_BF16, 8, nullptr),
           CR_ERR_INVALID_ARG);
    expect("s8s4 bias on i32", cr_gemm_s8s4_rowscale(Q<int8_t>(), 512, Q<float>(), Q<uint8_t>(), 256, Q<float>(),
                                                     Q<float>(), 8, 8, 512, P(), CR_I32, 8, nullptr),
           CR_ERR_INVALID_ARG);
    expect("s8s4 empty", cr_gemm_s8s4_rowscale(Q<int8_t>(), 512, Q<float>(), Q<uint8_t>(), 256, Q<float>(), nullptr,
                                               0, 8, 512, P(), CR_BF16, 8, nullptr), CR_OK);
    expect("w4a8 small workspace", cr_linear_w4a8(P(), CR_BF16, 512, 0, 300, 512, Q<uint8_t>(), 256, Q<float>(), 8,
                                                  nullptr, P(), CR_BF16, 8, P(), cr_linear_w4a8_workspace_bytes(300, 512) - 1,
                                                  0, nullptr), CR_ERR_TOO_LARGE);
    expect("w4a8 i32 out", cr_linear_w4a8(P(), CR_BF16, 512, 0, 300, 512, Q<uint8_t>(), 256, Q<float>(), 8, nullptr,
                                          P(), CR_I32, 8, P(), 1 << 20, 0, nullptr), CR_ERR_UNSUPPORTED_DTYPE);
    expect("w4a8 empty", cr_linear_w4a8(nullptr, CR_BF16, 512, 0, 0, 512, Q<uint8_t>(), 256, Q<float>(), 8, nullptr,
                                        nullptr, CR_BF16, 8, nullptr, 0, 0, nullptr), CR_OK);
    // W4A4
    expect("aw4 ld_s4 < K_pad/2", cr_quant_act_w4(P(), CR_BF16, 512, 0, 8, 512, Q<uint8_t>(), 240, Q<float>(), 0,
                                                  nullptr), CR_ERR_INVALID_ARG);
    expect("aw4 swiglu ld_x < 2K", cr_quant_act_w4(P(), CR_BF16, 1000, 1, 8, 512, Q<uint8_t>(), 256, Q<float>(), 0,
                                                   nullptr), CR_ERR_INVALID_ARG);
    expect("aw4 dtype", cr_quant_act_w4(P(), CR_I32, 512, 0, 8, 512, Q<uint8_t>(), 256, Q<float>(), 0, nullptr),
           CR_ERR_UNSUPPORTED_DTYPE);
    expect("aw4 empty", cr_quant_act_w4(nullptr, CR_BF16, 512, 0, 0, 512, nullptr, 256, nullptr, 0, nullptr), CR_OK);
    expect("s4s4 lda < K_pad/2", cr_gemm_s4s4_rowscale(Q<uint8_t>(), 240, Q<float>(), Q<uint8_t>(), 256, Q<float>(),
                                                       nullptr, 8, 8, 512, P(), CR_BF16, 8, nullptr),
           CR_ERR_INVALID_ARG);
    expect("s4s4 misaligned lda", cr_gemm_s4s4_rowscale(Q<uint8_t>(), 264, Q<float>(), Q<uint8_t>(), 256,
                                                        Q<float>(), nullptr, 8, 8, 512, P(), CR_BF16, 8, nullptr),
           CR_ERR_MISALIGNED);
    expect("s4s4 bias on i32", cr_gemm_s4s4_rowscale(Q<uint8_t>(), 256, Q<float>(), Q<uint8_t>(), 256, Q<float>(),
                                                     Q<float>(), 8, 8, 512, P(), CR_I32, 8, nullptr),
           CR_ERR_INVALID_ARG);
    expect("s4s4 empty", cr_gemm_s4s4_rowscale(Q<uint8_t>(), 256, Q<float>(), Q<uint8_t>(), 256, Q<float>(), nullptr,
                                               8, 0, 512, P(), CR_BF16, 8, nullptr), CR_OK);
    expect("w4a4 small workspace", cr_linear_w4a4(P(), CR_BF16, 512, 0, 300, 512, Q<uint8_t>(), 256, Q<float>(), 8,
                                                  nullptr, P(), CR_BF16, 8, P(), cr_linear_w4a4_workspace_bytes(300, 512) - 1,
                                                  0, nullptr), CR_ERR_TOO_LARGE);
    expect("w4a4 i32 out", cr_linear_w4a4(P(), CR_BF16, 512, 0, 300, 512, Q<uint8_t>(), 256, Q<float>(), 8, nullptr,
                                          P(), CR_I32, 8, P(), 1 << 20, 0, nullptr), CR_ERR_UNSUPPORTED_DTYPE);
    expect("w4a4 empty", cr_linear_w4a4(nullptr, CR_BF16, 512, 0, 0, 512, Q<uint8_t>(), 256, Q<float>(), 8, nullptr,
                                        nullptr, CR_BF16, 8, nullptr, 0, 0, nullptr), CR_OK);
    // W4A4, E2M3 form: quads of rows, 3 K_pad bytes each
    expect("f6w ld_f6 < 3K_pad", cr_quant_weight_w4_e2m3(P(), CR_FP32, 512, 8, 512, Q<uint8_t>(), 1520, Q<float>(), 0,
                                                        nullptr), CR_ERR_INVALID_ARG);
    expect("f6w misaligned ld", cr_quant_weight_w4_e2m3(P(), CR_FP32, 512, 8, 512, Q<uint8_t>(), 1544, Q<float>(), 0,
                                                        nullptr), CR_ERR_MISALIGNED);
    expect("f6w empty", cr_quant_weight_w4_e2m3(nullptr, CR_FP32, 512, 0, 512, nullptr, 1536, nullptr, 0, nullptr),
           CR_OK);
    expect("f6a swiglu ld_x < 2K", cr_quant_act_w4_e2m3(P(), CR_BF16, 1000, 1, 8, 512, Q<uint8_t>(), 1536, Q<float>(),
                                                        0, nullptr), CR_ERR_INVALID_ARG);
    expect("f6a dtype", cr_quant_act_w4_e2m3(P(), CR_I32, 512, 0, 8, 512, Q<uint8_t>(), 1536, Q<float>(), 0, nullptr),
           CR_ERR_UNSUPPORTED_DTYPE);
    expect("f6 gemm lda < 3K_pad", cr_gemm_e2m3_rowscale(Q<uint8_t>(), 1520, Q<float>(), Q<uint8_t>(), 1536,
                                                         Q<float>(), nullptr, 8, 8, 512, P(), CR_BF16, 8, nullptr),
           CR_ERR_INVALID_ARG);
    expect("f6 gemm bias on i32", cr_gemm_e2m3_rowscale(Q<uint8_t>(), 1536, Q<float>(), Q<uint8_t>(), 1536, Q<float>(),
                                                        Q<float>(), 8, 8, 512, P(), CR_I32, 8, nullptr),
           CR_ERR_INVALID_ARG);
    expect("f6 gemm K_pad not a multiple of 256", cr_gemm_e2m3_rowscale(Q<uint8_t>(), 1536, Q<float>(), Q<uint8_t>(),
                                                                        1536, Q<float>(), nullptr, 8, 8, 500, P(),
                                                                        CR_BF16, 8, nullptr), CR_ERR_INVALID_ARG);
    expect("f6 layer small workspace",
           cr_linear_w4a4_e2m3(P(), CR_BF16, 512, 0, 300, 512, Q<uint8_t>(), 1536, Q<float>(), 8, nullptr, P(), CR_BF16,
                               8, P(), cr_linear_w4a4_e2m3_workspace_bytes(300, 512) - 1, 0, nullptr),
           CR_ERR_TOO_LARGE);
    expect("repack ld_f6 < 3K_pad", cr_repack_w4_e2m3(Q<uint8_t>(), 256, 8, 512, Q<uint8_t>(), 1520, nullptr),
           CR_ERR_INVALID_ARG);
    expect("repack K_pad not a multiple of 256", cr_repack_w4_e2m3(Q<uint8_t>(), 256, 8, 500, Q<uint8_t>(), 1536,
                                                                   nullptr), CR_ERR_INVALID_ARG);
    expect("repack empty", cr_repack_w4_e2m3(nullptr, 256, 0, 512, nullptr, 1536, nullptr), CR_OK);
    expect("f6 layer empty", cr_linear_w4a4_e2m3(nullptr, CR_BF16, 512, 0, 0, 512, Q<uint8_t>(), 1536, Q<float>(), 8,
                                                 nullptr, nullptr, CR_BF16, 8, nullptr, 0, 0, nullptr), CR_OK);
    auto na = [&](int64_t M, int64_t N, int64_t K, size_t mt) {
        return cr_linear_nvfp4_noalloc(P(), CR_BF16, 5376, 0, M, K, nullptr, Q<uint8_t>(), 2688, Q<uint8_t>(), 336,
                                       Q<float>(), N, nullptr, P(), CR_BF16, 21504, mt, 0, nullptr);
    };
    expect("noalloc activation beyond the scratch", na(19989, 21504, 5376, 0), CR_ERR_TOO_LARGE);
    expect("noalloc tiles beyond the scratch", na(4096, 21504, 5376, (size_t)64 << 20), CR_ERR_TOO_LARGE);
    expect("noalloc empty", na(0, 21504, 5376, 0), CR_OK);
    expect("noalloc negative", na(-1, 21504, 5376, 0), CR_ERR_INVALID_ARG);
    if (ndev == 0) {
        expect("noalloc without a device", na(4096, 21504, 5376, 0), CR_ERR_NO_DEVICE);
        expect("w4a8 without a device", cr_linear_w4a8(P(), CR_BF16, 512, 0, 300, 512, Q<uint8_t>(), 256, Q<float>(),
                                                       8, nullptr, P(), CR_BF16, 8, P(), 1 << 20, 0, nullptr),
               CR_ERR_NO_DEVICE);
        expect("w4a4 without a device", cr_linear_w4a4(P(), CR_BF16, 512, 0, 300, 512, Q<uint8_t>(), 256, Q<float>(),
                                                       8, nullptr, P(), CR_BF16, 8, P(), 1 << 20, 0, nullptr),
               CR_ERR_NO_DEVICE);
        expect("f6 layer without a device",
               cr_linear_w4a4_e2m3(P(), CR_BF16, 512, 0, 300, 512, Q<uint8_t>(), 1536, Q<float>(), 8, nullptr, P(),
                                   CR_BF16, 8, P(), 1 << 20, 0, nullptr), CR_ERR_NO_DEVICE);
        expect("aw4 without a device", cr_quant_act_w4(P(), CR_BF16, 512, 0, 8, 512, Q<uint8_t>(), 256, Q<float>(), 0,
                                                       nullptr), CR_ERR_NO_DEVICE);
        expect("layer without a device", lin(300, 1000, 5376, CR_BF16, need, P()), CR_ERR_NO_DEVICE);
        expect("qa without a device", qa(P(), 0, 512, 4, 512, P(), 512, P(), 0), CR_ERR_NO_DEVICE);
    }
    if (failures) return 1;
    std::printf("C ABI host validation under sanitizers: ok\n");
    return 0;
}
