// C ABI of the rotated W8A8 NVFP4 linear layer: argument validation, device checks,
// launch configuration and the bounded-staging layer orchestration.
//
// Layer orchestration (ComfyUI Turing Utils README, "Load ConvRot DiT ..." bullet):
// the activation is prepared once; the weight is prepared in chunks of output rows into
// call-local S8 tiles of bounded size (two tiles alternate), each chunk followed by the
// GEMM that writes its column band of the output; with a second stream and several
// chunks, the preparation of chunk c+1 runs beside the GEMM of chunk c, ordered by
// producer/consumer events.  Short batches skip the S8 weight altogether: the GEMM decodes
// the weight blocks itself (decode-inside-GEMM).  Chunking, streams and the path taken
// change no value.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/convrot.h"
#include "kernels.hpp"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other (read-only cache)

cr_status current_device_ok()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return CR_ERR_NO_DEVICE;
    }
    int s = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (s == 0) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess) {
            (void)hipGetLastError();
            return CR_ERR_NO_DEVICE;
        }
        s = (std::strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_arch_ok[dev].store(s, std::memory_order_relaxed);
    }
    return s == 1 ? CR_OK : CR_ERR_NO_DEVICE;
}

inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

inline int64_t elem_size(cr_dtype d)
{
    switch (d) {
    case CR_BF16: case CR_FP16: return 2;
    case CR_FP32: case CR_I32: return 4;
    default: return 0;
    }
}

inline cr_status from_hip(hipError_t e) { return e == hipSuccess ? CR_OK : CR_ERR_LAUNCH; }

constexpr int64_t kMaxRows = 0x7fffffff;

inline int64_t pad256(int64_t k) { return ((k + 255) / 256) * 256; }

cr_status check_flags(uint32_t flags)
{
    return (flags & ~(uint32_t)(CR_FLAG_FORCE_TWO_PASS | CR_FLAG_BLOCK_TRANSPOSED)) ? CR_ERR_INVALID_ARG : CR_OK;
}

cr_status check_act(const void *x, cr_dtype dt, int64_t ld_x, int64_t M, int64_t K, int64_t cols,
                    int8_t *x_s8, int64_t ld_s8, float *x_scale, uint32_t flags)
{
    if (M > 0 && (!x || !x_s8 || !x_scale)) return CR_ERR_INVALID_ARG;   // M = 0: nothing is read or written
    if (dt != CR_BF16 && dt != CR_FP16 && dt != CR_FP32) return CR_ERR_UNSUPPORTED_DTYPE;
    if (M < 0 || K < 1 || M > kMaxRows) return CR_ERR_INVALID_ARG;
    if (check_flags(flags) != CR_OK) return CR_ERR_INVALID_ARG;
    const int64_t kp = pad256(K);
    if (kp > CR_MAX_K_PAD) return CR_ERR_TOO_LARGE;
    if (ld_x < cols || ld_s8 < kp) return CR_ERR_INVALID_ARG;
    const int64_t es = elem_size(dt);
    if (!aligned(x, 16) || (ld_x * es) % 16 != 0) return CR_ERR_MISALIGNED;
    if (!aligned(x_s8, 16) || ld_s8 % 16 != 0 || !aligned(x_scale, 4)) return CR_ERR_MISALIGNED;
    return CR_OK;
}

cr_status check_weight(const uint8_t *w_fp4, int64_t ld_fp4, const uint8_t *w_sf, int64_t ld_sf,
                       const float *g, int64_t n_rows, int64_t K, int8_t *w_s8, int64_t ld_s8,
                       float *w_scale, uint32_t flags)
{
    if (n_rows > 0 && (!w_fp4 || !w_sf || !g || !w_s8 || !w_scale)) return CR_ERR_INVALID_ARG;
    if (n_rows < 0 || K < 1 || n_rows > kMaxRows) return CR_ERR_INVALID_ARG;
    if (check_flags(flags) != CR_OK) return CR_ERR_INVALID_ARG;
    const int64_t kp = pad256(K);
    if (kp > CR_MAX_K_PAD) return CR_ERR_TOO_LARGE;
    if (ld_fp4 < (K + 1) / 2 || ld_sf < (K + 15) / 16 || ld_s8 < kp) return CR_ERR_INVALID_ARG;
    if (!aligned(w_fp4, 16) || ld_fp4 % 16 != 0) return CR_ERR_MISALIGNED;
    if (!aligned(g, 4) || !aligned(w_scale, 4)) return CR_ERR_MISALIGNED;
    if (!aligned(w_s8, 16) || ld_s8 % 16 != 0) return CR_ERR_MISALIGNED;
    return CR_OK;
}

cr_status check_gemm(const int8_t *a, int64_t lda, const float *sa, const int8_t *b, int64_t ldb,
                     const float *sb, int64_t M, int64_t N, int64_t K_pad, void *c, cr_dtype cdt,
                     int64_t ldc)
{
    if ((M > 0 && !a) || (N > 0 && !b) || (M > 0 && N > 0 && !c)) return CR_ERR_INVALID_ARG;
    if (cdt != CR_BF16 && cdt != CR_FP16 && cdt != CR_FP32 && cdt != CR_I32) return CR_ERR_UNSUPPORTED_DTYPE;
    if (cdt != CR_I32 && ((M > 0 && !sa) || (N > 0 && !sb))) return CR_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || K_pad < 1 || K_pad % 256 != 0) return CR_ERR_INVALID_ARG;
    if (M > kMaxRows || N > kMaxRows) return CR_ERR_INVALID_ARG;
    // one workgroup of 512 threads per 256 x 256 tile; a dispatch counts work-items in 32 bits
    if (((M + 255) / 256) * ((N + 255) / 256) > (int64_t)(UINT32_MAX / 512)) return CR_ERR_TOO_LARGE;
    if (K_pad > CR_MAX_K_PAD) return CR_ERR_TOO_LARGE;
    if (lda < K_pad || ldb < K_pad || ldc < N) return CR_ERR_INVALID_ARG;
    if (!aligned(a, 16) || !aligned(b, 16) || lda % 16 != 0 || ldb % 16 != 0) return CR_ERR_MISALIGNED;
    if (!aligned(c, (size_t)elem_size(cdt))) return CR_ERR_MISALIGNED;
    if ((sa && !aligned(sa, 4)) || (sb && !aligned(sb, 4))) return CR_ERR_MISALIGNED;
    return CR_OK;
}

cr_status check_fused(const int8_t *a_s8, int64_t lda, const float *a_scale, const uint8_t *w_fp4,
                      int64_t ld_fp4, const uint8_t *w_sf, int64_t ld_sf, const float *g, const float *w_amax,
                      const float *bias, int64_t M, int64_t N, int64_t K, void *c, cr_dtype c_dtype, int64_t ldc,
                      uint32_t flags)
{
    if ((M > 0 && !a_s8) || (N > 0 && (!w_fp4 || !w_sf || !g)) || (M > 0 && N > 0 && !c)) return CR_ERR_INVALID_ARG;
    if (c_dtype != CR_BF16 && c_dtype != CR_FP16 && c_dtype != CR_FP32 && c_dtype != CR_I32)
        return CR_ERR_UNSUPPORTED_DTYPE;
    if (c_dtype != CR_I32 && M > 0 && !a_scale) return CR_ERR_INVALID_ARG;
    if (bias && c_dtype == CR_I32) return CR_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || K < 1 || M > kMaxRows || N > kMaxRows) return CR_ERR_INVALID_ARG;
    if (check_flags(flags) != CR_OK) return CR_ERR_INVALID_ARG;
    const int64_t kp = pad256(K);
    if (kp > CR_MAX_K_PAD) return CR_ERR_TOO_LARGE;
    if ((M + 127) / 128 > 65535) return CR_ERR_TOO_LARGE;
    if ((N + 31) / 32 > (int64_t)(UINT32_MAX / 256)) return CR_ERR_TOO_LARGE;   // 32-bit work-item count
    if (lda < kp || ld_fp4 < (K + 1) / 2 || ld_sf < (K + 15) / 16 || ldc < N) return CR_ERR_INVALID_ARG;
    if (!aligned(a_s8, 16) || lda % 16 != 0) return CR_ERR_MISALIGNED;
    if (!aligned(w_fp4, 16) || ld_fp4 % 16 != 0) return CR_ERR_MISALIGNED;
    if (!aligned(g, 4) || (w_amax && !aligned(w_amax, 4))) return CR_ERR_MISALIGNED;
    if ((a_scale && !aligned(a_scale, 4)) || (bias && !aligned(bias, 4))) return CR_ERR_MISALIGNED;
    if (!aligned(c, (size_t)elem_size(c_dtype))) return CR_ERR_MISALIGNED;
    return CR_OK;
}

// Batches of at most this many activation rows run the layer with the weight decoded
// inside the GEMM (cr_gemm_nvfp4_fused, row maxima from its own first pass) instead of
// staging S8 weight tiles: with so few rows the decode dominates either way, and the
// staged path adds the S8 write and read of the whole weight and a GEMM with few tiles.
constexpr int64_t kFusedMaxRows = 64;

// Workspace layout of cr_linear_nvfp4 (every region 256-byte aligned):
//   staged: x_s8 [M, K_pad] | x_scale [M] | tile0 [R, K_pad] | tscale0 [R] | tile1 | tscale1
//   fused:  x_s8 [M, K_pad] | x_scale [M]
struct LayerPlan {
    bool fused;
    int64_t K_pad, R, nchunks;
    size_t off_xscale, off_tile[2], off_tscale[2], bytes;
};

inline size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

int current_cus()
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
        (void)hipGetLastError();
        return 256;
    }
    return cus;
}

// Rows per weight chunk, a multiple of the GEMM tile height.  The chunks' GEMMs run one
// after another, so each pays for whole rounds of workgroups over the CUs: a GEMM of
// t tiles takes ceil(t / cus) rounds.
// * When the tile bound forces several chunks, the chunk height within the bound is the
//   one whose GEMMs need the fewest rounds in total (the tallest of those on a tie).  With
//   M = 19989 (79 tile rows) and a 16 MiB bound on K_pad = 14336, 1024-row chunks would be
//   316-tile GEMMs of two rounds each (11 rounds for 5376 rows); 768-row chunks are
//   237-tile GEMMs of one round (7 rounds, as many as one unchunked GEMM).
// * When the whole weight fits one chunk it is still split in two whenever the two GEMMs
//   together need no more rounds than one GEMM would: with a second stream the second
//   chunk's preparation can then overlap the first chunk's GEMM, and staged serially the
//   split costs nothing (QKV at M = 19989: 1.93-1.95 ms for the two GEMMs against 1.94 ms
//   for one over the whole weight, same operands).
int64_t plan_rows(int64_t M, int64_t N, int64_t K_pad, size_t max_tile_bytes, int cus)
{
    const int64_t T = convrot::kGemmTileRows;
    int64_t kmax = (int64_t)(max_tile_bytes / (size_t)K_pad) / T;   // tile rows per chunk
    if (kmax < 1) kmax = 1;
    const int64_t tiles_n = (N + T - 1) / T;
    const int64_t tiles_m = (M + convrot::kGemmTileCols - 1) / convrot::kGemmTileCols;
    auto rounds = [&](int64_t tiles) { return (tiles + cus - 1) / cus; };
    if (kmax < tiles_n) {                               // chunked by the bound
        int64_t best_k = kmax, best = -1;
        for (int64_t k = kmax; k >= 1 && kmax - k < 4096; k--) {   // host time stays bounded
            const int64_t rem = tiles_n % k;
            const int64_t r = (tiles_n / k) * rounds(tiles_m * k) + (rem ? rounds(tiles_m * rem) : 0);
            if (best < 0 || r < best) { best = r; best_k = k; }
        }
        return best_k * T;
    }
    if (tiles_n < 2) return tiles_n * T;
    const int64_t t0 = (tiles_n + 1) / 2, t1 = tiles_n - t0;
    if (rounds(tiles_m * t0) + rounds(tiles_m * t1) <= rounds(tiles_m * tiles_n)) return t0 * T;
    return tiles_n * T;
}

LayerPlan plan_layer(int64_t M, int64_t N, int64_t K, size_t max_tile_bytes)
{
    LayerPlan p{};
    if (max_tile_bytes == 0) max_tile_bytes = CR_DEFAULT_MAX_TILE_BYTES;
    p.K_pad = pad256(K);
    if (M == 0 || N == 0) return p;                  // empty: no chunks, no workspace
    if (M <= kFusedMaxRows) {
        p.fused = true;
        p.off_xscale = up256((size_t)M * (size_t)p.K_pad);
        p.bytes = up256(p.off_xscale + (size_t)M * 4);
        return p;
    }
    p.R = plan_rows(M, N, p.K_pad, max_tile_bytes, current_cus());
    p.nchunks = (N + p.R - 1) / p.R;
    size_t off = up256((size_t)M * (size_t)p.K_pad);
    p.off_xscale = off;
    off = up256(off + (size_t)M * 4);
    const int ntiles = p.nchunks > 1 ? 2 : 1;
    for (int t = 0; t < 2; t++) {
        p.off_tile[t] = off;
        p.off_tscale[t] = up256(off + (size_t)p.R * (size_t)p.K_pad);
        if (t < ntiles) off = up256(p.off_tscale[t] + (size_t)p.R * 4);
    }
    p.bytes = off;
    return p;
}

// Events that order the staging stream against the main stream.  A layer call takes one
// set from a per-device pool and returns it once its work is enqueued: a wait enqueued on a
// stream refers to the event's most recent record at the time of the wait, so a set can be
// recorded again by the next call (on this thread or another) while earlier work is still
// in flight.  Sets are created on first need (as many as there are concurrent callers) and
// kept until the process ends; the pool is guarded by a mutex.
struct EventSet {
    hipEvent_t ev[5] = {nullptr, nullptr, nullptr, nullptr, nullptr};
};

std::mutex g_event_mu;
std::vector<EventSet *> g_event_pool[kMaxDevices];

class PooledEvents {
public:
    explicit PooledEvents(bool want)
    {
        if (!want) return;
        if (hipGetDevice(&dev_) != hipSuccess || dev_ < 0 || dev_ >= kMaxDevices) {
            (void)hipGetLastError();
            dev_ = -1;
            return;
        }
        {
            std::lock_guard<std::mutex> lk(g_event_mu);
            auto &pool = g_event_pool[dev_];
            if (!pool.empty()) {
                set_ = pool.back();
                pool.pop_back();
                return;
            }
        }
        auto *s = new (std::nothrow) EventSet;
        if (!s) return;
        for (auto &e : s->ev)
            if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
                (void)hipGetLastError();
                for (auto &d : s->ev)
                    if (d) (void)hipEventDestroy(d);
                delete s;
                return;
            }
        set_ = s;
    }
    ~PooledEvents()
    {
        if (!set_) return;
        std::lock_guard<std::mutex> lk(g_event_mu);
        g_event_pool[dev_].push_back(set_);
    }
    PooledEvents(const PooledEvents &) = delete;
    PooledEvents &operator=(const PooledEvents &) = delete;
    bool ok() const { return set_ != nullptr; }
    hipEvent_t operator[](int i) const { return set_->ev[i]; }

private:
    int dev_ = -1;
    EventSet *set_ = nullptr;
};

// Device scratch of cr_linear_nvfp4_noalloc: the layer's workspace for callers that cannot
// allocate.  One copy per GPU, created with the code object and held until the process
// ends.  In host code `scratch` names a host-side stand-in, not device memory: only the
// address that hipGetSymbolAddress returns for the current device may reach a kernel.
static __device__ __align__(256) int8_t scratch[CR_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device (guarded)

// The current device's copy of `scratch`, resolved on the first call on that device (with
// that device current) and kept.
cr_status scratch_for_current_device(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return CR_ERR_NO_DEVICE;
    }
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return CR_ERR_LAUNCH;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return CR_OK;
}

// The tile bound cr_linear_nvfp4_noalloc uses when the caller passes 0: the largest one for
// which the activation and two S8 weight tiles (with their scales) fit the scratch; 0 when
// not even the activation and two 256-row tiles fit.
size_t noalloc_tile_bound(int64_t M, int64_t K)
{
    const int64_t kp = pad256(K);
    const size_t act = up256((size_t)M * (size_t)kp) + up256((size_t)M * 4);
    if (act + 512 >= CR_NOALLOC_SCRATCH_BYTES) return 0;
    const size_t rem = CR_NOALLOC_SCRATCH_BYTES - act - 512;
    const int64_t T = convrot::kGemmTileRows;
    const int64_t rows = (int64_t)(rem / (2 * ((size_t)kp + 4))) / T * T;
    return rows < T ? 0 : (size_t)rows * (size_t)kp;
}

}  // namespace

extern "C" {

int cr_abi_version(void) { return CR_ABI_VERSION; }

const char *cr_status_string(cr_status s)
{
    switch (s) {
    case CR_OK: return "CR_OK";
    case CR_ERR_INVALID_ARG: return "CR_ERR_INVALID_ARG";
    case CR_ERR_UNSUPPORTED_DTYPE: return "CR_ERR_UNSUPPORTED_DTYPE";
    case CR_ERR_MISALIGNED: return "CR_ERR_MISALIGNED";
    case CR_ERR_TOO_LARGE: return "CR_ERR_TOO_LARGE";
    case CR_ERR_NO_DEVICE: return "CR_ERR_NO_DEVICE";
    case CR_ERR_LAUNCH: return "CR_ERR_LAUNCH";
    default: return "CR_ERR_UNKNOWN";
    }
}

int64_t cr_padded_k(int64_t k) { return k < 1 ? 0 : pad256(k); }

cr_status cr_prep_weight_nvfp4(const uint8_t *w_fp4, int64_t ld_fp4, const uint8_t *w_sf, int64_t ld_sf,
                               const float *global_scale, int64_t n_rows, int64_t K,
                               int8_t *w_s8, int64_t ld_s8, float *w_scale,
                               uint32_t flags, hipStream_t stream)
{
    cr_status s = check_weight(w_fp4, ld_fp4, w_sf, ld_sf, global_scale, n_rows, K, w_s8, ld_s8, w_scale, flags);
    if (s != CR_OK || n_rows == 0) return s;
    if ((s = current_device_ok()) != CR_OK) return s;
    return from_hip(convrot::launch_prep_weight(w_fp4, ld_fp4, w_sf, ld_sf, global_scale, n_rows, K, w_s8,
                                                ld_s8, w_scale, (flags & CR_FLAG_FORCE_TWO_PASS) != 0,
                                                (flags & CR_FLAG_BLOCK_TRANSPOSED) != 0, stream));
}

cr_status cr_quant_act_ex(const void *x, cr_dtype x_dtype, int64_t ld_x, int swiglu, int64_t M, int64_t K,
                          const float *pre_scale, int8_t *x_s8, int64_t ld_s8, float *x_scale,
                          uint32_t flags, hipStream_t stream)
{
    if (swiglu && K > (int64_t)1 << 40) return CR_ERR_TOO_LARGE;
    cr_status s = check_act(x, x_dtype, ld_x, M, K, swiglu ? 2 * K : K, x_s8, ld_s8, x_scale, flags);
    if (s != CR_OK) return s;
    if (pre_scale && !aligned(pre_scale, 4)) return CR_ERR_MISALIGNED;
    if (M == 0) return CR_OK;
    if ((s = current_device_ok()) != CR_OK) return s;
    const bool tp = (flags & CR_FLAG_FORCE_TWO_PASS) != 0;
    const bool tr = (flags & CR_FLAG_BLOCK_TRANSPOSED) != 0;
    return from_hip(swiglu
        ? convrot::launch_quant_act_swiglu(x, (int)x_dtype, ld_x, M, K, pre_scale, x_s8, ld_s8, x_scale, tp, tr, stream)
        : convrot::launch_quant_act(x, (int)x_dtype, ld_x, M, K, pre_scale, x_s8, ld_s8, x_scale, tp, tr, stream));
}

cr_status cr_quant_act(const void *x, cr_dtype x_dtype, int64_t ld_x, int64_t M, int64_t K,
                       int8_t *x_s8, int64_t ld_s8, float *x_scale, uint32_t flags, hipStream_t stream)
{
    return cr_quant_act_ex(x, x_dtype, ld_x, 0, M, K, nullptr, x_s8, ld_s8, x_scale, flags, stream);
}

cr_status cr_quant_act_swiglu(const void *h, cr_dtype h_dtype, int64_t ld_h, int64_t M, int64_t F,
                              int8_t *x_s8, int64_t ld_s8, float *x_scale, uint32_t flags, hipStream_t stream)
{
    return cr_quant_act_ex(h, h_dtype, ld_h, 1, M, F, nullptr, x_s8, ld_s8, x_scale, flags, stream);
}

cr_status cr_swiglu(const void *h, cr_dtype h_dtype, int64_t ld_h, int64_t M, int64_t F,
                    float *out, int64_t ld_out, hipStream_t stream)
{
    if (M > 0 && (!h || !out)) return CR_ERR_INVALID_ARG;
    if (h_dtype != CR_BF16 && h_dtype != CR_FP16 && h_dtype != CR_FP32) return CR_ERR_UNSUPPORTED_DTYPE;
    if (M < 0 || F < 1 || F > ((int64_t)1 << 40) || M > ((int64_t)1 << 40) / F) return CR_ERR_INVALID_ARG;
    if (ld_h < 2 * F || ld_out < F) return CR_ERR_INVALID_ARG;
    if (!aligned(h, (size_t)elem_size(h_dtype)) || !aligned(out, 4)) return CR_ERR_MISALIGNED;
    if (M == 0) return CR_OK;
    cr_status s = current_device_ok();
    if (s != CR_OK) return s;
    return from_hip(convrot::launch_swiglu(h, (int)h_dtype, ld_h, M, F, out, ld_out, stream));
}

cr_status cr_gemm_s8_rowscale_bias(const int8_t *a_s8, int64_t lda, const float *a_scale,
                                   const int8_t *b_s8, int64_t ldb, const float *b_scale,
                                   const float *bias, int64_t M, int64_t N, int64_t K_pad,
                                   void *c, cr_dtype c_dtype, int64_t ldc, hipStream_t stream)
{
    cr_status s = check_gemm(a_s8, lda, a_scale, b_s8, ldb, b_scale, M, N, K_pad, c, c_dtype, ldc);
    if (s != CR_OK) return s;
    if (bias && c_dtype == CR_I32) return CR_ERR_INVALID_ARG;
    if (bias && !aligned(bias, 4)) return CR_ERR_MISALIGNED;
    if (M == 0 || N == 0) return CR_OK;
    if ((s = current_device_ok()) != CR_OK) return s;
    return from_hip(convrot::launch_gemm_s8(a_s8, lda, a_scale, b_s8, ldb, b_scale, bias, M, N, K_pad, c,
                                            (int)c_dtype, ldc, stream));
}

cr_status cr_gemm_s8_rowscale(const int8_t *a_s8, int64_t lda, const float *a_scale,
                              const int8_t *b_s8, int64_t ldb, const float *b_scale,
                              int64_t M, int64_t N, int64_t K_pad,
                              void *c, cr_dtype c_dtype, int64_t ldc, hipStream_t stream)
{
    return cr_gemm_s8_rowscale_bias(a_s8, lda, a_scale, b_s8, ldb, b_scale, nullptr, M, N, K_pad, c,
                                    c_dtype, ldc, stream);
}

cr_status cr_weight_amax_nvfp4(const uint8_t *w_fp4, int64_t ld_fp4, const uint8_t *w_sf, int64_t ld_sf,
                               const float *global_scale, int64_t n_rows, int64_t K, float *w_amax,
                               uint32_t flags, hipStream_t stream)
{
    if (n_rows > 0 && (!w_fp4 || !w_sf || !global_scale || !w_amax)) return CR_ERR_INVALID_ARG;
    if (n_rows < 0 || K < 1 || n_rows > kMaxRows) return CR_ERR_INVALID_ARG;
    if (check_flags(flags) != CR_OK) return CR_ERR_INVALID_ARG;
    if (pad256(K) > CR_MAX_K_PAD) return CR_ERR_TOO_LARGE;
    if (ld_fp4 < (K + 1) / 2 || ld_sf < (K + 15) / 16) return CR_ERR_INVALID_ARG;
    if (!aligned(w_fp4, 16) || ld_fp4 % 16 != 0) return CR_ERR_MISALIGNED;
    if (!aligned(global_scale, 4) || !aligned(w_amax, 4)) return CR_ERR_MISALIGNED;
    if (n_rows == 0) return CR_OK;
    cr_status s = current_device_ok();
    if (s != CR_OK) return s;
    return from_hip(convrot::launch_weight_amax(w_fp4, ld_fp4, w_sf, ld_sf, global_scale, n_rows, K, w_amax,
                                                (flags & CR_FLAG_FORCE_TWO_PASS) != 0, stream));
}

cr_status cr_gemm_nvfp4_fused(const int8_t *a_s8, int64_t lda, const float *a_scale,
                              const uint8_t *w_fp4, int64_t ld_fp4, const uint8_t *w_sf, int64_t ld_sf,
                              const float *global_scale, const float *w_amax, const float *bias,
                              int64_t M, int64_t N, int64_t K, void *c, cr_dtype c_dtype, int64_t ldc,
                              uint32_t flags, hipStream_t stream)
{
    cr_status s0 = check_fused(a_s8, lda, a_scale, w_fp4, ld_fp4, w_sf, ld_sf, global_scale, w_amax, bias, M, N, K,
                               c, c_dtype, ldc, flags);
    if (s0 != CR_OK || M == 0 || N == 0) return s0;
    cr_status s = current_device_ok();
    if (s != CR_OK) return s;
    return from_hip(convrot::launch_gemm_nvfp4_fused(a_s8, lda, a_scale, w_fp4, ld_fp4, w_sf, ld_sf, global_scale,
                                                     w_amax, bias, M, N, K, c, (int)c_dtype, ldc,
                                                     (flags & CR_FLAG_BLOCK_TRANSPOSED) != 0, stream));
}

cr_status cr_linear_nvfp4_plan(int64_t M, int64_t N, int64_t K, size_t max_tile_bytes,
                               int64_t *rows_per_chunk, int64_t *nchunks)
{
    if (!rows_per_chunk || !nchunks) return CR_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || K < 1) return CR_ERR_INVALID_ARG;
    if (pad256(K) > CR_MAX_K_PAD) return CR_ERR_TOO_LARGE;
    const LayerPlan p = plan_layer(M, N, K, max_tile_bytes);
    *rows_per_chunk = p.R;
    *nchunks = p.nchunks;
    return CR_OK;
}

size_t cr_linear_nvfp4_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t max_tile_bytes)
{
    if (M < 1 || N < 1 || K < 1 || pad256(K) > CR_MAX_K_PAD) return 0;   // an empty layer needs none
    return plan_layer(M, N, K, max_tile_bytes).bytes;
}

cr_status cr_linear_nvfp4_ex(const void *x, cr_dtype x_dtype, int64_t ld_x, int swiglu,
                             int64_t M, int64_t K, const float *pre_scale,
                             const uint8_t *w_fp4, int64_t ld_fp4,
                             const uint8_t *w_sf, int64_t ld_sf, const float *global_scale,
                             int64_t N, const float *bias, void *out, cr_dtype out_dtype, int64_t ldc,
                             void *workspace, size_t ws_bytes, size_t max_tile_bytes,
                             uint32_t flags, hipStream_t s_main, hipStream_t s_aux)
{
    if (out_dtype == CR_I32) return CR_ERR_UNSUPPORTED_DTYPE;
    if (M < 0 || N < 0 || K < 1) return CR_ERR_INVALID_ARG;
    if (swiglu && K > (int64_t)1 << 40) return CR_ERR_TOO_LARGE;
    if (pad256(K) > CR_MAX_K_PAD) return CR_ERR_TOO_LARGE;
    if (M == 0 || N == 0) {
        // an empty layer: the arguments that do not depend on the empty extent are checked
        // as for any other call, and nothing is enqueued
        if (x_dtype != CR_BF16 && x_dtype != CR_FP16 && x_dtype != CR_FP32) return CR_ERR_UNSUPPORTED_DTYPE;
        if (out_dtype != CR_BF16 && out_dtype != CR_FP16 && out_dtype != CR_FP32) return CR_ERR_UNSUPPORTED_DTYPE;
        if (check_flags(flags) != CR_OK || ld_x < (swiglu ? 2 * K : K) || ldc < N) return CR_ERR_INVALID_ARG;
        if ((M > 0 && !x) || (N > 0 && (!w_fp4 || !w_sf || !global_scale))) return CR_ERR_INVALID_ARG;
        if (ld_fp4 < (K + 1) / 2 || ld_sf < (K + 15) / 16) return CR_ERR_INVALID_ARG;
        if (!aligned(x, 16) || (ld_x * elem_size(x_dtype)) % 16 != 0) return CR_ERR_MISALIGNED;
        if (!aligned(w_fp4, 16) || ld_fp4 % 16 != 0) return CR_ERR_MISALIGNED;
        return CR_OK;
    }
    if (!workspace || !out) return CR_ERR_INVALID_ARG;
    const LayerPlan p = plan_layer(M, N, K, max_tile_bytes);
    if (!aligned(workspace, 256)) return CR_ERR_MISALIGNED;
    if (ws_bytes < p.bytes) return CR_ERR_TOO_LARGE;
    int8_t *ws = static_cast<int8_t *>(workspace);
    int8_t *x_s8 = ws;
    float *x_scale = reinterpret_cast<float *>(ws + p.off_xscale);
    if (p.fused) {
        cr_status s = check_act(x, x_dtype, ld_x, M, K, swiglu ? 2 * K : K, x_s8, p.K_pad, x_scale, flags);
        if (s != CR_OK) return s;
        s = check_fused(x_s8, p.K_pad, x_scale, w_fp4, ld_fp4, w_sf, ld_sf, global_scale, nullptr, bias, M, N, K,
                        out, out_dtype, ldc, flags);
        if (s != CR_OK) return s;
        if (pre_scale && !aligned(pre_scale, 4)) return CR_ERR_MISALIGNED;
        if ((s = current_device_ok()) != CR_OK) return s;
        const bool tp = (flags & CR_FLAG_FORCE_TWO_PASS) != 0;
        // both launches on s_main: they are short, kernels running side by side on this
        // chip take as long as one after the other, and cross-stream waits would cost more
        // than the whole activation preparation
        hipError_t e = swiglu
            ? convrot::launch_quant_act_swiglu(x, (int)x_dtype, ld_x, M, K, pre_scale, x_s8, p.K_pad, x_scale, tp, true, s_main)
            : convrot::launch_quant_act(x, (int)x_dtype, ld_x, M, K, pre_scale, x_s8, p.K_pad, x_scale, tp, true, s_main);
        if (e != hipSuccess) return CR_ERR_LAUNCH;
        return from_hip(convrot::launch_gemm_nvfp4_fused(x_s8, p.K_pad, x_scale, w_fp4, ld_fp4, w_sf, ld_sf,
                                                         global_scale, nullptr, bias, M, N, K, out, (int)out_dtype,
                                                         ldc, true, s_main));
    }
    int8_t *tile[2] = {ws + p.off_tile[0], ws + p.off_tile[1]};
    float *tscale[2] = {reinterpret_cast<float *>(ws + p.off_tscale[0]),
                        reinterpret_cast<float *>(ws + p.off_tscale[1])};
    // validate every call of the plan before enqueueing anything
    cr_status s = check_act(x, x_dtype, ld_x, M, K, swiglu ? 2 * K : K, x_s8, p.K_pad, x_scale, flags);
    if (s != CR_OK) return s;
    s = check_weight(w_fp4, ld_fp4, w_sf, ld_sf, global_scale, p.R < N ? p.R : N, K, tile[0], p.K_pad,
                     tscale[0], flags);
    if (s != CR_OK) return s;
    s = check_gemm(x_s8, p.K_pad, x_scale, tile[0], p.K_pad, tscale[0], M, p.R < N ? p.R : N, p.K_pad,
                   out, out_dtype, ldc);
    if (s != CR_OK) return s;
    if ((pre_scale && !aligned(pre_scale, 4)) || (bias && !aligned(bias, 4))) return CR_ERR_MISALIGNED;
    if ((s = current_device_ok()) != CR_OK) return s;

    const bool tp = (flags & CR_FLAG_FORCE_TWO_PASS) != 0;
    const int64_t es = elem_size(out_dtype);
    // with a second stream and several chunks, chunk c+1 is prepared while chunk c
    // multiplies (and the first while the activation is prepared), the overlap a caller asks
    // for by passing s_aux.  On this chip it measured 1 % (two chunks) to 3.5 % (seven
    // chunks) slower than staging every chunk on s_main: a preparation kernel started beside
    // a running GEMM waits for the compute units the GEMM holds and delays the next GEMM's
    // workgroups.  A single chunk has only the activation preparation to run beside, which
    // gains nothing either, while the two cross-stream waits cost about as much as a small
    // layer's activation preparation.
    const bool overlap = s_aux != nullptr && s_aux != s_main && p.nchunks > 1;
    PooledEvents evs(overlap);
    if (overlap && !evs.ok()) return CR_ERR_LAUNCH;
    hipEvent_t ev_start = nullptr, ev_prep[2] = {nullptr, nullptr}, ev_gemm[2] = {nullptr, nullptr};
    if (overlap) {
        ev_start = evs[0];
        ev_prep[0] = evs[1]; ev_prep[1] = evs[2];
        ev_gemm[0] = evs[3]; ev_gemm[1] = evs[4];
    }

    if (overlap) {
        // the staging stream must not run ahead of work already queued on s_main
        if (hipEventRecord(ev_start, s_main) != hipSuccess) return CR_ERR_LAUNCH;
        if (hipStreamWaitEvent(s_aux, ev_start, 0) != hipSuccess) return CR_ERR_LAUNCH;
    }
    // both S8 operands live only in the workspace: they use the block-transposed column
    // order, which skips one LDS transposition per block and leaves every int32 sum as is
    hipError_t e = swiglu
        ? convrot::launch_quant_act_swiglu(x, (int)x_dtype, ld_x, M, K, pre_scale, x_s8, p.K_pad, x_scale, tp, true, s_main)
        : convrot::launch_quant_act(x, (int)x_dtype, ld_x, M, K, pre_scale, x_s8, p.K_pad, x_scale, tp, true, s_main);
    if (e != hipSuccess) return CR_ERR_LAUNCH;

    for (int64_t c = 0; c < p.nchunks; c++) {
        const int b = (int)(c & 1);
        const int64_t n0 = c * p.R;
        const int64_t rows = (N - n0) < p.R ? (N - n0) : p.R;
        hipStream_t sp = overlap ? s_aux : s_main;
        if (overlap && c >= 2 && hipStreamWaitEvent(s_aux, ev_gemm[b], 0) != hipSuccess) return CR_ERR_LAUNCH;
        e = convrot::launch_prep_weight(w_fp4 + n0 * ld_fp4, ld_fp4, w_sf + n0 * ld_sf, ld_sf, global_scale,
                                        rows, K, tile[b], p.K_pad, tscale[b], tp, true, sp);
        if (e != hipSuccess) return CR_ERR_LAUNCH;
        if (overlap) {
            if (hipEventRecord(ev_prep[b], s_aux) != hipSuccess) return CR_ERR_LAUNCH;
            if (hipStreamWaitEvent(s_main, ev_prep[b], 0) != hipSuccess) return CR_ERR_LAUNCH;
        }
        e = convrot::launch_gemm_s8(x_s8, p.K_pad, x_scale, tile[b], p.K_pad, tscale[b],
                                    bias ? bias + n0 : nullptr, M, rows, p.K_pad,
                                    static_cast<int8_t *>(out) + n0 * es, (int)out_dtype, ldc, s_main);
        if (e != hipSuccess) return CR_ERR_LAUNCH;
        if (overlap && hipEventRecord(ev_gemm[b], s_main) != hipSuccess) return CR_ERR_LAUNCH;
    }
    return CR_OK;
}

cr_status cr_linear_nvfp4(const void *x, cr_dtype x_dtype, int64_t ld_x, int swiglu,
                          int64_t M, int64_t K,
                          const uint8_t *w_fp4, int64_t ld_fp4,
                          const uint8_t *w_sf, int64_t ld_sf, const float *global_scale,
                          int64_t N, void *out, cr_dtype out_dtype, int64_t ldc,
                          void *workspace, size_t ws_bytes, size_t max_tile_bytes,
                          uint32_t flags, hipStream_t s_main, hipStream_t s_aux)
{
    return cr_linear_nvfp4_ex(x, x_dtype, ld_x, swiglu, M, K, nullptr, w_fp4, ld_fp4, w_sf, ld_sf,
                              global_scale, N, nullptr, out, out_dtype, ldc, workspace, ws_bytes,
                              max_tile_bytes, flags, s_main, s_aux);
}

cr_status cr_quant_weight_w4(const void *w, cr_dtype w_dtype, int64_t ld_w, int64_t N, int64_t K,
                             uint8_t *w_s4, int64_t ld_s4, float *w_scale, uint32_t flags, hipStream_t stream)
{
    if (N > 0 && (!w || !w_s4 || !w_scale)) return CR_ERR_INVALID_ARG;
    if (w_dtype != CR_BF16 && w_dtype != CR_FP16 && w_dtype != CR_FP32) return CR_ERR_UNSUPPORTED_DTYPE;
    if (N < 0 || K < 1 || N > kMaxRows) return CR_ERR_INVALID_ARG;
    if (check_flags(flags) != CR_OK) return CR_ERR_INVALID_ARG;
    const int64_t kp = pad256(K);
    if (kp > CR_MAX_K_PAD) return CR_ERR_TOO_LARGE;
    if (ld_w < K || ld_s4 < kp / 2) return CR_ERR_INVALID_ARG;
    if (!aligned(w, 16) || (ld_w * elem_size(w_dtype)) % 16 != 0) return CR_ERR_MISALIGNED;
    if (!aligned(w_s4, 16) || ld_s4 % 16 != 0 || !aligned(w_scale, 4)) return CR_ERR_MISALIGNED;
    if (N == 0) return CR_OK;
    cr_status s = current_device_ok();
    if (s != CR_OK) return s;
    return from_hip(convrot::launch_quant_weight_w4(w, (int)w_dtype, ld_w, N, K, w_s4, ld_s4, w_scale,
                                                    (flags & CR_FLAG_FORCE_TWO_PASS) != 0,
                                                    (flags & CR_FLAG_BLOCK_TRANSPOSED) != 0, stream));
}

cr_status cr_gemm_s8s4_rowscale(const int8_t *a_s8, int64_t lda, const float *a_scale,
                                const uint8_t *b_s4, int64_t ldb, const float *b_scale, const float *bias,
                                int64_t M, int64_t N, int64_t K_pad, void *c, cr_dtype c_dtype, int64_t ldc,
                                hipStream_t stream)
{
    if ((M > 0 && !a_s8) || (N > 0 && !b_s4) || (M > 0 && N > 0 && !c)) return CR_ERR_INVALID_ARG;
    if (c_dtype != CR_BF16 && c_dtype != CR_FP16 && c_dtype != CR_FP32 && c_dtype != CR_I32)
        return CR_ERR_UNSUPPORTED_DTYPE;
    if (c_dtype != CR_I32 && ((M > 0 && !a_scale) || (N > 0 && !b_scale))) return CR_ERR_INVALID_ARG;
    if (bias && c_dtype == CR_I32) return CR_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || K_pad < 1 || K_pad % 256 != 0 || M > kMaxRows || N > kMaxRows) return CR_ERR_INVALID_ARG;
    if (((M + 255) / 256) * ((N + 255) / 256) > (int64_t)(UINT32_MAX / 512)) return CR_ERR_TOO_LARGE;
    if (K_pad > CR_MAX_K_PAD) return CR_ERR_TOO_LARGE;
    if (lda < K_pad || ldb < K_pad / 2 || ldc < N) return CR_ERR_INVALID_ARG;   // ldb in bytes
    if (!aligned(a_s8, 16) || !aligned(b_s4, 16) || lda % 16 != 0 || ldb % 16 != 0) return CR_ERR_MISALIGNED;
    if (!aligned(c, (size_t)elem_size(c_dtype))) return CR_ERR_MISALIGNED;
    if ((a_scale && !aligned(a_scale, 4)) || (b_scale && !aligned(b_scale, 4)) || (bias && !aligned(bias, 4)))
        return CR_ERR_MISALIGNED;
    if (M == 0 || N == 0) return CR_OK;
    cr_status s = current_device_ok();
    if (s != CR_OK) return s;
    return from_hip(convrot::launch_gemm_s8s4(a_s8, lda, a_scale, b_s4, ldb, b_scale, bias, M, N, K_pad, c,
                                              (int)c_dtype, ldc, stream));
}

size_t cr_linear_w4a8_workspace_bytes(int64_t M, int64_t K)
{
    if (M < 1 || K < 1 || pad256(K) > CR_MAX_K_PAD) return 0;
    return up256(up256((size_t)M * (size_t)pad256(K)) + (size_t)M * 4);
}

cr_status cr_linear_w4a8(const void *x, cr_dtype x_dtype, int64_t ld_x, int swiglu, int64_t M, int64_t K,
                         const uint8_t *w_s4, int64_t ld_s4, const float *w_scale, int64_t N, const float *bias,
                         void *out, cr_dtype out_dtype, int64_t ldc, void *workspace, size_t ws_bytes,
                         uint32_t flags, hipStream_t stream)
{
    if (x_dtype != CR_BF16 && x_dtype != CR_FP16 && x_dtype != CR_FP32) return CR_ERR_UNSUPPORTED_DTYPE;
    if (out_dtype != CR_BF16 && out_dtype != CR_FP16 && out_dtype != CR_FP32) return CR_ERR_UNSUPPORTED_DTYPE;
    if (M < 0 || N < 0 || K < 1 || M > kMaxRows || N > kMaxRows) return CR_ERR_INVALID_ARG;
    if (check_flags(flags) != CR_OK) return CR_ERR_INVALID_ARG;
    if (swiglu && K > (int64_t)1 << 40) return CR_ERR_TOO_LARGE;
    const int64_t kp = pad256(K);
    if (kp > CR_MAX_K_PAD) return CR_ERR_TOO_LARGE;
    if (((M + 255) / 256) * ((N + 255) / 256) > (int64_t)(UINT32_MAX / 512)) return CR_ERR_TOO_LARGE;
    if (ld_x < (swiglu ? 2 * K : K) || ld_s4 < kp / 2 || ldc < N) return CR_ERR_INVALID_ARG;
    if ((M > 0 && !x) || (N > 0 && (!w_s4 || !w_scale)) || (M > 0 && N > 0 && !out)) return CR_ERR_INVALID_ARG;
    if (!aligned(x, 16) || (ld_x * elem_size(x_dtype)) % 16 != 0) return CR_ERR_MISALIGNED;
    if (!aligned(w_s4, 16) || ld_s4 % 16 != 0 || !aligned(w_scale, 4)) return CR_ERR_MISALIGNED;
    if ((bias && !aligned(bias, 4)) || !aligned(out, (size_t)elem_size(out_dtype))) return CR_ERR_MISALIGNED;
    if (M == 0 || N == 0) return CR_OK;       // an empty layer: nothing to enqueue, no workspace
    if (!workspace) return CR_ERR_INVALID_ARG;
    if (!aligned(workspace, 256)) return CR_ERR_MISALIGNED;
    if (ws_bytes < cr_linear_w4a8_workspace_bytes(M, K)) return CR_ERR_TOO_LARGE;
    cr_status s = current_device_ok();
    if (s != CR_OK) return s;
    int8_t *x_s8 = static_cast<int8_t *>(workspace);
    float *x_scale = reinterpret_cast<float *>(x_s8 + up256((size_t)M * (size_t)kp));
    const bool tp = (flags & CR_FLAG_FORCE_TWO_PASS) != 0;
    const bool tr = (flags & CR_FLAG_BLOCK_TRANSPOSED) != 0;
    hipError_t e = swiglu
        ? convrot::launch_quant_act_swiglu(x, (int)x_dtype, ld_x, M, K, nullptr, x_s8, kp, x_scale, tp, tr, stream)
        : convrot::launch_quant_act(x, (int)x_dtype, ld_x, M, K, nullptr, x_s8, kp, x_scale, tp, tr, stream);
    if (e != hipSuccess) return CR_ERR_LAUNCH;
    return from_hip(convrot::launch_gemm_s8s4(x_s8, kp, x_scale, w_s4, ld_s4, w_scale, bias, M, N, kp, out,
                                              (int)out_dtype, ldc, stream));
}

cr_status cr_quant_act_w4(const void *x, cr_dtype x_dtype, int64_t ld_x, int swiglu, int64_t M, int64_t K,
                          uint8_t *x_s4, int64_t ld_s4, float *x_scale, uint32_t flags, hipStream_t stream)
{
    if (M > 0 && (!x || !x_s4 || !x_scale)) return CR_ERR_INVALID_ARG;
    if (x_dtype != CR_BF16 && x_dtype != CR_FP16 && x_dtype != CR_FP32) return CR_ERR_UNSUPPORTED_DTYPE;
    if (M < 0 || K < 1 || M > kMaxRows) return CR_ERR_INVALID_ARG;
    if (check_flags(flags) != CR_OK) return CR_ERR_INVALID_ARG;
    if (swiglu && K > (int64_t)1 << 40) return CR_ERR_TOO_LARGE;
    const int64_t kp = pad256(K);
    if (kp > CR_MAX_K_PAD) return CR_ERR_TOO_LARGE;
    if (ld_x < (swiglu ? 2 * K : K) || ld_s4 < kp / 2) return CR_ERR_INVALID_ARG;
    if (!aligned(x, 16) || (ld_x * elem_size(x_dtype)) % 16 != 0) return CR_ERR_MISALIGNED;
    if (!aligned(x_s4, 16) || ld_s4 % 16 != 0 || !aligned(x_scale, 4)) return CR_ERR_MISALIGNED;
    if (M == 0) return CR_OK;
    cr_status s = current_device_ok();
    if (s != CR_OK) return s;
    return from_hip(convrot::launch_quant_act_w4(x, (int)x_dtype, ld_x, swiglu != 0, M, K, x_s4, ld_s4, x_scale,
                                                 (flags & CR_FLAG_FORCE_TWO_PASS) != 0,
                                                 (flags & CR_FLAG_BLOCK_TRANSPOSED) != 0, stream));
}

cr_status cr_gemm_s4s4_rowscale(const uint8_t *a_s4, int64_t lda, const float *a_scale,
                                const uint8_t *b_s4, int64_t ldb, const float *b_scale, const float *bias,
                                int64_t M, int64_t N, int64_t K_pad, void *c, cr_dtype c_dtype, int64_t ldc,
                                hipStream_t stream)
{
    if ((M > 0 && !a_s4) || (N > 0 && !b_s4) || (M > 0 && N > 0 && !c)) return CR_ERR_INVALID_ARG;
    if (c_dtype != CR_BF16 && c_dtype != CR_FP16 && c_dtype != CR_FP32 && c_dtype != CR_I32)
        return CR_ERR_UNSUPPORTED_DTYPE;
    if (c_dtype != CR_I32 && ((M > 0 && !a_scale) || (N > 0 && !b_scale))) return CR_ERR_INVALID_ARG;
    if (bias && c_dtype == CR_I32) return CR_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || K_pad < 1 || K_pad % 256 != 0 || M > kMaxRows || N > kMaxRows) return CR_ERR_INVALID_ARG;
    if (((M + 255) / 256) * ((N + 255) / 256) > (int64_t)(UINT32_MAX / 512)) return CR_ERR_TOO_LARGE;
    if (K_pad > CR_MAX_K_PAD) return CR_ERR_TOO_LARGE;
    if (lda < K_pad / 2 || ldb < K_pad / 2 || ldc < N) return CR_ERR_INVALID_ARG;   // lda, ldb in bytes
    if (!aligned(a_s4, 16) || !aligned(b_s4, 16) || lda % 16 != 0 || ldb % 16 != 0) return CR_ERR_MISALIGNED;
    if (!aligned(c, (size_t)elem_size(c_dtype))) return CR_ERR_MISALIGNED;
    if ((a_scale && !aligned(a_scale, 4)) || (b_scale && !aligned(b_scale, 4)) || (bias && !aligned(bias, 4)))
        return CR_ERR_MISALIGNED;
    if (M == 0 || N == 0) return CR_OK;
    cr_status s = current_device_ok();
    if (s != CR_OK) return s;
    return from_hip(convrot::launch_gemm_s4s4(a_s4, lda, a_scale, b_s4, ldb, b_scale, bias, M, N, K_pad, c,
                                              (int)c_dtype, ldc, stream));
}

size_t cr_linear_w4a4_workspace_bytes(int64_t M, int64_t K)
{
    if (M < 1 || K < 1 || pad256(K) > CR_MAX_K_PAD) return 0;
    return up256(up256((size_t)M * (size_t)(pad256(K) / 2)) + (size_t)M * 4);
}

cr_status cr_linear_w4a4(const void *x, cr_dtype x_dtype, int64_t ld_x, int swiglu, int64_t M, int64_t K,
                         const uint8_t *w_s4, int64_t ld_s4, const float *w_scale, int64_t N, const float *bias,
                         void *out, cr_dtype out_dtype, int64_t ldc, void *workspace, size_t ws_bytes,
                         uint32_t flags, hipStream_t stream)
{
    if (x_dtype != CR_BF16 && x_dtype != CR_FP16 && x_dtype != CR_FP32) return CR_ERR_UNSUPPORTED_DTYPE;
    if (out_dtype != CR_BF16 && out_dtype != CR_FP16 && out_dtype != CR_FP32) return CR_ERR_UNSUPPORTED_DTYPE;
    if (M < 0 || N < 0 || K < 1 || M > kMaxRows || N > kMaxRows) return CR_ERR_INVALID_ARG;
    if (check_flags(flags) != CR_OK) return CR_ERR_INVALID_ARG;
    if (swiglu && K > (int64_t)1 << 40) return CR_ERR_TOO_LARGE;
    const int64_t kp = pad256(K);
    if (kp > CR_MAX_K_PAD) return CR_ERR_TOO_LARGE;
    if (((M + 255) / 256) * ((N + 255) / 256) > (int64_t)(UINT32_MAX / 512)) return CR_ERR_TOO_LARGE;
    if (ld_x < (swiglu ? 2 * K : K) || ld_s4 < kp / 2 || ldc < N) return CR_ERR_INVALID_ARG;
    if ((M > 0 && !x) || (N > 0 && (!w_s4 || !w_scale)) || (M > 0 && N > 0 && !out)) return CR_ERR_INVALID_ARG;
    if (!aligned(x, 16) || (ld_x * elem_size(x_dtype)) % 16 != 0) return CR_ERR_MISALIGNED;
    if (!aligned(w_s4, 16) || ld_s4 % 16 != 0 || !aligned(w_scale, 4)) return CR_ERR_MISALIGNED;
    if ((bias && !aligned(bias, 4)) || !aligned(out, (size_t)elem_size(out_dtype))) return CR_ERR_MISALIGNED;
    if (M == 0 || N == 0) return CR_OK;       // an empty layer: nothing to enqueue, no workspace
    if (!workspace) return CR_ERR_INVALID_ARG;
    if (!aligned(workspace, 256)) return CR_ERR_MISALIGNED;
    if (ws_bytes < cr_linear_w4a4_workspace_bytes(M, K)) return CR_ERR_TOO_LARGE;
    cr_status s = current_device_ok();
    if (s != CR_OK) return s;
    uint8_t *x_s4 = static_cast<uint8_t *>(workspace);
    float *x_scale = reinterpret_cast<float *>(x_s4 + up256((size_t)M * (size_t)(kp / 2)));
    hipError_t e = convrot::launch_quant_act_w4(x, (int)x_dtype, ld_x, swiglu != 0, M, K, x_s4, kp / 2, x_scale,
                                                (flags & CR_FLAG_FORCE_TWO_PASS) != 0,
                                                (flags & CR_FLAG_BLOCK_TRANSPOSED) != 0, stream);
    if (e != hipSuccess) return CR_ERR_LAUNCH;
    return from_hip(convrot::launch_gemm_s4s4(x_s4, kp / 2, x_scale, w_s4, ld_s4, w_scale, bias, M, N, kp, out,
                                              (int)out_dtype, ldc, stream));
}

cr_status cr_quant_weight_w4_e2m3(const void *w, cr_dtype w_dtype, int64_t ld_w, int64_t N, int64_t K,
                                  uint8_t *w_f6, int64_t ld_f6, float *w_scale, uint32_t flags, hipStream_t stream)
{
    if (N > 0 && (!w || !w_f6 || !w_scale)) return CR_ERR_INVALID_ARG;
    if (w_dtype != CR_BF16 && w_dtype != CR_FP16 && w_dtype != CR_FP32) return CR_ERR_UNSUPPORTED_DTYPE;
    if (N < 0 || K < 1 || N > kMaxRows) return CR_ERR_INVALID_ARG;
    if (check_flags(flags) != CR_OK) return CR_ERR_INVALID_ARG;
    const int64_t kp = pad256(K);
    if (kp > CR_MAX_K_PAD) return CR_ERR_TOO_LARGE;
    if (ld_w < K || ld_f6 < 3 * kp) return CR_ERR_INVALID_ARG;
    if (!aligned(w, 16) || (ld_w * elem_size(w_dtype)) % 16 != 0) return CR_ERR_MISALIGNED;
    if (!aligned(w_f6, 16) || ld_f6 % 16 != 0 || !aligned(w_scale, 4)) return CR_ERR_MISALIGNED;
    if (N == 0) return CR_OK;
    cr_status s = current_device_ok();
    if (s != CR_OK) return s;
    return from_hip(convrot::launch_quant_weight_e2m3(w, (int)w_dtype, ld_w, N, K, w_f6, ld_f6, w_scale,
                                                      (flags & CR_FLAG_FORCE_TWO_PASS) != 0,
                                                      (flags & CR_FLAG_BLOCK_TRANSPOSED) != 0, stream));
}

cr_status cr_repack_w4_e2m3(const uint8_t *w_s4, int64_t ld_s4, int64_t N, int64_t K_pad, uint8_t *w_f6,
                            int64_t ld_f6, hipStream_t stream)
{
    if (N > 0 && (!w_s4 || !w_f6)) return CR_ERR_INVALID_ARG;
    if (N < 0 || N > kMaxRows || K_pad < 1 || K_pad % 256 != 0) return CR_ERR_INVALID_ARG;
    if (K_pad > CR_MAX_K_PAD) return CR_ERR_TOO_LARGE;
    if (ld_s4 < K_pad / 2 || ld_f6 < 3 * K_pad) return CR_ERR_INVALID_ARG;
    if (!aligned(w_s4, 16) || ld_s4 % 16 != 0 || !aligned(w_f6, 16) || ld_f6 % 16 != 0) return CR_ERR_MISALIGNED;
    if (N == 0) return CR_OK;
    cr_status s = current_device_ok();
    if (s != CR_OK) return s;
    return from_hip(convrot::launch_repack_w4_e2m3(w_s4, ld_s4, N, K_pad, w_f6, ld_f6, stream));
}

cr_status cr_quant_act_w4_e2m3(const void *x, cr_dtype x_dtype, int64_t ld_x, int swiglu, int64_t M, int64_t K,
                               uint8_t *x_f6, int64_t ld_f6, float *x_scale, uint32_t flags, hipStream_t stream)
{
    if (M > 0 && (!x || !x_f6 || !x_scale)) return CR_ERR_INVALID_ARG;
    if (x_dtype != CR_BF16 && x_dtype != CR_FP16 && x_dtype != CR_FP32) return CR_ERR_UNSUPPORTED_DTYPE;
    if (M < 0 || K < 1 || M > kMaxRows) return CR_ERR_INVALID_ARG;
    if (check_flags(flags) != CR_OK) return CR_ERR_INVALID_ARG;
    if (swiglu && K > (int64_t)1 << 40) return CR_ERR_TOO_LARGE;
    const int64_t kp = pad256(K);
    if (kp > CR_MAX_K_PAD) return CR_ERR_TOO_LARGE;
    if (ld_x < (swiglu ? 2 * K : K) || ld_f6 < 3 * kp) return CR_ERR_INVALID_ARG;
    if (!aligned(x, 16) || (ld_x * elem_size(x_dtype)) % 16 != 0) return CR_ERR_MISALIGNED;
    if (!aligned(x_f6, 16) || ld_f6 % 16 != 0 || !aligned(x_scale, 4)) return CR_ERR_MISALIGNED;
    if (M == 0) return CR_OK;
    cr_status s = current_device_ok();
    if (s != CR_OK) return s;
    return from_hip(convrot::launch_quant_act_e2m3(x, (int)x_dtype, ld_x, swiglu != 0, M, K, x_f6, ld_f6, x_scale,
                                                   (flags & CR_FLAG_FORCE_TWO_PASS) != 0,
                                                   (flags & CR_FLAG_BLOCK_TRANSPOSED) != 0, stream));
}

cr_status cr_gemm_e2m3_rowscale(const uint8_t *a_f6, int64_t lda, const float *a_scale,
                                const uint8_t *b_f6, int64_t ldb, const float *b_scale, const float *bias,
                                int64_t M, int64_t N, int64_t K_pad, void *c, cr_dtype c_dtype, int64_t ldc,
                                hipStream_t stream)
{
    if ((M > 0 && !a_f6) || (N > 0 && !b_f6) || (M > 0 && N > 0 && !c)) return CR_ERR_INVALID_ARG;
    if (c_dtype != CR_BF16 && c_dtype != CR_FP16 && c_dtype != CR_FP32 && c_dtype != CR_I32)
        return CR_ERR_UNSUPPORTED_DTYPE;
    if (c_dtype != CR_I32 && ((M > 0 && !a_scale) || (N > 0 && !b_scale))) return CR_ERR_INVALID_ARG;
    if (bias && c_dtype == CR_I32) return CR_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || K_pad < 1 || K_pad % 256 != 0 || M > kMaxRows || N > kMaxRows) return CR_ERR_INVALID_ARG;
    if (((M + 255) / 256) * ((N + 255) / 256) > (int64_t)(UINT32_MAX / 512)) return CR_ERR_TOO_LARGE;
    if (K_pad > CR_MAX_K_PAD) return CR_ERR_TOO_LARGE;
    if (lda < 3 * K_pad || ldb < 3 * K_pad || ldc < N) return CR_ERR_INVALID_ARG;   // bytes per quad of rows
    if (!aligned(a_f6, 16) || !aligned(b_f6, 16) || lda % 16 != 0 || ldb % 16 != 0) return CR_ERR_MISALIGNED;
    if (!aligned(c, (size_t)elem_size(c_dtype))) return CR_ERR_MISALIGNED;
    if ((a_scale && !aligned(a_scale, 4)) || (b_scale && !aligned(b_scale, 4)) || (bias && !aligned(bias, 4)))
        return CR_ERR_MISALIGNED;
    if (M == 0 || N == 0) return CR_OK;
    cr_status s = current_device_ok();
    if (s != CR_OK) return s;
    return from_hip(convrot::launch_gemm_e2m3(a_f6, lda, a_scale, b_f6, ldb, b_scale, bias, M, N, K_pad, c,
                                              (int)c_dtype, ldc, stream));
}

size_t cr_linear_w4a4_e2m3_workspace_bytes(int64_t M, int64_t K)
{
    if (M < 1 || K < 1 || pad256(K) > CR_MAX_K_PAD) return 0;
    return up256(up256((size_t)((M + 3) / 4) * (size_t)(3 * pad256(K))) + (size_t)M * 4);
}

cr_status cr_linear_w4a4_e2m3(const void *x, cr_dtype x_dtype, int64_t ld_x, int swiglu, int64_t M, int64_t K,
                              const uint8_t *w_f6, int64_t ld_f6, const float *w_scale, int64_t N,
                              const float *bias, void *out, cr_dtype out_dtype, int64_t ldc, void *workspace,
                              size_t ws_bytes, uint32_t flags, hipStream_t stream)
{
    if (x_dtype != CR_BF16 && x_dtype != CR_FP16 && x_dtype != CR_FP32) return CR_ERR_UNSUPPORTED_DTYPE;
    if (out_dtype != CR_BF16 && out_dtype != CR_FP16 && out_dtype != CR_FP32) return CR_ERR_UNSUPPORTED_DTYPE;
    if (M < 0 || N < 0 || K < 1 || M > kMaxRows || N > kMaxRows) return CR_ERR_INVALID_ARG;
    if (check_flags(flags) != CR_OK) return CR_ERR_INVALID_ARG;
    if (swiglu && K > (int64_t)1 << 40) return CR_ERR_TOO_LARGE;
    const int64_t kp = pad256(K);
    if (kp > CR_MAX_K_PAD) return CR_ERR_TOO_LARGE;
    if (((M + 255) / 256) * ((N + 255) / 256) > (int64_t)(UINT32_MAX / 512)) return CR_ERR_TOO_LARGE;
    if (ld_x < (swiglu ? 2 * K : K) || ld_f6 < 3 * kp || ldc < N) return CR_ERR_INVALID_ARG;
    if ((M > 0 && !x) || (N > 0 && (!w_f6 || !w_scale)) || (M > 0 && N > 0 && !out)) return CR_ERR_INVALID_ARG;
    if (!aligned(x, 16) || (ld_x * elem_size(x_dtype)) % 16 != 0) return CR_ERR_MISALIGNED;
    if (!aligned(w_f6, 16) || ld_f6 % 16 != 0 || !aligned(w_scale, 4)) return CR_ERR_MISALIGNED;
    if ((bias && !aligned(bias, 4)) || !aligned(out, (size_t)elem_size(out_dtype))) return CR_ERR_MISALIGNED;
    if (M == 0 || N == 0) return CR_OK;       // an empty layer: nothing to enqueue, no workspace
    if (!workspace) return CR_ERR_INVALID_ARG;
    if (!aligned(workspace, 256)) return CR_ERR_MISALIGNED;
    if (ws_bytes < cr_linear_w4a4_e2m3_workspace_bytes(M, K)) return CR_ERR_TOO_LARGE;
    cr_status s = current_device_ok();
    if (s != CR_OK) return s;
    const int64_t lf = 3 * kp;                  // one quad of rows
    uint8_t *x_f6 = static_cast<uint8_t *>(workspace);
    float *x_scale = reinterpret_cast<float *>(x_f6 + up256((size_t)((M + 3) / 4) * (size_t)lf));
    hipError_t e = convrot::launch_quant_act_e2m3(x, (int)x_dtype, ld_x, swiglu != 0, M, K, x_f6, lf, x_scale,
                                                  (flags & CR_FLAG_FORCE_TWO_PASS) != 0,
                                                  (flags & CR_FLAG_BLOCK_TRANSPOSED) != 0, stream);
    if (e != hipSuccess) return CR_ERR_LAUNCH;
    return from_hip(convrot::launch_gemm_e2m3(x_f6, lf, x_scale, w_f6, ld_f6, w_scale, bias, M, N, kp, out,
                                              (int)out_dtype, ldc, stream));
}

cr_status cr_linear_nvfp4_noalloc(const void *x, cr_dtype x_dtype, int64_t ld_x, int swiglu,
                                  int64_t M, int64_t K, const float *pre_scale,
                                  const uint8_t *w_fp4, int64_t ld_fp4,
                                  const uint8_t *w_sf, int64_t ld_sf, const float *global_scale,
                                  int64_t N, const float *bias, void *out, cr_dtype out_dtype, int64_t ldc,
                                  size_t max_tile_bytes, uint32_t flags, hipStream_t stream)
{
    if (M < 0 || N < 0 || K < 1) return CR_ERR_INVALID_ARG;
    if (pad256(K) > CR_MAX_K_PAD) return CR_ERR_TOO_LARGE;
    if (M == 0 || N == 0)    // an empty layer: argument checks only, as in cr_linear_nvfp4_ex
        return cr_linear_nvfp4_ex(x, x_dtype, ld_x, swiglu, M, K, pre_scale, w_fp4, ld_fp4, w_sf, ld_sf,
                                  global_scale, N, bias, out, out_dtype, ldc, nullptr, 0, max_tile_bytes, flags,
                                  stream, nullptr);
    size_t bound = max_tile_bytes;
    if (bound == 0 && M > kFusedMaxRows) {
        bound = noalloc_tile_bound(M, K);
        if (bound == 0) return CR_ERR_TOO_LARGE;
    }
    if (plan_layer(M, N, K, bound).bytes > CR_NOALLOC_SCRATCH_BYTES) return CR_ERR_TOO_LARGE;
    cr_status s = current_device_ok();
    if (s != CR_OK) return s;
    void *ws = nullptr;
    if ((s = scratch_for_current_device(&ws)) != CR_OK) return s;
    // serial staging on `stream`: no second stream, so no events are needed
    return cr_linear_nvfp4_ex(x, x_dtype, ld_x, swiglu, M, K, pre_scale, w_fp4, ld_fp4, w_sf, ld_sf, global_scale,
                              N, bias, out, out_dtype, ldc, ws, CR_NOALLOC_SCRATCH_BYTES, bound, flags, stream,
                              nullptr);
}

}  // extern "C"
