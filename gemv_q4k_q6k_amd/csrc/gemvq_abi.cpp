// C ABI of libgemvq.so (declared in include/gemvq.h).
//
// Each entry point validates every argument on the host first (so a rejected
// call touches no HIP state and a CPU-only test can exercise every error
// path), then looks up the CU count of the current device once, then enqueues
// the kernels on the caller's stream and checks the launch.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <stddef.h>
#include <stdint.h>

#include "../../include/gemvq.h"
#include "gemvq_launch.h"

namespace {

using gemvq::kMaxK;
constexpr int64_t kMaxQ8K = 65536;
constexpr int64_t kMaxN = 2147483647;

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

// Shape of a weight matrix; on success stores its byte size.
int check_shape(int64_t N, int64_t K, int64_t block_bytes, size_t *bytes)
{
    if (N < 1 || N > kMaxN || K < 256 || K > kMaxK || K % 256 != 0) return GEMVQ_ERR_SHAPE;
    const int64_t nb = K / 256;
    if (N > INT64_MAX / (nb * block_bytes)) return GEMVQ_ERR_SHAPE;
    *bytes = (size_t)(N * nb * block_bytes);
    return GEMVQ_OK;
}

// CU count of the current device, cached per device ordinal.
std::atomic<int> g_cus[64];

int device_cus(int *cus)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GEMVQ_ERR_HIP;
    if (dev >= 0 && dev < 64) {
        const int c = g_cus[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *cus = c;
            return GEMVQ_OK;
        }
    }
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1)
        return GEMVQ_ERR_HIP;
    if (dev >= 0 && dev < 64) g_cus[dev].store(c, std::memory_order_relaxed);
    *cus = c;
    return GEMVQ_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? GEMVQ_OK : GEMVQ_ERR_HIP; }

// Workspace of lm_head_argmax_noalloc: the 12,288 bytes lm_head_argmax takes
// from its caller (a done counter and the running key, then a reserved
// area), here a file-scope device array.  Every GPU the library runs on holds
// its own copy, at its own address, until the process ends.  In host code the
// name `scratch` is only a stand-in for the symbol: its device address comes
// from hipGetSymbolAddress, once per device, and only that address is ever
// passed to a kernel.
static __device__ __align__(256) uint8_t scratch[gemvq::kArgmaxWsBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];   // device address of `scratch` per device ordinal

// `scratch`'s address on the current device.  The first call for a device
// looks it up and clears the counters (first kArgmaxZeroBytes) with a fill
// kernel on `s`, which orders the clear before the argmax launch that
// follows on the same stream; every argmax launch leaves them zero again.
int scratch_on_current_device(hipStream_t s, void **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GEMVQ_ERR_HIP;
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GEMVQ_ERR_HIP;
        if (gemvq::launch_fill_zero(p, gemvq::kArgmaxZeroBytes, s) != hipSuccess) return GEMVQ_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return GEMVQ_OK;
}

}  // namespace

extern "C" {

const char *gemvq_strerror(int status)
{
    switch (status) {
    case GEMVQ_OK: return "ok";
    case GEMVQ_ERR_NULL: return "a required pointer is NULL";
    case GEMVQ_ERR_SHAPE: return "bad shape: need 1 <= N < 2^31, 256 <= K <= 32768, K % 256 == 0";
    case GEMVQ_ERR_ALIGN: return "misaligned pointer";
    case GEMVQ_ERR_WORKSPACE: return "workspace too small";
    case GEMVQ_ERR_ALIAS: return "an output overlaps an input";
    case GEMVQ_ERR_HIP: return "HIP runtime error at launch";
    case GEMVQ_ERR_VALUE: return "an argument value is out of range";
    default: return "unknown status";
    }
}

size_t gemvq_lm_head_argmax_ws_bytes(int64_t N, int64_t K)
{
    (void)N;
    (void)K;
    return gemvq::kArgmaxWsBytes;
}

int gemvq_tile_geometry(int kind, int64_t N, int64_t K, int64_t out[11])
{
    constexpr int kHookCus = 256;   // MI355X
    if (!out) return GEMVQ_ERR_NULL;
    if (kind < 0 || kind > 7) return GEMVQ_ERR_SHAPE;
    size_t wb = 0;
    if (int st = check_shape(N, K, (kind == 1 || kind == 4 || kind == 7) ? 210 : 144, &wb)) return st;
    if (kind == 5 && N % 32 != 0) return GEMVQ_ERR_SHAPE;
    const gemvq::Plan pl = kind == 5   ? gemvq::make_swiglu_q8_plan(N, K, kHookCus)
                           : kind >= 6 ? gemvq::make_batch_plan(N, K, kind == 6 ? 2 : 4,
                                                                gemvq::batch_slots(gemvq::kMaxBatch, kind == 7), nullptr)
                                       : gemvq::make_plan(N, K, kind, kHookCus);
    out[0] = pl.waves;
    out[1] = pl.rows_tile;
    out[2] = pl.tiles;
    out[3] = pl.wave_local;
    out[4] = pl.x_in_lds;
    out[5] = (int64_t)pl.lds_bytes;
    out[6] = pl.wave_local ? pl.steps : 1;
    out[7] = (pl.wave_local && !pl.rows_kernel) ? 1 : 0;
    out[8] = pl.resident;
    out[9] = pl.resident ? pl.phase : 0;
    out[10] = pl.resident ? pl.grid : 0;
    return GEMVQ_OK;
}

int q4k_gemv_multi(const void *const *W, const int64_t *N, float *const *y, const float *const *residual, int count,
                   const float *x, int64_t K, void *stream)
{
    if (!W || !N || !y || !x) return GEMVQ_ERR_NULL;
    if (count < 1 || count > gemvq::kMaxMulti) return GEMVQ_ERR_SHAPE;
    size_t wb[gemvq::kMaxMulti] = {0};
    int64_t total = 0;
    for (int i = 0; i < count; ++i) {
        if (!W[i] || !y[i]) return GEMVQ_ERR_NULL;
        if (int st = check_shape(N[i], K, 144, &wb[i])) return st;
        total += N[i];
    }
    if (K > gemvq::kMaxMultiK || total > kMaxN) return GEMVQ_ERR_SHAPE;
    if (!aligned(x, 16)) return GEMVQ_ERR_ALIGN;
    for (int i = 0; i < count; ++i) {
        if (!aligned(W[i], 16) || !aligned(y[i], 4)) return GEMVQ_ERR_ALIGN;
        if (residual && residual[i] && !aligned(residual[i], 4)) return GEMVQ_ERR_ALIGN;
    }
    const size_t nx = (size_t)K * 4;
    for (int i = 0; i < count; ++i) {
        const size_t ny = (size_t)N[i] * 4;
        if (overlap(y[i], ny, x, nx)) return GEMVQ_ERR_ALIAS;
        for (int j = 0; j < count; ++j) {
            if (overlap(y[i], ny, W[j], wb[j])) return GEMVQ_ERR_ALIAS;
            if (j != i && overlap(y[i], ny, y[j], (size_t)N[j] * 4)) return GEMVQ_ERR_ALIAS;
            // a residual may be its own output exactly (in-place add), nothing else
            const float *r = residual ? residual[j] : nullptr;
            if (r && overlap(y[i], ny, r, (size_t)N[j] * 4) && !(j == i && r == y[i])) return GEMVQ_ERR_ALIAS;
        }
    }
    int cus = 0;
    if (int st = device_cus(&cus)) return st;
    return status_of(gemvq::launch_q4k_gemv_multi(W, N, y, residual, count, x, K, cus, (hipStream_t)stream));
}

int q4k_gemv(const void *W, const float *x, float *y, int64_t N, int64_t K, void *stream)
{
    if (!W || !x || !y) return GEMVQ_ERR_NULL;
    size_t wb = 0;
    if (int st = check_shape(N, K, 144, &wb)) return st;
    if (!aligned(W, 16) || !aligned(x, 16) || !aligned(y, 4)) return GEMVQ_ERR_ALIGN;
    if (overlap(y, (size_t)N * 4, W, wb) || overlap(y, (size_t)N * 4, x, (size_t)K * 4)) return GEMVQ_ERR_ALIAS;
    int cus = 0;
    if (int st = device_cus(&cus)) return st;
    return status_of(gemvq::launch_q4k_gemv(W, x, y, N, K, cus, (hipStream_t)stream));
}

int q6k_gemv(const void *W, const float *x, float *y, int64_t N, int64_t K, void *stream)
{
    if (!W || !x || !y) return GEMVQ_ERR_NULL;
    size_t wb = 0;
    if (int st = check_shape(N, K, 210, &wb)) return st;
    if (!aligned(W, 4) || !aligned(x, 16) || !aligned(y, 4)) return GEMVQ_ERR_ALIGN;
    if (overlap(y, (size_t)N * 4, W, wb) || overlap(y, (size_t)N * 4, x, (size_t)K * 4)) return GEMVQ_ERR_ALIAS;
    int cus = 0;
    if (int st = device_cus(&cus)) return st;
    return status_of(gemvq::launch_q6k_gemv(W, x, y, N, K, cus, (hipStream_t)stream));
}

int q8_quantize(const float *x, int8_t *xq, uint16_t *xd, int64_t K, void *stream)
{
    if (!x || !xq || !xd) return GEMVQ_ERR_NULL;
    if (K < 32 || K > kMaxQ8K || K % 32 != 0) return GEMVQ_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(xd, 4)) return GEMVQ_ERR_ALIGN;
    const size_t nx = (size_t)K * 4, nq = (size_t)K, nd = (size_t)(K / 32) * 2;
    if (overlap(xq, nq, x, nx) || overlap(xd, nd, x, nx) || overlap(xq, nq, xd, nd)) return GEMVQ_ERR_ALIAS;
    return status_of(gemvq::launch_q8_quantize(x, xq, xd, K, (hipStream_t)stream));
}

int q4k_q8_gemv(const void *W, const int8_t *xq, const uint16_t *xd, float *y, int64_t N, int64_t K, void *stream)
{
    if (!W || !xq || !xd || !y) return GEMVQ_ERR_NULL;
    size_t wb = 0;
    if (int st = check_shape(N, K, 144, &wb)) return st;
    if (!aligned(W, 16) || !aligned(xq, 16) || !aligned(xd, 4) || !aligned(y, 4)) return GEMVQ_ERR_ALIGN;
    const size_t ny = (size_t)N * 4;
    if (overlap(y, ny, W, wb) || overlap(y, ny, xq, (size_t)K) || overlap(y, ny, xd, (size_t)(K / 32) * 2))
        return GEMVQ_ERR_ALIAS;
    int cus = 0;
    if (int st = device_cus(&cus)) return st;
    return status_of(gemvq::launch_q4k_q8_gemv(W, xq, xd, y, N, K, cus, (hipStream_t)stream));
}

int q4k_q8_gemv_from_f32(const void *W, const float *x, int8_t *xq, uint16_t *xd, float *y, int64_t N, int64_t K,
                         void *stream)
{
    if (!W || !x || !xq || !xd || !y) return GEMVQ_ERR_NULL;
    size_t wb = 0;
    if (int st = check_shape(N, K, 144, &wb)) return st;
    if (!aligned(W, 16) || !aligned(x, 16) || !aligned(xq, 16) || !aligned(xd, 4) || !aligned(y, 4))
        return GEMVQ_ERR_ALIGN;
    const size_t ny = (size_t)N * 4, nx = (size_t)K * 4, nq = (size_t)K, nd = (size_t)(K / 32) * 2;
    // outputs overlap neither the inputs nor each other
    if (overlap(y, ny, W, wb) || overlap(y, ny, x, nx) || overlap(y, ny, xq, nq) || overlap(y, ny, xd, nd) ||
        overlap(xq, nq, W, wb) || overlap(xq, nq, x, nx) || overlap(xq, nq, xd, nd) || overlap(xd, nd, W, wb) ||
        overlap(xd, nd, x, nx))
        return GEMVQ_ERR_ALIAS;
    int cus = 0;
    if (int st = device_cus(&cus)) return st;
    return status_of(gemvq::launch_q4k_q8_gemv_from_f32(W, x, xq, xd, y, N, K, cus, (hipStream_t)stream));
}

int q6k_q8_gemv(const void *W, const int8_t *xq, const uint16_t *xd, float *y, int64_t N, int64_t K, void *stream)
{
    if (!W || !xq || !xd || !y) return GEMVQ_ERR_NULL;
    size_t wb = 0;
    if (int st = check_shape(N, K, 210, &wb)) return st;
    if (!aligned(W, 4) || !aligned(xq, 16) || !aligned(xd, 4) || !aligned(y, 4)) return GEMVQ_ERR_ALIGN;
    const size_t ny = (size_t)N * 4;
    if (overlap(y, ny, W, wb) || overlap(y, ny, xq, (size_t)K) || overlap(y, ny, xd, (size_t)(K / 32) * 2))
        return GEMVQ_ERR_ALIAS;
    int cus = 0;
    if (int st = device_cus(&cus)) return st;
    return status_of(gemvq::launch_q6k_q8_gemv(W, xq, xd, y, N, K, cus, (hipStream_t)stream));
}

static int q8_gemv_batch_impl(bool q6k, const void *W, const int8_t *xq, const uint16_t *xd, float *y, int64_t N,
                              int64_t K, int m, void *stream)
{
    if (!W || !xq || !xd || !y) return GEMVQ_ERR_NULL;
    size_t wb = 0;
    if (int st = check_shape(N, K, q6k ? 210 : 144, &wb)) return st;
    if (m < 1 || m > gemvq::kMaxBatch || N * m > kMaxN) return GEMVQ_ERR_SHAPE;
    if (!aligned(W, q6k ? 4 : 16) || !aligned(xq, 16) || !aligned(xd, 4) || !aligned(y, 4)) return GEMVQ_ERR_ALIGN;
    const size_t ny = (size_t)N * m * 4, nq = (size_t)K * m, nd = (size_t)(K / 32) * 2 * m;
    if (overlap(y, ny, W, wb) || overlap(y, ny, xq, nq) || overlap(y, ny, xd, nd)) return GEMVQ_ERR_ALIAS;
    int cus = 0;
    if (int st = device_cus(&cus)) return st;
    return status_of(gemvq::launch_q8_gemv_batch(q6k, W, xq, xd, y, N, K, m, cus, (hipStream_t)stream));
}

int q4k_q8_gemv_batch(const void *W, const int8_t *xq, const uint16_t *xd, float *y, int64_t N, int64_t K, int m,
                      void *stream)
{
    return q8_gemv_batch_impl(false, W, xq, xd, y, N, K, m, stream);
}

int q6k_q8_gemv_batch(const void *W, const int8_t *xq, const uint16_t *xd, float *y, int64_t N, int64_t K, int m,
                      void *stream)
{
    return q8_gemv_batch_impl(true, W, xq, xd, y, N, K, m, stream);
}

int swiglu_gemv(const void *Wg, const void *Wu, const float *x, float *h, int64_t N, int64_t K, void *stream)
{
    if (!Wg || !Wu || !x || !h) return GEMVQ_ERR_NULL;
    size_t wb = 0;
    if (int st = check_shape(N, K, 144, &wb)) return st;
    if (!aligned(Wg, 16) || !aligned(Wu, 16) || !aligned(x, 16) || !aligned(h, 4)) return GEMVQ_ERR_ALIGN;
    const size_t nh = (size_t)N * 4;
    if (overlap(h, nh, Wg, wb) || overlap(h, nh, Wu, wb) || overlap(h, nh, x, (size_t)K * 4)) return GEMVQ_ERR_ALIAS;
    int cus = 0;
    if (int st = device_cus(&cus)) return st;
    return status_of(gemvq::launch_swiglu_gemv(Wg, Wu, x, h, N, K, cus, (hipStream_t)stream));
}

size_t gemvq_swiglu_q8_ws_bytes(int64_t N)
{
    if (N < 32 || N > kMaxN || N % 32 != 0) return 0;
    return gemvq::swiglu_q8_ws_bytes(N);
}

int swiglu_q8_gemv(const void *Wg, const void *Wu, const float *x, float *h, int8_t *hq, uint16_t *hd,
                   void *workspace, size_t ws_bytes, int64_t N, int64_t K, void *stream)
{
    if (!Wg || !Wu || !x || !hq || !hd || !workspace) return GEMVQ_ERR_NULL;
    size_t wb = 0;
    if (int st = check_shape(N, K, 144, &wb)) return st;
    if (N % 32 != 0) return GEMVQ_ERR_SHAPE;
    if (!aligned(Wg, 16) || !aligned(Wu, 16) || !aligned(x, 16) || (h && !aligned(h, 4)) || !aligned(hq, 16) ||
        !aligned(hd, 4) || !aligned(workspace, 256))
        return GEMVQ_ERR_ALIGN;
    if (ws_bytes < gemvq::swiglu_q8_ws_bytes(N)) return GEMVQ_ERR_WORKSPACE;
    const size_t nx = (size_t)K * 4, nh = h ? (size_t)N * 4 : 0, nq = (size_t)N, nd = (size_t)(N / 32) * 2;
    const void *ins[3] = {Wg, Wu, x};
    const size_t nins[3] = {wb, wb, nx};
    const void *outs[4] = {h, hq, hd, workspace};
    const size_t nouts[4] = {nh, nq, nd, ws_bytes};
    for (int o = 0; o < 4; ++o) {
        for (int i = 0; i < 3; ++i)
            if (overlap(outs[o], nouts[o], ins[i], nins[i])) return GEMVQ_ERR_ALIAS;
        for (int p = o + 1; p < 4; ++p)
            if (overlap(outs[o], nouts[o], outs[p], nouts[p])) return GEMVQ_ERR_ALIAS;
    }
    int cus = 0;
    if (int st = device_cus(&cus)) return st;
    return status_of(gemvq::launch_swiglu_q8_gemv(Wg, Wu, x, h, hq, hd, workspace, N, K, cus, (hipStream_t)stream));
}

// Shared checks of rms_norm_q8 and add_rms_norm_q8 (r and res both null for the former).
static int rms_norm_q8_impl(const float *x, const float *r, const float *w, float eps, float *res, float *y,
                            int8_t *xq, uint16_t *xd, int64_t K, void *stream)
{
    if (K < 32 || K > gemvq::kMaxNormK || K % 32 != 0) return GEMVQ_ERR_SHAPE;
    if (!(eps >= 0.0f) || eps > 3.0e38f) return GEMVQ_ERR_VALUE;   // rejects NaN, negative and infinite eps
    if (!aligned(x, 16) || (r && !aligned(r, 16)) || !aligned(w, 16) || (res && !aligned(res, 16)) ||
        (y && !aligned(y, 16)) || !aligned(xq, 16) || !aligned(xd, 4))
        return GEMVQ_ERR_ALIGN;
    const size_t nv = (size_t)K * 4, nq = (size_t)K, nd = (size_t)(K / 32) * 2;
    const void *ins[3] = {x, r, w};
    const size_t nins[3] = {nv, r ? nv : 0, nv};
    const void *outs[4] = {res, y, xq, xd};
    const size_t nouts[4] = {res ? nv : 0, y ? nv : 0, nq, nd};
    for (int o = 0; o < 4; ++o) {
        for (int i = 0; i < 3; ++i) {
            // the residual may be written over x or r exactly (in place), nothing else
            if (o == 0 && i < 2 && outs[0] == ins[i]) continue;
            if (overlap(outs[o], nouts[o], ins[i], nins[i])) return GEMVQ_ERR_ALIAS;
        }
        for (int p = o + 1; p < 4; ++p)
            if (overlap(outs[o], nouts[o], outs[p], nouts[p])) return GEMVQ_ERR_ALIAS;
    }
    return status_of(gemvq::launch_rms_norm_q8(x, r, w, eps, res, y, xq, xd, K, (hipStream_t)stream));
}

int rms_norm_q8(const float *x, const float *w, float eps, float *y, int8_t *xq, uint16_t *xd, int64_t K,
                void *stream)
{
    if (!x || !w || !xq || !xd) return GEMVQ_ERR_NULL;
    return rms_norm_q8_impl(x, nullptr, w, eps, nullptr, y, xq, xd, K, stream);
}

int add_rms_norm_q8(const float *x, const float *r, const float *w, float eps, float *res, float *y, int8_t *xq,
                    uint16_t *xd, int64_t K, void *stream)
{
    if (!x || !r || !w || !res || !xq || !xd) return GEMVQ_ERR_NULL;
    return rms_norm_q8_impl(x, r, w, eps, res, y, xq, xd, K, stream);
}

static int lm_head_argmax_impl(const void *W, const float *x, const uint32_t *mask, uint32_t *out_idx, float *out_max,
                               void *workspace, size_t ws_bytes, int64_t N, int64_t K, void *stream,
                               const gemvq::Timing &tm)
{
    if (!W || !x || !out_idx || !workspace) return GEMVQ_ERR_NULL;
    size_t wb = 0;
    if (int st = check_shape(N, K, 210, &wb)) return st;
    if (!aligned(W, 4) || !aligned(x, 16) || !aligned(out_idx, 4) || (out_max && !aligned(out_max, 4)) ||
        !aligned(workspace, 256) || (mask && !aligned(mask, 4)))
        return GEMVQ_ERR_ALIGN;
    if (ws_bytes < gemvq::kArgmaxWsBytes) return GEMVQ_ERR_WORKSPACE;
    const size_t nx = (size_t)K * 4;
    const size_t nm = mask ? (size_t)((N + 31) / 32) * 4 : 0;
    if (overlap(out_idx, 4, W, wb) || overlap(out_idx, 4, x, nx) || overlap(out_idx, 4, workspace, ws_bytes) ||
        overlap(out_idx, 4, mask, nm))
        return GEMVQ_ERR_ALIAS;
    if (out_max && (overlap(out_max, 4, W, wb) || overlap(out_max, 4, x, nx) ||
                    overlap(out_max, 4, workspace, ws_bytes) || overlap(out_max, 4, out_idx, 4) ||
                    overlap(out_max, 4, mask, nm)))
        return GEMVQ_ERR_ALIAS;
    if (overlap(workspace, ws_bytes, W, wb) || overlap(workspace, ws_bytes, x, nx) ||
        overlap(workspace, ws_bytes, mask, nm))
        return GEMVQ_ERR_ALIAS;
    int cus = 0;
    if (int st = device_cus(&cus)) return st;
    return status_of(gemvq::launch_lm_head_argmax(W, x, mask, out_idx, out_max, workspace, N, K, cus,
                                                  (hipStream_t)stream, tm));
}

int lm_head_argmax(const void *W, const float *x, uint32_t *out_idx, float *out_max, void *workspace, size_t ws_bytes,
                   int64_t N, int64_t K, void *stream)
{
    return lm_head_argmax_impl(W, x, nullptr, out_idx, out_max, workspace, ws_bytes, N, K, stream, gemvq::Timing{});
}

int lm_head_argmax_timed(const void *W, const float *x, uint32_t *out_idx, float *out_max, void *workspace,
                         size_t ws_bytes, int64_t N, int64_t K, void *stream, void *start_event, void *stop_event)
{
    gemvq::Timing tm;
    tm.start = (hipEvent_t)start_event;
    tm.stop = (hipEvent_t)stop_event;
    return lm_head_argmax_impl(W, x, nullptr, out_idx, out_max, workspace, ws_bytes, N, K, stream, tm);
}

int lm_head_argmax_noalloc(const void *W, const float *x, uint32_t *out_idx, float *out_max, int64_t N, int64_t K,
                           void *stream)
{
    if (!W || !x || !out_idx) return GEMVQ_ERR_NULL;
    size_t wb = 0;
    if (int st = check_shape(N, K, 210, &wb)) return st;
    if (!aligned(W, 4) || !aligned(x, 16) || !aligned(out_idx, 4) || (out_max && !aligned(out_max, 4)))
        return GEMVQ_ERR_ALIGN;
    const size_t nx = (size_t)K * 4;
    if (overlap(out_idx, 4, W, wb) || overlap(out_idx, 4, x, nx)) return GEMVQ_ERR_ALIAS;
    if (out_max && (overlap(out_max, 4, W, wb) || overlap(out_max, 4, x, nx) || overlap(out_max, 4, out_idx, 4)))
        return GEMVQ_ERR_ALIAS;
    int cus = 0;
    if (int st = device_cus(&cus)) return st;
    void *ws = nullptr;
    if (int st = scratch_on_current_device((hipStream_t)stream, &ws)) return st;
    return status_of(gemvq::launch_lm_head_argmax(W, x, nullptr, out_idx, out_max, ws, N, K, cus,
                                                  (hipStream_t)stream, gemvq::Timing{}));
}

int lm_head_argmax_masked(const void *W, const float *x, const uint32_t *mask, uint32_t *out_idx, float *out_max,
                          void *workspace, size_t ws_bytes, int64_t N, int64_t K, void *stream)
{
    if (!mask) return GEMVQ_ERR_NULL;
    return lm_head_argmax_impl(W, x, mask, out_idx, out_max, workspace, ws_bytes, N, K, stream, gemvq::Timing{});
}

int gemvq_stream_read(const void *p, int64_t bytes, int grid, int threads, uint32_t *sink, void *stream)
{
    if (!p || !sink) return GEMVQ_ERR_NULL;
    if (bytes < 16 || bytes % 16 != 0 || grid < 1 || grid > 65536) return GEMVQ_ERR_SHAPE;
    if (threads != 256 && threads != 1024) return GEMVQ_ERR_SHAPE;
    if (!aligned(p, 16) || !aligned(sink, 4)) return GEMVQ_ERR_ALIGN;
    if (overlap(sink, 1024, p, (size_t)bytes)) return GEMVQ_ERR_ALIAS;
    return status_of(gemvq::launch_stream_read(p, bytes, grid, threads, sink, (hipStream_t)stream));
}

int gemvq_q4k_q8_isums(const void *W, const int8_t *xq, int32_t *isums, int64_t N, int64_t K, void *stream)
{
    if (!W || !xq || !isums) return GEMVQ_ERR_NULL;
    size_t wb = 0;
    if (int st = check_shape(N, K, 144, &wb)) return st;
    if (N * (K / 32) > (int64_t)1 << 40) return GEMVQ_ERR_SHAPE;
    if (!aligned(W, 16) || !aligned(xq, 16) || !aligned(isums, 4)) return GEMVQ_ERR_ALIGN;
    const size_t ni = (size_t)N * (size_t)(K / 32) * 4;
    if (overlap(isums, ni, W, wb) || overlap(isums, ni, xq, (size_t)K)) return GEMVQ_ERR_ALIAS;
    return status_of(gemvq::launch_q4k_q8_isums(W, xq, isums, N, K, (hipStream_t)stream));
}

int gemvq_q6k_q8_isums(const void *W, const int8_t *xq, int32_t *isums, int64_t N, int64_t K, void *stream)
{
    if (!W || !xq || !isums) return GEMVQ_ERR_NULL;
    size_t wb = 0;
    if (int st = check_shape(N, K, 210, &wb)) return st;
    if (N * (K / 16) > (int64_t)1 << 40) return GEMVQ_ERR_SHAPE;
    if (!aligned(W, 4) || !aligned(xq, 16) || !aligned(isums, 4)) return GEMVQ_ERR_ALIGN;
    const size_t ni = (size_t)N * (size_t)(K / 16) * 4;
    if (overlap(isums, ni, W, wb) || overlap(isums, ni, xq, (size_t)K)) return GEMVQ_ERR_ALIAS;
    return status_of(gemvq::launch_q6k_q8_isums(W, xq, isums, N, K, (hipStream_t)stream));
}

}  // extern "C"
