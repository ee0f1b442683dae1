// Sanitizer driver for the library's host code (CPU only, no GPU needed):
// every entry point with arguments its checks reject (fake pointers that are
// never dereferenced; a rejected call makes no HIP call), and the launch-plan
// code through gemvq_tile_geometry over many shapes.  Built with host-side
// address and undefined-behaviour sanitizers (device code is not
// instrumented); exit 0 means every status was as expected and the run was
// clean.
#include <stdint.h>
#include <stdio.h>

#include "../../include/gemvq.h"

static int failures = 0;

static void expect(int got, int want, const char *what)
{
    if (got != want) {
        fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
        ++failures;
    }
}

#define P(v) ((void *)(uintptr_t)(v))
#define F(v) ((float *)(uintptr_t)(v))
static const uintptr_t A = 1ull << 20, B = 1ull << 30, C = 1ull << 34, D = 1ull << 38, E = 1ull << 42;

int main()
{
    // null pointers
    expect(q4k_gemv(nullptr, F(B), F(C), 4, 256, nullptr), GEMVQ_ERR_NULL, "q4k_gemv null W");
    expect(q6k_gemv(P(A), nullptr, F(C), 4, 256, nullptr), GEMVQ_ERR_NULL, "q6k_gemv null x");
    expect(q8_quantize(F(A), nullptr, (uint16_t *)P(C), 256, nullptr), GEMVQ_ERR_NULL, "q8_quantize null xq");
    expect(q4k_q8_gemv(P(A), (int8_t *)P(B), nullptr, F(D), 4, 256, nullptr), GEMVQ_ERR_NULL, "q4k_q8_gemv null xd");
    expect(swiglu_gemv(P(A), nullptr, F(C), F(D), 4, 256, nullptr), GEMVQ_ERR_NULL, "swiglu null Wu");
    expect(lm_head_argmax(P(A), F(B), nullptr, nullptr, P(E), 1 << 20, 4, 256, nullptr), GEMVQ_ERR_NULL, "lm_head null idx");
    expect(lm_head_argmax_noalloc(P(A), nullptr, (uint32_t *)P(C), nullptr, 4, 256, nullptr), GEMVQ_ERR_NULL,
           "noalloc null x");
    expect(q4k_q8_gemv_from_f32(P(A), F(B), nullptr, (uint16_t *)P(D), F(E), 4, 256, nullptr), GEMVQ_ERR_NULL,
           "from_f32 null xq");
    expect(gemvq_stream_read(nullptr, 1024, 256, 1024, (uint32_t *)P(C), nullptr), GEMVQ_ERR_NULL, "stream_read null");
    // shapes
    for (int64_t K : {0, 255, 300, 32768 + 256}) expect(q4k_gemv(P(A), F(B), F(C), 4, K, nullptr), GEMVQ_ERR_SHAPE, "K");
    expect(q6k_gemv(P(A), F(B), F(C), 0, 256, nullptr), GEMVQ_ERR_SHAPE, "N = 0");
    expect(q6k_gemv(P(A), F(B), F(C), (int64_t)1 << 40, 256, nullptr), GEMVQ_ERR_SHAPE, "N too large");
    expect(q8_quantize(F(A), (int8_t *)P(B), (uint16_t *)P(C), 33, nullptr), GEMVQ_ERR_SHAPE, "q8 K % 32");
    expect(gemvq_stream_read(P(A), 1000, 256, 1024, (uint32_t *)P(C), nullptr), GEMVQ_ERR_SHAPE, "stream_read bytes");
    expect(gemvq_stream_read(P(A), 1024, 256, 512, (uint32_t *)P(C), nullptr), GEMVQ_ERR_SHAPE, "stream_read threads");
    // alignment
    expect(q4k_gemv(P(A + 4), F(B), F(C), 4, 256, nullptr), GEMVQ_ERR_ALIGN, "q4k W 16 B");
    expect(q6k_gemv(P(A + 2), F(B), F(C), 4, 256, nullptr), GEMVQ_ERR_ALIGN, "q6k W 4 B");
    expect(lm_head_argmax(P(A), F(B), (uint32_t *)P(C), nullptr, P(E + 16), 1 << 20, 4, 256, nullptr),
           GEMVQ_ERR_ALIGN, "lm_head workspace 256 B");
    // workspace and aliasing
    expect(lm_head_argmax(P(A), F(B), (uint32_t *)P(C), nullptr, P(E), 100, 4, 256, nullptr), GEMVQ_ERR_WORKSPACE,
           "lm_head workspace size");
    expect(q4k_gemv(P(A), F(B), F(A + 64), 64, 512, nullptr), GEMVQ_ERR_ALIAS, "y inside W");
    expect(q4k_q8_gemv_from_f32(P(A), F(B), (int8_t *)P(C), (uint16_t *)P(C + 16), F(E), 64, 512, nullptr),
           GEMVQ_ERR_ALIAS, "xd inside xq");
    expect(rms_norm_q8(F(A), F(B), -1.0f, nullptr, (int8_t *)P(D), (uint16_t *)P(D + 4096), 256, nullptr),
           GEMVQ_ERR_VALUE, "negative eps");
    // launch plans of every kind over many shapes (host-only)
    int64_t out[12];
    long plans = 0;
    for (int kind = 0; kind <= 7; ++kind)
        for (int64_t N : {1, 2, 3, 5, 7, 16, 17, 31, 32, 64, 100, 257, 1000, 4096, 9728, 28672, 248320})
            for (int64_t K = 256; K <= 32768; K += (K < 4096 ? 256 : 1792)) {
                const int st = gemvq_tile_geometry(kind, N, K, out);
                if (st == GEMVQ_OK) {
                    ++plans;
                    if (out[0] < 1 || out[1] < 1 || out[2] < 1) {
                        fprintf(stderr, "bad plan kind %d N %ld K %ld\n", kind, (long)N, (long)K);
                        ++failures;
                    }
                }
            }
    expect(gemvq_tile_geometry(0, 0, 256, out), GEMVQ_ERR_SHAPE, "geometry N = 0");
    if (gemvq_strerror(12345) == nullptr) ++failures;
    printf("abi sanitizer run: %d failures, %ld plans\n", failures, plans);
    return failures ? 1 : 0;
}
