/* Sanitizer driver for oracle/oracle.c (CPU only): every exported function
 * on small seeded inputs of several shapes, including the edge sizes, built
 * with -fsanitize=address,undefined -fno-sanitize-recover=all so any
 * out-of-bounds access or undefined behaviour aborts the run.  It checks
 * nothing numerically (the pins do that); exit 0 means clean. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_fp16_to_f64(uint16_t h);
uint16_t orc_f32_to_fp16_rne(float f);
void orc_q4k_block(const uint8_t *blk, double *w);
void orc_q6k_block(const uint8_t *blk, double *w);
void orc_q4k_gemv(const uint8_t *W, const float *x, double *y, int64_t N, int64_t K);
void orc_q6k_gemv(const uint8_t *W, const float *x, double *y, int64_t N, int64_t K);
void orc_q6k_gemv_f64x(const uint8_t *W, const double *x, double *y, int64_t N, int64_t K);
void orc_swiglu(const uint8_t *Wg, const uint8_t *Wu, const float *x, double *h, double *g, double *u,
                int64_t N, int64_t K);
void orc_q8_quantize(const float *x, int8_t *q, uint16_t *dfp16, int64_t K);
void orc_q4k_q8_isums(const uint8_t *W, const int8_t *xq, int32_t *isums, int64_t N, int64_t K);
void orc_q4k_q8_gemv(const uint8_t *W, const int8_t *xq, const uint16_t *xd, double *y, int64_t N, int64_t K);
void orc_q6k_q8_isums(const uint8_t *W, const int8_t *xq, int32_t *isums, int64_t N, int64_t K);
void orc_q6k_q8_gemv(const uint8_t *W, const int8_t *xq, const uint16_t *xd, double *y, int64_t N, int64_t K);
int64_t orc_argmax_first_f64(const double *v, int64_t n);
int64_t orc_argmax_first_f32(const float *v, int64_t n);
int64_t orc_argmax_first_masked_f64(const double *v, const uint32_t *mask, int64_t n);
int64_t orc_argmax_first_masked_f32(const float *v, const uint32_t *mask, int64_t n);
int orc_num_threads(void);
void orc_set_num_threads(int n);

static uint64_t s = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void)
{
    s ^= s << 13;
    s ^= s >> 7;
    s ^= s << 17;
    return (uint32_t)(s >> 16);
}

/* exact-size heap buffers, so the address sanitizer sees every overrun */
static void *buf(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p) abort();
    return p;
}

static void fill_weights(uint8_t *W, size_t nblocks, size_t block)
{
    for (size_t i = 0; i < nblocks * block; ++i) W[i] = (uint8_t)rnd();
    for (size_t b = 0; b < nblocks; ++b) {   /* finite fp16 scales */
        uint8_t *p = W + b * block + (block == 144 ? 0 : 208);
        p[0] = (uint8_t)rnd();
        p[1] = (uint8_t)(0x10 + rnd() % 8);
        if (block == 144) {
            p[2] = (uint8_t)rnd();
            p[3] = (uint8_t)(0x10 + rnd() % 8);
        }
    }
}

static void run(int64_t N, int64_t K)
{
    const int64_t nb = K / 256;
    uint8_t *W4 = buf((size_t)(N * nb * 144)), *W4b = buf((size_t)(N * nb * 144));
    uint8_t *W6 = buf((size_t)(N * nb * 210));
    fill_weights(W4, (size_t)(N * nb), 144);
    fill_weights(W4b, (size_t)(N * nb), 144);
    fill_weights(W6, (size_t)(N * nb), 210);
    float *x = buf(sizeof(float) * (size_t)K);
    double *xd64 = buf(sizeof(double) * (size_t)K);
    for (int64_t k = 0; k < K; ++k) {
        x[k] = (float)((int32_t)(rnd() % 2001) - 1000) / 300.0f;
        xd64[k] = x[k];
    }
    double *y = buf(sizeof(double) * (size_t)N), *g = buf(sizeof(double) * (size_t)N), *u = buf(sizeof(double) * (size_t)N);
    orc_q4k_gemv(W4, x, y, N, K);
    orc_q6k_gemv(W6, x, y, N, K);
    orc_q6k_gemv_f64x(W6, xd64, y, N, K);
    orc_swiglu(W4, W4b, x, y, g, u, N, K);
    int8_t *q = buf((size_t)K);
    uint16_t *d = buf(sizeof(uint16_t) * (size_t)(K / 32));
    orc_q8_quantize(x, q, d, K);
    int32_t *is4 = buf(sizeof(int32_t) * (size_t)(N * (K / 32)));
    int32_t *is6 = buf(sizeof(int32_t) * (size_t)(N * (K / 16)));
    orc_q4k_q8_isums(W4, q, is4, N, K);
    orc_q4k_q8_gemv(W4, q, d, y, N, K);
    orc_q6k_q8_isums(W6, q, is6, N, K);
    orc_q6k_q8_gemv(W6, q, d, y, N, K);
    float *yf = buf(sizeof(float) * (size_t)N);
    for (int64_t n = 0; n < N; ++n) yf[n] = (float)y[n];
    uint32_t *mask = buf(sizeof(uint32_t) * (size_t)((N + 31) / 32));
    for (int64_t i = 0; i < (N + 31) / 32; ++i) mask[i] = rnd();
    volatile int64_t sink = orc_argmax_first_f64(y, N) + orc_argmax_first_f32(yf, N) +
                            orc_argmax_first_masked_f64(y, mask, N) + orc_argmax_first_masked_f32(yf, mask, N);
    (void)sink;
    double w[256];
    orc_q4k_block(W4, w);
    orc_q6k_block(W6 + 210 * (N * nb - 1), w);
    free(W4), free(W4b), free(W6), free(x), free(xd64), free(y), free(g), free(u), free(q), free(d);
    free(is4), free(is6), free(yf), free(mask);
}

int main(void)
{
    volatile double acc = 0.0;
    for (uint32_t h = 0; h < 65536; ++h) acc += isfinite(orc_fp16_to_f64((uint16_t)h)) ? 1.0 : 0.0;
    const float fs[] = {0.f, -0.f, 1.f, 65504.f, 65520.f, 1e-8f, -3.5e-5f, INFINITY, -INFINITY, NAN};
    for (size_t i = 0; i < sizeof(fs) / sizeof(fs[0]); ++i) acc += orc_f32_to_fp16_rne(fs[i]);
    const int64_t shapes[][2] = {{1, 256}, {3, 256}, {2, 512}, {5, 768}, {7, 1024}, {1, 2560}, {4, 9728}, {2, 32768}};
    for (int t = 1; t <= 2; ++t) {
        orc_set_num_threads(t);
        for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i) run(shapes[i][0], shapes[i][1]);
    }
    (void)acc;
    printf("oracle sanitizer run clean (%d threads available)\n", orc_num_threads());
    return 0;
}
