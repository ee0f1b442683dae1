/*
 * CPU oracle for the batch-1 quantized GEMV path (TEST INFRASTRUCTURE ONLY).
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  The product path (the HIP library) never calls it and
 * shares no code, header, table or constant with it.
 *
 * Design: plain definitions, written to be checked by eye.  Every super-block
 * is decoded exactly into f64 weights and every dot product is accumulated in
 * f64 in increasing k order.  This follows the "exact dequantized f64
 * reference" that the aprender-serve page (forward_qwen35_cuda.rs,
 * `attn_q_gemv_of_host_input`) puts both GPU and CPU GEMVs against.  Rows are
 * independent, so an OpenMP loop over rows changes no arithmetic.
 *
 * Block formats (the pages name the GGUF types Q4_K and Q6_K - qualiaDB
 * resident_decode.rs, the fused-FFN quant list - and pin the Q6_K size at
 * 210 bytes per 256 weights - "2520 B/row logits" for a 3072-wide row - but
 * never spell the bit layout out; the layout below is the public GGUF K-quant
 * layout, our reading):
 *
 *  Q4_K, 144 bytes / 256 weights:
 *    [0,2) d (fp16)   [2,4) dmin (fp16)   [4,16) s[12] packed 6-bit
 *    scale/min pairs for 8 sub-blocks of 32   [16,144) qs[128] 4-bit quants.
 *    sub-block j: j<4:  sc = s[j]&63, m = s[j+4]&63
 *                 j>=4: sc = (s[j+4]&15) | (s[j-4]>>6)<<4,
 *                       m  = (s[j+4]>>4) | (s[j]>>6)<<4
 *    quant of weight 32j+i: byte qs[32*(j/2)+i], low nibble if j even,
 *    high nibble if j odd.        w = d*sc*q - dmin*m
 *
 *  Q6_K, 210 bytes / 256 weights:
 *    [0,128) ql (low 4 bits)  [128,192) qh (high 2 bits)
 *    [192,208) sc[16] int8, one per 16 weights   [208,210) d (fp16)
 *    weight i = 128n + 32s + l (n in {0,1}, s in 0..3, l in 0..31):
 *      low 4 bits: ql[64n + 32*(s&1) + l], low nibble if s<2 else high nibble
 *      high 2 bits: (qh[32n + l] >> 2s) & 3
 *      w = d * sc[i/16] * (q - 32)
 *
 *  Q8 activation (32-element blocks, fp16 scale, int8 values):
 *    amax = max|x|, d = amax/127 (f32, correctly rounded),
 *    q = round-half-away-from-zero(x/d) (f32 division), scale stored as the
 *    fp16 (round-to-nearest-even) of d; amax == 0 gives d = 0 and q = 0.
 *    memra-engine decode.rs (`ffn_swiglu_decode` doc comment) names the
 *    "amax/127" rounding; the fp16 scale and 32-element block size come from
 *    the problem statement of the 70B-class FFN workload.
 *
 * Parity pins for every function live in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define Q4K_BLOCK_BYTES 144
#define Q6K_BLOCK_BYTES 210
#define QK 256

/* ---------------------------------------------------------------- fp16 */

/* IEEE-754 binary16 -> f64, from the definition: 1 sign bit, 5 exponent bits
 * (bias 15), 10 mantissa bits; exponent 0 = subnormal (m * 2^-24), exponent 31
 * = inf (m == 0) or NaN. */
double orc_fp16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = (m == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* f32 -> IEEE binary16 bits, round to nearest, ties to even, from the
 * definition: find the binary16 spacing (ulp) at |f|, divide (exact: both are
 * powers of two apart), round the quotient to an integer with ties to even,
 * then re-encode.  Overflow past the largest finite value rounds to inf. */
uint16_t orc_f32_to_fp16_rne(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    double a = fabs((double)f);
    if (isnan(f))
        return sign | 0x7E00;
    if (isinf(f))
        return sign | 0x7C00;
    if (a == 0.0)
        return sign;
    int ex;
    frexp(a, &ex);             /* a = fr * 2^ex, fr in [0.5, 1) */
    int E = ex - 1;            /* a in [2^E, 2^(E+1)) */
    if (E < -14)
        E = -14;               /* subnormal range shares the 2^-24 spacing */
    double ulp = ldexp(1.0, E - 10);
    double t = a / ulp;        /* exact */
    double fl = floor(t);
    double diff = t - fl;
    double r = fl;
    if (diff > 0.5 || (diff == 0.5 && fmod(fl, 2.0) != 0.0))
        r = fl + 1.0;
    double v = r * ulp;        /* the rounded magnitude */
    if (v >= 65536.0)
        return sign | 0x7C00;
    if (v < ldexp(1.0, -14))   /* subnormal (or rounded up to 2^-14, handled below) */
        return sign | (uint16_t)r;
    int ev;
    frexp(v, &ev);
    int e = ev - 1;            /* v in [2^e, 2^(e+1)) */
    uint16_t mant = (uint16_t)(v / ldexp(1.0, e - 10) - 1024.0);
    return sign | (uint16_t)((e + 15) << 10) | mant;
}

/* -------------------------------------------------------------- Q4_K */

/* Unpack one Q4_K super-block into its fields: d, dmin, the 8 (scale, min)
 * pairs and the 256 raw 4-bit quants in weight order. */
void orc_q4k_fields(const uint8_t *blk, double *d, double *dmin, int sc[8],
                    int mn[8], int q[256])
{
    const uint8_t *s = blk + 4;
    const uint8_t *qs = blk + 16;
    *d = orc_fp16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
    *dmin = orc_fp16_to_f64((uint16_t)(blk[2] | (blk[3] << 8)));
    for (int j = 0; j < 8; ++j) {
        if (j < 4) {
            sc[j] = s[j] & 63;
            mn[j] = s[j + 4] & 63;
        } else {
            sc[j] = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
            mn[j] = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
        }
    }
    for (int j = 0; j < 8; ++j) {
        for (int i = 0; i < 32; ++i) {
            uint8_t byte = qs[32 * (j / 2) + i];
            q[32 * j + i] = (j % 2 == 0) ? (byte & 15) : (byte >> 4);
        }
    }
}

/* Q4_K super-block -> 256 f64 weights: w = d*sc*q - dmin*m (exact in f64). */
void orc_q4k_block(const uint8_t *blk, double *w)
{
    double d, dmin;
    int sc[8], mn[8], q[256];
    orc_q4k_fields(blk, &d, &dmin, sc, mn, q);
    for (int i = 0; i < 256; ++i) {
        int j = i / 32;
        w[i] = d * sc[j] * q[i] - dmin * mn[j];
    }
}

/* -------------------------------------------------------------- Q6_K */

/* Unpack one Q6_K super-block: d, the 16 int8 scales and 256 quants 0..63. */
void orc_q6k_fields(const uint8_t *blk, double *d, int sc[16], int q[256])
{
    const uint8_t *ql = blk;
    const uint8_t *qh = blk + 128;
    const int8_t *s = (const int8_t *)(blk + 192);
    *d = orc_fp16_to_f64((uint16_t)(blk[208] | (blk[209] << 8)));
    for (int g = 0; g < 16; ++g)
        sc[g] = s[g];
    for (int i = 0; i < 256; ++i) {
        int n = i / 128, s4 = (i % 128) / 32, l = i % 32;
        uint8_t lowbyte = ql[64 * n + 32 * (s4 % 2) + l];
        int nib = (s4 < 2) ? (lowbyte & 15) : (lowbyte >> 4);
        int hi = (qh[32 * n + l] >> (2 * s4)) & 3;
        q[i] = nib | (hi << 4);
    }
}

/* Q6_K super-block -> 256 f64 weights: w = d * sc[i/16] * (q - 32). */
void orc_q6k_block(const uint8_t *blk, double *w)
{
    double d;
    int sc[16], q[256];
    orc_q6k_fields(blk, &d, sc, q);
    for (int i = 0; i < 256; ++i)
        w[i] = d * sc[i / 16] * (q[i] - 32);
}

/* --------------------------------------------------------------- GEMV */

/* y[n] = sum_k w[n,k] * x[k], W row-major: row n = blocks n*nb .. n*nb+nb-1. */
void orc_q4k_gemv(const uint8_t *W, const float *x, double *y, int64_t N, int64_t K)
{
    int64_t nb = K / QK;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double w[256];
        double acc = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            orc_q4k_block(W + (n * nb + b) * Q4K_BLOCK_BYTES, w);
            for (int i = 0; i < 256; ++i)
                acc += w[i] * (double)x[b * QK + i];
        }
        y[n] = acc;
    }
}

void orc_q6k_gemv(const uint8_t *W, const float *x, double *y, int64_t N, int64_t K)
{
    int64_t nb = K / QK;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double w[256];
        double acc = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            orc_q6k_block(W + (n * nb + b) * Q6K_BLOCK_BYTES, w);
            for (int i = 0; i < 256; ++i)
                acc += w[i] * (double)x[b * QK + i];
        }
        y[n] = acc;
    }
}

/* Same GEMVs over f64 activations (the SwiGLU down projection of an f64 h). */
void orc_q6k_gemv_f64x(const uint8_t *W, const double *x, double *y, int64_t N, int64_t K)
{
    int64_t nb = K / QK;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double w[256];
        double acc = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            orc_q6k_block(W + (n * nb + b) * Q6K_BLOCK_BYTES, w);
            for (int i = 0; i < 256; ++i)
                acc += w[i] * x[b * QK + i];
        }
        y[n] = acc;
    }
}

/* ------------------------------------------------------------- SwiGLU */

/* h = silu(Wg x) * (Wu x), silu(z) = z / (1 + e^-z) (memra-engine decode.rs,
 * `ffn_swiglu_decode`: down @ (silu(gate@z) * (up@z))).  g and u are the
 * exact f64 GEMVs; g and u are also returned for diagnostics. */
void orc_swiglu(const uint8_t *Wg, const uint8_t *Wu, const float *x, double *h,
                double *g, double *u, int64_t N, int64_t K)
{
    orc_q4k_gemv(Wg, x, g, N, K);
    orc_q4k_gemv(Wu, x, u, N, K);
    for (int64_t n = 0; n < N; ++n)
        h[n] = g[n] * u[n] / (1.0 + exp(-g[n]));
}

/* --------------------------------------------------------- Q8 quantize */

/* The decision that turns floats into integers is taken in f32, as the
 * method states it (amax/127, then a rounded quotient); only the stored
 * scale goes through fp16.  x must be finite. */
void orc_q8_quantize(const float *x, int8_t *q, uint16_t *dfp16, int64_t K)
{
    for (int64_t j = 0; j < K / 32; ++j) {
        const float *xb = x + 32 * j;
        float amax = 0.0f;
        for (int i = 0; i < 32; ++i) {
            float a = fabsf(xb[i]);
            if (a > amax)
                amax = a;
        }
        volatile float d = amax / 127.0f; /* f32, correctly rounded */
        for (int i = 0; i < 32; ++i) {
            int v = 0;
            if (d != 0.0f) {
                volatile float t = xb[i] / d;  /* f32 division */
                double r = round((double)t);   /* half away from zero */
                if (r > 127.0)
                    r = 127.0;
                if (r < -127.0)
                    r = -127.0;
                v = (int)r;
            }
            q[32 * j + i] = (int8_t)v;
        }
        dfp16[j] = orc_f32_to_fp16_rne(d);
    }
}

/* ------------------------------------------------------- Q4_K x Q8 path */

/* Integer part of the int8-dot path, exact: for row n and 32-element block j
 * (block j of the activation meets sub-block j%8 of super-block j/8),
 * isum[n][j] = sum_i q4[n][32j+i] * q8[32j+i]. */
void orc_q4k_q8_isums(const uint8_t *W, const int8_t *xq, int32_t *isums, int64_t N, int64_t K)
{
    int64_t nb = K / QK;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double d, dmin;
        int sc[8], mn[8], q[256];
        for (int64_t b = 0; b < nb; ++b) {
            orc_q4k_fields(W + (n * nb + b) * Q4K_BLOCK_BYTES, &d, &dmin, sc, mn, q);
            for (int j = 0; j < 8; ++j) {
                int32_t s = 0;
                for (int i = 0; i < 32; ++i)
                    s += q[32 * j + i] * (int32_t)xq[b * QK + 32 * j + i];
                isums[n * (K / 32) + b * 8 + j] = s;
            }
        }
    }
}

/* y = W * xdq with xdq[k] = fp16(d8[k/32]) * q8[k], the dequantized Q8
 * activation; f64 weights, f64 accumulation. */
void orc_q4k_q8_gemv(const uint8_t *W, const int8_t *xq, const uint16_t *xd, double *y,
                     int64_t N, int64_t K)
{
    int64_t nb = K / QK;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double w[256];
        double acc = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            orc_q4k_block(W + (n * nb + b) * Q4K_BLOCK_BYTES, w);
            for (int i = 0; i < 256; ++i) {
                int64_t k = b * QK + i;
                double xk = orc_fp16_to_f64(xd[k / 32]) * (double)xq[k];
                acc += w[i] * xk;
            }
        }
        y[n] = acc;
    }
}

/* ------------------------------------------------------- Q6_K x Q8 path */

/* Integer part of the Q6_K int8-dot path (the Q6_K x Q8 ffn_down of the
 * memra-engine decode.rs q8_1 fast path, `ffn_swiglu_decode`: the SwiGLU
 * epilogue emits a quantized activation that ffn_down consumes through
 * `matmul_pre`), exact: for row n and 16-element group g, the granularity
 * of the Q6_K scales, isum[n][g] = sum_i (q6[n][16g+i] - 32) * q8[16g+i]. */
void orc_q6k_q8_isums(const uint8_t *W, const int8_t *xq, int32_t *isums, int64_t N, int64_t K)
{
    int64_t nb = K / QK;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double d;
        int sc[16], q[256];
        for (int64_t b = 0; b < nb; ++b) {
            orc_q6k_fields(W + (n * nb + b) * Q6K_BLOCK_BYTES, &d, sc, q);
            for (int g = 0; g < 16; ++g) {
                int32_t s = 0;
                for (int i = 0; i < 16; ++i)
                    s += (q[16 * g + i] - 32) * (int32_t)xq[b * QK + 16 * g + i];
                isums[n * (K / 16) + b * 16 + g] = s;
            }
        }
    }
}

/* y = W * xdq over Q6_K rows, xdq the dequantized Q8 activation
 * (fp16(d8[k/32]) * q8[k]); f64 weights, f64 accumulation. */
void orc_q6k_q8_gemv(const uint8_t *W, const int8_t *xq, const uint16_t *xd, double *y,
                     int64_t N, int64_t K)
{
    int64_t nb = K / QK;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double w[256];
        double acc = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            orc_q6k_block(W + (n * nb + b) * Q6K_BLOCK_BYTES, w);
            for (int i = 0; i < 256; ++i) {
                int64_t k = b * QK + i;
                double xk = orc_fp16_to_f64(xd[k / 32]) * (double)xq[k];
                acc += w[i] * xk;
            }
        }
        y[n] = acc;
    }
}

/* ------------------------------------------------------------- argmax */

/* First index of the maximum over the non-NaN values; 0 when every value is
 * NaN.  -0 and +0 compare equal, so the smaller index wins between them.
 * First index of an exact maximum: the tie rule of the greedy GPU argmax in
 * aprender PR #4332 ("What changed", item (b)) and of the host candidate merge
 * in qualiaDB resident_decode.rs (`run_resident_token`). */
int64_t orc_argmax_first_f64(const double *v, int64_t n)
{
    int64_t best = -1;
    for (int64_t i = 0; i < n; ++i) {
        if (isnan(v[i]))
            continue;
        if (best < 0 || v[i] > v[best])
            best = i;
    }
    return best < 0 ? 0 : best;
}

int64_t orc_argmax_first_f32(const float *v, int64_t n)
{
    int64_t best = -1;
    for (int64_t i = 0; i < n; ++i) {
        if (isnan(v[i]))
            continue;
        if (best < 0 || v[i] > v[best])
            best = i;
    }
    return best < 0 ? 0 : best;
}

/* Masked argmax (memra-engine decode.rs, `decode_step_dc_cap_masked`: a
 * grammar mask bans tokens before the argmax reads the row).  Row i is banned
 * when bit (i % 32) of mask[i / 32] is set; banned and NaN rows are skipped;
 * the first index of the largest remaining value wins; none left gives 0. */
static int orc_banned(const uint32_t *mask, int64_t i)
{
    return (int)((mask[i / 32] >> (i % 32)) & 1u);
}

int64_t orc_argmax_first_masked_f64(const double *v, const uint32_t *mask, int64_t n)
{
    int64_t best = -1;
    for (int64_t i = 0; i < n; ++i) {
        if (isnan(v[i]) || orc_banned(mask, i))
            continue;
        if (best < 0 || v[i] > v[best])
            best = i;
    }
    return best < 0 ? 0 : best;
}

int64_t orc_argmax_first_masked_f32(const float *v, const uint32_t *mask, int64_t n)
{
    int64_t best = -1;
    for (int64_t i = 0; i < n; ++i) {
        if (isnan(v[i]) || orc_banned(mask, i))
            continue;
        if (best < 0 || v[i] > v[best])
            best = i;
    }
    return best < 0 ? 0 : best;
}

/* Number of OpenMP threads a parallel region uses (1 without OpenMP). */
int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
