/*
 * gemvq -- batch-1 quantized GEMV for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libgemvq.so.  Every entry point enqueues its kernels on the
 * caller's HIP stream and returns without synchronising; stream order is the
 * only dependency between calls (the aprender-serve page, forward_qwen35_cuda.rs,
 * enqueues every projection GEMV on one stream with no host sync).  No call
 * allocates device or host memory, reads device memory on the host or keeps
 * state between calls (aprender PR #4332, "What changed": zero per-token host
 * and device allocations, a 4-byte download per token).
 *
 * Shapes and layout.  N = rows = output length, K = columns = input length
 * (the weight handle on the aprender-serve page, `CudaQuantWeight`, carries
 * n = out_dim and k = in_dim).  K is a multiple of 256: each row is K/256
 * super-blocks stored back to back, rows back to back (row n starts at byte
 * n * (K/256) * block_bytes).  Block formats are GGUF Q4_K (144 bytes per
 * 256 weights) and Q6_K (210 bytes per 256 weights); the Q8 activation is
 * int8 values plus one fp16 scale per 32 values.
 *
 * Pointers.  Every pointer argument is a DEVICE pointer owned by the caller
 * (the library never frees or keeps one).  `stream` is a hipStream_t passed as
 * void* (NULL = the null stream).  fp16 values are passed as their uint16_t
 * bit patterns.
 *
 * Errors.  Every argument check happens on the host BEFORE any HIP call, so a
 * rejected call has no effect on the device.  A launch failure reported by
 * the runtime after the launch returns GEMVQ_ERR_HIP.
 *
 * Limits.  1 <= N <= 2^31 - 1; 256 <= K <= 32768; N * (K/256) * block_bytes
 * must fit in 63 bits.  Alignment: weights 16 B (Q4_K) or 4 B (Q6_K), float
 * vectors 16 B (inputs) / 4 B (outputs; the norms' outputs 16 B), int8 Q8
 * vector 16 B, Q8 scales 4 B.  Outputs may not overlap any input, except
 * where an entry point below allows an exact in-place update (a residual
 * output over its residual input).
 */
#ifndef GEMVQ_H
#define GEMVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define GEMVQ_OK            0
#define GEMVQ_ERR_NULL      1  /* a required pointer is NULL */
#define GEMVQ_ERR_SHAPE     2  /* N < 1, K < 256, K % 256 != 0, K > 32768, size overflow */
#define GEMVQ_ERR_ALIGN     3  /* a pointer violates the alignment above */
#define GEMVQ_ERR_WORKSPACE 4  /* workspace too small */
#define GEMVQ_ERR_ALIAS     5  /* an output overlaps an input */
#define GEMVQ_ERR_HIP       6  /* the HIP runtime reported an error at launch */
#define GEMVQ_ERR_VALUE     7  /* a scalar argument is out of range (eps) */

/*
 * y[n] = sum_k W[n,k] * x[k] over a Q4_K matrix, f32 activation, f32 result.
 * The float (non-int8) GEMV: the aprender-serve page pins the float Q4_K/Q6_K
 * variants (`pin_float_gemv`, "Q4kVariant::Mwv") as the correctness default.
 *   W: N*(K/256)*144 bytes.  x: float[K].  y: float[N] (written).
 */
int q4k_gemv(const void *W, const float *x, float *y, int64_t N, int64_t K, void *stream);

/*
 * Several Q4_K matrices of the same K against one x in a single launch, with
 * an optional residual added to each output: y_i = W_i x (+ residual_i)
 * (memra-engine decode.rs: the q, k and v projections share their input and
 * run as one launch, split by block offset, and the small beta/alpha pair
 * likewise, so launch-latency-sized GEMVs stop paying a launch each;
 * qualiaDB resident_decode.rs: the output projection adds the residual in the
 * GEMV's epilogue, `coop_gemv_residual`).  One pass streams all matrices,
 * every row reduced inside one wave.
 *   W, N, y: host arrays of `count` (1..4) device pointers / row counts;
 *   W[i]: Q4_K N[i] x K; y[i]: float[N[i]] (written).
 *   residual: NULL, or a host array of `count` device pointers, each NULL or
 *   float[N[i]]; residual[i] may equal y[i] (in-place add), no other overlap.
 *   x: float[K], 256 <= K <= 14336 (x and its sums are staged in LDS).
 * Errors as q4k_gemv; count outside 1..4 or a larger K is GEMVQ_ERR_SHAPE.
 */
int q4k_gemv_multi(const void *const *W, const int64_t *N, float *const *y, const float *const *residual,
                   int count, const float *x, int64_t K, void *stream);

/*
 * Same over a Q6_K matrix (210-byte blocks): the ffn_down projection and the
 * unfused lm_head (aprender-serve forward_qwen35_cuda.rs, the lm_head
 * `gemv_dispatch` at the end of `forward_single`).
 *   W: N*(K/256)*210 bytes.  x: float[K].  y: float[N].
 * Row results are bit-identical to the row values lm_head_argmax compares.
 */
int q6k_gemv(const void *W, const float *x, float *y, int64_t N, int64_t K, void *stream);

/*
 * Quantize an f32 activation to Q8 (memra-engine decode.rs, `quantize_q8_1`
 * and the "amax/127" rounding named in `ffn_swiglu_decode`): per 32-element
 * block, d = max|x|/127 in f32 (correctly rounded), q = round-half-away-from-
 * zero(x/d) with an f32 division, scale stored as fp16 (round to nearest
 * even); a block of zeros gives d = 0 and q = 0.  x must be finite.
 *   x: float[K] (K % 32 == 0, 32 <= K <= 65536).  xq: int8[K].  xd: uint16[K/32].
 */
int q8_quantize(const float *x, int8_t *xq, uint16_t *xd, int64_t K, void *stream);

/*
 * Q4_K x Q8 integer-dot GEMV: the approximate fast variant that quantizes the
 * activation first (aprender-serve `pin_reference_gemv` doc comment: the int8
 * activation path is an intentional approximation; memra-engine `matmul_pre`
 * on a pre-quantized activation).  Per 32-block j of row n the integer sum
 * isum = sum q4*q8 is exact; y[n] = sum_j d8_j*(d*sc_j*isum_j - dmin*m_j*sum q8).
 *   W: Q4_K N x K.  xq, xd: the output of q8_quantize for the same K.  y: float[N].
 */
int q4k_q8_gemv(const void *W, const int8_t *xq, const uint16_t *xd, float *y,
                int64_t N, int64_t K, void *stream);

/*
 * q8_quantize followed by q4k_q8_gemv as one call on an f32 activation (the
 * problem statement's configuration: activations quantized on the device to
 * Q8, then int8 dot products; memra-engine decode.rs `ffn_swiglu_decode`
 * quantizes the activation right before the pre-quantized GEMV).  Where
 * q4k_q8_gemv runs its wave-unit kernel (K/256 a power of two up to 16, or
 * K = 8192), every workgroup quantizes x in its own prologue, with the
 * encoder q8_quantize uses, while its first weight loads are in flight, and
 * no separate quantize launch exists; other shapes run the two launches.
 * Either way xq, xd receive exactly q8_quantize(x) and y exactly
 * q4k_q8_gemv(W, xq, xd) (bit for bit).
 *   W: Q4_K N x K.  x: float[K], finite.  xq: int8[K] (16-B aligned).
 *   xd: uint16[K/32].  y: float[N].  Outputs overlap no input and each other.
 */
int q4k_q8_gemv_from_f32(const void *W, const float *x, int8_t *xq, uint16_t *xd, float *y,
                         int64_t N, int64_t K, void *stream);

/*
 * Q6_K x Q8 integer-dot GEMV, the int8 ffn_down: on the pages' q8 fast path
 * the down projection consumes an already quantized activation (memra-engine
 * decode.rs `ffn_swiglu_decode`: the SwiGLU epilogue emits the q8 form of its
 * product and ffn_down reads it through `matmul_pre`).  Per 16-element group
 * g of row n the integer sum isum_g = sum (q6 - 32) * q8 is exact;
 * y[n] = d * sum_g sc_g * isum_g * d8_(g/2), with d8 the scale of the Q8 block
 * the group lies in.
 *   W: Q6_K N x K.  xq, xd: a Q8 activation of length K (q8_quantize,
 *   rms_norm_q8 or swiglu_q8_gemv output).  y: float[N].
 */
int q6k_q8_gemv(const void *W, const int8_t *xq, const uint16_t *xd, float *y,
                int64_t N, int64_t K, void *stream);

/*
 * Fused gate/up SwiGLU GEMV: h[n] = silu(g[n]) * u[n], g = Wg x, u = Wu x,
 * silu(z) = z / (1 + e^-z), both matrices read in one pass that shares x
 * (memra-engine decode.rs `ffn_swiglu_decode`: down @ (silu(gate@z) * (up@z));
 * qualiaDB resident_decode.rs: the fused FFN pass needs gate and up of the
 * same type and dims).  Follow with q6k_gemv(Wd, h) for the down projection.
 *   Wg, Wu: Q4_K N x K.  x: float[K].  h: float[N].
 */
int swiglu_gemv(const void *Wg, const void *Wu, const float *x, float *h,
                int64_t N, int64_t K, void *stream);

/*
 * Batched int8-activation GEMV: Y[j] = W * xdq_j for m activation vectors,
 * one pass over the weights (memra-engine decode.rs: the lockstep
 * multi-stream decode advances m streams through one walk of the layers,
 * and `full_attn_decode_batched` runs the weight-bound projections once for
 * all m streams, one weight read serving m tokens).  Each output row is the
 * single-vector Q8 GEMV of its vector, computed the same way whatever m and
 * whatever the other vectors hold.
 *   W: Q4_K (q4k_q8_gemv_batch) or Q6_K (q6k_q8_gemv_batch) N x K.
 *   xq: int8[m][K], xd: uint16[m][K/32] (m Q8 activations back to back, e.g.
 *   q8_quantize of the m vectors stored back to back as one vector of m*K).
 *   y: float[m][N].  1 <= m <= 8.  A Q6_K launch takes at most 4 vectors
 *   (their int8 slices next to the Q6_K blocks fill the register file), so
 *   q6k_q8_gemv_batch with m > 4 reads the weights twice; so does
 *   q4k_q8_gemv_batch for large matrices (more than 200 KB of weights per
 *   compute unit), where two passes of 4 vectors beat one of 8.
 */
int q4k_q8_gemv_batch(const void *W, const int8_t *xq, const uint16_t *xd, float *y,
                      int64_t N, int64_t K, int m, void *stream);
int q6k_q8_gemv_batch(const void *W, const int8_t *xq, const uint16_t *xd, float *y,
                      int64_t N, int64_t K, int m, void *stream);

/*
 * SwiGLU GEMV that emits its product as a Q8 activation: the producer-side
 * quantization of memra-engine decode.rs `ffn_swiglu_decode` (the SwiGLU
 * epilogue writes the q8 form of silu(gate)*up, `silu_mul_scaled_q8_1`, and
 * the down projection reads it directly, with no separate quantize launch),
 * stated there to be bit-identical to the unfused sequence.  Here hq/hd equal
 * q8_quantize applied to the h that swiglu_gemv writes whenever swiglu_gemv
 * runs its tile kernel for the same N x K (every K/256 that is not a power of
 * two up to 16, e.g. K = 2560); for other K the rows are summed in another
 * order and only the parity bound holds.  Pair with q6k_q8_gemv.
 *   Wg, Wu: Q4_K N x K.  x: float[K].  N % 32 == 0.
 *   h: float[N] or NULL (the f32 product is also written when given).
 *   hq: int8[N], hd: uint16[N/32] (fp16 scale bits), as q8_quantize writes.
 *   workspace: >= gemvq_swiglu_q8_ws_bytes(N) bytes, 256-byte aligned; its
 *   first N/32 * 4 bytes (per-block counters) must be zero before the first
 *   call, and every call leaves them zero; the rest needs no initial value.
 *   Calls that share a workspace must not run concurrently.
 */
int swiglu_q8_gemv(const void *Wg, const void *Wu, const float *x, float *h, int8_t *hq, uint16_t *hd,
                   void *workspace, size_t ws_bytes, int64_t N, int64_t K, void *stream);

/* Workspace bytes swiglu_q8_gemv needs for N rows (0 if N is not a positive
 * multiple of 32).  Host-only. */
size_t gemvq_swiglu_q8_ws_bytes(int64_t N);

/*
 * RMS norm that emits a Q8 activation (memra-engine decode.rs
 * `rms_norm_q8_1`: the attention-input norm writes the quantized activation
 * of the following projections directly).  The pages name the norm and its
 * eps without writing it out; this is the usual RMS norm,
 *   y[i] = w[i] * x[i] / sqrt(sum_j x[j]^2 / K + eps),
 * followed by the Q8 encoding of y exactly as q8_quantize does it.
 *   x, w: float[K], K % 32 == 0, 32 <= K <= 32768.  eps >= 0 and finite.
 *   y: float[K] or NULL (the f32 norm is also written when given).
 *   xq: int8[K], xd: uint16[K/32].
 *   Alignment: every float vector (x, w, y, and r, res below) 16 bytes.
 * Runs as one workgroup (a latency-bound vector op).
 */
int rms_norm_q8(const float *x, const float *w, float eps, float *y, int8_t *xq, uint16_t *xd, int64_t K,
                void *stream);

/*
 * Residual add, RMS norm and Q8 encoding in one launch (memra-engine
 * decode.rs `add_rms_norm_q8_1`: the post-attention residual add, the FFN
 * norm and its quantization; the sum is the new residual stream).
 *   res[i] = x[i] + r[i] (f32, written); then rms_norm_q8 of res.
 *   res may be x or r itself (in-place update); no other overlap.
 */
int add_rms_norm_q8(const float *x, const float *r, const float *w, float eps, float *res, float *y, int8_t *xq,
                    uint16_t *xd, int64_t K, void *stream);

/*
 * lm_head GEMV over Q6_K rows with an on-device argmax: writes the FIRST index
 * of the maximum row value (NaN rows never win; -0 == +0; all-NaN gives 0) to
 * out_idx[0] and, if out_max is not NULL, that value to out_max[0].  No logits
 * are written anywhere; the caller downloads 4 bytes (aprender PR #4332: the
 * tie fix keeps the first index of an exact maximum, and the download drops
 * from 248,320 f32 logits to a 4-byte token id; memra-engine decode.rs
 * `argmax_token_device_into`: the id stays in a persistent device word).
 * Two stages in one kernel: every workgroup reduces its rows to one (value,
 * index) candidate kept as an order-keeping 64-bit key and merges it into a
 * running key in the workspace with an atomic max; the last workgroup to
 * finish (a done counter) reads the running key, writes the result and sets
 * both words back to zero (memra-engine decode.rs names the same split,
 * `argmax_partial_f32` + `argmax_final_f32`; qualiaDB's top-1 per block and
 * candidate merge).
 *   W: Q6_K N x K.  x: float[K].  out_idx: uint32[1].  out_max: float[1] or NULL.
 *   workspace: device memory of at least gemvq_lm_head_argmax_ws_bytes(N, K)
 *   (12,288) bytes, 256-B aligned.  Its first 4096 bytes (the counters)
 *   must be zero before the first call; every call leaves them zero again, so
 *   one workspace serves any number of calls in stream order (also inside a
 *   captured graph).  The rest is reserved and needs no initial value.  Calls
 *   that share a workspace must not run concurrently.
 */
int lm_head_argmax(const void *W, const float *x, uint32_t *out_idx, float *out_max,
                   void *workspace, size_t ws_bytes, int64_t N, int64_t K, void *stream);

/*
 * lm_head_argmax with device timestamps: the same work, checks and errors.
 * start_event and stop_event are hipEvent_t handles (passed as void*) that
 * the caller created with timing enabled, or NULL.  When given, the GEMV
 * kernel's own start and end are recorded into them (hipExtLaunchKernel), so
 * hipEventElapsedTime(start_event, stop_event) is the kernel's duration
 * without the gaps around it: the per-launch time that a bandwidth figure
 * needs (aprender PR #4332 times decode per token; this times the lm_head
 * call itself).  The events stay owned by the caller.
 */
int lm_head_argmax_timed(const void *W, const float *x, uint32_t *out_idx, float *out_max,
                         void *workspace, size_t ws_bytes, int64_t N, int64_t K, void *stream,
                         void *start_event, void *stop_event);

/*
 * lm_head_argmax over the rows a mask allows: rows whose bit is set in `mask`
 * are banned and never win, exactly as if their value were NaN (memra-engine
 * decode.rs `decode_step_dc_cap_masked`: a grammar mask bans tokens before
 * the argmax reads the row, and the masked device argmax equals the masked
 * host argmax).  The result is the first index of the largest value among the
 * allowed, non-NaN rows; if there is none, 0 (out_max NaN).
 *   mask: uint32[ceil(N/32)], device memory, 4-B aligned; bit (i % 32) of
 *   word i / 32 bans row i; bits past N are ignored.  Other arguments,
 *   workspace rules and errors as lm_head_argmax; mask NULL is GEMVQ_ERR_NULL.
 */
int lm_head_argmax_masked(const void *W, const float *x, const uint32_t *mask, uint32_t *out_idx,
                          float *out_max, void *workspace, size_t ws_bytes, int64_t N, int64_t K,
                          void *stream);

/*
 * lm_head_argmax for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernel, result, checks and errors, but the workspace is the
 * library's own file-scope device array of gemvq_lm_head_argmax_ws_bytes()
 * (12,288) bytes, one per GPU, held until the process ends; no call
 * allocates.  The first call on a GPU looks up the array's address and clears
 * its counters with a small kernel on `stream`, ordered before the argmax
 * launch; every call leaves them zero.  Any shape lm_head_argmax accepts fits
 * the array (the argmax grid, and so the workspace, has a fixed maximum).
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (concurrent streams, or threads without ordering) race and give wrong
 * results; calls ordered on one stream, or in one captured graph, are safe.
 *   W, x, out_idx, out_max, N, K, stream: as lm_head_argmax.
 */
int lm_head_argmax_noalloc(const void *W, const float *x, uint32_t *out_idx, float *out_max,
                           int64_t N, int64_t K, void *stream);

/* Workspace bytes lm_head_argmax needs for an N x K call (host-only, no HIP call). */
size_t gemvq_lm_head_argmax_ws_bytes(int64_t N, int64_t K);

/*
 * Test hook for the exactness of the int8 path: writes the integer sums
 * isums[n][j] = sum_{i<32} q4[n][32j+i] * xq[32j+i] computed by the same
 * device decode and dot code as q4k_q8_gemv (before any scaling).
 *   isums: int32[N][K/32].
 */
int gemvq_q4k_q8_isums(const void *W, const int8_t *xq, int32_t *isums,
                       int64_t N, int64_t K, void *stream);

/*
 * Test hook for the Q6_K x Q8 path: isums[n][g] = sum_{i<16}
 * (q6[n][16g+i] - 32) * xq[16g+i] from the same device decode and dot code as
 * q6k_q8_gemv.
 *   isums: int32[N][K/16].
 */
int gemvq_q6k_q8_isums(const void *W, const int8_t *xq, int32_t *isums,
                       int64_t N, int64_t K, void *stream);

/*
 * Launch geometry of the GEMV kernels for an N x K matrix (host-only, no HIP
 * call; for tests and tuning).  kind: 0 = Q4_K (q4k_gemv), 1 = Q6_K (q6k_gemv,
 * lm_head_argmax), 2 = Q4_K x Q8 (q4k_q8_gemv), 3 = SwiGLU (swiglu_gemv),
 * 4 = Q6_K x Q8 (q6k_q8_gemv), 5 = SwiGLU with Q8 emission (swiglu_q8_gemv,
 * N % 32 == 0), 6 / 7 = batched Q4_K / Q6_K x Q8 (the geometry and the LDS of
 * 8 vector slots).
 * out[0] = waves per workgroup, out[1] = rows per tile, out[2] = tiles,
 * out[3] = 1 if a row's partial sums reduce inside one wave, out[4] = 1 if the
 * activation is staged through LDS, out[5] = dynamic LDS bytes, out[6] =
 * steps.  When out[3] is 1 a tile is one wave's rows, taken by the waves of
 * one workgroup per CU, and out[0] is the most waves such a workgroup has (the
 * launch uses as many as fit on a CU): with out[6] = 1 a tile is
 * 64 / (4*K/256) rows side by side; with out[6] = 2 (Q4_K x Q8 at
 * K = 8192) it is one row whose lane l takes quarter l%4 of super-blocks
 * l/4 and 16 + l/4.  out[7] = 1 for the wave-unit kernel: there a lane's
 * byte offset within a unit never changes, and on a ragged matrix the last
 * unit starts at row N - rows (its lanes whose rows the unit before covered
 * are idle); with N < rows, lanes past N read the unit's first super-block.
 * out[8] = 1 for the tile kernel's CU-resident form (one workgroup per CU at
 * most, each owning contiguous tiles, out[9] of them or fewer, all in flight
 * at once; workgroup w owns tiles [w*q + min(w, r), ...) with q, r the
 * quotient and remainder of the tiles over the out[10] workgroups), 0 for
 * the ring form (out[9] = out[10] = 0).  The resident choice depends on the
 * device's CU count; this hook assumes 256 (MI355X).
 * Returns GEMVQ_ERR_SHAPE for shapes the GEMV entry points reject.
 */
int gemvq_tile_geometry(int kind, int64_t N, int64_t K, int64_t out[11]);

/*
 * Measurement hook: a plain streaming read of `bytes` (a multiple of 16,
 * 16-B aligned) at device address p, each byte read once with 16-byte
 * loads by `grid` workgroups of `threads` threads (256 or 1024;
 * grid-stride).  It is the ceiling the GEMVs' achieved bandwidth is
 * compared with at the same byte count (its best time over workgroup sizes
 * and grids).  sink: device uint32[256], written only if the folded data
 * equals one fixed value (in practice never).
 * Returns GEMVQ_ERR_SHAPE for bytes < 16, not a multiple of 16, grid
 * outside [1, 65536] or threads other than 256 and 1024.
 */
int gemvq_stream_read(const void *p, int64_t bytes, int grid, int threads, uint32_t *sink, void *stream);

/* Static description of a status code (never NULL). */
const char *gemvq_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* GEMVQ_H */
