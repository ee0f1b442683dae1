// gfx950 kernels of the batch-1 quantized GEMV path and their launchers.
//
// One kernel template serves the f32-activation Q4_K and Q6_K GEMVs, the
// fused gate/up SwiGLU GEMV, the Q4_K x Q8 integer-dot GEMV and the lm_head
// GEMV with argmax.  Lane geometry is described in gemvq_device.h: each lane
// owns one quarter of one super-block column of the rows in a tile and keeps
// the 64 activation values of that quarter in registers, so the steady state
// streams weight bytes only.  A row's value is the sum of its 4*(K/256) lane
// partials; the summation tree depends only on K, never on which workgroup,
// wave or tile holds the row, so equal rows give bit-identical values (the
// argmax tie rule relies on this) and q6k_gemv's outputs are exactly the values
// lm_head_argmax compares.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "gemvq_device.h"
#include "gemvq_launch.h"

namespace gemvq {

enum Kind : int { kQ4K = 0, kQ6K = 1, kQ4KQ8 = 2, kSwiglu = 3, kQ6KQ8 = 4 };
constexpr bool is_q8(int kind) { return kind == kQ4KQ8 || kind == kQ6KQ8; }   // int8 activation
constexpr bool is_q6(int kind) { return kind == kQ6K || kind == kQ6KQ8; }     // Q6_K weights
// kQ8Emit: the tile kernel's rows are also encoded as a Q8 activation (the
// SwiGLU product feeding an int8 down projection)
enum Epi : int { kStore = 0, kArgmax = 1, kArgmaxMasked = 2, kQ8Emit = 3 };
constexpr bool is_argmax(int epi) { return epi == kArgmax || epi == kArgmaxMasked; }


struct GemvArgs {
    const uint8_t *W;      // matrix (gate matrix for SwiGLU)
    const uint8_t *W2;     // up matrix for SwiGLU
    const float *x;        // f32 activation
    const int8_t *xq;      // Q8 activation values
    const uint16_t *xd;    // Q8 activation scales (fp16 bits)
    float *y;              // output (h for SwiGLU)
    uint32_t *out_idx;     // argmax result
    float *out_max;        // argmax value or nullptr
    uint8_t *ws;           // argmax workspace
    const uint32_t *mask;  // masked argmax: bit (i & 31) of word i >> 5 set = row i banned
    int64_t N;
    int tiles;             // ceil(N / rows_tile)
    int tiles_q, tiles_r;  // tiles per workgroup: tiles_q, plus one for the first tiles_r workgroups
    int nb;                // super-blocks per row
    int lanes_row;         // lanes per row: 4 * nb (64 for the two-step wave kernel)
    uint32_t lanes_row_magic;  // ceil(2^32 / lanes_row): tid / lanes_row == umulhi(tid, magic) for tid < 1024
    int rows_tile;         // rows per tile (P)
    int x_in_lds;          // stage the activation (and its 16-element sums) through LDS first
    int steps;             // row-stream kernel: 16-super-block steps per row
    int chunk_shift;       // wave/row-stream kernels: units are dealt in chunks of 1 << chunk_shift
    // multi-output launches (gemv_rows_kernel<..., MULTI = 1>): up to kMaxMulti
    // matrices of the same K; units [ustart[m], ustart[m+1]) belong to matrix m
    const uint8_t *Wm[kMaxMulti];
    float *ym[kMaxMulti];
    const float *rm[kMaxMulti];   // residual added to y, or nullptr
    int64_t Nm[kMaxMulti];
    int ustart[kMaxMulti + 1];
    // Q8 emission (EPI == kQ8Emit): codes and scales of the rows, the byte
    // offset of the row values in the workspace (ws), and of the workgroup's
    // row buffer in LDS
    int8_t *hq;
    uint16_t *hd;
    uint32_t emit_vals_off;
    uint32_t emit_lds_off;
    // batched GEMV (gemv_batch_kernel): vectors, and how many are staged in
    // LDS per round
    int batch;
    int batch_round;
    // tile kernel: byte offset of the row-reduction buffer in LDS
    uint32_t red_off;
    // threads per workgroup (blockDim.x), set by the launch.  The tile and
    // batch kernels read it from here: blockDim.x comes from the implicit
    // kernel arguments through a vector load that the compiler may issue
    // after the weight loads, and vector-memory counters retire in order, so
    // its wait then waited for every weight load issued before it.
    int threads;
};

// ------------------------------------------------------- activation setup

template <int KIND>
struct XSlice;
template <> struct XSlice<kQ4K> { Q4KX v; };
template <> struct XSlice<kSwiglu> { Q4KX v; };
template <> struct XSlice<kQ6K> { Q6KX v; };
template <> struct XSlice<kQ4KQ8> { Q8X v; };
template <> struct XSlice<kQ6KQ8> { Q6Q8X v; };
// Slices in fixed point: the wave-unit kernel holds Q6_K activations as
// Q6KFX, the row-stream kernel f32 Q4_K ones as Q4KFX, and the tile kernel
// Q6_K ones as Q6KFX when it stages x in LDS; everything else uses XSlice.
struct FXSlice { Q6KFX v; };
template <int KIND> struct WaveSlice { using T = XSlice<KIND>; };
template <> struct WaveSlice<kQ6K> { using T = FXSlice; };
struct FX4Slice { Q4KFX v; };
template <int KIND> struct RowsSlice { using T = XSlice<KIND>; };
template <> struct RowsSlice<kQ4K> { using T = FX4Slice; };
template <int KIND, bool FX> struct TileSlice { using T = XSlice<KIND>; };
template <> struct TileSlice<kQ6K, true> { using T = FXSlice; };
template <> struct TileSlice<kQ4K, true> { using T = FX4Slice; };
template <> struct TileSlice<kSwiglu, true> { using T = FX4Slice; };

// Activation form of the tile kernel when it stages x in LDS: fixed point
// (true) or f32.  Q6_K always takes fixed point (its f32 dot needs two more
// byte permutes per four weights).  The resident Q4_K forms (single matrix
// and SwiGLU pair) take it too: their dot products run after the weight
// stream has arrived (f32: ~1.75 VALU operations per weight, fixed point
// ~1.1), and the conversion runs under the first tile's loads.  Measured
// against the f32 form at 2560 x 9728, 9728 x 2560 and 4096 x 2560:
// 5.94 -> 5.12, 5.60 -> 5.05 and 4.40 -> 4.01 us.  The ring form keeps f32:
// its many short-lived workgroups each pay the conversion at start-up.
constexpr bool tile_fx(int kind, bool xlds, bool res)
{
    return xlds && (kind == kQ6K || (res && (kind == kSwiglu || kind == kQ4K)));
}

// Layout of the activation staged in LDS: 16 bytes of padding after every
// 256 bytes.  A lane's slice is 64 consecutive bytes (Q8) or 64 consecutive
// floats (Q4_K), and lanes read slices 64 or 256 bytes apart; unpadded, all
// lanes of a read pass would hit the same four LDS banks (up to 16-way
// conflicts).  The padding shifts consecutive lanes onto different banks.
// Every 16-byte chunk, 16-float segment or 64-byte slice the kernels read
// starts and ends inside one 256-byte span, so it stays contiguous.
__device__ __forceinline__ uint32_t lds_pad(uint32_t byte_off) { return byte_off + ((byte_off >> 8) << 4); }

// Address of activation element i: straight (global x) or in the padded LDS
// layout.
template <bool PADDED>
__device__ __forceinline__ const float *x_at(const float *base, int i)
{
    if constexpr (PADDED)
        return (const float *)((const unsigned char *)base + lds_pad(4u * (uint32_t)i));
    else
        return base + i;
}

__device__ __forceinline__ void load_x_f32(float *dst, const float *src, int n)
{
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
        if (i < n) {
            const float4 v = *(const float4 *)(src + i);
            dst[i] = v.x;
            dst[i + 1] = v.y;
            dst[i + 2] = v.z;
            dst[i + 3] = v.w;
        }
    }
}

// Sum of 16 consecutive activation values, added in index order.  Every
// activation sum the kernels use is built from these, whether a lane adds
// its own slice or a workgroup precomputes them in LDS, so both give the
// same bits.
__device__ __forceinline__ float sum16(const float *v)
{
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) t += v[i];
    return t;
}

// Q4_K part c of block b: xl = x[256b + 64c + i], xh = x[256b + 64c + 32 + i].
template <bool PADDED = false>
__device__ __forceinline__ void load_x(Q4KX &xs, const float *xsrc, int b, int c)
{
    const int o = kQK * b + 64 * c;
#pragma unroll
    for (int i = 0; i < 32; i += 16) {
        load_x_f32(xs.xl + i, x_at<PADDED>(xsrc, o + i), 16);
        load_x_f32(xs.xh + i, x_at<PADDED>(xsrc, o + 32 + i), 16);
    }
}

// The slice's two 32-element sums: from `sums` (16-element sums of x held in
// LDS) or, when it is null, added here from the slice.
__device__ __forceinline__ void finish_x(Q4KX &xs, const float *sums, int b, int c)
{
    float sl, sh;
    if (sums) {
        const float *q = sums + 16 * b + 4 * c;
        sl = q[0] + q[1];
        sh = q[2] + q[3];
    } else {
        sl = sum16(xs.xl) + sum16(xs.xl + 16);
        sh = sum16(xs.xh) + sum16(xs.xh + 16);
    }
    pin(sl);
    pin(sh);
    xs.sxl = sl;
    xs.sxh = sh;
}

// Q6_K part u of block b: xs[s][i] = x[256b + 128n + 32s + l0 + i].
template <bool PADDED = false>
__device__ __forceinline__ void load_x(Q6KX &xs, const float *xsrc, int b, int u)
{
    const int n = u >> 1, l0 = 16 * (u & 1);
    const int o = kQK * b + 128 * n + l0;
#pragma unroll
    for (int s = 0; s < 4; ++s) load_x_f32(xs.xs[s], x_at<PADDED>(xsrc, o + 32 * s), 16);
}

__device__ __forceinline__ void finish_x(Q6KX &xs, const float *sums, int b, int u)
{
    const int n = u >> 1;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        float t = sums ? sums[16 * b + 8 * n + 2 * s + (u & 1)] : sum16(xs.xs[s]);
        pin(t);
        xs.sx[s] = t;
    }
}

// Q8 part c of block b: 32 int8 of sub-blocks 8b+2c and 8b+2c+1, their scales.
template <bool PADDED = false>
__device__ __forceinline__ void load_x(Q8X &xs, const int8_t *qsrc, const uint16_t *dsrc, int b, int c)
{
    const uint32_t o = (uint32_t)(kQK * b + 64 * c);
    const uint32_t *p = (const uint32_t *)(qsrc + (PADDED ? lds_pad(o) : o));
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        xs.ql[k] = p[k];
        xs.qh[k] = p[8 + k];
    }
    xs.dl = xs.dh = 0.f;
    if (dsrc) {
        const int j = 8 * b + 2 * c;
        xs.dl = (float)__builtin_bit_cast(_Float16, dsrc[j]);
        xs.dh = (float)__builtin_bit_cast(_Float16, dsrc[j + 1]);
    }
}

// The fp16 scale words of a lane's Q8 slice, loaded on their own so that
// they can go out with the activation codes, before any weight load: the
// two scales of Q8X part c of block b (one dword: scales 8b+2c, 8b+2c+1), or
// the four of Q6Q8X part u (two dwords: scales 8b+4n .. 8b+4n+3).  The
// scale array is 4-byte aligned.
__device__ __forceinline__ void load_xd(uint32_t (&w)[2], const uint16_t *dsrc, const Q8X *, int b, int c)
{
    w[0] = *(const uint32_t *)(dsrc + 8 * b + 2 * c);
    w[1] = 0u;
}
__device__ __forceinline__ void load_xd(uint32_t (&w)[2], const uint16_t *dsrc, const Q6Q8X *, int b, int u)
{
    const uint32_t *dp = (const uint32_t *)(dsrc + 8 * b + 4 * (u >> 1));
    w[0] = dp[0];
    w[1] = dp[1];
}
// The slice's scales from those words (the same values load_x reads).
__device__ __forceinline__ void set_xd(Q8X &xs, const uint32_t (&w)[2])
{
    xs.dl = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[0] & 0xFFFFu));
    xs.dh = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[0] >> 16));
}
__device__ __forceinline__ void set_xd(Q6Q8X &xs, const uint32_t (&w)[2])
{
    xs.d2[0] = w[0];
    xs.d2[1] = w[1];
}

// Integer sums of the slice's two Q8 blocks.
__device__ __forceinline__ void finish_x(Q8X &xs)
{
    int32_t sl = 0, sh = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        sl = __builtin_amdgcn_sdot4((int)xs.ql[k], 0x01010101, sl, false);
        sh = __builtin_amdgcn_sdot4((int)xs.qh[k], 0x01010101, sh, false);
    }
    pin(sl);
    pin(sh);
    xs.sl = sl;
    xs.sh = sh;
}

// Q8 part u of a Q6_K block b: group s = x[256b + 128n + 32s + l0 + i], i < 16,
// and the scale of Q8 block 8b + 4n + s.
template <bool PADDED = false>
__device__ __forceinline__ void load_x(Q6Q8X &xs, const int8_t *qsrc, const uint16_t *dsrc, int b, int u)
{
    const int n = u >> 1, l0 = 16 * (u & 1);
    const uint32_t o = (uint32_t)(kQK * b + 128 * n + l0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint32_t os = o + 32u * (uint32_t)s;
        const uint32_t *p = (const uint32_t *)(qsrc + (PADDED ? lds_pad(os) : os));
#pragma unroll
        for (int k = 0; k < 4; ++k) xs.q[s][k] = p[k];
    }
    // the group scales are those of Q8 blocks 8b + 4n .. 8b + 4n + 3
    xs.d2[0] = xs.d2[1] = 0u;
    if (dsrc) {
        const uint16_t *dp = dsrc + 8 * b + 4 * n;
        xs.d2[0] = (uint32_t)dp[0] | ((uint32_t)dp[1] << 16);
        xs.d2[1] = (uint32_t)dp[2] | ((uint32_t)dp[3] << 16);
    }
}

// Integer sums of the slice's four 16-element groups, two to a dword.
__device__ __forceinline__ void finish_x(Q6Q8X &xs)
{
    int32_t t[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        t[s] = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) t[s] = __builtin_amdgcn_sdot4((int)xs.q[s][k], 0x01010101, t[s], false);
    }
    int32_t a = (int32_t)(((uint32_t)t[0] & 0xFFFFu) | ((uint32_t)t[1] << 16));
    int32_t c = (int32_t)(((uint32_t)t[2] & 0xFFFFu) | ((uint32_t)t[3] << 16));
    pin(a);
    pin(c);
    xs.sx2[0] = (uint32_t)a;
    xs.sx2[1] = (uint32_t)c;
}

// ------------------------------------------------------- per-kind traits

template <int KIND> struct Traits;
template <> struct Traits<kQ4K> {
    typedef Q4KRaw Raw;
    static constexpr int kBytes = kQ4KBytes;
    static constexpr int kOuts = 1;
};
template <> struct Traits<kQ4KQ8> {
    typedef Q4KRaw Raw;
    static constexpr int kBytes = kQ4KBytes;
    static constexpr int kOuts = 1;
};
template <> struct Traits<kQ6K> {
    typedef Q6KRaw Raw;
    static constexpr int kBytes = kQ6KBytes;
    static constexpr int kOuts = 1;
};
template <> struct Traits<kQ6KQ8> {
    typedef Q6KRaw Raw;
    static constexpr int kBytes = kQ6KBytes;
    static constexpr int kOuts = 1;
};
template <> struct Traits<kSwiglu> {
    typedef Q4KRaw Raw;
    static constexpr int kBytes = kQ4KBytes;
    static constexpr int kOuts = 2;
};

template <int KIND>
struct RawSet {
    typename Traits<KIND>::Raw r[Traits<KIND>::kOuts];
};

template <int KIND>
__device__ __forceinline__ void zero_raw(RawSet<KIND> &rs)
{
    if constexpr (is_q6(KIND)) {
        q6k_zero(rs.r[0]);
    } else {
        q4k_zero(rs.r[0]);
        if constexpr (KIND == kSwiglu) q4k_zero(rs.r[1]);
    }
}

template <int KIND, class XS>
__device__ __forceinline__ void dot_raw(const RawSet<KIND> &rs, const XS &xs, int part, float (&out)[2])
{
    if constexpr (KIND == kQ6K) {
        out[0] = q6k_dot(rs.r[0], xs.v, part);
    } else if constexpr (KIND == kQ6KQ8) {
        out[0] = q6k_q8_dot(rs.r[0], xs.v, part);
    } else if constexpr (KIND == kQ4KQ8) {
        out[0] = q4k_q8_dot(rs.r[0], xs.v, part);
    } else {
        out[0] = q4k_dot(rs.r[0], xs.v, part);
        if constexpr (KIND == kSwiglu) out[1] = q4k_dot(rs.r[1], xs.v, part);
    }
}

// ---------------------------------------------------------------- epilogue

// Running argmax of a thread: the largest key (argmax_key) of the rows it has
// emitted; NaN rows are skipped, and so are banned rows of a masked argmax
// (`mword` is the mask word holding the row's bit), 0 means none.
template <int KIND, int EPI>
__device__ __forceinline__ void emit_row(const GemvArgs &a, int64_t row, const float (&v)[2], uint64_t &best,
                                         uint32_t mword = 0)
{
    if constexpr (is_argmax(EPI)) {
        const bool banned = EPI == kArgmaxMasked && ((mword >> (row & 31)) & 1u);
        const uint64_t k = (v[0] != v[0] || banned) ? 0ull : argmax_key(v[0], (uint32_t)row);
        best = k > best ? k : best;
    } else if constexpr (KIND == kSwiglu) {
        const float g = v[0], u = v[1];
        a.y[row] = g * u / (1.0f + expf(-g));
    } else {
        a.y[row] = v[0];
    }
}

// Workspace of lm_head_argmax (offsets in bytes; each word on a 128-byte line
// of its own):
//   [0, 4)      done counter: workgroups that have published their key
//   [128, 136)  running key: the largest key published so far
// Both are zero between calls.
__device__ __forceinline__ uint32_t *ws_count(uint8_t *ws) { return (uint32_t *)ws; }
__device__ __forceinline__ uint64_t *ws_key(uint8_t *ws) { return (uint64_t *)(ws + kArgmaxKeyOff); }

// Grid-level argmax: the threads' running keys meet in LDS (one barrier) and
// wave 0 folds them with DPP and lane reads.  Thread 0 then merges the
// workgroup's key into the running key with a returning atomic max (device
// scope) and counts the workgroup done.  The max's returned value is consumed
// behind a compiler memory barrier before the count is issued, so the count
// leaves the CU only after the max has been performed at the device's
// coherence point; the workgroup whose count completes the grid then reads
// the running key there with a device-scope load and sees every merged key.
// It writes the 4-byte result and sets both words back to zero.  Keys are
// order-keeping (argmax_key), so the largest key is the largest value with
// the smallest index, whatever order the workgroups finish in.  A release
// add and an acquire load would state the same order in the memory model,
// but on this target they write back and invalidate the XCD's L2 (measured:
// the timed lm_head 37.12 -> 37.80 us); device-scope atomics need neither to
// be coherent across the XCDs.  The last workgroup waits for three dependent
// round trips (max, count, read).
// `holders` threads (0..holders-1) carry running keys.
__device__ void argmax_finish(const GemvArgs &a, uint64_t best, int holder, int holders)
{
    __shared__ uint64_t s_key[kMaxThreads];
    if (holder >= 0) s_key[holder] = best;
    __syncthreads();
    if (threadIdx.x >= 64) return;   // wave 0 finishes
    uint64_t k = 0;
    for (int h = (int)threadIdx.x; h < holders; h += 64) k = s_key[h] > k ? s_key[h] : k;
    k = wave_max_key(k);
    if (threadIdx.x != 0) return;
    if (k) {
        const uint64_t old = __hip_atomic_fetch_max(ws_key(a.ws), k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("" ::"v"(old) : "memory");   // consumed: the max is performed before the count
    }
    const uint32_t prev = __hip_atomic_fetch_add(ws_count(a.ws), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev != gridDim.x - 1) return;
    const uint64_t top = __hip_atomic_load(ws_key(a.ws), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    a.out_idx[0] = top ? argmax_key_index(top) : 0u;
    if (a.out_max) a.out_max[0] = top ? argmax_key_value(top) : __builtin_nanf("");
    __hip_atomic_store(ws_key(a.ws), 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(ws_count(a.ws), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------ Q8 emission

// Q8 encoding of one 32-element block held one value per lane of a 32-lane
// half-wave (lane l holds element l): amax by a lane-max tree (exact,
// order-free), d = amax/127 and q = round(v/d) in f32 with correctly rounded
// division (the HIP default), q rounded half away from zero (roundf) and
// clamped to [-127, 127]; the scale is stored as the fp16 of d (round to
// nearest even).  Every producer of Q8 activations uses this one function,
// so their codes agree bit for bit on equal inputs.
__device__ __forceinline__ float q8_scale(float amax) { return amax / 127.0f; }
__device__ __forceinline__ uint16_t q8_scale_bits(float d) { return __builtin_bit_cast(uint16_t, (_Float16)d); }
__device__ __forceinline__ int q8_code(float v, float d)
{
    int q = 0;
    if (d != 0.0f) {
        float r = roundf(v / d);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        q = (int)r;
    }
    return q;
}

__device__ __forceinline__ int8_t q8_encode(float v, uint16_t &dbits)
{
    float amax = fabsf(v);
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 32));
    const float d = q8_scale(amax);
    dbits = q8_scale_bits(d);
    return (int8_t)q8_code(v, d);
}

// The codes q8_code gives for NV values of one block (scale d), packed four
// to a word (value 4k + j in byte j of word k), with one division per block
// instead of one per value.  Each quotient is taken as q = v * (1/d), both
// products rounded to nearest: |q - v/d| <= (2^-23 + 2^-48) |v/d|, and the
// correctly rounded v/d that q8_code rounds is within 2^-24 |v/d| of v/d.
// Since |v/d| <= 127 (1 + 2^-23), q and q8_code's quotient differ by less than
// 2^-15, so both round to the same integer unless a half-integer lies within
// that distance.  A value whose q has a fractional part within 2^-13 of 0.5
// (or is not a number), or a block whose d is zero, subnormal or not finite,
// takes q8_code itself for all NV values.  The codes are q8_code's bit for
// bit (checked on the CPU against the exact division over adversarial
// quotients next to every k + 0.5).
template <int NV>
__device__ __forceinline__ void q8_codes_fast(const float (&v)[NV], float d, uint32_t (&w)[NV / 4])
{
    const float y = 1.0f / d;
    bool slow = !(d >= 0x1p-126f && d <= 0x1p+126f);
    int c[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const float q = v[i] * y;
        const float t = truncf(q);
        const float f = fabsf(q - t);   // exact for |q| < 2^23
        slow = slow || !(fabsf(f - 0.5f) >= 0x1p-13f);
        const float r = f >= 0.5f ? t + copysignf(1.0f, q) : t;   // half away from zero, as roundf
        c[i] = (int)fminf(fmaxf(r, -127.0f), 127.0f);
    }
    if (slow) {
#pragma unroll
        for (int i = 0; i < NV; ++i) c[i] = q8_code(v[i], d);
    }
#pragma unroll
    for (int k = 0; k < NV / 4; ++k)
        w[k] = (uint32_t)(c[4 * k] & 0xFF) | ((uint32_t)(c[4 * k + 1] & 0xFF) << 8) |
               ((uint32_t)(c[4 * k + 2] & 0xFF) << 16) | ((uint32_t)(c[4 * k + 3] & 0xFF) << 24);
}

// Q8 encoding of the rows a workgroup of the tile kernel computed, [r0, r1)
// (values in LDS).  A 32-row block that lies inside the range is encoded
// right here.  A block shared with other workgroups goes through the
// workspace: each sharer publishes its rows with returning atomic exchanges
// (device scope, coherent across the XCDs, performed before the count),
// then adds its row count to the block's counter; the sharer whose count
// completes 32 reads the block back, encodes it and clears the counter, so
// every counter is zero again between calls.  No workgroup waits for
// another.  Workspace: counters (u32 per block) at ws[0], row values at
// ws[emit_vals_off].  As in argmax_finish, the order of the exchanges before
// the count comes from consuming their returned values behind a compiler
// memory barrier; a release add and acquire loads measured 10.5 -> 13.8 us
// at 9728 x 2560 (L2 writeback and invalidation).
__device__ void q8_emit_finish(const GemvArgs &a, const float *s_h, int64_t r0, int64_t r1)
{
    __syncthreads();   // every row of the range is in LDS
    if (r1 <= r0) return;
    const int l = threadIdx.x & 31;
    const int hw = (int)(threadIdx.x >> 5), nhw = a.threads >> 5;
    uint32_t *cnt = (uint32_t *)a.ws;
    uint32_t *vals = (uint32_t *)(a.ws + a.emit_vals_off);
    const int64_t jb = r0 >> 5, je = (r1 - 1) >> 5;
    for (int64_t j = jb + hw; j <= je; j += nhw) {   // uniform over the half-wave
        const int64_t b0 = j << 5;
        const int64_t lo = b0 > r0 ? b0 : r0;
        const int64_t hi = b0 + 32 < r1 ? b0 + 32 : r1;
        const int64_t row = b0 + l;
        const bool mine = row >= lo && row < hi;
        float v = mine ? s_h[row - r0] : 0.f;
        if (lo != b0 || hi != b0 + 32) {
            if (mine) {
                const uint32_t old = __hip_atomic_exchange(vals + row, __float_as_uint(v), __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
                asm volatile("" ::"v"(old) : "memory");   // consumed: performed before the count below
            }
            uint32_t prev = 0;
            if (l == 0)
                prev = __hip_atomic_fetch_add(cnt + j, (uint32_t)(hi - lo), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            prev = (uint32_t)__shfl((int)prev, 0, 32);
            if (prev + (uint32_t)(hi - lo) != 32u) continue;   // another sharer completes the block
            v = __uint_as_float(__hip_atomic_load(vals + row, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            if (l == 0) __hip_atomic_store(cnt + j, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        uint16_t dbits;
        const int8_t q = q8_encode(v, dbits);
        a.hq[row] = q;
        if (l == 0) a.hd[j] = dbits;
    }
}

// ------------------------------------------------------------------ kernel

// Fixed-point activation of the row-stream and tile kernels, in LDS: the high,
// middle and low byte arrays of X (K bytes each, padded layout), then the
// 16-element f32 sums (K/16), then the per-part exponents (K/64 ints).
__device__ __forceinline__ uint32_t fx4_sums_off(int K) { return 3u * lds_pad((uint32_t)K); }
__device__ __forceinline__ uint32_t fx4_exps_off(int K) { return fx4_sums_off(K) + 4u * (uint32_t)(K / 16); }

// Group g (16 values v, in registers) of the activation: its f32 sum (added
// in index order, as sum16 does) and its fixed-point bytes.  The four groups
// of one 64-value part sit in one quad of lanes and share the part's largest
// |x| by DPP; the quad's first lane (lead) writes the part's exponent at index
// eidx.  Call with whole quads active.
__device__ void fx_stage_group(unsigned char *smem, int K, int g, int eidx, bool lead, const float (&v)[16])
{
    float t = 0.f, m = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        t += v[i];
        m = fmaxf(m, fabsf(v[i]));
    }
    ((float *)(smem + fx4_sums_off(K)))[g] = t;
    m = fmaxf(m, dpp_f<kDppQuadXor1>(m));
    m = fmaxf(m, dpp_f<kDppQuadXor2>(m));
    const int e = (m > 0.f && m <= 3.402823466e38f) ? 22 - __builtin_amdgcn_frexp_expf(m) : 0;
    uint32_t hi[4], mid[4], lo[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        int X[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) X[j] = (int)rintf(__builtin_amdgcn_ldexpf(v[4 * k + j], e));
        const uint32_t p01 = __builtin_amdgcn_perm((uint32_t)X[1], (uint32_t)X[0], 0x05010400u);
        const uint32_t p23 = __builtin_amdgcn_perm((uint32_t)X[3], (uint32_t)X[2], 0x05010400u);
        const uint32_t r01 = __builtin_amdgcn_perm((uint32_t)X[1], (uint32_t)X[0], 0x07030602u);
        const uint32_t r23 = __builtin_amdgcn_perm((uint32_t)X[3], (uint32_t)X[2], 0x07030602u);
        lo[k] = __builtin_amdgcn_perm(p23, p01, 0x05040100u);
        mid[k] = __builtin_amdgcn_perm(p23, p01, 0x07060302u);
        hi[k] = __builtin_amdgcn_perm(r23, r01, 0x05040100u);
    }
    const uint32_t stride = lds_pad((uint32_t)K);
    const uint32_t o = lds_pad(16u * (uint32_t)g);
    *(u32x4 *)(smem + o) = u32x4{hi[0], hi[1], hi[2], hi[3]};
    *(u32x4 *)(smem + stride + o) = u32x4{mid[0], mid[1], mid[2], mid[3]};
    *(u32x4 *)(smem + 2 * stride + o) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    if (lead) ((int *)(smem + fx4_exps_off(K)))[eidx] = e;
}

// Lane slice of part c of block b from the staged fixed-point activation.
__device__ __forceinline__ void fx4_load(Q4KFX &xs, const unsigned char *smem, int K, int b, int c)
{
    const uint32_t stride = lds_pad((uint32_t)K);
    const int P = 4 * b + c;   // the part's 64 values start at element 64P
    const uint32_t o = lds_pad(64u * (uint32_t)P);   // 64 bytes inside one padded 256-byte span
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const u32x4 h = *(const u32x4 *)(smem + o + 16 * q);
        const u32x4 m = *(const u32x4 *)(smem + stride + o + 16 * q);
        const u32x4 l = *(const u32x4 *)(smem + 2 * stride + o + 16 * q);
        xs.hi[4 * q] = h.x; xs.hi[4 * q + 1] = h.y; xs.hi[4 * q + 2] = h.z; xs.hi[4 * q + 3] = h.w;
        xs.mid[4 * q] = m.x; xs.mid[4 * q + 1] = m.y; xs.mid[4 * q + 2] = m.z; xs.mid[4 * q + 3] = m.w;
        xs.lo[4 * q] = l.x; xs.lo[4 * q + 1] = l.y; xs.lo[4 * q + 2] = l.z; xs.lo[4 * q + 3] = l.w;
    }
    const float *sums = (const float *)(smem + fx4_sums_off(K));
    float sl = sums[4 * P] + sums[4 * P + 1], sh = sums[4 * P + 2] + sums[4 * P + 3];
    pin(sl);
    pin(sh);
    xs.sxl = sl;
    xs.sxh = sh;
    xs.e = -((const int *)(smem + fx4_exps_off(K)))[P];
}

// The same layout for Q6_K parts (tile kernel): part slot t (block t >> 4,
// part (t >> 2) & 3, group t & 3 of the part) is 16-element group g of the
// activation; the exponent sits at the part's index 4*block + part = t >> 2.
__device__ __forceinline__ int fx6_group_of_slot(int t)
{
    const int blk = t >> 4, u = (t >> 2) & 3, sg = t & 3;
    return 16 * blk + 8 * (u >> 1) + 2 * sg + (u & 1);
}

__device__ __forceinline__ void fx6_load(Q6KFX &xs, const unsigned char *smem, int K, int b, int u)
{
    const int n = u >> 1;
    const uint32_t stride = lds_pad((uint32_t)K);
    const int e = ((const int *)(smem + fx4_exps_off(K)))[4 * b + u];
    const float *sums = (const float *)(smem + fx4_sums_off(K));
#pragma unroll
    for (int sg = 0; sg < 4; ++sg) {
        const int g = 16 * b + 8 * n + 2 * sg + (u & 1);
        const uint32_t o = lds_pad(16u * (uint32_t)g);
        const u32x4 h = *(const u32x4 *)(smem + o);
        const u32x4 m = *(const u32x4 *)(smem + stride + o);
        const u32x4 l = *(const u32x4 *)(smem + 2 * stride + o);
        xs.hi[sg][0] = h.x; xs.hi[sg][1] = h.y; xs.hi[sg][2] = h.z; xs.hi[sg][3] = h.w;
        xs.mid[sg][0] = m.x; xs.mid[sg][1] = m.y; xs.mid[sg][2] = m.z; xs.mid[sg][3] = m.w;
        xs.lo[sg][0] = l.x; xs.lo[sg][1] = l.y; xs.lo[sg][2] = l.z; xs.lo[sg][3] = l.w;
        float t = -32.f * __builtin_amdgcn_ldexpf(sums[g], e);
        pin(t);
        xs.m[sg] = t;
    }
    xs.e = -e;
}

// Stages the f32 activation of a tile or row-stream launch in fixed point:
// thread tid converts slot tid and slot tid + blockDim from the values it
// loaded first (xg0, xg1), then any further slots straight from x.
template <int KIND>
__device__ __forceinline__ void fx_stage_all(unsigned char *smem, const float *x, int K, const float (&xg0)[16],
                                             const float (&xg1)[16])
{
    const int slots = K / 16, tid = (int)threadIdx.x, bd = (int)blockDim.x;
    auto stage = [&](int t, const float (&v)[16]) {
        if constexpr (KIND == kQ6K) fx_stage_group(smem, K, fx6_group_of_slot(t), t >> 2, (t & 3) == 0, v);
        else fx_stage_group(smem, K, t, t >> 2, (t & 3) == 0, v);
    };
    if (tid < slots) stage(tid, xg0);
    if (tid + bd < slots) stage(tid + bd, xg1);
    for (int t = tid + 2 * bd; t < slots; t += bd) {
        const int g = KIND == kQ6K ? fx6_group_of_slot(t) : t;
        float v[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 f = *(const float4 *)(x + 16 * g + 4 * q);
            v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
        }
        stage(t, v);
    }
}

// The 16 values of slot t of the activation (t < K/16), for the preload.
template <int KIND>
__device__ __forceinline__ void fx_preload(float (&v)[16], const float *x, int K, int t)
{
    if (t < K / 16) {
        const int g = KIND == kQ6K ? fx6_group_of_slot(t) : t;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 f = *(const float4 *)(x + 16 * g + 4 * q);
            v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
        }
    }
}

// Tile kernel, for rows that do not fit an aligned power-of-two lane group of
// one wave: a tile of rows spans the workgroup, each super-block's quad sum
// goes through LDS and one thread per row adds the K/256 block sums in order.
// PHASE: tiles in flight per lane (software pipeline depth); 1 for grids in
// which workgroups own a single tile.  XLDS: the activation (and its
// 16-element sums) is staged through LDS because several rows of a tile
// share it; otherwise each lane reads its own slice.
// RES: the CU-resident form, for mid-size matrices (a few tiles per CU).
// At most one workgroup per CU; it owns PHASE tiles or fewer and issues the
// loads of all of them before anything else waits, so the CU's whole share
// of the matrix is in flight at once.  Every tile's block sums then go to a
// buffer of their own and one barrier precedes the row sums, which are
// added in the same order as in the ring form (same bits).
// MULTI (CU-resident Q4_K store only): up to kMaxMulti matrices of the same
// K sharing x, their tiles numbered one matrix after the other (a.ustart[m]
// is matrix m's first tile; a tile holds rows of one matrix only), each with
// its own output and optional residual.
template <int KIND, int EPI, int PHASE, bool XLDS, bool RES, bool MULTI>
__device__ __forceinline__ void gemv_tile_body(GemvArgs a)
{
    static_assert(!MULTI || (RES && KIND == kQ4K && EPI == kStore), "multi-output tiles: resident Q4_K store");
    constexpr int kPhase = PHASE;
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int BYTES = Traits<KIND>::kBytes;
    constexpr int OUTS = Traits<KIND>::kOuts;
    const int tid = threadIdx.x;
    // threads per workgroup, from the arguments (see GemvArgs::threads)
    auto nthr = [&]() -> int { return a.threads; };
    const int p = (int)__umulhi((uint32_t)tid, a.lanes_row_magic);   // row within the tile
    const int rr = tid - p * a.lanes_row;     // lane within the row
    const int b = rr >> 2;                    // super-block column
    const int part = rr & 3;                  // quarter of the super-block
    const bool lane_on = p < a.rows_tile;
    const int K = a.nb * kQK;

    const int bid = blockIdx.x;
    const int t_begin = bid * a.tiles_q + (bid < a.tiles_r ? bid : a.tiles_r);
    const int t_end = t_begin + a.tiles_q + (bid < a.tiles_r ? 1 : 0);
    // rows of the last tile that exist (the tail may be ragged)
    const int last_rows = (int)(a.N - (a.tiles - 1) * a.rows_tile);
    const int64_t tile_stride = (int64_t)a.rows_tile * a.nb * BYTES;   // bytes per tile
    const uint32_t lane_off = (uint32_t)((p * a.nb + b) * BYTES);      // < tile_stride

    // multi-output: the matrix of tile t (workgroup-uniform)
    auto mat_of = [&](int t) {
        int m = 0;
        if constexpr (MULTI) {
#pragma unroll
            for (int j = 1; j < kMaxMulti; ++j) m += t >= a.ustart[j] ? 1 : 0;
        }
        return m;
    };
    auto valid_tile = [&](int t) {
        if constexpr (MULTI) {
            const int m = mat_of(t);
            return lane_on && t < t_end && (int64_t)(t - a.ustart[m]) * a.rows_tile + p < a.Nm[m];
        }
        return lane_on && t < t_end && (t < a.tiles - 1 || p < last_rows);
    };
    // Loads are unconditional so no branch surrounds them (a branch, even a
    // uniform one, makes the compiler drain every outstanding load at the loop
    // head): a tile past this workgroup's range re-reads its last tile (an L2
    // hit), a lane with nothing to do reads the first super-block of the tile
    // (always in bounds), and the partial sums of both are discarded.
    auto fetch = [&](RawSet<KIND> &rs, int t) {
        const int tt = t < t_end ? t : t_end - 1;
        const uint32_t off = valid_tile(t) ? lane_off : 0u;
        if constexpr (MULTI) {
            const int m = mat_of(tt);
            q4k_load(rs.r[0], a.Wm[m] + (int64_t)(tt - a.ustart[m]) * tile_stride, off, part);
            return;
        }
        const int64_t tb = (int64_t)tt * tile_stride;
        if constexpr (is_q6(KIND)) {
            q6k_load(rs.r[0], a.W + tb, off, part);
        } else {
            q4k_load(rs.r[0], a.W + tb, off, part);
            if constexpr (KIND == kSwiglu) q4k_load(rs.r[1], a.W2 + tb, off, part);
        }
    };

    // The activation's global loads go first, then the first weight tiles:
    // vector-memory counters retire in issue order, so staging x waits only
    // for x while the weight tiles stay in flight behind it.
    // A fixed-point activation (tile_fx) is staged from two slots of 16
    // values per thread, loaded first and converted once the x loads are in.
    // In the ring form Q4_K and the SwiGLU pair keep f32: their launches of
    // many short-lived workgroups are bound by start-up, which the
    // conversion lengthens (measured slower at 2560 x 9728 and 9728 x 2560).
    constexpr bool kFx = tile_fx(KIND, XLDS, RES);
    // A resident workgroup with a fixed-point activation issues its first
    // tile's weight loads, converts x while they are in flight, and issues the
    // remaining tiles right after the staging barrier, before its own slice
    // reads (6.80 -> 6.55 us at 2560 x 9728 against after the slice).  Issue is throttled by
    // the memory pipeline (a wave waits at each load until the CU accepts it),
    // so with every tile issued first the conversion started only once most
    // of the stream was out, and the dot products waited for it; with x
    // converted before any weight load the stream started late.  Measured
    // with device timestamps at 2560 x 9728 (Q6_K) and 9728 x 2560 (SwiGLU):
    // x staged at ~2.8 us instead of ~4.2 (all tiles first) and 7.6 -> 6.8,
    // 8.7 -> 8.3 us per call.  The other forms issue every tile first.
    constexpr int kPre = (RES && kFx) ? 1 : kPhase;   // tiles fetched before the conversion
    static_assert(kFx || kPre == kPhase, "only the fixed-point form defers tiles");
    float xg0[16], xg1[16];
    if constexpr (kFx) {
        fx_preload<KIND>(xg0, a.x, K, tid);
        fx_preload<KIND>(xg1, a.x, K, tid + nthr());
    }
    // float4 (or 16 int8) staged per thread through registers; a resident
    // workgroup has 768 threads, so 4 cover K <= 12288 in f32
    constexpr int kXRegs = kFx ? 1 : (RES ? 4 : 8);
    u32x4 xr[kXRegs];
    if constexpr (XLDS && !kFx) {
        const int step = is_q8(KIND) ? 16 : 4;   // elements per 16-byte load
        const uint8_t *src = is_q8(KIND) ? (const uint8_t *)a.xq : (const uint8_t *)a.x;
        const int esz = is_q8(KIND) ? 1 : 4;
#pragma unroll
        for (int r = 0; r < kXRegs; ++r) {
            const int i = (tid + r * nthr()) * step;
            if (i < K) xr[r] = *(const u32x4 *)(src + (size_t)i * esz);
        }
    }
    typename TileSlice<KIND, kFx>::T xs;
    const int xb = lane_on ? b : 0;
    if constexpr (!XLDS) {
        // each lane reads its own slice (no other lane of the tile shares it)
        if constexpr (is_q8(KIND))
            load_x(xs.v, a.xq, nullptr, xb, part);
        else
            load_x(xs.v, a.x, xb, part);
    }
    // the lane's Q8 scale words go out with the codes, before the weights: a
    // scale load issued after them would wait for every one of them
    uint32_t xdw[2];
    if constexpr (is_q8(KIND)) load_xd(xdw, a.xd, &xs.v, xb, part);
    if constexpr (!XLDS && is_q8(KIND)) set_xd(xs.v, xdw);
    RawSet<KIND> ring[kPhase];
    // A large activation (K > 4096: over 16 KB of f32, the same for every
    // CU) gets a head start of ~0.2 us (s_sleep 8 = 512 cycles) before the
    // first tile's weight loads, so it is not queued behind them and the
    // conversion starts earlier.  Measured at 2560 x 9728 (Q4_K, Q6_K) against
    // issuing the weights at once: 5.7-5.9 -> 5.2-5.3 us (Q4_K) and 7.07 ->
    // 6.58 us (Q6_K); s_sleep 4 and 16 did less well over the FFN and the
    // attention projections.  Small activations arrive quickly without it.
    if constexpr (RES && kFx) {
        if (K > 4096) __builtin_amdgcn_s_sleep(8);
    }
#pragma unroll
    for (int d = 0; d < kPre; ++d) fetch(ring[d], t_begin + d);

    // ---- activation slice into registers (through LDS when several rows of
    // a tile share it).  The two branches keep the source pointer's address
    // space visible to the compiler (LDS reads stay ds_read, global reads stay
    // global_load) instead of a generic pointer that would turn both into flat
    // loads waiting on every outstanding memory operation.
    if constexpr (kFx) {
        fx_stage_all<KIND>(smem, a.x, K, xg0, xg1);
        __syncthreads();
#pragma unroll
        for (int d = kPre; d < kPhase; ++d) fetch(ring[d], t_begin + d);
        if constexpr (KIND == kQ6K) fx6_load(xs.v, smem, K, xb, part);
        else fx4_load(xs.v, smem, K, xb, part);
    } else if constexpr (XLDS) {
        // registers staged above, then any remainder straight through
        const int step = is_q8(KIND) ? 16 : 4;
        const uint8_t *src = is_q8(KIND) ? (const uint8_t *)a.xq : (const uint8_t *)a.x;
        const int esz = is_q8(KIND) ? 1 : 4;
#pragma unroll
        for (int r = 0; r < kXRegs; ++r) {
            const int i = (tid + r * nthr()) * step;
            if (i < K) *(u32x4 *)(smem + lds_pad((uint32_t)(i * esz))) = xr[r];
        }
        for (int i = (tid + kXRegs * nthr()) * step; i < K; i += nthr() * step)
            *(u32x4 *)(smem + lds_pad((uint32_t)(i * esz))) = *(const u32x4 *)(src + (size_t)i * esz);
        __syncthreads();
    }
    if constexpr (kFx) {
        // slice loaded above
    } else if constexpr (is_q8(KIND)) {
        if constexpr (XLDS) {
            load_x<true>(xs.v, (const int8_t *)smem, nullptr, xb, part);
            set_xd(xs.v, xdw);
        }
        finish_x(xs.v);
    } else {
        if constexpr (XLDS) {
            // K/16 sums of 16 consecutive activation values, once per workgroup
            const float *sx = (const float *)smem;
            float *ssum = (float *)(smem + lds_pad(4u * (uint32_t)K));
            for (int g = tid; g < K / 16; g += nthr()) ssum[g] = sum16(x_at<true>(sx, 16 * g));
            __syncthreads();
            load_x<true>(xs.v, sx, xb, part);
            finish_x(xs.v, (const float *)ssum, xb, part);
        } else {
            finish_x(xs.v, (const float *)nullptr, xb, part);
        }
    }
    // LDS is reused for row reductions below (the resident form keeps them
    // in a region of their own, past the staged activation)
    if constexpr (!RES) __syncthreads();

    float *red = (float *)(smem + a.red_off);   // ring: [2][OUTS][rows_tile][nb]; resident: [PHASE][...]
    const int red_stride = OUTS * a.rows_tile * a.nb;
    // Q8 emission: the workgroup's rows [r_begin, r_end) are kept in LDS
    float *s_h = (float *)(smem + a.emit_lds_off);
    const int64_t r_begin = (int64_t)t_begin * a.rows_tile;
    const int64_t r_end = (int64_t)t_end * a.rows_tile < a.N ? (int64_t)t_end * a.rows_tile : a.N;
    uint64_t best = 0;   // running argmax key (argmax kernels)
    int buf = 0;
    // this lane's quarter-block sums of tile t into the reduction buffer rb
    auto block_sums = [&](const RawSet<KIND> &rs, int t, float *rb) {
        float ps[2];
        dot_raw<KIND>(rs, xs, part, ps);
        const bool v = valid_tile(t);
#pragma unroll
        for (int o = 0; o < OUTS; ++o) {
            const float q = quad_sum(v ? ps[o] : 0.f);
            if (part == 0 && lane_on) rb[(o * a.rows_tile + p) * a.nb + b] = q;
        }
    };
    // epilogue of one row from its sums r (one lane per row)
    auto row_epi = [&](int64_t row, const float (&r)[2]) {
        if constexpr (EPI == kQ8Emit) {
            // the SwiGLU product exactly as the store epilogue writes it
            const float g = r[0], u = r[1];
            const float hv = g * u / (1.0f + expf(-g));
            s_h[row - r_begin] = hv;
            if (a.y) a.y[row] = hv;
        } else {
            uint32_t mw = 0;
            if constexpr (EPI == kArgmaxMasked) mw = a.mask[row >> 5];
            emit_row<KIND, EPI>(a, row, r, best, mw);
        }
    };
    // row pr of tile t from its block sums in rb: added in column order
    // (loads issued four at a time), then the epilogue
    auto row_out = [&](const float *rb, int t, int pr) {
        const int64_t row = (int64_t)t * a.rows_tile + pr;
        if (row >= a.N) return;
        float r[2];
#pragma unroll
        for (int o = 0; o < OUTS; ++o) {
            const float *src = rb + (o * a.rows_tile + pr) * a.nb;
            float acc = 0.f;
            int c = 0;
            for (; c + 4 <= a.nb; c += 4) {
                const float v0 = src[c], v1 = src[c + 1], v2 = src[c + 2], v3 = src[c + 3];
                acc = (((acc + v0) + v1) + v2) + v3;
            }
            for (; c < a.nb; ++c) acc += src[c];
            r[o] = acc;
        }
        row_epi(row, r);
    };
    // The same row summed by an aligned group of L lanes (4, 8 or 16; lane s
    // of the group): lane s adds columns s, s + L, s + 2L, ... in that order,
    // the group's partial sums are then added by group_sum (a fixed pairing,
    // the same bits in every lane), and lane 0 of the group runs the
    // epilogue.  Loads are unconditional (column 0 stands in past the row's
    // end) and contribute +0 there: a partial sum that starts at +0 is never
    // -0, so adding +0 leaves it unchanged.  Uniform across the group.
    auto row_out_group = [&](const float *rb, int t, int pr, int s, int L) {
        int64_t row = (int64_t)t * a.rows_tile + pr;
        int m = 0;
        if constexpr (MULTI) {
            // the matrix's fields picked by constant index: the lane groups of
            // a wave hold rows of different tiles, and a lane-varying index
            // into the argument arrays loads them with waited vector loads
            m = mat_of(t);
            int us = a.ustart[0];
            int64_t nm = a.Nm[0];
#pragma unroll
            for (int j = 1; j < kMaxMulti; ++j) {
                us = m == j ? a.ustart[j] : us;
                nm = m == j ? a.Nm[j] : nm;
            }
            row = (int64_t)(t - us) * a.rows_tile + pr;
            if (row >= nm) return;
        }
        if (row >= a.N) return;
        float r[2];
#pragma unroll
        for (int o = 0; o < OUTS; ++o) {
            const float *src = rb + (o * a.rows_tile + pr) * a.nb;
            float acc = 0.f;
            for (int c0 = s; c0 < a.nb; c0 += 4 * L) {
                float v[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = c0 + i * L;
                    v[i] = src[c < a.nb ? c : 0];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) acc += c0 + i * L < a.nb ? v[i] : 0.f;
            }
            r[o] = group_sum(acc, L);
        }
        if constexpr (MULTI) {
            // the residual (possibly the output itself) is read before the
            // output is written, by the same lane
            float *ym = a.ym[0];
            const float *rm = a.rm[0];
#pragma unroll
            for (int j = 1; j < kMaxMulti; ++j) {
                ym = m == j ? a.ym[j] : ym;
                rm = m == j ? a.rm[j] : rm;
            }
            if (s == 0) ym[row] = rm ? r[0] + rm[row] : r[0];
        } else {
            if (s == 0) row_epi(row, r);
        }
    };
    // dot, row reduction and epilogue of tile t (workgroup-uniform control flow)
    auto process = [&](const RawSet<KIND> &rs, int t) {
        float *rb = red + buf * red_stride;
        block_sums(rs, t, rb);
        __syncthreads();
        if (tid < a.rows_tile && t < t_end) row_out(rb, t, tid);
        buf ^= 1;   // the next tile writes the other half; one barrier per tile suffices
    };

    if constexpr (RES) {
        // every tile of the range is already in flight: block sums of each
        // into a buffer of its own, one barrier, then one thread per row
#pragma unroll
        for (int d = 0; d < kPhase; ++d)
            if (t_begin + d < t_end) block_sums(ring[d], t_begin + d, red + d * red_stride);   // uniform
        __syncthreads();
        // a group of lanes per row, sized so each lane adds a few columns
        const int nrows = kPhase * a.rows_tile;
        const int lg = a.nb <= 16 ? 2 : (a.nb <= 32 ? 3 : 4);
        const int L = 1 << lg, s = tid & (L - 1);
        for (int j = tid >> lg; j < nrows; j += nthr() >> lg) {
            const int d = j / a.rows_tile;
            if (t_begin + d < t_end) row_out_group(red + d * red_stride, t_begin + d, j - d * a.rows_tile, s, L);
        }
        if constexpr (is_argmax(EPI)) {
            // every wave folds its threads' keys first (all lanes active here)
            const int lane = tid & 63;
            best = wave_max_key(best);
            argmax_finish(a, best, lane == 0 ? (tid >> 6) : -1, (int)(nthr() >> 6));
        }
        if constexpr (EPI == kQ8Emit) q8_emit_finish(a, s_h, r_begin, r_end);
        return;
    }

    // ring of kPhase tiles in flight per lane: tile t+kPhase is fetched right
    // after tile t is consumed
    for (int t = t_begin; t < t_end; t += kPhase) {
#pragma unroll
        for (int d = 0; d < kPhase; ++d) {
            if (t + d < t_end) process(ring[d], t + d);   // workgroup-uniform
            // unconditional, so every iteration issues the same loads and the
            // compiler's wait for a slot counts only the loads issued after
            // it (a guarded fetch makes it drain every load at the loop head)
            fetch(ring[d], t + d + kPhase);
        }
    }

    if constexpr (is_argmax(EPI)) {
        // the row-sum threads hold the keys
        argmax_finish(a, best, tid < a.rows_tile ? tid : -1, a.rows_tile);
    }
    if constexpr (EPI == kQ8Emit) q8_emit_finish(a, s_h, r_begin, r_end);
}

template <int KIND, int EPI, int PHASE, bool XLDS, bool RES = false>
__global__ __launch_bounds__(RES ? kResThreads : kMaxThreads) void gemv_kernel(GemvArgs a)
{
    gemv_tile_body<KIND, EPI, PHASE, XLDS, RES, false>(a);
}

// CU-resident tiles of several Q4_K matrices sharing x (q4k_gemv_multi).
template <int PHASE>
__global__ __launch_bounds__(kResThreads) void gemv_kernel_multi(GemvArgs a)
{
    gemv_tile_body<kQ4K, kStore, PHASE, true, true, true>(a);
}

// ------------------------------------------------------ wave-unit kernel

// Shapes whose rows fit one wave run with one workgroup per CU, holding as
// many waves as the CU can keep resident at this kernel's register use.  A
// row fits one wave when its 4*K/256 lanes are a power of two up to 64
// (STEPS = 1: a wave unit is 64/lanes_row rows), or when it is 32 super-blocks
// wide (STEPS = 2: a unit is one row, and every lane takes one quarter
// super-block in each half of the row).  The matrix is cut into units, dealt
// to the workgroups in turn; a workgroup's waves take its units from an LDS
// counter.  Waves that the CU issues less often (the arbiter favours older
// waves) then simply take fewer units, and the CU finishes its share as a
// whole instead of waiting for its slowest wave or workgroup.  The activation
// is staged in LDS once per CU.  A row's value is reduced the same way
// wherever it sits (fixed lane layout, halves added in order), so equal rows
// give equal bits.
template <int KIND>
constexpr int wave_max_threads() { return (is_q8(KIND) || KIND == kQ4K) ? 1024 : 768; }
constexpr int kWaveMaxThreads = 1024;   // the largest of wave_max_threads
constexpr int kHalvesWaves = 8;          // waves per CU of the two-half (STEPS = 2) wave-unit kernel
// The same kernel quantizing x in its prologue runs 16: the prologue's work
// is shared by more waves (28,672 x 8192, duplicated builds interleaved:
// 25.12 / 25.20 us with 8 waves, 24.66 / 24.64 with 16; the plain Q8 launch
// goes the other way, 23.9 against 24.4 us).
constexpr int kQuantHalvesWaves = 16;

// QUANT (Q4_K x Q8 only): the activation arrives as f32 (a.x) and every
// workgroup quantizes it to Q8 in its prologue, with the encoder every Q8
// producer uses (q8_scale, q8_code, q8_scale_bits), so its codes and scales
// equal q8_quantize's bit for bit; workgroup 0 also writes them to a.hq and
// a.hd.  The codes go to LDS as the int8 activation, the scales to LDS past
// them.
template <int KIND, int EPI, int STEPS, bool QUANT = false>
__global__ __launch_bounds__(wave_max_threads<KIND>()) void gemv_wave_kernel(GemvArgs a)
{
    // one unit in flight per wave (the next unit's loads are issued as soon
    // as the current one is consumed): with 8-16 waves per CU that keeps
    // ~37-70 KB per CU in flight, and measured faster than two units per
    // wave (lm_head 36.4 against 37.6 us, Q4_K x Q8 28,672 x 8192 24.8
    // against 26.3 us, both with 12-16 waves): more outstanding requests
    // only queue at the memory side.
    constexpr int kPhase = 1;
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ uint32_t s_next;   // next unit to hand out, relative to the range
    constexpr int BYTES = Traits<KIND>::kBytes;
    constexpr int OUTS = Traits<KIND>::kOuts;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: unit bases stay scalar
    const int waves = (int)(blockDim.x >> 6);
    // STEPS == 1: a.lanes_row lanes per row, rows side by side; STEPS == 2:
    // one row, lanes_row == 64, block b + 16*s in step s
    const int p = STEPS == 1 ? (int)__umulhi((uint32_t)lane, a.lanes_row_magic) : 0;   // row within the unit
    const int rr = lane - p * a.lanes_row;
    const int b = rr >> 2;
    const int part = rr & 3;
    const int K = a.nb * kQK;

    // this workgroup's units: units are dealt to the workgroups in turn, in
    // chunks of 1 << chunk_shift units (the fewest whose bytes fill whole
    // 128-byte lines, so no line is fetched by two CUs), and its waves take
    // them in order through the LDS counter.  At any moment the whole grid
    // reads one window of the matrix, the access pattern the HBM serves
    // fastest.  umap(v) is the workgroup's v-th unit, or `units` once past
    // the end (it grows with v).
    // QUANT: workgroup b takes position (b mod 8) * G/8 + b / 8 of each round
    // instead of b (a permutation of the grid when G is a multiple of 8), so
    // the workgroups of one XCD (workgroup b runs on XCD b mod 8) read one
    // contiguous eighth of the round's window.  Measured at 28,672 x 8192:
    // 24.0-24.2 -> 23.4-23.5 us; the same order made the Q6_K lm_head
    // 0.2-0.4 us slower and left the Q4_K x Q8 GEMV unchanged, so the other
    // forms keep the plain one.
    const int64_t units = a.tiles;
    const int u_end = (int)units;
    const int last_rows = (int)(a.N - (units - 1) * a.rows_tile);
    const int64_t wpos = (QUANT && (gridDim.x & 7u) == 0u)
                             ? (int64_t)((blockIdx.x & 7u) * (gridDim.x >> 3) + (blockIdx.x >> 3))
                             : (int64_t)blockIdx.x;
    auto umap = [&](int v) {
        const int sh = a.chunk_shift;
        const int64_t u = ((((int64_t)(v >> sh)) * gridDim.x + wpos) << sh) | (v & ((1 << sh) - 1));
        return (int)(u < units ? u : units);
    };

    // Rows of unit u start at rbase(u).  On a ragged matrix the last unit is
    // moved back to end at row N, and its lanes whose row the unit before
    // already covered are not valid: every lane of every unit then reads
    // inside the matrix at a lane offset that never changes (only with
    // N < rows_tile do lanes past N read the unit's first super-block).
    const bool shift_last = last_rows < a.rows_tile && a.N >= a.rows_tile;
    const int64_t row_bytes = (int64_t)a.nb * BYTES;
    auto rbase = [&](int u) -> int64_t {
        return (shift_last && u == u_end - 1) ? a.N - a.rows_tile : (int64_t)u * a.rows_tile;
    };
    auto valid_unit = [&](int u) {
        return u < u_end - 1 || (u == u_end - 1 && (shift_last ? p >= a.rows_tile - last_rows : p < last_rows));
    };
    uint32_t lane_off[STEPS];
#pragma unroll
    for (int st = 0; st < STEPS; ++st) lane_off[st] = p < a.N ? (uint32_t)((p * a.nb + b + 16 * st) * BYTES) : 0u;
    // unconditional loads, as in gemv_kernel: a unit past the end re-reads
    // the unit `prev` this wave has just processed (still in its CU's cache)
    auto fetch = [&](RawSet<KIND> (&rs)[STEPS], int u, int prev) {
        const int uu = u < u_end ? u : prev;
        const int64_t ub = rbase(uu) * row_bytes;
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            const uint32_t off = lane_off[st];
            if constexpr (is_q6(KIND)) {
                q6k_load(rs[st].r[0], a.W + ub, off, part);
            } else {
                q4k_load(rs[st].r[0], a.W + ub, off, part);
                if constexpr (KIND == kSwiglu) q4k_load(rs[st].r[1], a.W2 + ub, off, part);
            }
        }
    };

    // activation loads first, then the first unit of every wave (a register
    // or two per thread cover x for any workgroup of 4+ waves; smaller
    // workgroups load the rest below).  Q6_K takes the activation in fixed
    // point: each thread loads two 16-value slots and converts them once the
    // weight loads are out.
    constexpr bool kFx = KIND == kQ6K;
    float xg0[16], xg1[16];
    if constexpr (kFx) {
        fx_preload<KIND>(xg0, a.x, K, tid);
        fx_preload<KIND>(xg1, a.x, K, tid + (int)blockDim.x);
    }
    constexpr int kXRegs = (kFx || QUANT) ? 0 : (is_q8(KIND) ? 1 : 2);
    const int step = is_q8(KIND) ? 16 : 4;
    const int esz = is_q8(KIND) ? 1 : 4;
    const uint8_t *src = is_q8(KIND) ? (const uint8_t *)a.xq : (const uint8_t *)a.x;
    u32x4 xr[kXRegs > 0 ? kXRegs : 1];
#pragma unroll
    for (int r = 0; r < kXRegs; ++r) {
        const int i = (tid + r * (int)blockDim.x) * step;
        if (i < K) xr[r] = *(const u32x4 *)(src + (size_t)i * esz);
    }
    // QUANT: thread t takes values [8t, 8t + 8) of x, a quarter of a 32-value
    // Q8 block (the quad t & ~3 holds the block), so every wave of a 1024-thread
    // workgroup shares the encoding at K = 8192; the first round is loaded
    // before the weights
    float xv[QUANT ? 8 : 1];
    if constexpr (QUANT) {
        if (tid * 8 < K) load_x_f32(xv, a.x + 8 * tid, 8);
    }
    // Q8 activation without QUANT: the lane's scale words of each step go out
    // before the weights (a scale load issued after them waits for all of them)
    uint32_t xdw[(is_q8(KIND) && !QUANT) ? STEPS : 1][2];
    if constexpr (is_q8(KIND) && !QUANT) {
#pragma unroll
        for (int st = 0; st < STEPS; ++st)
            load_xd(xdw[st], a.xd, (const decltype(XSlice<KIND>::v) *)nullptr, b + 16 * st, part);
    }
    int unit[kPhase];
    RawSet<KIND> ring[kPhase][STEPS];
    // masked argmax: each unit's mask word (the word of the lane's row,
    // clamped to the last row) is loaded just before its weights, from the
    // uniform mask base plus a 32-bit lane offset, so the wait for the
    // weights covers it.  Issued after them, it took a wait of its own for
    // the weights first (its destination reused a weight load's address
    // register), one more round trip per unit: 43.2 against 36.6 us for the
    // unmasked launch at 248,320 x 1024.
    uint32_t mword[kPhase];
    auto fetch_mask = [&](int d, int u, int prev) {
        if constexpr (EPI == kArgmaxMasked) {
            int64_t row = rbase(u < u_end ? u : prev) + p;
            row = row < a.N ? row : a.N - 1;
            uint32_t off = (uint32_t)(row >> 5) * 4u;
            asm volatile("" : "+v"(off));
            mword[d] = *(const uint32_t *)((const uint8_t *)a.mask + off);
        } else {
            mword[d] = 0;
        }
    };
#pragma unroll
    for (int d = 0; d < kPhase; ++d) {
        unit[d] = umap(d * waves + wave);
        fetch_mask(d, unit[d], u_end - 1);
        fetch(ring[d], unit[d], u_end - 1);
    }
    // QUANT: a second unit per wave goes out before the prologue encodes x and
    // is consumed right after the first, so the weight stream keeps going
    // while x is encoded; afterwards one unit per wave is in flight, as in
    // every other form (28,672 x 8192: 0.1-0.3 us faster in interleaved
    // trials, bit-identical)
    static_assert(!QUANT || EPI == kStore, "the quantizing form stores its rows");
    RawSet<KIND> pre[QUANT ? STEPS : 1];
    int upre = u_end;
    if constexpr (QUANT) {
        upre = umap(kPhase * waves + wave);
        fetch(pre, upre, u_end - 1);
    }
    if (tid == 0) s_next = (uint32_t)((QUANT ? kPhase + 1 : kPhase) * waves);
    // QUANT: the scales sit in LDS past the padded codes
    const uint16_t *xd_src = a.xd;
    if constexpr (QUANT) {
        uint16_t *s_xd = (uint16_t *)(smem + lds_pad((uint32_t)K));
        xd_src = s_xd;
        for (int t = tid; t * 8 < K; t += (int)blockDim.x) {   // quads (t & ~3 .. t | 3) share an iteration
            if (t != tid) load_x_f32(xv, a.x + 8 * t, 8);
            float m = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(xv[i]));
            m = fmaxf(m, dpp_f<kDppQuadXor1>(m));   // the block's other quarters
            m = fmaxf(m, dpp_f<kDppQuadXor2>(m));
            const float d = q8_scale(m);
            uint32_t w[2];
            q8_codes_fast<8>(xv, d, w);
            const u32x2 codes = u32x2{w[0], w[1]};
            *(u32x2 *)(smem + lds_pad(8u * (uint32_t)t)) = codes;
            const uint16_t dbits = q8_scale_bits(d);
            if ((t & 3) == 0) s_xd[t >> 2] = dbits;
            if (blockIdx.x == 0) {
                *(u32x2 *)(a.hq + 8 * t) = codes;
                if ((t & 3) == 0) a.hd[t >> 2] = dbits;
            }
        }
    } else if constexpr (kFx) {
        fx_stage_all<KIND>(smem, a.x, K, xg0, xg1);
    } else {
#pragma unroll
        for (int r = 0; r < kXRegs; ++r) {
            const int i = (tid + r * (int)blockDim.x) * step;
            if (i < K) *(u32x4 *)(smem + lds_pad((uint32_t)(i * esz))) = xr[r];
        }
        for (int i = (tid + kXRegs * (int)blockDim.x) * step; i < K; i += (int)blockDim.x * step)
            *(u32x4 *)(smem + lds_pad((uint32_t)(i * esz))) = *(const u32x4 *)(src + (size_t)i * esz);
    }
    __syncthreads();
    typename WaveSlice<KIND>::T xs[STEPS];
    if constexpr (kFx) {
#pragma unroll
        for (int st = 0; st < STEPS; ++st) fx6_load(xs[st].v, smem, K, b + 16 * st, part);
    } else if constexpr (is_q8(KIND)) {
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            if constexpr (QUANT) {
                load_x<true>(xs[st].v, (const int8_t *)smem, xd_src, b + 16 * st, part);
            } else {
                load_x<true>(xs[st].v, (const int8_t *)smem, nullptr, b + 16 * st, part);
                set_xd(xs[st].v, xdw[st]);
            }
            finish_x(xs[st].v);
        }
    } else {
        const float *sx = (const float *)smem;
        float *ssum = (float *)(smem + lds_pad(4u * (uint32_t)K));
        for (int g = tid; g < K / 16; g += blockDim.x) ssum[g] = sum16(x_at<true>(sx, 16 * g));
        __syncthreads();
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            load_x<true>(xs[st].v, sx, b + 16 * st, part);
            finish_x(xs[st].v, (const float *)ssum, b + 16 * st, part);
        }
    }

    // argmax: the running best row of the lane.  Every lane of a row's group
    // holds the row's value (the reductions end with the same bits in each),
    // and a lane meets its rows in increasing index order (claims only grow),
    // so a strictly larger value replaces the best and the first index of a
    // maximum is kept.  bv starts as NaN (no row yet): the first non-NaN row
    // is taken; NaN rows and banned rows never are.
    float bv = __builtin_nanf("");
    uint32_t bi = 0;
    // keep taking units until every ring slot comes back past the range (the
    // counter only grows, so once one claim is past it every later one is)
    auto active = [&]() {
        bool any = false;
#pragma unroll
        for (int d = 0; d < kPhase; ++d) any = any || unit[d] < u_end;
        return any;
    };
    // one unit's rows: the lane's dot products, reduced over the row's lanes,
    // then stored or folded into the running argmax (mw: the unit's mask word)
    auto consume = [&](const RawSet<KIND> (&rs)[STEPS], int u, uint32_t mw) {
        float ps[2] = {0.f, 0.f};
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            float q[2];
            dot_raw<KIND>(rs[st], xs[st], part, q);
#pragma unroll
            for (int o = 0; o < OUTS; ++o) ps[o] = st == 0 ? q[o] : ps[o] + q[o];
        }
        const bool v = valid_unit(u);
        float r[2];
#pragma unroll
        for (int o = 0; o < OUTS; ++o) r[o] = group_sum(v ? ps[o] : 0.f, a.lanes_row);
        if constexpr (is_argmax(EPI)) {
            const uint32_t row = (uint32_t)(rbase(u) + p);
            bool take = v && !(r[0] <= bv) && r[0] == r[0];
            if constexpr (EPI == kArgmaxMasked) take = take && !((mw >> (row & 31)) & 1u);
            bv = take ? r[0] : bv;
            bi = take ? row : bi;
        } else {
            uint64_t unused = 0;
            if (rr == 0 && v) emit_row<KIND, EPI>(a, rbase(u) + p, r, unused, mw);
        }
    };
    // claim the wave's next unit from the workgroup's counter and issue its loads
    auto advance = [&](int d) {
        uint32_t c = 0;
        if (lane == 0) c = __hip_atomic_fetch_add(&s_next, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const int done = unit[d];
        unit[d] = umap((int)__builtin_amdgcn_readfirstlane(c));
        fetch_mask(d, unit[d], done);
        fetch(ring[d], unit[d], done);
    };
    if constexpr (QUANT) {
        if (unit[0] < u_end) {   // wave-uniform
            consume(ring[0], unit[0], mword[0]);
            advance(0);
        }
        if (upre < u_end) consume(pre, upre, 0u);
    }
    while (active()) {
#pragma unroll
        for (int d = 0; d < kPhase; ++d) {
            if (unit[d] < u_end) {   // wave-uniform
                consume(ring[d], unit[d], mword[d]);
                advance(d);
            }
        }
    }

    if constexpr (is_argmax(EPI)) {
        // each wave's largest key reaches lane 0, then the workgroup's
        uint64_t best = bv == bv ? argmax_key(bv, bi) : 0ull;
        best = wave_max_key(best);
        argmax_finish(a, best, lane == 0 ? wave : -1, waves);
    }
}

// ---------------------------------------------------- row-stream kernel

// Every other shape (K/256 not a power of two up to 16, or more than 16
// super-blocks): a wave takes whole rows and walks each one in steps of 16
// super-blocks, lane l taking quarter l%4 of super-block l/4 of the step
// (lanes past the row's last super-block idle).  Rows of up to 16 super-blocks
// are one step; a power-of-two group of lanes holds each, so a wave unit is
// 64/group rows.  Longer rows are one row per unit and S = ceil(K/4096) steps.
// As in the wave-unit kernel there is one workgroup per CU, its waves take
// units from an LDS counter, and the activation is staged in LDS once; the
// slice of a step is re-read from LDS when a row has several steps.  Each wave
// runs a pipeline of (unit, step) pairs, one in flight; a row's step sums are
// added in step order and reduced over its lane group, the same way for every
// row.
template <int KIND, int EPI, int MULTI>
__global__ __launch_bounds__(wave_max_threads<KIND>()) void gemv_rows_kernel(GemvArgs a)
{
    constexpr int kPhase = 1;   // one (unit, step) in flight per wave, as in the wave-unit kernel (measured faster)
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ uint32_t s_next;   // next unit to hand out, relative to the range
    constexpr int BYTES = Traits<KIND>::kBytes;
    constexpr int OUTS = Traits<KIND>::kOuts;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int waves = (int)(blockDim.x >> 6);
    const int group = a.lanes_row;                                      // lanes per row (power of two)
    const int p = (int)__umulhi((uint32_t)lane, a.lanes_row_magic);    // row within the unit
    const int rr = lane - p * group;
    const int b = rr >> 2;
    const int part = rr & 3;
    const int K = a.nb * kQK;
    const int S = a.steps;

    // units dealt to the workgroups in turn, as in the wave-unit kernel
    const int64_t units = a.tiles;
    const int u_end = (int)units;
    const int last_rows = (int)(a.N - (units - 1) * a.rows_tile);
    const int64_t unit_stride = (int64_t)a.rows_tile * a.nb * BYTES;
    auto umap = [&](int v) {
        const int sh = a.chunk_shift;
        const int64_t u = ((((int64_t)(v >> sh)) * gridDim.x + blockIdx.x) << sh) | (v & ((1 << sh) - 1));
        return (int)(u < units ? u : units);
    };

    // super-block of this lane in step s, or -1 past the row's end
    auto block_of = [&](int st) { const int c = b + 16 * st; return c < a.nb ? c : -1; };
    // multi-output: the matrix of unit u (wave-uniform) and the unit's index in it
    auto mat_of = [&](int u) {
        int m = 0;
        if constexpr (MULTI) {
#pragma unroll
            for (int j = 1; j < kMaxMulti; ++j) m += u >= a.ustart[j] ? 1 : 0;
        }
        return m;
    };
    auto valid_row = [&](int u) {
        if constexpr (MULTI) {
            const int m = mat_of(u);
            return u < u_end && (int64_t)(u - a.ustart[m]) * a.rows_tile + p < a.Nm[m];
        } else {
            return u < u_end && (u < units - 1 || p < last_rows);
        }
    };
    // unconditional loads: past the range the unit `prev` is re-read (still
    // cached), an idle lane reads the unit's first super-block
    auto fetch = [&](RawSet<KIND> &rs, int u, int st, int prev) {
        const int uu = u < u_end ? u : prev;
        const int c = block_of(st);
        const uint32_t off = (valid_row(u) && c >= 0) ? (uint32_t)((p * a.nb + c) * BYTES) : 0u;
        const uint8_t *Wb = a.W;
        int64_t ub = (int64_t)uu * unit_stride;
        if constexpr (MULTI) {
            const int m = mat_of(uu);
            Wb = a.Wm[m];
            ub = (int64_t)(uu - a.ustart[m]) * unit_stride;
        }
        if constexpr (is_q6(KIND)) {
            q6k_load(rs.r[0], Wb + ub, off, part);
        } else {
            q4k_load(rs.r[0], Wb + ub, off, part);
            if constexpr (KIND == kSwiglu) q4k_load(rs.r[1], a.W2 + ub, off, part);
        }
    };
    // multi-output residual of the lane's row in unit u (loaded with the unit's
    // first step; a launch without residual re-reads y, which is discarded)
    auto fetch_res = [&](int u, int prev) {
        float r = 0.f;
        if constexpr (MULTI) {
            const int uu = u < u_end ? u : prev;
            const int m = mat_of(uu);
            int64_t row = (int64_t)(uu - a.ustart[m]) * a.rows_tile + p;
            row = row < a.Nm[m] ? row : a.Nm[m] - 1;
            const float *src = a.rm[m] ? a.rm[m] : a.ym[m];
            r = src[row];
        }
        return r;
    };

    // f32 Q4_K takes the activation in fixed point (Q4KFX): each thread
    // loads two 16-value groups first, and converts them after the first
    // weight loads are out
    constexpr bool kFx = KIND == kQ4K;
    float xg0[16], xg1[16];
    if constexpr (kFx) {
        fx_preload<KIND>(xg0, a.x, K, tid);
        fx_preload<KIND>(xg1, a.x, K, tid + (int)blockDim.x);
    }
    // activation loads first
    constexpr int kXRegs = kFx ? 0 : (is_q8(KIND) ? 1 : 2);
    const int xstep = is_q8(KIND) ? 16 : 4;
    const int esz = is_q8(KIND) ? 1 : 4;
    const uint8_t *src = is_q8(KIND) ? (const uint8_t *)a.xq : (const uint8_t *)a.x;
    u32x4 xr[kXRegs > 0 ? kXRegs : 1];
#pragma unroll
    for (int r = 0; r < kXRegs; ++r) {
        const int i = (tid + r * (int)blockDim.x) * xstep;
        if (i < K) xr[r] = *(const u32x4 *)(src + (size_t)i * esz);
    }

    // the fetch cursor walks (unit, step) pairs: the first two units of the
    // wave are fixed, later ones come from the counter when their first step
    // is fetched
    int fu = umap(wave), fs = 0;
    int next_fixed = umap(waves + wave);   // second fixed unit, then -1
    int ring_u[kPhase], ring_s[kPhase];
    RawSet<KIND> ring[kPhase];
    float ring_r[kPhase];   // multi-output: residual of the lane's row
    auto advance = [&]() {
        if (++fs == S) {
            fs = 0;
            if (next_fixed >= 0) {
                fu = next_fixed;
                next_fixed = -1;
            } else {
                uint32_t c = 0;
                if (lane == 0) c = __hip_atomic_fetch_add(&s_next, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                fu = umap((int)__builtin_amdgcn_readfirstlane(c));
            }
        }
    };
    if (tid == 0) s_next = (uint32_t)(2 * waves);
    __syncthreads();   // the counter is set before any wave claims
#pragma unroll
    for (int d = 0; d < kPhase; ++d) {
        ring_u[d] = fu;
        ring_s[d] = fs;
        fetch(ring[d], fu, fs, u_end - 1);
        ring_r[d] = fetch_res(fu, u_end - 1);
        advance();
    }

    if constexpr (kFx) {
        fx_stage_all<KIND>(smem, a.x, K, xg0, xg1);
        __syncthreads();
    } else {
#pragma unroll
        for (int r = 0; r < kXRegs; ++r) {
            const int i = (tid + r * (int)blockDim.x) * xstep;
            if (i < K) *(u32x4 *)(smem + lds_pad((uint32_t)(i * esz))) = xr[r];
        }
        for (int i = (tid + kXRegs * (int)blockDim.x) * xstep; i < K; i += (int)blockDim.x * xstep)
            *(u32x4 *)(smem + lds_pad((uint32_t)(i * esz))) = *(const u32x4 *)(src + (size_t)i * esz);
        __syncthreads();
    }
    const float *sx = (const float *)smem;
    const float *ssum = (const float *)(smem + lds_pad(4u * (uint32_t)K));
    if constexpr (!is_q8(KIND) && !kFx) {
        float *w = (float *)ssum;
        for (int g = tid; g < K / 16; g += blockDim.x) w[g] = sum16(x_at<true>(sx, 16 * g));
        __syncthreads();
    }
    typename RowsSlice<KIND>::T xs;
    auto slice = [&](int st) {
        const int c = block_of(st);
        const int cb = c >= 0 ? c : 0;   // idle lanes read any valid slice
        if constexpr (kFx) {
            fx4_load(xs.v, smem, K, cb, part);
        } else if constexpr (is_q8(KIND)) {
            load_x<true>(xs.v, (const int8_t *)smem, a.xd, cb, part);
            finish_x(xs.v);
        } else {
            load_x<true>(xs.v, sx, cb, part);
            finish_x(xs.v, ssum, cb, part);
        }
    };
    if (S == 1) slice(0);

    uint64_t best = 0;
    float acc[2] = {0.f, 0.f};
    bool done = false;
    while (!done) {
#pragma unroll
        for (int d = 0; d < kPhase; ++d) {
            if (!done) {
                const int u = ring_u[d], st = ring_s[d];
                if (u >= u_end) {   // wave-uniform; every later pair is past the range too
                    done = true;
                } else {
                    if (S > 1) slice(st);
                    float q[2];
                    dot_raw<KIND>(ring[d], xs, part, q);
                    const bool lv = block_of(st) >= 0;
#pragma unroll
                    for (int o = 0; o < OUTS; ++o) {
                        const float t = lv ? q[o] : 0.f;
                        acc[o] = st == 0 ? t : acc[o] + t;
                    }
                    if (st == S - 1) {
                        const bool v = valid_row(u);
                        float r[2];
#pragma unroll
                        for (int o = 0; o < OUTS; ++o) r[o] = group_sum(acc[o], group);
                        if (rr == 0 && v) {
                            if constexpr (MULTI) {
                                const int m = mat_of(u);
                                const int64_t row = (int64_t)(u - a.ustart[m]) * a.rows_tile + p;
                                a.ym[m][row] = a.rm[m] ? r[0] + ring_r[d] : r[0];
                            } else {
                                const int64_t row = (int64_t)u * a.rows_tile + p;
                                uint32_t mw = 0;
                                if constexpr (EPI == kArgmaxMasked) mw = a.mask[row >> 5];
                                emit_row<KIND, EPI>(a, row, r, best, mw);
                            }
                        }
                    }
                    ring_u[d] = fu;
                    ring_s[d] = fs;
                    fetch(ring[d], fu, fs, u);
                    ring_r[d] = fetch_res(fu, u);
                    advance();
                }
            }
        }
    }

    if constexpr (is_argmax(EPI)) {
        best = wave_max_key(best);
        argmax_finish(a, best, lane == 0 ? wave : -1, waves);
    }
}

// ------------------------------------------------------ batched kernel

// Batched int8-activation GEMV: y[j][n] = sum_k W[n,k] * xdq_j[k] for the
// a.batch <= M vectors j (memra-engine decode.rs, lockstep multi-stream
// decode: one weight read serves m streams).  The tile kernel's geometry and
// row reduction, with M outputs per row: each lane dequantizes its quarter
// super-block once and dots it against the M activation slices it keeps in
// registers, so the weight stream is read once for all vectors.  The
// vectors are staged through LDS a.batch_round at a time (at most ~60 KiB
// per round) and each lane copies its slices into registers; slots past
// a.batch repeat the last vector and are never stored.  A row's value for
// vector j is summed exactly as the tile kernel sums it (quad sums, then the
// K/256 block sums in column order), whatever M, the batch or the row's
// position: results do not depend on the other vectors.
template <int KIND, int M, int PHASE>
__global__ __launch_bounds__(kMaxThreads) void gemv_batch_kernel(GemvArgs a)
{
    static_assert(is_q8(KIND), "batched GEMV takes Q8 activations");
    constexpr int kPhase = PHASE;
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int BYTES = Traits<KIND>::kBytes;
    const int tid = threadIdx.x;
    const int p = (int)__umulhi((uint32_t)tid, a.lanes_row_magic);   // row within the tile
    const int rr = tid - p * a.lanes_row;
    const int b = rr >> 2;
    const int part = rr & 3;
    const bool lane_on = p < a.rows_tile;
    const int K = a.nb * kQK;
    const int P = a.rows_tile;

    const int bid = blockIdx.x;
    const int t_begin = bid * a.tiles_q + (bid < a.tiles_r ? bid : a.tiles_r);
    const int t_end = t_begin + a.tiles_q + (bid < a.tiles_r ? 1 : 0);
    const int last_rows = (int)(a.N - (a.tiles - 1) * P);
    const int64_t tile_stride = (int64_t)P * a.nb * BYTES;
    const uint32_t lane_off = (uint32_t)((p * a.nb + b) * BYTES);
    auto valid_tile = [&](int t) { return lane_on && t < t_end && (t < a.tiles - 1 || p < last_rows); };
    // unconditional loads, as in gemv_kernel
    auto fetch = [&](RawSet<KIND> &rs, int t) {
        const int tt = t < t_end ? t : t_end - 1;
        const uint32_t off = valid_tile(t) ? lane_off : 0u;
        const int64_t tb = (int64_t)tt * tile_stride;
        if constexpr (is_q6(KIND))
            q6k_load(rs.r[0], a.W + tb, off, part);
        else
            q4k_load(rs.r[0], a.W + tb, off, part);
    };

    // every vector's Q8 scale words of the lane go out first: loaded after the
    // weights, each waited for every weight load, one vector after another
    XSlice<KIND> xs[M];
    const int xb = lane_on ? b : 0;
    uint32_t xdw[M][2];
#pragma unroll
    for (int j = 0; j < M; ++j) {
        const int jv = j < a.batch ? j : a.batch - 1;
        load_xd(xdw[j], a.xd + (size_t)jv * (K / 32), &xs[j].v, xb, part);
    }

    RawSet<KIND> ring[kPhase];
#pragma unroll
    for (int d = 0; d < kPhase; ++d) fetch(ring[d], t_begin + d);

    // activation slices, staged a.batch_round vectors at a time; a vector
    // occupies K + K/16 bytes of LDS (lds_pad layout)
    const int vbytes = K + K / 16;
    for (int j0 = 0; j0 < M; j0 += a.batch_round) {   // workgroup-uniform
        const int nv = M - j0 < a.batch_round ? M - j0 : a.batch_round;
        for (int i = tid * 16; i < nv * K; i += a.threads * 16) {
            const int jj = i / K, kk = i - jj * K;
            const int jv = j0 + jj < a.batch ? j0 + jj : a.batch - 1;
            *(u32x4 *)(smem + jj * vbytes + lds_pad((uint32_t)kk)) = *(const u32x4 *)(a.xq + (size_t)jv * K + kk);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < M; ++j) {
            if (j >= j0 && j < j0 + nv) {
                load_x<true>(xs[j].v, (const int8_t *)(smem + (j - j0) * vbytes), nullptr, xb, part);
                set_xd(xs[j].v, xdw[j]);
                finish_x(xs[j].v);
            }
        }
        __syncthreads();   // LDS is rewritten by the next round (or reused below)
    }

    float *red = (float *)smem;   // [2][M][rows_tile][nb]
    const int red_stride = M * P * a.nb;
    int buf = 0;
    auto process = [&](const RawSet<KIND> &rs, int t) {
        float ps[M];
        const bool v = valid_tile(t);
#pragma unroll
        for (int j = 0; j < M; ++j) {
            float q[2];
            dot_raw<KIND>(rs, xs[j], part, q);
            ps[j] = v ? q[0] : 0.f;
        }
        float *rb = red + buf * red_stride;
#pragma unroll
        for (int j = 0; j < M; ++j) {
            const float q = quad_sum(ps[j]);
            if (part == 0 && lane_on) rb[(j * P + p) * a.nb + b] = q;
        }
        __syncthreads();
        // P * M <= 2 * a.threads (a row has at least 4 lanes and M <= 8):
        // two fixed passes, so the number of stores per tile is static and
        // the ring loads keep their counted waits
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int i = tid + it * a.threads;
            const int j = i / P, pr = i - j * P;
            const int64_t row = (int64_t)t * P + pr;
            if (t < t_end && j < a.batch && row < a.N) {
                const float *src = rb + (j * P + pr) * a.nb;
                float acc = 0.f;
                int c = 0;
                for (; c + 4 <= a.nb; c += 4) {
                    const float v0 = src[c], v1 = src[c + 1], v2 = src[c + 2], v3 = src[c + 3];
                    acc = (((acc + v0) + v1) + v2) + v3;
                }
                for (; c < a.nb; ++c) acc += src[c];
                a.y[(size_t)j * a.N + row] = acc;
            }
        }
        buf ^= 1;
    };

    for (int t = t_begin; t < t_end; t += kPhase) {
#pragma unroll
        for (int d = 0; d < kPhase; ++d) {
            if (t + d < t_end) process(ring[d], t + d);
            fetch(ring[d], t + d + kPhase);   // unconditional, as in gemv_kernel
        }
    }
}

// --------------------------------------------------------- Q8 quantize

// One 32-lane half-wave per 32-element block.
__global__ __launch_bounds__(256) void q8_quantize_kernel(const float *__restrict__ x, int8_t *__restrict__ xq,
                                                         uint16_t *__restrict__ xd, int K)
{
    const int gid = blockIdx.x * blockDim.x + threadIdx.x;
    const bool on = gid < K;
    const float v = on ? x[gid] : 0.f;
    uint16_t dbits;
    const int8_t q = q8_encode(v, dbits);
    if (on) {
        xq[gid] = q;
        if ((gid & 31) == 0) xd[gid >> 5] = dbits;
    }
}

// ------------------------------------------------------ RMS norm -> Q8

// y = w * x / sqrt(mean(x^2) + eps), then the Q8 encoding of y (memra-engine
// decode.rs `rms_norm_q8_1`, and `add_rms_norm_q8_1` with ADD: x is first
// replaced by x + r, which is also written to res as the new residual).  One
// workgroup of 1024 threads; in pass p thread t holds the four elements from
// 4096p + 4t (16-byte loads), so a 32-element Q8 block sits in 8 consecutive
// lanes and is encoded there (the block maximum by a 3-step xor tree, then
// the same q8_scale / q8_code as every other producer).  All loads are issued
// up front, clamped to the vector's last four elements (no branch separates
// them); PASSES is the power of two >= K/4096.  The sum of squares is added
// per lane in element order, then by a fixed shuffle tree, then over the 16
// waves in order.  res may be x or r itself (each element is read, then
// written, by one lane; those pointers carry no __restrict__ for that reason).
constexpr int kNormThreads = 1024;
constexpr int kNormSpan = 4 * kNormThreads;   // elements per pass

template <bool ADD, int PASSES>
__global__ __launch_bounds__(kNormThreads) void rms_norm_q8_kernel(const float *x, const float *r,
                                                                  const float *__restrict__ w, float eps,
                                                                  float *res, float *__restrict__ y,
                                                                  int8_t *__restrict__ xq, uint16_t *__restrict__ xd,
                                                                  int K)
{
    __shared__ float s_part[kNormThreads / 64];
    const int tid = threadIdx.x;
    float4 v[PASSES], wv[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int e = kNormSpan * p + 4 * tid;
        const int ec = e < K ? e : K - 4;
        v[p] = *(const float4 *)(x + ec);
        if constexpr (ADD) {
            const float4 t = *(const float4 *)(r + ec);
            v[p] = make_float4(v[p].x + t.x, v[p].y + t.y, v[p].z + t.z, v[p].w + t.w);
        }
        wv[p] = *(const float4 *)(w + ec);
    }
    float ss = 0.f;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const bool on = kNormSpan * p + 4 * tid < K;
        const float4 a = v[p];
        const float q = (((a.x * a.x) + (a.y * a.y)) + (a.z * a.z)) + (a.w * a.w);
        ss += on ? q : 0.f;
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) ss += __shfl_xor(ss, off);
    if ((tid & 63) == 0) s_part[tid >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < kNormThreads / 64; ++i) tot += s_part[i];
    const float inv = 1.0f / sqrtf(tot / (float)K + eps);
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int e = kNormSpan * p + 4 * tid;
        if (e < K) {   // uniform over each 8-lane block group (K % 32 == 0)
            if constexpr (ADD) *(float4 *)(res + e) = v[p];
            const float4 a = v[p], b = wv[p];
            const float4 yv = make_float4((a.x * inv) * b.x, (a.y * inv) * b.y, (a.z * inv) * b.z, (a.w * inv) * b.w);
            if (y) *(float4 *)(y + e) = yv;
            float amax = fmaxf(fmaxf(fabsf(yv.x), fabsf(yv.y)), fmaxf(fabsf(yv.z), fabsf(yv.w)));
#pragma unroll
            for (int m = 1; m < 8; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 8));
            const float d = q8_scale(amax);
            const uint32_t packed = (uint32_t)(uint8_t)q8_code(yv.x, d) | ((uint32_t)(uint8_t)q8_code(yv.y, d) << 8) |
                                    ((uint32_t)(uint8_t)q8_code(yv.z, d) << 16) |
                                    ((uint32_t)(uint8_t)q8_code(yv.w, d) << 24);
            *(uint32_t *)(xq + e) = packed;
            if ((tid & 7) == 0) xd[e >> 5] = q8_scale_bits(d);
        }
    }
}

// ---------------------------------------------------- Q4_K x Q8 isums hook

// Integer sums of every (row, 32-block) with the same decode and dot code as
// the Q8 GEMV (q4k_load + q4k_q8_isums); one thread per (row, block, part).
__global__ __launch_bounds__(256) void q4k_q8_isums_kernel(const uint8_t *__restrict__ W, const int8_t *__restrict__ xq,
                                                          int32_t *__restrict__ isums, int64_t N, int nb)
{
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = N * nb * kParts;
    if (gid >= total) return;
    const int part = (int)(gid & 3);
    const int64_t blk = gid >> 2;   // row * nb + b
    const int b = (int)(blk % nb);
    Q8X xs;
    load_x(xs, xq, nullptr, b, part);
    finish_x(xs);
    Q4KRaw r;
    q4k_load(r, W + blk * kQ4KBytes, 0u, part);
    int32_t isl, ish;
    q4k_q8_isums(r, xs, isl, ish);
    isums[blk * 8 + 2 * part] = isl;
    isums[blk * 8 + 2 * part + 1] = ish;
}

// Integer sums of every (row, 16-element group) of the Q6_K x Q8 GEMV with
// its decode and dot code (q6k_load + q6k_q8_isums); one thread per (row,
// block, part), each part covering 4 groups.
__global__ __launch_bounds__(256) void q6k_q8_isums_kernel(const uint8_t *__restrict__ W, const int8_t *__restrict__ xq,
                                                          int32_t *__restrict__ isums, int64_t N, int nb)
{
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = N * nb * kParts;
    if (gid >= total) return;
    const int part = (int)(gid & 3);
    const int64_t blk = gid >> 2;   // row * nb + b
    const int b = (int)(blk % nb);
    Q6Q8X xs;
    load_x(xs, xq, nullptr, b, part);
    finish_x(xs);
    Q6KRaw r;
    q6k_load(r, W + blk * kQ6KBytes, 0u, part);
    int32_t is[4];
    q6k_q8_isums(r, xs, is);
    // group s of part u is 16-element group 8n + 2s + (u & 1) of the block
    const int n = part >> 1;
#pragma unroll
    for (int s = 0; s < 4; ++s) isums[blk * 16 + 8 * n + 2 * s + (part & 1)] = is[s];
}

// ------------------------------------------------------------ launch plan

// Plan of a wave-unit or row-stream launch (every row reduced inside one
// wave), or false when the shape goes to the tile kernel.
// Shared tail of a wave-unit or row-stream plan (steps and lanes_row set).
static bool finish_wave_plan(Plan &pl, int64_t N, int64_t K, int kind)
{
    pl.wave_local = 1;
    pl.waves = (kind == kQ4KQ8 && !pl.rows_kernel && pl.steps == 2)
                   ? kHalvesWaves
                   : (is_q8(kind) || (kind == kQ4K && pl.steps == 2) ? 1024 : 768) / 64;   // the most; the launch decides
    pl.threads = pl.waves * 64;
    pl.rows_tile = 64 / pl.lanes_row;
    pl.tiles = (N + pl.rows_tile - 1) / pl.rows_tile;
    // chunk of units whose bytes are a whole number of 128-byte lines
    const int64_t unit_bytes = (int64_t)pl.rows_tile * pl.nb * (is_q6(kind) ? 210 : 144);
    pl.chunk_shift = 0;
    while (((unit_bytes << pl.chunk_shift) & 127) != 0) ++pl.chunk_shift;
    const size_t xb = is_q8(kind) ? (size_t)K : (size_t)K * 4;
    pl.x_in_lds = 1;
    pl.lds_bytes = xb + xb / 16 + (is_q8(kind) ? 0 : (size_t)(K / 16) * 4);
    pl.grid = 0;
    return pl.lds_bytes <= 65536;   // larger x (f32, K > ~15000) goes to the tile kernel
}

// Row-stream plan: rows walked in steps of 16 super-blocks, each row inside a
// power-of-two lane group of one wave.
static bool plan_rows(Plan &pl, int64_t N, int64_t K, int kind)
{
    pl.nb = (int)(K / kQK);
    pl.rows_kernel = 1;
    pl.steps = (pl.nb + 15) / 16;
    int g = 4;
    while (g < 4 * pl.nb && g < 64) g *= 2;
    pl.lanes_row = g;   // lanes per row: a power of two holding min(nb, 16) super-blocks
    if (kind != kQ4K) return finish_wave_plan(pl, N, K, kind);
    finish_wave_plan(pl, N, K, kind);
    // f32 Q4_K: fixed-point activation (three padded byte arrays, the
    // 16-element sums and the part exponents) instead of the f32 copy
    pl.lds_bytes = 3 * ((size_t)K + (size_t)K / 16) + (size_t)(K / 16) * 4 + (size_t)(K / 64) * 4;
    return pl.lds_bytes <= 65536;
}

// Plan of a wave-unit or row-stream launch (every row reduced inside one
// wave), or false when the shape goes to the tile kernel.
static bool plan_in_wave(Plan &pl, int64_t N, int64_t K, int kind)
{
    pl.nb = (int)(K / kQK);
    pl.lanes_row = kParts * pl.nb;
    const bool fits = pl.lanes_row <= 64 && (pl.lanes_row & (pl.lanes_row - 1)) == 0;
    // two halves need the x slices of both in registers: only the int8 path
    // has room for them without spilling
    const bool halves = pl.nb == 32 && kind == kQ4KQ8;
    // The row-stream kernel wins (measured) for f32 Q4_K rows of two halves,
    // and for one-step rows of a single Q6_K or Q8 matrix when each CU gets a
    // couple of dozen rows at most; with more rows per CU, longer rows, the
    // SwiGLU pair or a single f32 Q4_K matrix (resident fixed-point tile:
    // 4096 x 2560 4.48 -> 4.01 us), the tile kernel wins.
    const bool stream = (kind == kQ4K && pl.nb == 32) || (pl.nb < 16 && kind != kSwiglu && kind != kQ4K && N <= 6144);
    if (!fits && !halves && !stream) return false;
    if (!fits && !halves) return plan_rows(pl, N, K, kind);
    // gemv_wave_kernel: the row's lanes are a power-of-two group (or two halves)
    pl.rows_kernel = 0;
    if (fits) {
        pl.steps = 1;
    } else {
        pl.steps = 2;
        pl.lanes_row = 64;
    }
    const bool ok = finish_wave_plan(pl, N, K, kind);
    // Q6_K: fixed-point activation (three padded byte arrays, the 16-element
    // sums and the part exponents) instead of the f32 copy
    if (kind == kQ6K) pl.lds_bytes = 3 * ((size_t)K + (size_t)K / 16) + (size_t)(K / 16) * 4 + (size_t)(K / 64) * 4;
    return ok && pl.lds_bytes <= 65536;
}

// Most tiles a CU-resident workgroup holds in flight, by kind: the raw
// blocks of every tile and the activation slice stay in registers (at most
// 168 VGPRs with three waves per SIMD), so the SwiGLU pair (two matrices per
// tile) takes two.
static int res_max_phase(int kind) { return kind == kSwiglu ? 2 : kResMaxPhase; }

// Bytes of LDS the tile kernel stages the activation in (f32 padded copy and
// its 16-element sums; int8 padded copy; or the fixed-point Q6_K form).
static size_t tile_staged_bytes(int64_t K, int kind, bool res)
{
    const size_t xbytes = is_q8(kind) ? (size_t)K : (size_t)K * 4;
    const size_t sums = is_q8(kind) ? 0 : (size_t)(K / 16) * 4;
    if (tile_fx(kind, true, res)) return 3 * ((size_t)K + (size_t)K / 16) + sums + (size_t)(K / 64) * 4;
    return xbytes + xbytes / 16 + sums;   // 16 bytes of padding per 256 (lds_pad)
}

// CU-resident tile plan (gemv_kernel<..., RES = true>), or false.  Waves per
// workgroup w in {4, 8, 12} (one workgroup per CU, whole SIMDs); each w gives
// rows per tile R = 64w / (4 nb) and a busiest CU of ceil(tiles / cus) tiles.
// The plan takes the w whose busiest CU has the fewest rows (then the fewest
// idle lanes, then fewer waves), if that CU's tiles fit in flight at once.
// The grid is the fewest workgroups that keep to that many tiles each.
static bool plan_resident(Plan &pl, int64_t N, int64_t K, int kind, size_t extra_lds, int cus)
{
    int best_w = 0, best_per = 0;
    int64_t best_rows = INT64_MAX;
    double best_u = -1.0;
    for (int w = 4; w <= kResThreads / 64; w += 4) {
        const int rows = 64 * w / pl.lanes_row;
        if (rows < 1) continue;
        const int64_t tiles = (N + rows - 1) / rows;
        const int64_t per = (tiles + cus - 1) / cus;
        if (per > res_max_phase(kind)) continue;
        const int64_t busiest = per * rows;
        const double util = (double)(rows * pl.lanes_row) / (64.0 * w);
        if (busiest < best_rows || (busiest == best_rows && util > best_u + 1e-9)) {
            best_rows = busiest;
            best_u = util;
            best_w = w;
            best_per = (int)per;
        }
    }
    if (!best_w) return false;
    pl.waves = best_w;
    pl.threads = 64 * best_w;
    pl.rows_tile = pl.threads / pl.lanes_row;
    pl.tiles = (N + pl.rows_tile - 1) / pl.rows_tile;
    pl.phase = best_per;
    pl.grid = (int)((pl.tiles + best_per - 1) / best_per);
    const int outs = (kind == kSwiglu) ? 2 : 1;
    const size_t red = (size_t)pl.phase * outs * pl.rows_tile * pl.nb * 4;
    const size_t staged = (tile_staged_bytes(K, kind, true) + 15) & ~(size_t)15;
    if (red + extra_lds > 65536) return false;
    pl.x_in_lds = (pl.rows_tile > 1 && staged + red + extra_lds <= 65536) ? 1 : 0;
    pl.red_off = pl.x_in_lds ? staged : 0;
    pl.lds_bytes = pl.red_off + red;
    pl.resident = 1;
    return true;
}

// Tile-kernel plan; `extra_lds` bytes of LDS are reserved past the kernel's
// own (the Q8 emission's row buffer), and x is staged through LDS only if
// everything fits in 64 KiB.  With `resident` the CU-resident form is taken
// when a CU's share of the tiles fits in flight at once; otherwise the ring
// form walks contiguous tile ranges.
static Plan make_tile_plan(int64_t N, int64_t K, int kind, size_t extra_lds, int cus, bool resident)
{
    Plan pl{};
    pl.nb = (int)(K / kQK);
    pl.wave_local = 0;
    pl.rows_kernel = 0;
    pl.steps = 1;
    pl.lanes_row = kParts * pl.nb;
    if (resident && plan_resident(pl, N, K, kind, extra_lds, cus)) return pl;
    pl.resident = 0;
    pl.phase = 0;
    pl.red_off = 0;
    // tile kernel: 1, 2, 4 or 8 waves (a workgroup of another size leaves SIMDs
    // unevenly loaded and fewer workgroups fit on a CU); fewest idle lanes,
    // ties to fewer waves; at least one row per tile
    int best_w = 0;
    double best_u = -1.0;
    for (int w = 1; w <= kMaxThreads / 64; w *= 2) {
        const int rows = 64 * w / pl.lanes_row;
        if (rows < 1) continue;
        const double util = (double)(rows * pl.lanes_row) / (64.0 * w);
        if (util > best_u + 1e-9) {
            best_u = util;
            best_w = w;
        }
    }
    pl.waves = best_w;
    pl.threads = 64 * pl.waves;
    pl.rows_tile = pl.threads / pl.lanes_row;
    pl.tiles = (N + pl.rows_tile - 1) / pl.rows_tile;
    const int outs = (kind == kSwiglu) ? 2 : 1;
    const size_t red = (size_t)2 * outs * pl.rows_tile * pl.nb * 4;   // two buffers
    // Staging x through LDS pays when several rows of a tile read the same
    // slice; with one row per tile every element has a single reader.  Q6_K
    // activations go to LDS in fixed point (three padded byte arrays, the
    // 16-element sums and the part exponents).
    const size_t staged = tile_staged_bytes(K, kind, false);
    pl.x_in_lds = (pl.rows_tile > 1 && staged + extra_lds <= 65536) ? 1 : 0;
    pl.lds_bytes = (pl.x_in_lds ? staged : 0);
    if (red > pl.lds_bytes) pl.lds_bytes = red;
    pl.grid = 0;   // set by the launcher from the occupancy
    return pl;
}

Plan make_plan(int64_t N, int64_t K, int kind, int cus)
{
    Plan pl{};
    if (plan_in_wave(pl, N, K, kind)) return pl;
    return make_tile_plan(N, K, kind, 0, cus, true);
}

Plan make_swiglu_q8_plan(int64_t N, int64_t K, int cus)
{
    return make_tile_plan(N, K, kSwiglu, (size_t)4 * kEmitRows + 16, cus, true);
}

// Batched GEMV plan: the tile kernel's geometry (4 lanes per super-block, a
// row across the workgroup), LDS for a round of staged vectors or the M-way
// row reduction, whichever is larger.
Plan make_batch_plan(int64_t N, int64_t K, int kind, int M, int *round)
{
    Plan pl = make_tile_plan(N, K, kind, 0, 0, false);
    const size_t vbytes = (size_t)K + (size_t)K / 16;
    int r = (int)(kBatchStageBytes / vbytes);
    r = r < 1 ? 1 : (r > M ? M : r);
    if (round) *round = r;
    pl.x_in_lds = 1;
    const size_t red = (size_t)2 * M * pl.rows_tile * pl.nb * 4;
    pl.lds_bytes = (size_t)r * vbytes > red ? (size_t)r * vbytes : red;
    return pl;
}

// Resident workgroups per CU of a kernel at a block size and LDS size,
// cached (occupancy depends only on those and the compiled kernel).
static int occupancy(const void *fn, int threads, size_t lds)
{
    struct Entry { const void *fn; int threads; size_t lds; int occ; };
    static std::mutex mu;
    static Entry cache[64];
    static int n = 0;
    {
        std::lock_guard<std::mutex> g(mu);
        for (int i = 0; i < n; ++i)
            if (cache[i].fn == fn && cache[i].threads == threads && cache[i].lds == lds) return cache[i].occ;
    }
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, threads, lds) != hipSuccess || occ < 1) occ = 1;
    std::lock_guard<std::mutex> g(mu);
    if (n < 64) cache[n++] = Entry{fn, threads, lds, occ};
    return occ;
}

// At most one resident wave of workgroups (persistent grid), and at least
// `min_tiles` tiles per workgroup: a workgroup's start-up (activation staging,
// first-tile latency) costs several tile times, so short grids run faster
// with fewer, longer-lived workgroups.
static int grid_for(const Plan &pl, const void *fn, int cus, int min_tiles)
{
    int64_t g = (int64_t)cus * occupancy(fn, pl.threads, pl.lds_bytes);
    const int64_t by_tiles = (pl.tiles + min_tiles - 1) / min_tiles;
    if (g > by_tiles) g = by_tiles;
    if (g < 1) g = 1;
    return (int)g;
}

static GemvArgs base_args(const Plan &pl, int64_t N)
{
    GemvArgs a{};
    a.N = N;
    a.tiles = (int)pl.tiles;
    a.nb = pl.nb;
    a.lanes_row = pl.lanes_row;
    a.lanes_row_magic = (uint32_t)((((uint64_t)1 << 32) + (uint64_t)pl.lanes_row - 1) / (uint64_t)pl.lanes_row);
    a.rows_tile = pl.rows_tile;
    a.x_in_lds = pl.x_in_lds;
    a.steps = pl.steps;
    a.chunk_shift = pl.chunk_shift;
    a.red_off = (uint32_t)pl.red_off;
    return a;
}

// Launch on stream s; with a start or stop event the kernel's own start and
// end are recorded into them (hipExtLaunchKernel), so their elapsed time is
// the kernel's duration.
template <typename Kern>
static void launch_on(Kern k, const Plan &pl, const GemvArgs &a_in, hipStream_t s, const Timing &tm)
{
    GemvArgs a = a_in;
    a.threads = pl.threads;
    if (tm.start || tm.stop)
        hipExtLaunchKernelGGL(k, dim3(pl.grid), dim3(pl.threads), (uint32_t)pl.lds_bytes, s, tm.start, tm.stop, 0u, a);
    else
        hipLaunchKernelGGL(k, dim3(pl.grid), dim3(pl.threads), pl.lds_bytes, s, a);
}

// CU-resident tile launch: pl.grid workgroups of pl.threads, each owning at
// most pl.phase contiguous tiles (all in flight at once).
template <int KIND, int EPI, bool XLDS>
static hipError_t launch_resident(Plan &pl, GemvArgs a, hipStream_t s, const Timing &tm)
{
    a.tiles_q = (int)(pl.tiles / pl.grid);
    a.tiles_r = (int)(pl.tiles % pl.grid);
    switch (pl.phase) {
    case 1: launch_on(gemv_kernel<KIND, EPI, 1, XLDS, true>, pl, a, s, tm); break;
    case 2: launch_on(gemv_kernel<KIND, EPI, 2, XLDS, true>, pl, a, s, tm); break;
    default:
        if constexpr (KIND != kSwiglu) {
            if (pl.phase == 3) launch_on(gemv_kernel<KIND, EPI, 3, XLDS, true>, pl, a, s, tm);
            else launch_on(gemv_kernel<KIND, EPI, kResMaxPhase, XLDS, true>, pl, a, s, tm);
        }
        break;
    }
    return hipGetLastError();
}

template <int KIND, int EPI, bool XLDS>
static hipError_t launch_mode(Plan &pl, GemvArgs a, int cus, hipStream_t s, const Timing &tm)
{
    if (pl.resident) return launch_resident<KIND, EPI, XLDS>(pl, a, s, tm);
    // the occupancy of the deeper-pipelined kernel sizes the grid; if that
    // leaves at most one tile per workgroup the single-tile kernel runs
    const void *fn2 = (const void *)gemv_kernel<KIND, EPI, 2, XLDS>;
    // Fewest tiles per workgroup: a workgroup's start-up is mostly its copy
    // of x, so a short x (<= 16 KiB: K <= 4096 in f32) is worth spreading
    // over more workgroups of 3 tiles, a long one over fewer of 4 (measured:
    // 9728 x 2560 6.85 us with 3 against 7.15 us with 4; 2560 x 9728 8.9 us
    // with 3 against 7.2 us with 4).  The SwiGLU pair doubles a tile's work.
    const int64_t x_bytes = (int64_t)pl.nb * kQK * (is_q8(KIND) ? 1 : 4);
    pl.grid = grid_for(pl, fn2, cus, KIND == kSwiglu ? 2 : (x_bytes <= 16384 ? 3 : 4));
    if (is_argmax(EPI) && pl.grid > kArgmaxMaxGrid) pl.grid = kArgmaxMaxGrid;
    if constexpr (EPI == kQ8Emit) {
        // a workgroup's rows must fit its LDS row buffer
        const int64_t per = kEmitRows / pl.rows_tile;
        const int64_t need = (pl.tiles + per - 1) / per;
        if (pl.grid < need) pl.grid = (int)need;
    }
    a.tiles_q = (int)(pl.tiles / pl.grid);
    a.tiles_r = (int)(pl.tiles % pl.grid);
    // the SwiGLU pair keeps one tile in flight (its tile is two matrices'
    // worth of loads already; measured 10.2 against 10.4 us at 9728 x 2560)
    if (KIND != kSwiglu && (a.tiles_q >= 2 || (a.tiles_q == 1 && a.tiles_r > 0)))
        launch_on(gemv_kernel<KIND, EPI, 2, XLDS>, pl, a, s, tm);
    else
        launch_on(gemv_kernel<KIND, EPI, 1, XLDS>, pl, a, s, tm);
    return hipGetLastError();
}

// Waves of gemv_wave_kernel<KIND, EPI> one workgroup can have while one such
// workgroup still fits on a CU (registers, LDS), cached per LDS size.
static int wave_kernel_waves(const void *fn, size_t lds, int max_waves)
{
    struct Entry { const void *fn; size_t lds; int waves; };
    static std::mutex mu;
    static Entry cache[32];
    static int n = 0;
    {
        std::lock_guard<std::mutex> g(mu);
        for (int i = 0; i < n; ++i)
            if (cache[i].fn == fn && cache[i].lds == lds) return cache[i].waves;
    }
    int waves = 1;
    for (int w = max_waves; w >= 1; --w) {
        int occ = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, 64 * w, lds) == hipSuccess && occ >= 1) {
            waves = w;
            break;
        }
    }
    std::lock_guard<std::mutex> g(mu);
    if (n < 32) cache[n++] = Entry{fn, lds, waves};
    return waves;
}

// One workgroup per CU (at most one per unit), each with as many waves as fit
// on a CU next to nothing else, but no more waves than it has units.
template <typename Kern>
static hipError_t launch_per_cu(Kern k, int max_waves, Plan &pl, const GemvArgs &a, int cus, hipStream_t s,
                                const Timing &tm)
{
    const int wmax = wave_kernel_waves((const void *)k, pl.lds_bytes, max_waves);
    int64_t grid = pl.tiles < cus ? pl.tiles : cus;
    if (grid > kArgmaxMaxGrid) grid = kArgmaxMaxGrid;
    const int64_t per = (pl.tiles + grid - 1) / grid;   // units per workgroup
    pl.grid = (int)grid;
    pl.waves = (int)(per < wmax ? per : wmax);
    pl.threads = 64 * pl.waves;
    launch_on(k, pl, a, s, tm);
    return hipGetLastError();
}

template <int KIND, int EPI, int STEPS>
static hipError_t launch_wave(Plan &pl, const GemvArgs &a, int cus, hipStream_t s, const Timing &tm)
{
    // rows of two halves (Q4_K x Q8 at K = 8192) run 8 waves per CU, each
    // walking twice the rows, rather than 16 (measured at 28672 x 8192,
    // interleaved on one device: 24.0 against 24.7 us; 6 waves 29.2 us)
    constexpr int kWaves = STEPS == 2 ? kHalvesWaves : wave_max_threads<KIND>() / 64;
    return launch_per_cu(gemv_wave_kernel<KIND, EPI, STEPS>, kWaves, pl, a, cus, s, tm);
}

template <int KIND, int EPI>
static hipError_t launch(Plan &pl, const GemvArgs &a, int cus, hipStream_t s, const Timing &tm = Timing{})
{
    if (pl.wave_local) {
        if (pl.rows_kernel) return launch_per_cu(gemv_rows_kernel<KIND, EPI, 0>, pl.waves, pl, a, cus, s, tm);
        if constexpr (KIND == kQ4KQ8)
            if (pl.steps == 2) return launch_wave<KIND, EPI, 2>(pl, a, cus, s, tm);
        return launch_wave<KIND, EPI, 1>(pl, a, cus, s, tm);
    }
    return pl.x_in_lds ? launch_mode<KIND, EPI, true>(pl, a, cus, s, tm) : launch_mode<KIND, EPI, false>(pl, a, cus, s, tm);
}

hipError_t launch_q4k_gemv(const void *W, const float *x, float *y, int64_t N, int64_t K, int cus, hipStream_t s)
{
    Plan pl = make_plan(N, K, kQ4K, cus);
    GemvArgs a = base_args(pl, N);
    a.W = (const uint8_t *)W;
    a.x = x;
    a.y = y;
    return launch<kQ4K, kStore>(pl, a, cus, s);
}

hipError_t launch_q6k_gemv(const void *W, const float *x, float *y, int64_t N, int64_t K, int cus, hipStream_t s)
{
    Plan pl = make_plan(N, K, kQ6K, cus);
    GemvArgs a = base_args(pl, N);
    a.W = (const uint8_t *)W;
    a.x = x;
    a.y = y;
    return launch<kQ6K, kStore>(pl, a, cus, s);
}

hipError_t launch_swiglu_gemv(const void *Wg, const void *Wu, const float *x, float *h, int64_t N, int64_t K, int cus,
                              hipStream_t s)
{
    Plan pl = make_plan(N, K, kSwiglu, cus);
    GemvArgs a = base_args(pl, N);
    a.W = (const uint8_t *)Wg;
    a.W2 = (const uint8_t *)Wu;
    a.x = x;
    a.y = h;
    return launch<kSwiglu, kStore>(pl, a, cus, s);
}

hipError_t launch_q4k_q8_gemv(const void *W, const int8_t *xq, const uint16_t *xd, float *y, int64_t N, int64_t K,
                              int cus, hipStream_t s)
{
    Plan pl = make_plan(N, K, kQ4KQ8, cus);
    GemvArgs a = base_args(pl, N);
    a.W = (const uint8_t *)W;
    a.xq = xq;
    a.xd = xd;
    a.y = y;
    return launch<kQ4KQ8, kStore>(pl, a, cus, s);
}

hipError_t launch_q4k_q8_gemv_from_f32(const void *W, const float *x, int8_t *xq, uint16_t *xd, float *y, int64_t N,
                                       int64_t K, int cus, hipStream_t s)
{
    Plan pl = make_plan(N, K, kQ4KQ8, cus);
    if (pl.wave_local && !pl.rows_kernel) {
        // wave-unit kernel: the quantization runs in its prologue; the
        // scales take K/16 bytes of LDS past the codes
        GemvArgs a = base_args(pl, N);
        a.W = (const uint8_t *)W;
        a.x = x;
        a.hq = xq;
        a.hd = xd;
        a.y = y;
        pl.lds_bytes = ((pl.lds_bytes + 15) & ~(size_t)15) + (size_t)(K / 16);
        if (pl.steps == 2)
            return launch_per_cu(gemv_wave_kernel<kQ4KQ8, kStore, 2, true>, kQuantHalvesWaves, pl, a, cus, s, Timing{});
        return launch_per_cu(gemv_wave_kernel<kQ4KQ8, kStore, 1, true>, wave_max_threads<kQ4KQ8>() / 64, pl, a, cus,
                             s, Timing{});
    }
    // other shapes: the quantize launch, then the GEMV on its output (the
    // same codes, the same GEMV)
    const hipError_t e = launch_q8_quantize(x, xq, xd, K, s);
    if (e != hipSuccess) return e;
    return launch_q4k_q8_gemv(W, xq, xd, y, N, K, cus, s);
}

hipError_t launch_swiglu_q8_gemv(const void *Wg, const void *Wu, const float *x, float *h, int8_t *hq, uint16_t *hd,
                                 void *ws, int64_t N, int64_t K, int cus, hipStream_t s)
{
    Plan pl = make_swiglu_q8_plan(N, K, cus);
    GemvArgs a = base_args(pl, N);
    a.W = (const uint8_t *)Wg;
    a.W2 = (const uint8_t *)Wu;
    a.x = x;
    a.y = h;
    a.hq = hq;
    a.hd = hd;
    a.ws = (uint8_t *)ws;
    a.emit_vals_off = (uint32_t)swiglu_q8_vals_offset(N);
    a.emit_lds_off = (uint32_t)((pl.lds_bytes + 15) & ~(size_t)15);
    pl.lds_bytes = a.emit_lds_off + (size_t)4 * kEmitRows;
    return pl.x_in_lds ? launch_mode<kSwiglu, kQ8Emit, true>(pl, a, cus, s, Timing{})
                       : launch_mode<kSwiglu, kQ8Emit, false>(pl, a, cus, s, Timing{});
}

template <int KIND, int M>
static hipError_t launch_batch_m(Plan &pl, GemvArgs a, int cus, hipStream_t s)
{
    const void *fn2 = (const void *)gemv_batch_kernel<KIND, M, 2>;
    pl.grid = grid_for(pl, fn2, cus, 4);
    a.tiles_q = (int)(pl.tiles / pl.grid);
    a.tiles_r = (int)(pl.tiles % pl.grid);
    if (a.tiles_q >= 2 || (a.tiles_q == 1 && a.tiles_r > 0))
        launch_on(gemv_batch_kernel<KIND, M, 2>, pl, a, s, Timing{});
    else
        launch_on(gemv_batch_kernel<KIND, M, 1>, pl, a, s, Timing{});
    return hipGetLastError();
}

template <int KIND>
static hipError_t launch_batch_kind(Plan &pl, const GemvArgs &a, int M, int cus, hipStream_t s)
{
    switch (M) {
    case 1: return launch_batch_m<KIND, 1>(pl, a, cus, s);
    case 2: return launch_batch_m<KIND, 2>(pl, a, cus, s);
    case 4: return launch_batch_m<KIND, 4>(pl, a, cus, s);
    default:
        if constexpr (KIND == kQ4KQ8) return launch_batch_m<KIND, 8>(pl, a, cus, s);
        return hipErrorInvalidValue;   // not reached: batch_slots caps Q6_K at 4
    }
}

// Vector slots of one launch for m vectors: 1, 2, 4 or 8.  Eight Q6_K x Q8
// slices (20 registers each) next to the Q6_K blocks in flight exceed the
// register file, so Q6_K launches take at most 4 and larger batches run in
// launches of 4.
int batch_slots(int m, bool q6k)
{
    const int cap = q6k ? 4 : kMaxBatch;
    const int M = m <= 1 ? 1 : m <= 2 ? 2 : m <= 4 ? 4 : 8;
    return M < cap ? M : cap;
}

hipError_t launch_q8_gemv_batch(bool q6k, const void *W, const int8_t *xq, const uint16_t *xd, float *y, int64_t N,
                                int64_t K, int m, int cus, hipStream_t s)
{
    int M = batch_slots(m, q6k);
    int round = 1;
    Plan pl = make_batch_plan(N, K, q6k ? kQ6KQ8 : kQ4KQ8, M, &round);
    // Eight slots make a long-running launch VALU- and register-bound: with
    // a lot of weight per compute unit two launches of four are faster
    // (28,672 x 8192, 460 KB per CU: 88 us against 107 us); short launches,
    // bound by start-up, keep the single pass over the weights (9728 x 2560,
    // 55 KB per CU: 13.9 us against 19.0 us).
    const int64_t wbytes = N * (K / kQK) * (q6k ? kQ6KBytes : kQ4KBytes);
    if (M == 8 && wbytes >= (int64_t)kBatchSplitBytesPerCu * cus) {
        M = 4;
        pl = make_batch_plan(N, K, q6k ? kQ6KQ8 : kQ4KQ8, M, &round);
    }
    for (int j0 = 0; j0 < m; j0 += M) {
        Plan p = pl;
        GemvArgs a = base_args(p, N);
        a.W = (const uint8_t *)W;
        a.xq = xq + (size_t)j0 * K;
        a.xd = xd + (size_t)j0 * (K / 32);
        a.y = y + (size_t)j0 * N;
        a.batch = m - j0 < M ? m - j0 : M;
        a.batch_round = round;
        const hipError_t e =
            q6k ? launch_batch_kind<kQ6KQ8>(p, a, M, cus, s) : launch_batch_kind<kQ4KQ8>(p, a, M, cus, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_q6k_q8_gemv(const void *W, const int8_t *xq, const uint16_t *xd, float *y, int64_t N, int64_t K,
                              int cus, hipStream_t s)
{
    Plan pl = make_plan(N, K, kQ6KQ8, cus);
    GemvArgs a = base_args(pl, N);
    a.W = (const uint8_t *)W;
    a.xq = xq;
    a.xd = xd;
    a.y = y;
    return launch<kQ6KQ8, kStore>(pl, a, cus, s);
}

hipError_t launch_lm_head_argmax(const void *W, const float *x, const uint32_t *mask, uint32_t *out_idx,
                                 float *out_max, void *ws, int64_t N, int64_t K, int cus, hipStream_t s,
                                 const Timing &tm)
{
    Plan pl = make_plan(N, K, kQ6K, cus);
    GemvArgs a = base_args(pl, N);
    a.W = (const uint8_t *)W;
    a.x = x;
    a.ws = (uint8_t *)ws;
    a.out_idx = out_idx;
    a.out_max = out_max;
    a.mask = mask;
    if (mask) return launch<kQ6K, kArgmaxMasked>(pl, a, cus, s, tm);
    return launch<kQ6K, kArgmax>(pl, a, cus, s, tm);
}

// Multi-output launch on CU-resident tiles, where one matrix of all the
// rows would take that form: waves per workgroup w in {4, 8, 12}, each
// matrix's rows in tiles of its own (R = 64w / (4 nb) rows), the w whose
// busiest CU has the fewest rows with its tiles all in flight (at most
// kResMaxPhase) and x staged in LDS.  False if there is none.
static bool launch_multi_resident(const void *const *W, const int64_t *N, float *const *y, const float *const *r,
                                  int count, const float *x, int64_t total, int64_t K, int cus, hipStream_t s,
                                  hipError_t &err)
{
    const Plan single = make_plan(total, K, kQ4K, cus);
    if (single.wave_local || !single.resident) return false;
    Plan pl = single;
    int64_t best_rows = INT64_MAX, best_tiles = 0, best_per = 0;
    int best_w = 0;
    for (int w = 4; w <= kResThreads / 64; w += 4) {
        const int rows = 64 * w / pl.lanes_row;
        if (rows < 2) continue;   // x is staged in LDS only when rows share it
        int64_t tiles = 0;
        for (int m = 0; m < count; ++m) tiles += (N[m] + rows - 1) / rows;
        const int64_t per = (tiles + cus - 1) / cus;
        if (per > kResMaxPhase) continue;
        const size_t red = (size_t)per * rows * pl.nb * 4;
        const size_t staged = (tile_staged_bytes(K, kQ4K, true) + 15) & ~(size_t)15;
        if (staged + red > 65536) continue;
        if (per * rows < best_rows) {
            best_rows = per * rows;
            best_w = w;
            best_tiles = tiles;
            best_per = per;
        }
    }
    if (!best_w) return false;
    pl.waves = best_w;
    pl.threads = 64 * best_w;
    pl.rows_tile = pl.threads / pl.lanes_row;
    pl.phase = (int)best_per;
    pl.tiles = best_tiles;
    pl.grid = (int)((best_tiles + best_per - 1) / best_per);
    pl.x_in_lds = 1;
    pl.red_off = (tile_staged_bytes(K, kQ4K, true) + 15) & ~(size_t)15;
    pl.lds_bytes = pl.red_off + (size_t)best_per * pl.rows_tile * pl.nb * 4;
    GemvArgs a = base_args(pl, total);
    a.x = x;
    int64_t t = 0;
    for (int m = 0; m < kMaxMulti; ++m) {
        a.ustart[m] = m < count ? (int)t : INT32_MAX;
        a.Wm[m] = m < count ? (const uint8_t *)W[m] : nullptr;
        a.ym[m] = m < count ? y[m] : nullptr;
        a.rm[m] = (m < count && r) ? r[m] : nullptr;
        a.Nm[m] = m < count ? N[m] : 0;
        if (m < count) t += (N[m] + pl.rows_tile - 1) / pl.rows_tile;
    }
    a.ustart[kMaxMulti] = INT32_MAX;
    a.W = a.Wm[0];
    a.y = a.ym[0];
    a.tiles_q = (int)(pl.tiles / pl.grid);
    a.tiles_r = (int)(pl.tiles % pl.grid);
    switch (pl.phase) {
    case 1: launch_on(gemv_kernel_multi<1>, pl, a, s, Timing{}); break;
    case 2: launch_on(gemv_kernel_multi<2>, pl, a, s, Timing{}); break;
    case 3: launch_on(gemv_kernel_multi<3>, pl, a, s, Timing{}); break;
    default: launch_on(gemv_kernel_multi<kResMaxPhase>, pl, a, s, Timing{}); break;
    }
    err = hipGetLastError();
    return true;
}

hipError_t launch_q4k_gemv_multi(const void *const *W, const int64_t *N, float *const *y, const float *const *r,
                                 int count, const float *x, int64_t K, int cus, hipStream_t s)
{
    int64_t total = 0;
    for (int m = 0; m < count; ++m) total += N[m];
    // CU-resident tiles where one matrix of all the rows would take them
    // (q, k and v of 4096 + 1024 + 1024 rows at K = 2560, graph replay:
    // 6.82 us on the row-stream kernel, 6.26 us on 8-wave resident tiles;
    // 4 waves with 5 tiles each measured 0.2 us slower)
    hipError_t err = hipSuccess;
    if (launch_multi_resident(W, N, y, r, count, x, total, K, cus, s, err)) return err;
    // otherwise one row-stream plan for the stacked matrices (every row inside one wave)
    Plan pl{};
    plan_rows(pl, total, K, kQ4K);
    GemvArgs a = base_args(pl, total);
    a.x = x;
    int64_t u = 0;
    for (int m = 0; m < kMaxMulti; ++m) {
        a.ustart[m] = (int)u;
        if (m < count) {
            a.Wm[m] = (const uint8_t *)W[m];
            a.ym[m] = y[m];
            a.rm[m] = r ? r[m] : nullptr;
            a.Nm[m] = N[m];
            u += (N[m] + pl.rows_tile - 1) / pl.rows_tile;
        } else {
            a.Wm[m] = nullptr;
            a.ym[m] = nullptr;
            a.rm[m] = nullptr;
            a.Nm[m] = 0;
        }
    }
    for (int m = count; m < kMaxMulti; ++m) a.ustart[m] = INT32_MAX;
    a.ustart[kMaxMulti] = INT32_MAX;
    pl.tiles = u;
    a.tiles = (int)u;
    a.W = a.Wm[0];
    a.y = a.ym[0];
    return launch_per_cu(gemv_rows_kernel<kQ4K, kStore, 1>, pl.waves, pl, a, cus, s, Timing{});
}

__global__ __launch_bounds__(256) void fill_zero_kernel(u32x4 *p, int n16)
{
    for (int i = (int)threadIdx.x; i < n16; i += (int)blockDim.x) p[i] = u32x4{0u, 0u, 0u, 0u};
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s)
{
    if (bytes % 16 != 0 || bytes > 65536 || ((uintptr_t)p & 15) != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(1), dim3(256), 0, s, (u32x4 *)p, (int)(bytes / 16));
    return hipGetLastError();
}

// Plain streaming read, the measured ceiling the GEMVs are compared with:
// every byte of p[0, n16 * 16) is read once with 16-byte loads, grid-stride
// over the whole buffer, and folded into one word that is stored only if it
// equals a value no seeded input produces (so the loads cannot be dropped
// and nothing is written in practice).  One load per thread per iteration,
// in workgroups of 256 or 1024 threads; the benchmark keeps the best over
// both sizes and a range of grids.  In a sweep at 132 and 209 MB (1, 2, 4, 8
// or 16 loads per thread per iteration, 256 or 1024 threads, grids of 256 to
// 16384, with and without the nontemporal hint) this form was among the
// fastest (20.8 and 32.4 us), against 22.1 and 34.6 us for four loads per
// iteration in 256-thread workgroups.
__global__ __launch_bounds__(1024) void stream_read_kernel(const u32x4 *__restrict__ p, int64_t n16,
                                                                   uint32_t *__restrict__ sink)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) acc ^= p[i];
    const uint32_t w = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (w == 0x9E3779B9u) sink[threadIdx.x & 255] = w;
}

hipError_t launch_stream_read(const void *p, int64_t bytes, int grid, int threads, uint32_t *sink, hipStream_t s)
{
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(threads), 0, s, (const u32x4 *)p, bytes / 16, sink);
    return hipGetLastError();
}

hipError_t launch_q8_quantize(const float *x, int8_t *xq, uint16_t *xd, int64_t K, hipStream_t s)
{
    const int threads = 256;
    const int blocks = (int)((K + threads - 1) / threads);
    hipLaunchKernelGGL(q8_quantize_kernel, dim3(blocks), dim3(threads), 0, s, x, xq, xd, (int)K);
    return hipGetLastError();
}

hipError_t launch_q4k_q8_isums(const void *W, const int8_t *xq, int32_t *isums, int64_t N, int64_t K, hipStream_t s)
{
    const int nb = (int)(K / kQK);
    const int64_t total = N * nb * kParts;
    const int threads = 256;
    const int64_t blocks = (total + threads - 1) / threads;
    hipLaunchKernelGGL(q4k_q8_isums_kernel, dim3((unsigned)blocks), dim3(threads), 0, s, (const uint8_t *)W, xq, isums,
                       N, nb);
    return hipGetLastError();
}

}  // namespace gemvq

namespace gemvq {

hipError_t launch_q6k_q8_isums(const void *W, const int8_t *xq, int32_t *isums, int64_t N, int64_t K, hipStream_t s)
{
    const int nb = (int)(K / kQK);
    const int64_t total = N * nb * kParts;
    const int threads = 256;
    const int64_t blocks = (total + threads - 1) / threads;
    hipLaunchKernelGGL(q6k_q8_isums_kernel, dim3((unsigned)blocks), dim3(threads), 0, s, (const uint8_t *)W, xq, isums,
                       N, nb);
    return hipGetLastError();
}

}  // namespace gemvq

namespace gemvq {

template <bool ADD>
static void launch_norm(const float *x, const float *r, const float *w, float eps, float *res, float *y, int8_t *xq,
                        uint16_t *xd, int K, hipStream_t s)
{
    const int passes = (K + kNormSpan - 1) / kNormSpan;
    const dim3 g(1), b(kNormThreads);
    if (passes <= 1)
        hipLaunchKernelGGL((rms_norm_q8_kernel<ADD, 1>), g, b, 0, s, x, r, w, eps, res, y, xq, xd, K);
    else if (passes <= 2)
        hipLaunchKernelGGL((rms_norm_q8_kernel<ADD, 2>), g, b, 0, s, x, r, w, eps, res, y, xq, xd, K);
    else if (passes <= 4)
        hipLaunchKernelGGL((rms_norm_q8_kernel<ADD, 4>), g, b, 0, s, x, r, w, eps, res, y, xq, xd, K);
    else
        hipLaunchKernelGGL((rms_norm_q8_kernel<ADD, 8>), g, b, 0, s, x, r, w, eps, res, y, xq, xd, K);
}

hipError_t launch_rms_norm_q8(const float *x, const float *r, const float *w, float eps, float *res, float *y,
                              int8_t *xq, uint16_t *xd, int64_t K, hipStream_t s)
{
    if (r)
        launch_norm<true>(x, r, w, eps, res, y, xq, xd, (int)K, s);
    else
        launch_norm<false>(x, r, w, eps, res, y, xq, xd, (int)K, s);
    return hipGetLastError();
}

}  // namespace gemvq
