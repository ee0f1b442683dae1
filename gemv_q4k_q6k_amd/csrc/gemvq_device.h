// Device-side building blocks of the gfx950 GEMV kernels: super-block loads,
// in-register dequantisation + dot products, wave reductions.
//
// Lane geometry shared by every GEMV kernel.  A row of K weights is K/256
// super-blocks; four lanes ("parts") share each super-block, so a row occupies
// lanes_row = 4 * (K/256) consecutive lanes of the workgroup.  A workgroup of W
// waves holds P = floor(64*W / lanes_row) rows at a time (a "tile").  A lane's
// (row-in-tile, block, part) never changes while the workgroup walks its
// tiles, so each lane loads the 64 activation values its part multiplies once
// and keeps them in VGPRs; per tile it streams only weight bytes.
//
//   Q4_K part c (0..3): quant bytes qs[32c, 32c+32) = low nibbles of sub-block
//     2c (weights 64c + i) and high nibbles of sub-block 2c+1 (64c + 32 + i).
//   Q6_K part u (0..3), n = u>>1, l0 = 16*(u&1): ql[64n+l0, +16),
//     ql[64n+32+l0, +16) and qh[32n+l0, +16) = weights 128n + 32s + l0 + i for
//     s = 0..3, i < 16, one int8 scale per s.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// No multiply is fused into an add unless the code says so (fmaf): with the
// compiler free to contract, two kernels built from the same device code
// (another tile geometry template, the multi-output form, the Q8-emitting
// epilogue) could round a row differently, and the library promises equal
// bits wherever the row arithmetic is the same.
#pragma clang fp contract(off)

namespace gemvq {

constexpr int kQK = 256;
constexpr int kQ4KBytes = 144;
constexpr int kQ6KBytes = 210;
constexpr int kParts = 4;                 // lanes per super-block
constexpr uint32_t kNoIndex = 0xFFFFFFFFu;

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// f16 "magic" conversion: OR-ing a 10-bit integer m into the mantissa of
// 1024.0h (0x6400) gives the exact half value 1024 + m.  Two such halves per
// dword feed v_fma_mix_f32 directly (f16 operand, f32 accumulate).
constexpr uint32_t kMagic2 = 0x64006400u;

__device__ __forceinline__ h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }

// (v & mask) | other in one v_and_or_b32.  gfx9 VOP3 encodings take no
// literal constants, so the compiler otherwise splits this into a VOP2 and +
// or pair; the mask goes in an SGPR and `other` in a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t v, uint32_t mask, uint32_t other)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(v), "s"(mask), "v"(other));
    return r;
}

__device__ __forceinline__ float half_lo(uint32_t v) { return (float)as_h2(v).x; }
__device__ __forceinline__ float half_hi(uint32_t v) { return (float)as_h2(v).y; }

// ---------------------------------------------------------------- DPP
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Sum over the 4 lanes of a quad; every lane of the quad gets the same bits
// (each step adds a value to its mirror partner, a commutative pair).
__device__ __forceinline__ float quad_sum(float v)
{
    v += dpp_f<kDppQuadXor1>(v);
    v += dpp_f<kDppQuadXor2>(v);
    return v;
}

// Sum over aligned groups of `group` lanes (4, 8, 16, 32 or 64), same bits in
// every lane of a group.  Lane groups start at multiples of `group`.
__device__ __forceinline__ float group_sum(float v, int group)
{
    v = quad_sum(v);
    if (group >= 8) v += dpp_f<kDppRowHalfMirror>(v);
    if (group >= 16) v += dpp_f<kDppRowMirror>(v);
    if (group >= 32) v += __shfl_xor(v, 16);
    if (group >= 64) v += __shfl_xor(v, 32);
    return v;
}

// ------------------------------------------------------------- argmax
// Argmax candidates are ordered so that NaN never wins, a larger value wins,
// and of two equal values (-0 == +0) the smaller index wins.  The 64-bit key
// below has exactly that unsigned order: the high word maps the float
// monotonically to an unsigned integer (-0 folded onto +0), the low word is
// ~index.  Key 0 means "no candidate" (no real candidate maps to it; NaN rows
// are never keyed).
__device__ __forceinline__ uint64_t argmax_key(float v, uint32_t i)
{
    uint32_t f = __float_as_uint(v == 0.f ? 0.f : v);
    f = (f & 0x80000000u) ? ~f : (f | 0x80000000u);
    return ((uint64_t)f << 32) | (uint64_t)(~i);
}

__device__ __forceinline__ float argmax_key_value(uint64_t k)
{
    const uint32_t f = (uint32_t)(k >> 32);
    return __uint_as_float((f & 0x80000000u) ? (f & 0x7FFFFFFFu) : ~f);
}

__device__ __forceinline__ uint32_t argmax_key_index(uint64_t k) { return ~(uint32_t)k; }

// Largest unsigned value over a fully active wave, returned uniformly: the
// maximum within each row of 16 lanes by DPP (quad swaps, half-row and row
// mirrors), then across the four rows by lane reads.  No LDS round trip, so
// the chain is a few dozen cycles instead of the ~100-cycle latency of each
// ds_bpermute step of a shuffle tree.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, dpp_u<0xB1>(v));    // quad_perm [1,0,3,2]
    v = max(v, dpp_u<0x4E>(v));    // quad_perm [2,3,0,1]
    v = max(v, dpp_u<0x141>(v));   // row_half_mirror
    v = max(v, dpp_u<0x140>(v));   // row_mirror
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(r0, r1), max(r2, r3));
}

// Largest argmax key over a fully active wave: the largest high word, then
// the largest low word among the lanes that hold it.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k)
{
    const uint32_t hi = wave_max_u32((uint32_t)(k >> 32));
    const uint32_t lo = wave_max_u32((uint32_t)(k >> 32) == hi ? (uint32_t)k : 0u);
    return ((uint64_t)hi << 32) | lo;
}

// Keeps a computed value in a register (stops the compiler from recomputing
// it inside a loop to save registers).
__device__ __forceinline__ void pin(float &v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin(int32_t &v) { asm volatile("" : "+v"(v)); }

// ---------------------------------------------------------------- Q4_K

struct Q4KRaw {
    u32x4 hdr;   // d | dmin<<16, scale bytes 0..3, 4..7, 8..11
    u32x4 q0;    // quant bytes [32c, 32c+16)
    u32x4 q1;    // quant bytes [32c+16, 32c+32)
};

// `tile` is workgroup-uniform (scalar registers) and `off` the lane's 32-bit
// byte offset of its super-block inside the tile, so every load is one
// global_load with an SGPR base, a VGPR offset and an immediate.
__device__ __forceinline__ void q4k_load(Q4KRaw &r, const uint8_t *__restrict__ tile, uint32_t off, int c)
{
    // 32-bit offsets from the uniform base, pinned where they are used (see
    // q6k_load)
    uint32_t oh = off, oq = off + 32u * (uint32_t)c + 16u;
    asm volatile("" : "+v"(oh), "+v"(oq));
    r.hdr = *(const u32x4 *)(tile + oh);
    r.q0 = *(const u32x4 *)(tile + oq);
    r.q1 = *(const u32x4 *)(tile + oq + 16u);
}

__device__ __forceinline__ void q4k_zero(Q4KRaw &r)
{
    r.hdr = u32x4{0, 0, 0, 0};
    r.q0 = r.hdr;
    r.q1 = r.hdr;
}

// Scale and min of sub-blocks 2c and 2c+1 from the 12 packed bytes.
// j < 4: scale = s[j] & 63, min = s[j+4] & 63;
// j >= 4: scale = (s[j+4] & 15) | (s[j-4] >> 6) << 4, min = (s[j+4] >> 4) | (s[j] >> 6) << 4.
__device__ __forceinline__ void q4k_scales(const u32x4 &hdr, int c, uint32_t &sc0, uint32_t &sc1,
                                           uint32_t &m0, uint32_t &m1)
{
    const uint32_t sh = (uint32_t)(c & 1) * 16u;
    const uint32_t A = hdr.y >> sh;      // s[2(c&1)], s[2(c&1)+1]
    const uint32_t B = hdr.z >> sh;      // s[4+2(c&1)], ...
    const uint32_t C = hdr.w >> sh;      // s[8+2(c&1)], ...
    if (c < 2) {
        sc0 = A & 63u;
        sc1 = (A >> 8) & 63u;
        m0 = B & 63u;
        m1 = (B >> 8) & 63u;
    } else {
        sc0 = (C & 15u) | ((A >> 2) & 0x30u);
        sc1 = ((C >> 8) & 15u) | ((A >> 10) & 0x30u);
        m0 = ((C >> 4) & 15u) | ((B >> 2) & 0x30u);
        m1 = ((C >> 12) & 15u) | ((B >> 10) & 0x30u);
    }
}

// Activation slice of a Q4_K part: xl = x[64c + i], xh = x[64c + 32 + i].
struct Q4KX {
    float xl[32];
    float xh[32];
    float sxl, sxh;   // sums of xl and xh
};

// Dot product of one Q4_K part with its activation slice (f32 accumulate).
// Quants enter as exact halves 1024+q (low nibble) and 1024+16q (high nibble),
// so acc_lo = sum q x + 1024 sum x and acc_hi = 16 sum q x + 1024 sum x; the
// offsets are removed with the precomputed sums.
__device__ __forceinline__ float q4k_dot(const Q4KRaw &r, const Q4KX &x, int c)
{
    uint32_t sc0, sc1, m0, m1;
    q4k_scales(r.hdr, c, sc0, sc1, m0, m1);
    const float d = half_lo(r.hdr.x);
    const float dmin = half_hi(r.hdr.x);
    const uint32_t w[8] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w};
    const uint32_t magic = kMagic2;
    float aL0 = 0.f, aL1 = 0.f, aH0 = 0.f, aH1 = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t v = w[k];
        const uint32_t v8 = v >> 8;
        const h2_t t0 = as_h2(and_or(v, 0x000F000Fu, magic));    // lo(b0), lo(b2)
        const h2_t t1 = as_h2(and_or(v, 0x00F000F0u, magic));    // 16hi(b0), 16hi(b2)
        const h2_t t2 = as_h2(and_or(v8, 0x000F000Fu, magic));   // lo(b1), lo(b3)
        const h2_t t3 = as_h2(and_or(v8, 0x00F000F0u, magic));   // 16hi(b1), 16hi(b3)
        aL0 = __builtin_fmaf((float)t0.x, x.xl[4 * k + 0], aL0);
        aL1 = __builtin_fmaf((float)t2.x, x.xl[4 * k + 1], aL1);
        aL0 = __builtin_fmaf((float)t0.y, x.xl[4 * k + 2], aL0);
        aL1 = __builtin_fmaf((float)t2.y, x.xl[4 * k + 3], aL1);
        aH0 = __builtin_fmaf((float)t1.x, x.xh[4 * k + 0], aH0);
        aH1 = __builtin_fmaf((float)t3.x, x.xh[4 * k + 1], aH1);
        aH0 = __builtin_fmaf((float)t1.y, x.xh[4 * k + 2], aH0);
        aH1 = __builtin_fmaf((float)t3.y, x.xh[4 * k + 3], aH1);
    }
    const float qxl = (aL0 + aL1) - 1024.f * x.sxl;             // sum q x, low sub-block
    const float qxh = ((aH0 + aH1) - 1024.f * x.sxh) * 0.0625f; // sum q x, high sub-block
    const float dl = d * (float)sc0, dh = d * (float)sc1;
    const float ml = dmin * (float)m0, mh = dmin * (float)m1;
    return (dl * qxl - ml * x.sxl) + (dh * qxh - mh * x.sxh);
}

// Activation slice of a Q4_K part in fixed point (row-stream and resident
// SwiGLU tile kernels): the part's 64 values (x[256b + 64c + i], i < 64: the
// low sub-block's 32, then the high one's) share one scale,
// X_i = rint(x_i * 2^(22-E)) with E the binary exponent of the part's largest
// |x| (frexp: largest |x| = f 2^E, 1/2 <= f < 1, so |X_i| <= 2^22 and the
// rounding error 2^(E-23) is at most 2^-22 of that value), split into a
// signed high byte and unsigned
// middle and low bytes, four elements to a dword (dwords 0..7 low sub-block,
// 8..15 high).  e = E - 22 undoes the scale; sxl and sxh are the f32 sums
// of the two sub-blocks for the min term.
struct Q4KFX {
    uint32_t hi[16], mid[16], lo[16];
    float sxl, sxh;
    int e;
};

// Dot product of one Q4_K part against a fixed-point slice: the nibbles of
// each quant dword (low nibbles: the low sub-block, high nibbles: the high
// one) go through one sdot4 with the signed high bytes and two udot4 with the
// unsigned middle and low bytes, exact in integers; each sub-block's three
// sums are joined in f32, scaled by d*sc and back by 2^e, and the min term is
// taken with the f32 sums.
__device__ __forceinline__ float q4k_dot(const Q4KRaw &r, const Q4KFX &x, int c)
{
    uint32_t sc0, sc1, m0, m1;
    q4k_scales(r.hdr, c, sc0, sc1, m0, m1);
    const float d = half_lo(r.hdr.x);
    const float dmin = half_hi(r.hdr.x);
    const uint32_t w[8] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w};
    int32_t lh = 0, hh = 0;
    uint32_t lm = 0u, ll = 0u, hm = 0u, hl = 0u;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t qn = w[k] & 0x0F0F0F0Fu;           // low nibbles: weights 4k..4k+3 of the low sub-block
        const uint32_t qm = (w[k] >> 4) & 0x0F0F0F0Fu;    // high nibbles: the same of the high sub-block
        lh = __builtin_amdgcn_sdot4((int)qn, (int)x.hi[k], lh, false);
        lm = __builtin_amdgcn_udot4(qn, x.mid[k], lm, false);
        ll = __builtin_amdgcn_udot4(qn, x.lo[k], ll, false);
        hh = __builtin_amdgcn_sdot4((int)qm, (int)x.hi[8 + k], hh, false);
        hm = __builtin_amdgcn_udot4(qm, x.mid[8 + k], hm, false);
        hl = __builtin_amdgcn_udot4(qm, x.lo[8 + k], hl, false);
    }
    // |lh| <= 32*15*64 and lm*256 + ll < 2^25: exact or one f32 rounding
    const float ql = __builtin_fmaf((float)lh, 65536.f, (float)((lm << 8) + ll));
    const float qh = __builtin_fmaf((float)hh, 65536.f, (float)((hm << 8) + hl));
    const float dl = d * (float)sc0, dh = d * (float)sc1;
    const float ml = dmin * (float)m0, mh = dmin * (float)m1;
    return __builtin_amdgcn_ldexpf(dl * ql + dh * qh, x.e) - (ml * x.sxl + mh * x.sxh);
}

// ------------------------------------------------------------ Q4_K x Q8

// Q8 activation slice of a Q4_K part: 32 int8 for each of sub-blocks 2c and
// 2c+1 packed in dwords, their fp16 scales as f32, and their integer sums.
struct Q8X {
    uint32_t ql[8];
    uint32_t qh[8];
    float dl, dh;
    int32_t sl, sh;
};

// Exact integer sums of one part: isl = sum q4*q8 over sub-block 2c, ish over 2c+1.
__device__ __forceinline__ void q4k_q8_isums(const Q4KRaw &r, const Q8X &x, int32_t &isl, int32_t &ish)
{
    const uint32_t w[8] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w};
    int32_t a = 0, b = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        a = __builtin_amdgcn_sdot4((int)(w[k] & 0x0F0F0F0Fu), (int)x.ql[k], a, false);
        b = __builtin_amdgcn_sdot4((int)((w[k] >> 4) & 0x0F0F0F0Fu), (int)x.qh[k], b, false);
    }
    isl = a;
    ish = b;
}

__device__ __forceinline__ float q4k_q8_dot(const Q4KRaw &r, const Q8X &x, int c)
{
    uint32_t sc0, sc1, m0, m1;
    q4k_scales(r.hdr, c, sc0, sc1, m0, m1);
    const float d = half_lo(r.hdr.x);
    const float dmin = half_hi(r.hdr.x);
    int32_t isl, ish;
    q4k_q8_isums(r, x, isl, ish);
    const float lo = d * (float)sc0 * (float)isl - dmin * (float)m0 * (float)x.sl;
    const float hi = d * (float)sc1 * (float)ish - dmin * (float)m1 * (float)x.sh;
    return x.dl * lo + x.dh * hi;
}

// ---------------------------------------------------------------- Q6_K

// A Q6_K block starts 2 bytes off a dword boundary when its flat index is odd.
// Its fields are loaded with dword loads at their true (2-byte aligned)
// addresses: the HSA code-object ABI for gfx9 runs the shader memory path in
// unaligned mode, so a global dword load needs only byte alignment (the
// compiler itself emits such loads for 2-byte aligned packed data on this
// target).  Every byte read lies inside the block.
struct Q6KRaw {
    uint32_t a[4];   // ql[64n+l0 .. +16)
    uint32_t b[4];   // ql[64n+32+l0 .. +16)
    uint32_t h[4];   // qh[32n+l0 .. +16)
    uint32_t s[2];   // scale window sc[8n .. 8n+8)
    uint32_t dbits;  // fp16 d in the low 16 bits
};

struct __attribute__((packed, aligned(2))) U32x4A2 { uint32_t v[4]; };
struct __attribute__((packed, aligned(2))) U32x2A2 { uint32_t v[2]; };

__device__ __forceinline__ void load4(uint32_t (&o)[4], const uint8_t *p)
{
    const U32x4A2 v = *(const U32x4A2 *)p;
    o[0] = v.v[0];
    o[1] = v.v[1];
    o[2] = v.v[2];
    o[3] = v.v[3];
}

// `tile` is the workgroup-uniform start of the unit or tile, `off` the lane's
// byte offset of its block in it; part u = 2n + (l0 / 16) of the block.
__device__ __forceinline__ void q6k_load(Q6KRaw &r, const uint8_t *__restrict__ tile, uint32_t off, int u)
{
    // one 32-bit lane offset per field from the uniform base, so each load
    // takes the scalar-base form (no 64-bit address arithmetic per lane).  The
    // empty asm marks each offset as (re)defined where it is used: when the
    // offsets do not change across a loop, the compiler would otherwise
    // widen them to 64 bits outside it and add them to the base with a
    // 64-bit VALU add per load.
    const uint32_t n = (uint32_t)(u >> 1), l0 = 16u * (uint32_t)(u & 1);
    uint32_t oa = off + 64u * n + l0, ob = off + 64u * n + 32u + l0, oh = off + 128u + 32u * n + l0;
    uint32_t os = off + 192u + 8u * n, od = off + 208u;
    asm volatile("" : "+v"(oa), "+v"(ob), "+v"(oh), "+v"(os), "+v"(od));
    load4(r.a, tile + oa);
    load4(r.b, tile + ob);
    load4(r.h, tile + oh);
    const U32x2A2 sc = *(const U32x2A2 *)(tile + os);
    r.s[0] = sc.v[0];
    r.s[1] = sc.v[1];
    r.dbits = *(const uint16_t *)(tile + od);
}

__device__ __forceinline__ void q6k_zero(Q6KRaw &r)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) r.a[i] = r.b[i] = r.h[i] = 0u;
    r.s[0] = r.s[1] = 0u;
    r.dbits = 0u;
}

// Activation slice of a Q6_K part: xs[s][i] = x[128n + 32s + l0 + i].
struct Q6KX {
    float xs[4][16];
    float sx[4];     // sum over i of xs[s][i]
};

// Quants of dword k of a Q6_K part: byte j of q[s] is the 6-bit quant (0..63)
// of weight 128n + 32s + l0 + 4k + j, assembled from its ql nibble and its qh
// bit pair with one v_and_or_b32 each.
__device__ __forceinline__ void q6k_quants(const Q6KRaw &r, int k, uint32_t (&q)[4])
{
    const uint32_t a = r.a[k], b = r.b[k], h = r.h[k];
    q[0] = and_or(h << 4, 0x30303030u, a & 0x0F0F0F0Fu);
    q[1] = and_or(h << 2, 0x30303030u, b & 0x0F0F0F0Fu);
    q[2] = and_or(h, 0x30303030u, (a >> 4) & 0x0F0F0F0Fu);
    q[3] = and_or(h >> 2, 0x30303030u, (b >> 4) & 0x0F0F0F0Fu);
}

// The four int8 scales of part u: sc[s] = sc[8n + (u&1) + 2s], bytes (u&1) + 2s
// of the 8-byte scale window.
__device__ __forceinline__ void q6k_scales(const Q6KRaw &r, int u, int (&sc)[4])
{
    const uint32_t s0 = r.s[0], s1 = r.s[1];
    const uint32_t bo = (uint32_t)(u & 1) * 8u;
    sc[0] = __builtin_amdgcn_sbfe((int)s0, bo, 8);
    sc[1] = __builtin_amdgcn_sbfe((int)s0, bo + 16u, 8);
    sc[2] = __builtin_amdgcn_sbfe((int)s1, bo, 8);
    sc[3] = __builtin_amdgcn_sbfe((int)s1, bo + 16u, 8);
}

// Dot product of one Q6_K part: quant bytes are assembled per dword (4 quants
// of one group s), spread into halves 1024+q with v_perm_b32 and multiplied in
// f32.  sum (q-32) x = acc - 1056 * sum x.
__device__ __forceinline__ float q6k_dot(const Q6KRaw &r, const Q6KX &x, int u)
{
    float acc[4][2];
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[s][0] = acc[s][1] = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t q[4];
        q6k_quants(r, k, q);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            // bytes 0,2 and 1,3 of q[s] under the 0x64 exponent byte -> halves 1024+q
            const h2_t e = as_h2(__builtin_amdgcn_perm(0x64646464u, q[s], 0x04020400u));
            const h2_t o = as_h2(__builtin_amdgcn_perm(0x64646464u, q[s], 0x04030401u));
            acc[s][0] = __builtin_fmaf((float)e.x, x.xs[s][4 * k + 0], acc[s][0]);
            acc[s][1] = __builtin_fmaf((float)o.x, x.xs[s][4 * k + 1], acc[s][1]);
            acc[s][0] = __builtin_fmaf((float)e.y, x.xs[s][4 * k + 2], acc[s][0]);
            acc[s][1] = __builtin_fmaf((float)o.y, x.xs[s][4 * k + 3], acc[s][1]);
        }
    }
    int sc[4];
    q6k_scales(r, u, sc);
    const float d = half_lo(r.dbits);
    const float t0 = (float)sc[0] * ((acc[0][0] + acc[0][1]) - 1056.f * x.sx[0]);
    const float t1 = (float)sc[1] * ((acc[1][0] + acc[1][1]) - 1056.f * x.sx[1]);
    const float t2 = (float)sc[2] * ((acc[2][0] + acc[2][1]) - 1056.f * x.sx[2]);
    const float t3 = (float)sc[3] * ((acc[3][0] + acc[3][1]) - 1056.f * x.sx[3]);
    return d * ((t0 + t1) + (t2 + t3));
}

// Activation slice of a Q6_K part in fixed point (wave-unit kernel).  The
// part's 64 values (groups s = 0..3, x[128n + 32s + l0 + i], i < 16) share
// one scale: X_i = rint(x_i * 2^(22-E)) with E the binary exponent of the
// part's largest |x| (frexp), so |X_i| <= 2^22 and the rounding error,
// 2^(E-23), is at most 2^-22 of that largest value.  Each X_i is split into
// three bytes, X_i = 65536*hi + 256*mid + lo (hi signed, mid and lo unsigned), four
// elements to a dword, so a group's dot product with the 6-bit quants is
// three exact integer dot products.  m[s] = -32 * sum_s * 2^(22-E) takes the
// quants' offset off in the scaled domain, and e = E - 22 undoes the scale
// once per part (a non-finite activation makes m non-finite, and with it
// every row value).
struct Q6KFX {
    uint32_t hi[4][4], mid[4][4], lo[4][4];
    float m[4];
    int e;
};

// Dot product of one Q6_K part against a fixed-point slice: per group, the
// quant bytes (assembled as in q6k_dot) go through one sdot4 with the signed
// high bytes and two udot4 with the unsigned middle and low bytes (all sums
// exact); the three sums are joined in f32, the offset added, the group
// scaled by its int8 scale, and the part's sum scaled back by 2^e and d.
__device__ __forceinline__ float q6k_dot(const Q6KRaw &r, const Q6KFX &x, int u)
{
    int32_t sh[4];
    uint32_t sm[4], sl[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        sh[s] = 0;
        sm[s] = sl[s] = 0u;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t q[4];
        q6k_quants(r, k, q);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            sh[s] = __builtin_amdgcn_sdot4((int)q[s], (int)x.hi[s][k], sh[s], false);
            sm[s] = __builtin_amdgcn_udot4(q[s], x.mid[s][k], sm[s], false);
            sl[s] = __builtin_amdgcn_udot4(q[s], x.lo[s][k], sl[s], false);
        }
    }
    int sc[4];
    q6k_scales(r, u, sc);
    const float d = half_lo(r.dbits);
    float t[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        // |sh| <= 16*63*64 and sm*256 + sl < 2^27: both convert exactly or
        // within one f32 rounding
        const float v = __builtin_fmaf((float)sh[s], 65536.f, (float)((sm[s] << 8) + sl[s]));
        t[s] = (float)sc[s] * (v + x.m[s]);
    }
    return d * __builtin_amdgcn_ldexpf((t[0] + t[1]) + (t[2] + t[3]), x.e);
}

// ------------------------------------------------------------ Q6_K x Q8

// Q8 activation slice of a Q6_K part u: group s holds the 16 int8 values
// x[128n + 32s + l0 + i] in four dwords; the fp16 scales of the 32-element Q8
// blocks the groups lie in (block 4n + s of the super-block) and the groups'
// integer sums (|sum| <= 16 * 127) are kept two to a dword, so a slice takes
// 20 registers (the batched kernel holds up to eight).
struct Q6Q8X {
    uint32_t q[4][4];
    uint32_t d2[2];    // fp16 scale of group s in half s & 1 of d2[s >> 1]
    uint32_t sx2[2];   // int16 sum of group s in half s & 1 of sx2[s >> 1]
};

__device__ __forceinline__ float q6q8_scale(const Q6Q8X &x, int s)
{
    return (s & 1) ? half_hi(x.d2[s >> 1]) : half_lo(x.d2[s >> 1]);
}

__device__ __forceinline__ int32_t q6q8_sum(const Q6Q8X &x, int s)
{
    return __builtin_amdgcn_sbfe((int)x.sx2[s >> 1], (uint32_t)(16 * (s & 1)), 16);
}

// Exact integer sums of one part: is[s] = sum_i (q6 - 32) * q8 over group s.
// The 6-bit quants (0..63) are valid signed bytes, so v_dot4_i32_i8 takes
// them as they are and the -32 offset is removed with the group's q8 sum.
__device__ __forceinline__ void q6k_q8_isums(const Q6KRaw &r, const Q6Q8X &x, int32_t (&is)[4])
{
    int32_t acc[4] = {0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t q[4];
        q6k_quants(r, k, q);
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[s] = __builtin_amdgcn_sdot4((int)q[s], (int)x.q[s][k], acc[s], false);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) is[s] = acc[s] - 32 * q6q8_sum(x, s);
}

// |sc * isum| <= 128 * 16 * 32 * 127 < 2^24, so each group term is exact in
// f32 before its Q8 scale is applied.
__device__ __forceinline__ float q6k_q8_dot(const Q6KRaw &r, const Q6Q8X &x, int u)
{
    int32_t is[4];
    q6k_q8_isums(r, x, is);
    int sc[4];
    q6k_scales(r, u, sc);
    const float d = half_lo(r.dbits);
    const float t0 = (float)(sc[0] * is[0]) * q6q8_scale(x, 0);
    const float t1 = (float)(sc[1] * is[1]) * q6q8_scale(x, 1);
    const float t2 = (float)(sc[2] * is[2]) * q6q8_scale(x, 2);
    const float t3 = (float)(sc[3] * is[3]) * q6q8_scale(x, 3);
    return d * ((t0 + t1) + (t2 + t3));
}

}  // namespace gemvq
