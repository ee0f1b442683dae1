// Internal interface between the C ABI (gemvq_abi.cpp) and the kernels
// (gemvq_kernels.hip).  Launchers assume validated arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gemvq {

// Largest workgroup of the GEMV kernels (8 waves; lets a lane use up to 256
// VGPRs) and hence the widest row: 512 lanes = 128 super-blocks, K <= 32768.
constexpr int kMaxThreads = 512;
constexpr int64_t kMaxK = 32768;

// lm_head_argmax workspace: a done counter and the running key, each on a
// 128-byte line of its own inside the first kArgmaxZeroBytes (zero between
// calls).  The argmax launches use at most kArgmaxMaxGrid workgroups.
constexpr size_t kArgmaxKeyOff = 128;
constexpr size_t kArgmaxZeroBytes = 4096;
constexpr int kArgmaxMaxGrid = 1024;
constexpr size_t kArgmaxWsBytes = kArgmaxZeroBytes + 8 * (size_t)kArgmaxMaxGrid;

// Matrices one multi-output GEMV launch can take; x (f32) must fit in LDS.
constexpr int kMaxMulti = 4;
constexpr int64_t kMaxMultiK = 14336;   // 4.5 K bytes of LDS (padded x and its sums) <= 64 KiB

// Launch geometry of the GEMV kernel template (pure function of N, K, the
// CU count and the kernel kind).
struct Plan {
    int nb;          // super-blocks per row
    int lanes_row;   // lanes per row (4 per super-block)
    int wave_local;  // rows reduce inside one wave (gemv_wave_kernel)
    int steps;       // 16-super-block steps per row (wave and row-stream kernels)
    int rows_kernel; // 1: gemv_rows_kernel, 0: gemv_wave_kernel (when wave_local)
    int chunk_shift; // wave/row-stream kernels: units dealt in chunks of 1 << chunk_shift
    int waves;       // waves per workgroup
    int threads;     // 64 * waves
    int rows_tile;   // rows per tile
    int64_t tiles;   // ceil(N / rows_tile)
    int x_in_lds;    // activation staged through LDS
    size_t lds_bytes;
    int grid;        // workgroups (one resident wave; set at launch)
    // tile kernel, CU-resident form: one workgroup per CU (at most), each
    // with all `phase` tiles of its row range in flight from the start; the
    // row-reduction buffer then sits at red_off, past the staged activation
    int resident;
    int phase;
    size_t red_off;
};

// Threads of a CU-resident tile workgroup (12 waves, three per SIMD) and the
// most tiles one holds in flight.
constexpr int kResThreads = 768;
constexpr int kResMaxPhase = 4;

// `cus`: compute units of the device the launch runs on (the tile kernel's
// CU-resident form splits the rows over them)
Plan make_plan(int64_t N, int64_t K, int kind, int cus);
Plan make_swiglu_q8_plan(int64_t N, int64_t K, int cus);   // always the tile kernel
// batched int8 GEMV: vectors per call, LDS bytes a round of staged vectors
// may take, the kernel's vector slots for m vectors (1, 2, 4 or 8; Q6_K at
// most 4, larger batches in launches of 4), and its plan (round = vectors
// staged per round)
constexpr int kMaxBatch = 8;
constexpr size_t kBatchStageBytes = 61440;
constexpr int64_t kBatchSplitBytesPerCu = 200 * 1024;   // weight bytes per CU above which 8 slots run as 2 x 4
int batch_slots(int m, bool q6k);
Plan make_batch_plan(int64_t N, int64_t K, int kind, int M, int *round);

// Optional device timestamps of one launch: the kernel's own start and end
// are recorded into these caller-created events when they are not null.
struct Timing {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

hipError_t launch_q4k_gemv(const void *W, const float *x, float *y, int64_t N, int64_t K, int cus, hipStream_t s);
hipError_t launch_q6k_gemv(const void *W, const float *x, float *y, int64_t N, int64_t K, int cus, hipStream_t s);
hipError_t launch_swiglu_gemv(const void *Wg, const void *Wu, const float *x, float *h, int64_t N, int64_t K, int cus,
                              hipStream_t s);
hipError_t launch_q4k_q8_gemv(const void *W, const int8_t *xq, const uint16_t *xd, float *y, int64_t N, int64_t K,
                              int cus, hipStream_t s);
hipError_t launch_q6k_q8_gemv(const void *W, const int8_t *xq, const uint16_t *xd, float *y, int64_t N, int64_t K,
                              int cus, hipStream_t s);
// q4k_q8_gemv_from_f32: quantize x (writing xq, xd) and run the Q4_K x Q8 GEMV
hipError_t launch_q4k_q8_gemv_from_f32(const void *W, const float *x, int8_t *xq, uint16_t *xd, float *y, int64_t N,
                                       int64_t K, int cus, hipStream_t s);
// mask: nullptr, or the banned-row bitmask of lm_head_argmax_masked
hipError_t launch_lm_head_argmax(const void *W, const float *x, const uint32_t *mask, uint32_t *out_idx,
                                 float *out_max, void *ws, int64_t N, int64_t K, int cus, hipStream_t s,
                                 const Timing &tm = Timing{});
hipError_t launch_q4k_gemv_multi(const void *const *W, const int64_t *N, float *const *y, const float *const *r,
                                 int count, const float *x, int64_t K, int cus, hipStream_t s);
hipError_t launch_q8_quantize(const float *x, int8_t *xq, uint16_t *xd, int64_t K, hipStream_t s);
// measurement hook: read bytes (a multiple of 16) at p once with `grid`
// workgroups of 256 threads; sink: uint32[256], written only on an
// impossible fold value
hipError_t launch_stream_read(const void *p, int64_t bytes, int grid, int threads, uint32_t *sink, hipStream_t s);
// zero `bytes` (a multiple of 16, at most 65536) at a 16-byte aligned device address with a fill kernel
hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s);
hipError_t launch_q6k_q8_isums(const void *W, const int8_t *xq, int32_t *isums, int64_t N, int64_t K, hipStream_t s);
// swiglu_q8_gemv: rows a tile-kernel workgroup keeps in LDS for the Q8
// emission; workspace = one u32 counter per 32-row block, then the N row
// values from offset swiglu_q8_vals_offset(N).
constexpr int kEmitRows = 2048;
constexpr size_t swiglu_q8_vals_offset(int64_t N) { return (((size_t)(N / 32) * 4) + 255) & ~(size_t)255; }
constexpr size_t swiglu_q8_ws_bytes(int64_t N) { return swiglu_q8_vals_offset(N) + (size_t)N * 4; }
hipError_t launch_swiglu_q8_gemv(const void *Wg, const void *Wu, const float *x, float *h, int8_t *hq, uint16_t *hd,
                                 void *ws, int64_t N, int64_t K, int cus, hipStream_t s);
// r == nullptr: rms_norm_q8; otherwise add_rms_norm_q8 (res receives x + r).  K % 32 == 0, K <= kMaxNormK.
constexpr int64_t kMaxNormK = 32768;
hipError_t launch_rms_norm_q8(const float *x, const float *r, const float *w, float eps, float *res, float *y,
                              int8_t *xq, uint16_t *xd, int64_t K, hipStream_t s);
hipError_t launch_q8_gemv_batch(bool q6k, const void *W, const int8_t *xq, const uint16_t *xd, float *y, int64_t N,
                                int64_t K, int m, int cus, hipStream_t s);
hipError_t launch_q4k_q8_isums(const void *W, const int8_t *xq, int32_t *isums, int64_t N, int64_t K, hipStream_t s);

}  // namespace gemvq
