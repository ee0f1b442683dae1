#!/usr/bin/env python3
"""Benchmark of the batch-1 quantized GEMV path on one MI355X.

One step = one pass of the whole hot path over the five workloads' shapes, all
enqueued on one stream in decode order (the layers' GEMVs, then the lm_head
with its argmax, last as in a decoder):
  1. Q4_K GEMV 1024x1024 (config 1)
  2. Q4_K GEMV  4096x2560, 2560x9728, 9728x2560 (4B-class decode shapes)
  3. fused gate/up SwiGLU GEMV (2 x Q4_K 9728x2560) + ffn_down Q6_K 2560x9728
  4. Q8 quantize of an f32[8192] activation + Q4_K x Q8 GEMV 28672x8192 (one
     launch: q4k_q8_gemv_from_f32 quantizes in the GEMV's prologue)
  5. lm_head Q6_K 248,320 x 1024 GEMV + fused first-index argmax (4-byte result)
Weights are seeded synthetic data with the workloads' distributions.  Two
copies of every weight buffer alternate between steps, so each buffer is
re-read only after ~0.85 GB of other traffic and the 256 MB Infinity Cache
cannot serve it.

Prints ONE JSON line: value = effective weight GB/s of the whole step (weight
bytes streamed per step / time per step), plus the lm_head-argmax calls/s,
a roofline entry for the dominant kernel (its algorithmic bytes / its average
kernel duration: the lm_head launch itself records its start and end into HIP
events on the launch stream, inside the timed region) and the CPU oracle timed
on the host on a bounded sample.  `configs` reports each workload on its own
(us per call, GEMV/s, weight GB/s, fraction of 8 TB/s and of a plain
streaming read of the same byte count, the oracle's time on one host thread
and on all of them); `kernels` is the per-kernel breakdown.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Q4_K GEMV effective HBM GB/s (% of peak) + lm_head-argmax calls/sec"
HBM_PEAK_GBS = 8000.0
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic_lm_head_argmax_q6k_248320x1024.json")
KERNEL_SOURCES = [os.path.join(ROOT, "gemv_q4k_q6k_amd", "csrc", f) for f in
                  ("gemvq_kernels.hip", "gemvq_device.h", "gemvq_launch.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def build_workload(dev):
    """Seeded inputs (CPU numpy) and their device copies (two weight sets)."""
    import torch
    import synth

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    t0 = time.time()
    c1 = synth.c1_inputs(0)
    c2 = [synth.c2_inputs(i) for i in range(3)]
    c3 = synth.c3_inputs(0)
    c4 = synth.c4_inputs(0)
    c5 = synth.c5_inputs(0)
    host = {"c1": c1, "c2": c2, "c3": c3, "c4": c4, "c5": c5}
    sets = []
    for copy in range(2):
        s = {
            "c1W": up(c1[0]),
            "c2W": [up(W) for W, _ in c2],
            "c3W": up(c3[0]),
            "c4Wg": up(c4[0]), "c4Wu": up(c4[1]), "c4Wd": up(c4[2]),
            "c5W": up(c5[0]),
        }
        sets.append(s)
    vec = {
        "c1x": up(c1[1]),
        "c1y": torch.empty(synth.C1_Q4K[0], dtype=torch.float32, device=dev),
        "c2x": [up(x) for _, x in c2],
        "c3x": up(c3[1]),
        "c4x": up(c4[3]),
        "c5x": up(c5[1]),
        "h": torch.empty(synth.C4_SWIGLU[0], dtype=torch.float32, device=dev),
        "yd": torch.empty(synth.C4_SWIGLU[1], dtype=torch.float32, device=dev),
        "c2y": [torch.empty(N, dtype=torch.float32, device=dev) for N, _ in synth.C2_Q4K],
        "c5y": torch.empty(synth.C5_Q8[0], dtype=torch.float32, device=dev),
        "xq": torch.empty(synth.C5_Q8[1], dtype=torch.int8, device=dev),
        "xd": torch.empty(synth.C5_Q8[1] // 32, dtype=torch.int16, device=dev),
        "idx": torch.empty(1, dtype=torch.int32, device=dev),
        "ws": torch.zeros(0, dtype=torch.uint8, device=dev),
    }
    torch.cuda.synchronize()
    log(f"workload built in {time.time() - t0:.1f}s")
    return host, sets, vec


def weight_bytes():
    import synth
    b = {}
    N, K = synth.C1_Q4K
    b["c1"] = N * K // 256 * 144
    b["c2"] = sum(N * K // 256 * 144 for N, K in synth.C2_Q4K)
    N, K = synth.C3_LM_HEAD
    b["c3"] = N * K // 256 * 210
    N, K = synth.C4_SWIGLU
    b["c4"] = 2 * N * K // 256 * 144 + K * N // 256 * 210
    N, K = synth.C5_Q8
    b["c5"] = N * K // 256 * 144
    return b


def lm_head_algorithmic_bytes():
    import synth
    N, K = synth.C3_LM_HEAD
    return N * K // 256 * 210 + 4 * K + 4


def step_calls(gq, s, v):
    """The hot path of one step as pre-bound C-ABI calls (raw pointers and
    the current stream), so the timed loop spends ~1 us of host time per
    launch.  Every argument was validated once by the binding (self_check
    runs the same buffers through it).  Returns (calls, index of the lm_head
    call)."""
    import torch
    import synth
    L = gq.lib()
    st = torch.cuda.current_stream().cuda_stream
    calls = []
    N, K = synth.C1_Q4K
    calls.append((L.q4k_gemv, (s["c1W"].data_ptr(), v["c1x"].data_ptr(), v["c1y"].data_ptr(), N, K, st)))
    for i, (N, K) in enumerate(synth.C2_Q4K):
        calls.append((L.q4k_gemv, (s["c2W"][i].data_ptr(), v["c2x"][i].data_ptr(), v["c2y"][i].data_ptr(), N, K, st)))
    N, K = synth.C4_SWIGLU
    calls.append((L.swiglu_gemv, (s["c4Wg"].data_ptr(), s["c4Wu"].data_ptr(), v["c4x"].data_ptr(),
                                  v["h"].data_ptr(), N, K, st)))
    calls.append((L.q6k_gemv, (s["c4Wd"].data_ptr(), v["h"].data_ptr(), v["yd"].data_ptr(), K, N, st)))
    N, K = synth.C5_Q8
    calls.append((L.q4k_q8_gemv_from_f32, (s["c5W"].data_ptr(), v["c5x"].data_ptr(), v["xq"].data_ptr(),
                                           v["xd"].data_ptr(), v["c5y"].data_ptr(), N, K, st)))
    N, K = synth.C3_LM_HEAD
    lm = len(calls)
    # the timed variant: identical work, and the kernel's own start/end go
    # into the events run_calls passes (None, None outside the timed region)
    calls.append((L.lm_head_argmax_timed, (s["c3W"].data_ptr(), v["c3x"].data_ptr(), v["idx"].data_ptr(), None,
                                           v["ws"].data_ptr(), v["ws"].numel(), N, K, st)))
    return calls, lm


def run_calls(calls, lm, events=None):
    """One step.  events = (start, stop) raw hipEvent_t handles that receive
    the lm_head kernel's own start and end, or None."""
    for j, (fn, args) in enumerate(calls):
        rc = fn(*args, *(events if events is not None else (None, None))) if j == lm else fn(*args)
        if rc != 0:
            raise RuntimeError(f"{fn.__name__} returned {rc}")


def run_step(gq, s, v):
    """One pass of the hot path through the checked binding."""
    import synth
    N, K = synth.C1_Q4K
    gq.q4k_gemv(s["c1W"], v["c1x"], N, K, y=v["c1y"])
    for i, (N, K) in enumerate(synth.C2_Q4K):
        gq.q4k_gemv(s["c2W"][i], v["c2x"][i], N, K, y=v["c2y"][i])
    N, K = synth.C4_SWIGLU
    gq.swiglu_gemv(s["c4Wg"], s["c4Wu"], v["c4x"], N, K, h=v["h"])
    gq.q6k_gemv(s["c4Wd"], v["h"], K, N, y=v["yd"])
    N, K = synth.C5_Q8
    gq.q4k_q8_gemv_from_f32(s["c5W"], v["c5x"], N, K, xq=v["xq"], xd=v["xd"], y=v["c5y"])
    N, K = synth.C3_LM_HEAD
    gq.lm_head_argmax(s["c3W"], v["c3x"], N, K, v["ws"], out_idx=v["idx"])


def graph_step_ms(gq, sets, v, steps):
    """ms per step when each step is one replay of a HIP graph holding the
    whole step (one graph per weight copy, replayed alternately): the same
    kernels without per-launch host work."""
    import torch
    graphs = []
    for s in sets:
        run_step(gq, s, v)   # warm-up outside capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run_step(gq, s, v)
        graphs.append(g)
    for k in range(4):
        graphs[k % 2].replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for k in range(steps):
        graphs[k % 2].replay()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    del graphs
    return ms


def sync_rate(prepared, v, n=400):
    """lm_head calls per second when every call is followed by the 4-byte
    download of the token id and a host sync (a greedy decode loop's
    per-token pattern), alternating the two weight copies."""
    import torch
    for k in range(10):
        calls, lm = prepared[k % 2]
        fn, a = calls[lm]
        fn(*a, None, None)
        int(v["idx"].item())
    t0 = time.perf_counter()
    for k in range(n):
        calls, lm = prepared[k % 2]
        fn, a = calls[lm]
        rc = fn(*a, None, None)
        if rc != 0:
            raise RuntimeError(f"lm_head_argmax_timed returned {rc}")
        int(v["idx"].item())
    torch.cuda.synchronize()
    return n / (time.perf_counter() - t0)


def self_check(gq, sets, v):
    """Sanity of the benchmarked buffers without the oracle (the parity suite
    against the oracle lives in tests/): the fused argmax must equal the
    first-index argmax of q6k_gemv's own logits on both weight copies."""
    import torch
    import synth
    N, K = synth.C3_LM_HEAD
    ok = True
    for s in sets:
        run_step(gq, s, v)
        logits = gq.q6k_gemv(s["c3W"], v["c3x"], N, K)
        m = logits.max()
        first = int(torch.nonzero(logits == m)[0].item())
        ok = ok and int(v["idx"].item()) == first
    torch.cuda.synchronize()
    return bool(ok)


MIN_ROTATE_BYTES = 640 << 20     # weight copies per timed kernel: beyond the 256 MB Infinity Cache


def graph_us(fn, ws, reps=24):
    """Per-call device time of fn: `reps` calls (rotating through the
    per-copy argument tuples ws) captured in one HIP graph, four warm
    replays, then the median of 7 trials of 3 replays between two HIP events
    (no host launch overhead).  Every copy is touched twice before the
    capture (first touches of fresh copies run slower)."""
    import torch
    for r in range(2 * len(ws)):
        fn(ws[r % len(ws)])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for r in range(reps):
            fn(ws[r % len(ws)])
    for _ in range(4):
        g.replay()
    torch.cuda.synchronize()
    trials = []
    for _ in range(7):
        st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st.record()
        for _ in range(3):
            g.replay()
        en.record()
        torch.cuda.synchronize()
        trials.append(st.elapsed_time(en) * 1000.0 / (reps * 3))
    del g
    return float(np.median(trials))


READ_SHAPES = tuple((1024, g) for g in (128, 256, 512, 1024, 2048, 4096)) + \
              tuple((256, g) for g in (1024, 2048, 4096, 8192, 16384))   # (threads, grid)


def read_ceiling(gq, dev, sizes, in_cache=()):
    """Streaming-read time of each byte count: the library's plain read
    kernel (16-byte loads, grid-stride) over slices of one pool, rotating
    through >= 640 MB of slices (sizes listed in in_cache: one slice, read
    again and again, as the in-cache config it matches), best over workgroup
    sizes and grids.  {bytes: {"us", "GBps", "grid", "threads", "in_cache"}}."""
    import torch
    pool = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    out = {}
    for S in sizes:
        S16 = S - S % 16
        stride = -(-S16 // 256) * 256
        n = 1 if S in in_cache else max(2, min(pool.numel() // stride, -(-MIN_ROTATE_BYTES // S16)))
        bufs = [(pool[i * stride:i * stride + S16],) for i in range(n)]
        best = None
        for thr, grid in READ_SHAPES:
            us = graph_us(lambda w, grid=grid, thr=thr: gq.stream_read(w[0], grid, sink, threads=thr), bufs)
            if best is None or us < best[0]:
                best = (us, grid, thr)
        out[S] = {"us": round(best[0], 2), "GBps": round(S16 / best[0] / 1e3, 1), "grid": best[1],
                  "threads": best[2], "in_cache": S in in_cache}
    del pool
    torch.cuda.empty_cache()
    return out


def breakdown(gq, sets, v, reps=24):
    """Per-call device time of each kernel, not part of `value`: `reps`
    launches are captured in a HIP graph and replayed between two HIP events
    (no host launch overhead in the measurement; median of 7 trials).  Each kernel rotates through
    enough device-side copies of its weights (>= 640 MB in total) that the
    256 MB Infinity Cache cannot serve a repeat.  rocprofv3 kernel traces are
    the cross-check."""
    import torch
    import synth
    out = {}
    dev = v["h"].device
    yl = torch.empty(synth.C3_LM_HEAD[0], dtype=torch.float32, device=dev)
    min_bytes = 640 << 20

    def copies(t):
        n = max(2, -(-min_bytes // t.numel()))
        return [t] + [t.clone() for _ in range(n - 1)]

    def timeit(name, fn, ws, nbytes, weight_bytes=None, in_cache=False):
        """ws: list of per-copy weight tuples; nbytes: algorithmic bytes per
        call; weight_bytes: the matrix bytes it streams (the read ceiling is
        matched to them)."""
        us = graph_us(fn, ws, reps)
        out[name] = {"us": round(us, 2), "GBps": round(nbytes / us / 1e3, 1),
                     "frac_hbm_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4), "weight_copies": len(ws),
                     "weight_bytes": weight_bytes}
        if in_cache:
            out[name]["in_cache"] = True

    s0 = sets[0]
    # config 1: 1024 x 1024 (590 KB) is read from the Infinity Cache after the
    # first call; reported as such, not against the HBM roofline
    N, K = synth.C1_Q4K
    timeit("c1_q4k_gemv_1024x1024_in_cache", lambda w: gq.q4k_gemv(w[0], v["c1x"], N, K, y=v["c1y"]),
           [(s0["c1W"],)], N * K // 256 * 144 + 4 * (N + K), N * K // 256 * 144, in_cache=True)
    # config 2: the three decode shapes back to back, each rotating its copies
    trip = list(zip(*[copies(s0["c2W"][i]) for i in range(3)]))

    def c2_triple(w):
        for i, (N, K) in enumerate(synth.C2_Q4K):
            gq.q4k_gemv(w[i], v["c2x"][i], N, K, y=v["c2y"][i])
    c2_bytes = sum(N * K // 256 * 144 for N, K in synth.C2_Q4K)
    timeit("c2_q4k_gemv_triple", c2_triple, trip, c2_bytes + sum(4 * (N + K) for N, K in synth.C2_Q4K), c2_bytes)
    del trip
    for i, (N, K) in enumerate(synth.C2_Q4K):
        ws = [(w,) for w in copies(s0["c2W"][i])]
        timeit(f"q4k_gemv_{N}x{K}", lambda w, i=i, N=N, K=K: gq.q4k_gemv(w[0], v["c2x"][i], N, K, y=v["c2y"][i]),
               ws, N * K // 256 * 144 + 4 * (N + K), N * K // 256 * 144)
        del ws
    N, K = synth.C3_LM_HEAD
    ws = [(w,) for w in copies(s0["c3W"])]
    timeit("q6k_gemv_248320x1024", lambda w: gq.q6k_gemv(w[0], v["c3x"], N, K, y=yl), ws,
           N * K // 256 * 210 + 4 * (N + K), N * K // 256 * 210)
    timeit("lm_head_argmax_248320x1024", lambda w: gq.lm_head_argmax(w[0], v["c3x"], N, K, v["ws"], out_idx=v["idx"]),
           ws, lm_head_algorithmic_bytes(), N * K // 256 * 210)
    # the masked variant: a seeded ban mask over ~1% of the vocabulary, one
    # 4-byte mask word per 32 rows read with the weights
    banned = np.random.default_rng(11).random(N) < 0.01
    mask = torch.from_numpy(np.packbits(np.concatenate([banned, np.zeros((-N) % 32, bool)]),
                                        bitorder="little").view(np.int32)).to(v["c3x"].device)
    ws_m = torch.zeros_like(v["ws"])
    timeit("lm_head_argmax_masked_248320x1024",
           lambda w: gq.lm_head_argmax_masked(w[0], v["c3x"], mask, N, K, ws_m, out_idx=v["idx"]),
           ws, lm_head_algorithmic_bytes() + 4 * ((N + 31) // 32), N * K // 256 * 210)
    del ws
    N, K = synth.C4_SWIGLU
    ws = list(zip(copies(s0["c4Wg"]), copies(s0["c4Wu"])))
    timeit("swiglu_gemv_9728x2560", lambda w: gq.swiglu_gemv(w[0], w[1], v["c4x"], N, K, h=v["h"]), ws,
           2 * N * K // 256 * 144 + 4 * (N + K), 2 * N * K // 256 * 144)
    del ws
    ws = [(w,) for w in copies(s0["c4Wd"])]
    timeit("q6k_gemv_2560x9728", lambda w: gq.q6k_gemv(w[0], v["h"], K, N, y=v["yd"]), ws,
           K * N // 256 * 210 + 4 * (N + K), K * N // 256 * 210)
    del ws
    N, K = synth.C5_Q8
    timeit("q8_quantize_8192", lambda w: gq.q8_quantize(v["c5x"], xq=v["xq"], xd=v["xd"]), [()],
           K * 4 + K + K // 16)
    ws = [(w,) for w in copies(s0["c5W"])]
    timeit("q4k_q8_gemv_28672x8192", lambda w: gq.q4k_q8_gemv(w[0], v["xq"], v["xd"], N, K, y=v["c5y"]), ws,
           N * K // 256 * 144 + K + K // 16 + 4 * N, N * K // 256 * 144)

    def c5(w):
        gq.q8_quantize(v["c5x"], xq=v["xq"], xd=v["xd"])
        gq.q4k_q8_gemv(w[0], v["xq"], v["xd"], N, K, y=v["c5y"])
    timeit("c5_q8_quantize+q4k_q8_gemv_28672x8192", c5, ws,
           N * K // 256 * 144 + 4 * K + 2 * (K + K // 16) + 4 * N, N * K // 256 * 144)
    timeit("c5_q4k_q8_gemv_from_f32_28672x8192",
           lambda w: gq.q4k_q8_gemv_from_f32(w[0], v["c5x"], N, K, xq=v["xq"], xd=v["xd"], y=v["c5y"]), ws,
           N * K // 256 * 144 + 4 * K + K + K // 16 + 4 * N, N * K // 256 * 144)
    timeit("q4k_gemv_28672x8192", lambda w: gq.q4k_gemv(w[0], v["c5x"], N, K, y=v["c5y"]), ws,
           N * K // 256 * 144 + 4 * (N + K), N * K // 256 * 144)
    del ws
    # the fused q/k/v projection of a 4B-class attention block (one launch for
    # three Q4_K matrices sharing x) against three separate launches
    K = 2560
    qkv = (4096, 1024, 1024)
    r = synth.rng_for(77)
    mats = [torch.from_numpy(synth.q4k_weights(r, n, K)).to(dev) for n in qkv]
    xq = torch.from_numpy(synth.activation(r, K)).to(dev)
    ys = [torch.empty(n, dtype=torch.float32, device=dev) for n in qkv]
    nbytes = sum(n * K // 256 * 144 for n in qkv) + 4 * (K + sum(qkv))
    sets_ = list(zip(*[copies(m) for m in mats]))
    timeit("q4k_gemv_multi_qkv_4096+1024+1024x2560",
           lambda w: gq.q4k_gemv_multi(list(w), list(qkv), xq, K, ys=ys), sets_, nbytes)

    def three(w):
        for m, n, y in zip(w, qkv, ys):
            gq.q4k_gemv(m, xq, n, K, y=y)
    timeit("q4k_gemv_x3_separate_4096+1024+1024x2560", three, sets_, nbytes)
    del sets_, mats
    # producer-side Q8 emission on the SwiGLU FFN of the 4B-class layer: the
    # int8 down projection, the SwiGLU that emits Q8 itself, and the whole FFN
    # (gate/up + down) on the f32 path, the unfused int8 path and the fused one
    N, K = synth.C4_SWIGLU
    hq = torch.empty(N, dtype=torch.int8, device=dev)
    hd = torch.empty(N // 32, dtype=torch.int16, device=dev)
    wsq = torch.zeros(gq.swiglu_q8_ws_bytes(N), dtype=torch.uint8, device=dev)
    gq.swiglu_gemv(s0["c4Wg"], s0["c4Wu"], v["c4x"], N, K, h=v["h"])
    gq.q8_quantize(v["h"], xq=hq, xd=hd)
    ffn = list(zip(copies(s0["c4Wg"]), copies(s0["c4Wu"]), copies(s0["c4Wd"])))
    gu_bytes = 2 * N * K // 256 * 144
    d_bytes = K * N // 256 * 210
    timeit("q6k_q8_gemv_2560x9728", lambda w: gq.q6k_q8_gemv(w[2], hq, hd, K, N, y=v["yd"]), ffn,
           d_bytes + N + N // 16 + 4 * K)
    timeit("swiglu_q8_gemv_9728x2560", lambda w: gq.swiglu_q8_gemv(w[0], w[1], v["c4x"], N, K, wsq, hq=hq, hd=hd),
           ffn, gu_bytes + 4 * K + N + N // 16)

    def ffn_f32(w):
        gq.swiglu_gemv(w[0], w[1], v["c4x"], N, K, h=v["h"])
        gq.q6k_gemv(w[2], v["h"], K, N, y=v["yd"])

    def ffn_q8_unfused(w):
        gq.swiglu_gemv(w[0], w[1], v["c4x"], N, K, h=v["h"])
        gq.q8_quantize(v["h"], xq=hq, xd=hd)
        gq.q6k_q8_gemv(w[2], hq, hd, K, N, y=v["yd"])

    def ffn_q8_fused(w):
        gq.swiglu_q8_gemv(w[0], w[1], v["c4x"], N, K, wsq, hq=hq, hd=hd)
        gq.q6k_q8_gemv(w[2], hq, hd, K, N, y=v["yd"])
    for name, fn in (("ffn_f32_swiglu+q6k", ffn_f32), ("ffn_q8_swiglu+quantize+q6k_q8", ffn_q8_unfused),
                     ("ffn_q8_swiglu_q8+q6k_q8", ffn_q8_fused)):
        timeit(name, fn, ffn, gu_bytes + d_bytes, gu_bytes + d_bytes)
    del ffn
    # batched int8 GEMV: m Q8 activation vectors through one weight read, on
    # the 70B-class FFN matrix and on the Q6_K lm_head
    for name, fn, W_, (N, K), bpr in (
            ("q4k_q8_gemv_batch_28672x8192", gq.q4k_q8_gemv_batch, s0["c5W"], synth.C5_Q8, 144),
            ("q6k_q8_gemv_batch_248320x1024", gq.q6k_q8_gemv_batch, s0["c3W"], synth.C3_LM_HEAD, 210)):
        xqb, xdb = synth.q8_activations(synth.rng_for(79), 8, K)
        dq = torch.from_numpy(xqb.reshape(-1)).to(dev)
        dd = torch.from_numpy(xdb.reshape(-1).view(np.int16)).to(dev)
        yb = torch.empty(8 * N, dtype=torch.float32, device=dev)
        wsb = [(w,) for w in copies(W_)]
        for m in (1, 2, 4, 8):
            timeit(f"{name}_m{m}",
                   lambda w, m=m: fn(w[0], dq[:m * K], dd[:m * K // 32], N, K, m, y=yb[:m * N]), wsb,
                   N * K // 256 * bpr + m * (K + K // 16 + 4 * N))
        del wsb
    # norm producers at the 70B-class hidden size (K = 8192)
    K = synth.C5_Q8[1]
    r = synth.rng_for(78)
    z = torch.from_numpy(synth.activation(r, K)).to(dev)
    z2 = torch.from_numpy(synth.activation(r, K)).to(dev)
    wn = torch.from_numpy(r.uniform(0.5, 1.5, K).astype(np.float32)).to(dev)
    res = torch.empty(K, dtype=torch.float32, device=dev)
    timeit("rms_norm_q8_8192", lambda w: gq.rms_norm_q8(z, wn, 1e-5, xq=v["xq"], xd=v["xd"]), [()],
           2 * 4 * K + K + K // 16)
    timeit("add_rms_norm_q8_8192",
           lambda w: gq.add_rms_norm_q8(z, z2, wn, 1e-5, res=res, xq=v["xq"], xd=v["xd"]), [()],
           4 * 4 * K + K + K // 16)
    torch.cuda.empty_cache()
    return out


CALIB_MIB = 256
CALIB_TAG = "neg_kernel"        # the calibration copy is torch's elementwise negation


def calibration_copy(dev, mib=CALIB_MIB, reps=6):
    """A plain streaming copy of known size: `reps` launches of torch's
    elementwise negation over mib MiB of f32 (mib MiB read, mib MiB written
    per launch).  Run under rocprofv3 --pmc, its FETCH_SIZE/WRITE_SIZE give the
    factors that turn those counters into bytes."""
    import torch
    a = torch.ones((mib << 20) // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(reps):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    del a, b


def _counter_means(db, counter):
    """{kernel name: mean over dispatches of the counter's per-dispatch total}
    from a rocprofv3 (rocpd SQLite) database."""
    import sqlite3
    import collections
    c = sqlite3.connect(db)
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for name, disp, val in c.execute(
            "select kernel_name, dispatch_id, value from counters_collection where counter_name = ?", (counter,)):
        per[name][disp] += val
    c.close()
    return {k: (sum(v.values()) / len(v), len(v)) for k, v in per.items()}


def _pick(means, pred, what):
    hits = [(k, v) for k, v in means.items() if pred(k)]
    if len(hits) != 1:
        raise SystemExit(f"expected one {what} kernel in the counter database, found {[k for k, _ in hits]}")
    return hits[0]


def traffic_kernels():
    """(tag, demangled-name pattern of the kernel's one instantiation in the
    step, algorithmic bytes per launch, record path) of the kernels whose
    HBM traffic is recorded."""
    import synth
    out = [("lm_head_argmax", r"gemv_(wave_)?kernel<1, 1,", lm_head_algorithmic_bytes(), PROFILE_TRAFFIC)]
    N, K = synth.C4_SWIGLU
    out.append(("swiglu_gemv_9728x2560", r"gemv_kernel<3, 0, \d, true, true>", 2 * N * K // 256 * 144 + 4 * (N + K),
                os.path.join(ROOT, "profiles", "traffic_swiglu_gemv_9728x2560.json")))
    out.append(("q6k_gemv_2560x9728", r"gemv_kernel<1, 0, \d, true, true>", K * N // 256 * 210 + 4 * (N + K),
                os.path.join(ROOT, "profiles", "traffic_q6k_gemv_2560x9728.json")))
    # config 2: 4096x2560 is the step's only three-tile resident instantiation;
    # 2560x9728 and 9728x2560 share one (two tiles) and equal byte counts, so
    # one record, under both breakdown entries ('+'-joined tag), covers both
    N, K = synth.C2_Q4K[0]
    out.append(("q4k_gemv_4096x2560", r"gemv_kernel<0, 0, 3, true, true>", N * K // 256 * 144 + 4 * (N + K),
                os.path.join(ROOT, "profiles", "traffic_q4k_gemv_4096x2560.json")))
    N, K = synth.C2_Q4K[1]
    assert tuple(synth.C2_Q4K[2]) == (K, N)
    out.append(("q4k_gemv_2560x9728+q4k_gemv_9728x2560", r"gemv_kernel<0, 0, 2, true, true>",
                N * K // 256 * 144 + 4 * (N + K),
                os.path.join(ROOT, "profiles", "traffic_q4k_gemv_2560x9728_and_9728x2560.json")))
    N, K = synth.C5_Q8
    # f32 x in, its Q8 codes and scales out (one workgroup writes them), y out
    out.append(("c5_q4k_q8_gemv_from_f32_28672x8192", r"gemv_wave_kernel<2, 0, 2, true>",
                N * K // 256 * 144 + 4 * K + K + K // 16 + 4 * N,
                os.path.join(ROOT, "profiles", "traffic_q4k_q8_gemv_from_f32_28672x8192.json")))
    return out


def write_traffic(fetch_db, write_db, command):
    """Turn two rocprofv3 --pmc runs of `bench.py --calibration-copy` (one
    with FETCH_SIZE, one with WRITE_SIZE) into HBM bytes per launch of each
    recorded kernel, scaled by what the same counters read for the
    calibration copy, and store each next to the kernel-source hash it was
    taken on."""
    known = CALIB_MIB << 20
    is_cal = lambda k: CALIB_TAG in k
    fm, wm = _counter_means(fetch_db, "FETCH_SIZE"), _counter_means(write_db, "WRITE_SIZE")
    cal_name, (cal_f, _) = _pick(fm, is_cal, "calibration")
    _, (cal_w, _) = _pick(wm, is_cal, "calibration")
    f_fac = known / (cal_f * 1024.0)
    w_fac = known / (cal_w * 1024.0)
    for tag, pat, alg, path in traffic_kernels():
        is_k = lambda k, pat=pat: re.search(pat, k) is not None
        if tag != "lm_head_argmax" and not any(is_k(k) for k in fm):
            continue     # counters taken on a step without this kernel
        k_name, (k_f, n_f) = _pick(fm, is_k, tag)
        _, (k_w, n_w) = _pick(wm, is_k, tag)
        fetch_b = k_f * 1024.0 * f_fac
        write_b = k_w * 1024.0 * w_fac
        out = {
            "kernel": k_name, "workload": tag, "dispatches": {"fetch": n_f, "write": n_w},
            "fetch_size_kib_per_dispatch": round(k_f, 1), "write_size_kib_per_dispatch": round(k_w, 1),
            "calibration": {"kernel": cal_name, "bytes_read": known, "bytes_written": known,
                            "fetch_size_kib": round(cal_f, 1), "write_size_kib": round(cal_w, 1),
                            "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4)},
            "hbm_fetch_bytes_per_launch": int(round(fetch_b)), "hbm_write_bytes_per_launch": int(round(write_b)),
            "bytes_per_launch": int(round(fetch_b + write_b)),
            "algorithmic_bytes_per_launch": alg,
            "traffic_over_algorithmic": round((fetch_b + write_b) / alg, 4),
            "kernel_source_hash": kernel_source_hash(),
            "command": command,
        }
        os.makedirs(os.path.dirname(path), exist_ok=True)
        with open(path, "w") as f:
            json.dump(out, f, indent=1)
            f.write("\n")
        print(json.dumps(out))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_config_calls(host):
    """{config: (one call of the oracle on that workload, weight bytes)}: the
    f64 oracle's own functions on the seeded inputs the GPU runs."""
    import oracle
    import synth
    wb = weight_bytes()

    def c1():
        N, K = synth.C1_Q4K
        oracle.q4k_gemv(host["c1"][0], host["c1"][1], N, K)

    def c2():
        for i, (N, K) in enumerate(synth.C2_Q4K):
            oracle.q4k_gemv(host["c2"][i][0], host["c2"][i][1], N, K)

    def c3():
        N, K = synth.C3_LM_HEAD
        oracle.argmax_first(oracle.q6k_gemv(host["c3"][0], host["c3"][1], N, K))

    def c4():
        Wg, Wu, Wd, x = host["c4"]
        N, K = synth.C4_SWIGLU
        h, _, _ = oracle.swiglu(Wg, Wu, x, N, K)
        oracle.q6k_gemv_f64x(Wd, h, K, N)

    def c5():
        W, x = host["c5"]
        N, K = synth.C5_Q8
        q, d = oracle.q8_quantize(x)
        oracle.q4k_q8_gemv(W, q, d, N, K)
    return {"c1": (c1, wb["c1"]), "c2": (c2, wb["c2"]), "c3": (c3, wb["c3"]), "c4": (c4, wb["c4"]),
            "c5": (c5, wb["c5"])}


def cpu_baseline(host, budget_s=(1.0, 0.6)):
    """The oracle as it stands, timed on the host on each workload: on one
    thread and on all of its OpenMP threads, repeating each config's call
    until budget_s (one thread, all threads) seconds have passed (at least
    one call).  `value` is the whole step's weight GB/s on all threads (the
    sum of the configs' per-call times)."""
    import oracle
    calls = oracle_config_calls(host)
    all_threads = oracle.num_threads()
    per = {}
    t_start = time.time()
    for name, (fn, nbytes) in calls.items():
        row = {"weight_bytes": nbytes}
        for label, threads, budget in (("one_thread", 1, budget_s[0]), ("all_threads", all_threads, budget_s[1])):
            oracle.set_num_threads(threads)
            n = 0
            t0 = time.perf_counter()
            while True:
                fn()
                n += 1
                if time.perf_counter() - t0 >= budget:
                    break
            ms = (time.perf_counter() - t0) * 1e3 / n
            row[label] = {"threads": threads, "ms_per_call": round(ms, 3), "calls_per_s": round(1e3 / ms, 2),
                          "weight_GBps": round(nbytes / ms / 1e6, 3), "calls_timed": n}
        per[name] = row
    oracle.set_num_threads(all_threads)
    step_ms = sum(r["all_threads"]["ms_per_call"] for r in per.values())
    wb = sum(weight_bytes().values())
    return {"value": round(wb / step_ms / 1e6, 3), "unit": "GB/s", "cores": all_threads, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0)),
            "sample": (f"each of the five workloads' oracle calls (f64) repeated for >= {budget_s[0]} s on one "
                       f"thread and >= {budget_s[1]} s on {all_threads} threads ({time.time() - t_start:.1f} s in "
                       f"all); value = the whole step's weight bytes / the sum of the per-config times on "
                       f"{all_threads} threads"),
            "per_config": per}


def c5_q8_accuracy(gq, host, v):
    """The Q8 path's result (GPU, config 5) against the exact-x f64 result
    (reported, not gated; the pages quote cosine 0.9887 for their DP4A path
    against 0.9999 for the float one)."""
    import oracle
    import synth
    W, x = host["c5"]
    N, K = synth.C5_Q8
    y8, _, _ = gq.q4k_q8_gemv_from_f32(v["c5W"], v["c5x"], N, K, xq=v["xq"], xd=v["xd"])
    y8 = y8.cpu().numpy().astype(np.float64)
    exact = oracle.q4k_gemv(W, x, N, K)
    q, d = oracle.q8_quantize(x)
    q8hat = oracle.q4k_q8_gemv(W, q, d, N, K)
    cos = float(np.dot(y8, exact) / (np.linalg.norm(y8) * np.linalg.norm(exact)))
    return {"cosine_vs_exact_x": round(cos, 6),
            "e_inf_vs_exact_x": float(f"{np.max(np.abs(y8 - exact)) / np.max(np.abs(exact)):.3e}"),
            "e_inf_vs_oracle_q8_path": float(f"{np.max(np.abs(y8 - q8hat)) / np.max(np.abs(q8hat)):.3e}"),
            "oracle_q8_cosine_vs_exact_x": round(float(np.dot(q8hat, exact) / (np.linalg.norm(q8hat) *
                                                                               np.linalg.norm(exact))), 6)}


CONFIG_KERNELS = {
    # config: (breakdown entry, weight bytes per call, the read launches its ceiling counts, label)
    "c1": ("c1_q4k_gemv_1024x1024_in_cache", ("c1",), "Q4_K 1024x1024 (in cache: 590 KB, not HBM-bound)"),
    "c2": ("c2_q4k_gemv_triple", ("c2a", "c2b", "c2c"), "Q4_K 4096x2560 + 2560x9728 + 9728x2560 back to back"),
    "c3": ("lm_head_argmax_248320x1024", ("c3",), "lm_head Q6_K 248320x1024 + argmax"),
    "c4": ("ffn_f32_swiglu+q6k", ("c4g", "c4d"), "SwiGLU 2x Q4_K 9728x2560 + Q6_K 2560x9728 (two launches)"),
    "c5": ("c5_q4k_q8_gemv_from_f32_28672x8192", ("c5",),
           "Q8 quantize + Q4_K x Q8 28672x8192 (one launch: the quantization in the GEMV's prologue)"),
}


def read_sizes():
    import synth
    sz = {}
    N, K = synth.C1_Q4K
    sz["c1"] = N * K // 256 * 144
    for tag, (N, K) in zip(("c2a", "c2b", "c2c"), synth.C2_Q4K):
        sz[tag] = N * K // 256 * 144
    N, K = synth.C3_LM_HEAD
    sz["c3"] = N * K // 256 * 210
    N, K = synth.C4_SWIGLU
    sz["c4g"] = 2 * N * K // 256 * 144
    sz["c4d"] = K * N // 256 * 210
    N, K = synth.C5_Q8
    sz["c5"] = N * K // 256 * 144
    return sz


def config_algorithmic_bytes():
    """Bytes a config must move per call: its weights plus the f32 vectors
    it reads and writes (config 4: h written and read back between the two
    launches; config 5, one launch: x read, the Q8 codes and fp16 scales
    written once, the GEMV reading them from LDS, y written)."""
    import synth
    wb = weight_bytes()
    N, K = synth.C1_Q4K
    out = {"c1": wb["c1"] + 4 * (N + K)}
    out["c2"] = wb["c2"] + sum(4 * (N + K) for N, K in synth.C2_Q4K)
    N, K = synth.C3_LM_HEAD
    out["c3"] = wb["c3"] + 4 * K + 4
    N, K = synth.C4_SWIGLU
    out["c4"] = wb["c4"] + 4 * K + 2 * 4 * N + 4 * K
    N, K = synth.C5_Q8
    out["c5"] = wb["c5"] + 4 * K + K + K // 16 + 4 * N
    return out


def device_facts(dev):
    """The device's own account of itself (torch's view of
    hipGetDeviceProperties), for the report."""
    import torch
    pr = torch.cuda.get_device_properties(dev)
    keys = ("name", "gcnArchName", "multi_processor_count", "warp_size", "total_memory", "L2_cache_size",
            "shared_memory_per_multiprocessor", "shared_memory_per_block", "max_threads_per_multi_processor")
    return {k: getattr(pr, k) for k in keys if hasattr(pr, k)}


def config_summary(kern, ceil, cpu):
    """Per-config figures from the breakdown, the read ceilings and the CPU
    oracle timings."""
    sz = read_sizes()
    wb = weight_bytes()
    alg = config_algorithmic_bytes()
    out = {}
    for name, (entry, reads, label) in CONFIG_KERNELS.items():
        k = kern.get(entry)
        if k is None:
            continue
        us = k["us"]
        read_us = sum(ceil[sz[r]]["us"] for r in reads) if ceil else None
        row = {"workload": label, "us_per_call": us, "gemv_per_s": round(1e6 / us, 1),
               "weight_GBps": round(wb[name] / us / 1e3, 1),
               "algorithmic_bytes": alg[name], "algorithmic_GBps": round(alg[name] / us / 1e3, 1),
               "frac_hbm_peak": round(wb[name] / us / 1e3 / HBM_PEAK_GBS, 4),
               "read_ceiling_us": round(read_us, 2) if read_us else None,
               "frac_read_ceiling": round(read_us / us, 4) if read_us else None}
        if name == "c1":
            row["in_cache"] = True
        if cpu:
            c = cpu["per_config"][name]
            row["oracle_ms_per_call"] = {"one_thread": c["one_thread"]["ms_per_call"],
                                         "all_threads": c["all_threads"]["ms_per_call"]}
            row["gpu_vs_oracle_all_threads"] = round(c["all_threads"]["ms_per_call"] * 1e3 / us, 1)
        out[name] = row
    return out


def attach_traffic(kern):
    """Each recorded kernel's HBM bytes per launch (None if its record is
    stale) under its breakdown entries; a '+'-joined tag names several
    entries that share one kernel instantiation and one record."""
    for tag, _, alg_b, path in traffic_kernels()[1:]:
        for t in tag.split("+"):
            if t in kern:
                kern[t]["traffic"] = traffic_entry(alg_b, path)


def traffic_entry(alg_bytes, path=None):
    """HBM bytes per launch from a committed rocprofv3 counter record (the
    lm_head's by default), if it was taken on the current kernel sources."""
    try:
        with open(path or PROFILE_TRAFFIC) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="first run a plain 256 MiB device copy six times (counter calibration for rocprofv3)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="no GPU work: summarise two rocprofv3 --pmc databases (FETCH_SIZE, WRITE_SIZE) of "
                         "'bench.py --calibration-copy' into the lm_head traffic record under profiles/")
    ap.add_argument("--traffic-command", default="", help="the profiling commands, stored with the record")
    args = ap.parse_args()
    if args.traffic_from:
        write_traffic(*args.traffic_from, args.traffic_command)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the path is a single-GPU kernel library); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gemv_q4k_q6k_amd as gq
    import synth

    dev = torch.device("cuda:0")
    gq.lib()
    if args.calibration_copy:
        calibration_copy(dev)
    host, sets, v = build_workload(dev)
    N, K = synth.C3_LM_HEAD
    v["ws"] = torch.zeros(gq.lm_head_argmax_ws_bytes(N, K), dtype=torch.uint8, device=dev)
    parity_ok = self_check(gq, sets, v)   # both copies go through the checked binding once
    log(f"self-check of the benchmarked buffers: {'ok' if parity_ok else 'FAILED'}")

    prepared = [step_calls(gq, sets[c], v) for c in range(2)]
    for w in range(args.warmup):
        run_calls(*prepared[w % 2])
    torch.cuda.synchronize()

    # per-step (start, stop) events for the lm_head kernel; recording each once
    # creates its HIP handle
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in ev:
        a.record()
        b.record()
    handles = [(a.cuda_event, b.cuda_event) for a, b in ev]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    gc.disable()   # no collector pause between launches inside the timed region
    wall0 = time.perf_counter()
    t_start.record()
    for k in range(args.steps):
        calls, lm = prepared[k % 2]
        run_calls(calls, lm, handles[k])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gc.enable()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    lm_us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1000.0

    wb = weight_bytes()
    step_bytes = sum(wb.values())
    gms = graph_step_ms(gq, sets, v, args.steps)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    alg = lm_head_algorithmic_bytes()
    achieved = alg / (lm_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_entry(alg),
                "kernel": "lm_head_argmax Q6_K 248320x1024", "algorithmic_bytes_per_launch": alg,
                "avg_launch_us": round(lm_us, 2)}
    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded GGUF Q4_K/Q6_K blocks, f32 activations)",
        "config": {"workload": "decode hot path, in decode order: Q4_K 1024x1024; Q4_K 4096x2560+2560x9728+"
                               "9728x2560; SwiGLU 2x Q4_K 9728x2560 + Q6_K 2560x9728; Q8 quantize + Q4_K x Q8 "
                               "28672x8192 (one launch); Q6_K lm_head 248320x1024 + argmax",
                   "weight_bytes_per_step": step_bytes,
                   "value_is": "weight bytes of the whole step / step time (every config's GEMVs; see configs "
                               "for each one)",
                   "weight_copies": 2, "parallelism": "single GPU"},
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "lm_head_argmax_calls_per_s": round(1e6 / lm_us, 1),
        "lm_head_argmax_sync_calls_per_s": round(sync_rate(prepared, v), 1),
        "graph_ms_per_step": round(gms, 4),
        "graph_value": round(step_bytes / (gms * 1e-3) / 1e9, 1),
        "self_check_ok": parity_ok,
        "device": device_facts(dev),
        "wall_s": round(wall, 3),
        "roofline": roofline,
    }
    kern, ceil, cpu = None, None, None
    if not args.no_breakdown:
        kern = breakdown(gq, sets, v)
        sizes = sorted(set(read_sizes().values()))
        ceil = read_ceiling(gq, dev, sizes, in_cache=(read_sizes()["c1"],))
        for k in kern.values():   # each kernel against a read of its matrix bytes
            wbk = k.get("weight_bytes")
            if wbk in ceil:
                k["frac_read_ceiling"] = round(ceil[wbk]["us"] / k["us"], 4)
        attach_traffic(kern)
        result["kernels"] = kern
        result["read_ceiling"] = {str(S): c for S, c in ceil.items()}
        result["c5_q8_accuracy"] = c5_q8_accuracy(gq, host, {**v, "c5W": sets[0]["c5W"]})
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(host)
        result["cpu_baseline"] = cpu
    if kern is not None:
        result["configs"] = config_summary(kern, ceil, cpu)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
