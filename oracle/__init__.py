"""CPU oracle for the batch-1 quantized GEMV path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (``gemv_q4k_q6k_amd`` and
its HIP library) never does, and the two share no code.

The GEMV and quantizer arithmetic lives in ``oracle.c`` (plain C, f64
accumulation, exact super-block decoding; see that file's header for the
block formats and the readings they rest on); this module builds it with gcc,
loads it with ctypes and converts numpy arrays.  The RMS norms are plain
numpy in f64 here.  Every function is pinned by
``tests/test_oracle_pins.py`` against closed forms, hand-packed blocks,
library routines (numpy float16, numpy matmul, numpy nanargmax) and brute
force.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

Q4K_BLOCK_BYTES = 144
Q6K_BLOCK_BYTES = 210
QK = 256


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (-O2, OpenMP, no fast-math, no FMA
    contraction so every f64/f32 operation rounds once)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-std=c11", "-Wall", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        sig = {
            "orc_fp16_to_f64": (ctypes.c_double, [ctypes.c_uint16]),
            "orc_f32_to_fp16_rne": (ctypes.c_uint16, [ctypes.c_float]),
            "orc_q4k_block": (None, [P, P]),
            "orc_q6k_block": (None, [P, P]),
            "orc_q4k_gemv": (None, [P, P, P, I64, I64]),
            "orc_q6k_gemv": (None, [P, P, P, I64, I64]),
            "orc_q6k_gemv_f64x": (None, [P, P, P, I64, I64]),
            "orc_swiglu": (None, [P, P, P, P, P, P, I64, I64]),
            "orc_q8_quantize": (None, [P, P, P, I64]),
            "orc_q4k_q8_isums": (None, [P, P, P, I64, I64]),
            "orc_q4k_q8_gemv": (None, [P, P, P, P, I64, I64]),
            "orc_q6k_q8_isums": (None, [P, P, P, I64, I64]),
            "orc_q6k_q8_gemv": (None, [P, P, P, P, I64, I64]),
            "orc_argmax_first_f64": (I64, [P, I64]),
            "orc_argmax_first_f32": (I64, [P, I64]),
            "orc_argmax_first_masked_f64": (I64, [P, P, I64]),
            "orc_argmax_first_masked_f32": (I64, [P, P, I64]),
            "orc_num_threads": (ctypes.c_int, []),
            "orc_set_num_threads": (None, [ctypes.c_int]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _blocks(W: np.ndarray, N: int, K: int, block_bytes: int) -> np.ndarray:
    W = np.ascontiguousarray(W, dtype=np.uint8)
    if K % QK or W.size != N * (K // QK) * block_bytes:
        raise ValueError("weight buffer size does not match N x K")
    return W


def _vec(x, dtype) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=dtype)


# ------------------------------------------------------------------ scalars
def fp16_to_f64(bits: int) -> float:
    return _load().orc_fp16_to_f64(int(bits) & 0xFFFF)


def f32_to_fp16_bits(v: float) -> int:
    return int(_load().orc_f32_to_fp16_rne(float(np.float32(v))))


# ------------------------------------------------------------------- blocks
def q4k_decode_block(blk: np.ndarray) -> np.ndarray:
    blk = np.ascontiguousarray(blk, dtype=np.uint8)
    assert blk.size == Q4K_BLOCK_BYTES
    w = np.empty(256, np.float64)
    _load().orc_q4k_block(_ptr(blk), _ptr(w))
    return w


def q6k_decode_block(blk: np.ndarray) -> np.ndarray:
    blk = np.ascontiguousarray(blk, dtype=np.uint8)
    assert blk.size == Q6K_BLOCK_BYTES
    w = np.empty(256, np.float64)
    _load().orc_q6k_block(_ptr(blk), _ptr(w))
    return w


def q4k_dequantize(W: np.ndarray, N: int, K: int) -> np.ndarray:
    """Whole N x K Q4_K matrix -> f64 (small sizes only)."""
    W = _blocks(W, N, K, Q4K_BLOCK_BYTES).reshape(-1, Q4K_BLOCK_BYTES)
    return np.concatenate([q4k_decode_block(b) for b in W]).reshape(N, K)


def q6k_dequantize(W: np.ndarray, N: int, K: int) -> np.ndarray:
    W = _blocks(W, N, K, Q6K_BLOCK_BYTES).reshape(-1, Q6K_BLOCK_BYTES)
    return np.concatenate([q6k_decode_block(b) for b in W]).reshape(N, K)


# -------------------------------------------------------------------- GEMVs
def q4k_gemv(W, x, N: int, K: int) -> np.ndarray:
    W = _blocks(W, N, K, Q4K_BLOCK_BYTES)
    x = _vec(x, np.float32)
    y = np.empty(N, np.float64)
    _load().orc_q4k_gemv(_ptr(W), _ptr(x), _ptr(y), N, K)
    return y


def q6k_gemv(W, x, N: int, K: int) -> np.ndarray:
    W = _blocks(W, N, K, Q6K_BLOCK_BYTES)
    x = _vec(x, np.float32)
    y = np.empty(N, np.float64)
    _load().orc_q6k_gemv(_ptr(W), _ptr(x), _ptr(y), N, K)
    return y


def q6k_gemv_f64x(W, x, N: int, K: int) -> np.ndarray:
    W = _blocks(W, N, K, Q6K_BLOCK_BYTES)
    x = _vec(x, np.float64)
    y = np.empty(N, np.float64)
    _load().orc_q6k_gemv_f64x(_ptr(W), _ptr(x), _ptr(y), N, K)
    return y


def swiglu(Wg, Wu, x, N: int, K: int):
    """Returns (h, g, u) in f64."""
    Wg = _blocks(Wg, N, K, Q4K_BLOCK_BYTES)
    Wu = _blocks(Wu, N, K, Q4K_BLOCK_BYTES)
    x = _vec(x, np.float32)
    h, g, u = (np.empty(N, np.float64) for _ in range(3))
    _load().orc_swiglu(_ptr(Wg), _ptr(Wu), _ptr(x), _ptr(h), _ptr(g), _ptr(u), N, K)
    return h, g, u


def q8_quantize(x):
    """Returns (q int8[K], d fp16 bits uint16[K/32])."""
    x = _vec(x, np.float32)
    K = x.size
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    q = np.empty(K, np.int8)
    d = np.empty(K // 32, np.uint16)
    _load().orc_q8_quantize(_ptr(x), _ptr(q), _ptr(d), K)
    return q, d


def q4k_q8_isums(W, xq, N: int, K: int) -> np.ndarray:
    W = _blocks(W, N, K, Q4K_BLOCK_BYTES)
    xq = _vec(xq, np.int8)
    out = np.empty((N, K // 32), np.int32)
    _load().orc_q4k_q8_isums(_ptr(W), _ptr(xq), _ptr(out), N, K)
    return out


def q4k_q8_gemv(W, xq, xd, N: int, K: int) -> np.ndarray:
    W = _blocks(W, N, K, Q4K_BLOCK_BYTES)
    xq = _vec(xq, np.int8)
    xd = _vec(xd, np.uint16)
    y = np.empty(N, np.float64)
    _load().orc_q4k_q8_gemv(_ptr(W), _ptr(xq), _ptr(xd), _ptr(y), N, K)
    return y


def q6k_q8_isums(W, xq, N: int, K: int) -> np.ndarray:
    """Exact integer sums of the Q6_K x Q8 path, int32[N, K/16]: one per
    16-element group (the Q6_K scale granularity), quants offset by -32."""
    W = _blocks(W, N, K, Q6K_BLOCK_BYTES)
    xq = _vec(xq, np.int8)
    out = np.empty((N, K // 16), np.int32)
    _load().orc_q6k_q8_isums(_ptr(W), _ptr(xq), _ptr(out), N, K)
    return out


def q6k_q8_gemv(W, xq, xd, N: int, K: int) -> np.ndarray:
    """y = W * xdq over Q6_K rows (xdq the dequantized Q8 activation), f64."""
    W = _blocks(W, N, K, Q6K_BLOCK_BYTES)
    xq = _vec(xq, np.int8)
    xd = _vec(xd, np.uint16)
    y = np.empty(N, np.float64)
    _load().orc_q6k_q8_gemv(_ptr(W), _ptr(xq), _ptr(xd), _ptr(y), N, K)
    return y


def q8_gemv_batch(fmt: str, W, xq, xd, N: int, K: int, m: int) -> np.ndarray:
    """Batched int8-activation GEMV (memra-engine decode.rs, the lockstep
    multi-stream decode and `full_attn_decode_batched`: one weight read
    serves m activation vectors): Y[j] = W * xdq_j for j < m, each row of Y
    the single-vector GEMV of that vector.  xq: int8[m, K], xd: fp16 bits
    [m, K/32], fmt "q4k" or "q6k".  Returns f64 [m, N]."""
    gemv = {"q4k": q4k_q8_gemv, "q6k": q6k_q8_gemv}[fmt]
    xq = np.asarray(xq, np.int8).reshape(m, K)
    xd = np.asarray(xd, np.uint16).reshape(m, K // 32)
    return np.stack([gemv(W, xq[j], xd[j], N, K) for j in range(m)])


# ------------------------------------------------ norms and Q8 emission
# memra-engine decode.rs names the producers that emit a quantized activation
# directly: `rms_norm_q8_1` (norm, then quantize), `add_rms_norm_q8_1`
# (residual add, norm, quantize; the sum is also returned as the new
# residual) and `silu_mul_scaled_q8_1` (the SwiGLU product, then quantize),
# each stated to equal the unfused sequence.  The pages name the norm and its
# eps (`cfg.rms_eps`) without writing it out; the reading here is the usual
# RMS norm, y_i = w_i * x_i / sqrt(mean_j x_j^2 + eps).


def rms_norm(x, w, eps: float) -> np.ndarray:
    """y = w * x / sqrt(mean(x^2) + eps) in f64 from f32 x, w and eps."""
    x = _vec(x, np.float32).astype(np.float64)
    w = _vec(w, np.float32).astype(np.float64)
    if x.shape != w.shape or x.size == 0:
        raise ValueError("x and w must be non-empty and of one length")
    e = float(np.float32(eps))
    ms = float(np.sum(x * x)) / x.size
    return w * (x / math.sqrt(ms + e))


def add_rms_norm(x, r, w, eps: float):
    """(res, y): res = x + r rounded once to f32 (the residual stream keeps
    f32), y = rms_norm(res, w, eps) in f64."""
    res = (_vec(x, np.float32) + _vec(r, np.float32)).astype(np.float32)
    return res, rms_norm(res, w, eps)


def rms_norm_q8(x, w, eps: float, r=None):
    """(res or None, y, q, d): the norm (after the residual add when r is
    given), then the Q8 quantization of y as an f32 vector.  The quantizer
    takes its decisions on f32 values, as q8_quantize does."""
    res = None
    if r is None:
        y = rms_norm(x, w, eps)
    else:
        res, y = add_rms_norm(x, r, w, eps)
    q, d = q8_quantize(y.astype(np.float32))
    return res, y, q, d


def swiglu_q8(Wg, Wu, x, N: int, K: int):
    """(h, q, d): the SwiGLU product h (f64), then the Q8 quantization of h as
    an f32 vector (N a multiple of 32)."""
    h, _, _ = swiglu(Wg, Wu, x, N, K)
    q, d = q8_quantize(h.astype(np.float32))
    return h, q, d


# ------------------------------------------------------------------- argmax
def q4k_gemv_multi(Ws, Ns, x, K, residuals=None):
    """y_i = W_i x (+ residual_i) for each matrix, each a plain q4k_gemv in
    f64 plus the f32 residual widened to f64."""
    out = []
    for i, (W, N) in enumerate(zip(Ws, Ns)):
        y = q4k_gemv(W, x, N, K)
        if residuals is not None and residuals[i] is not None:
            y = y + np.asarray(residuals[i], np.float64)
        out.append(y)
    return out


def argmax_first(v) -> int:
    """First index of the maximum over non-NaN values; 0 if all are NaN."""
    v = np.asarray(v)
    if v.dtype == np.float32:
        v = np.ascontiguousarray(v)
        return int(_load().orc_argmax_first_f32(_ptr(v), v.size))
    v = _vec(v, np.float64)
    return int(_load().orc_argmax_first_f64(_ptr(v), v.size))


def argmax_first_masked(v, mask_words) -> int:
    """First index of the maximum over non-NaN rows the mask allows (bit
    i % 32 of word i // 32 set bans row i); 0 if none is left."""
    v = np.asarray(v)
    m = np.ascontiguousarray(np.asarray(mask_words).view(np.uint32))
    assert m.size * 32 >= v.size
    if v.dtype == np.float32:
        v = np.ascontiguousarray(v)
        return int(_load().orc_argmax_first_masked_f32(_ptr(v), _ptr(m), v.size))
    v = _vec(v, np.float64)
    return int(_load().orc_argmax_first_masked_f64(_ptr(v), _ptr(m), v.size))


def top2_gap(v) -> float:
    """Largest minus second largest value at distinct indices (f64)."""
    v = np.asarray(v, dtype=np.float64)
    i = argmax_first(v)
    rest = np.delete(v, i)
    return float(v[i] - np.nanmax(rest))


def num_threads() -> int:
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    _load().orc_set_num_threads(int(n))
