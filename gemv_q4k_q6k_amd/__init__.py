"""Python binding of libgemvq.so, the gfx950 batch-1 quantized GEMV library.

Argument marshalling only: every function checks tensor dtype, device, size
and contiguity, passes raw device pointers and the current HIP stream of the
tensors' device to the C ABI (include/gemvq.h), and raises GemvqError on a
non-zero status.  All arithmetic happens in the HIP kernels; there is no CPU
fallback, and importing the functions fails loudly when the library has not
been built (``python -m gemv_q4k_q6k_amd.build``).

Layout: a weight matrix is a uint8 tensor holding N rows of K/256
super-blocks (144 bytes each for Q4_K, 210 for Q6_K), rows back to back.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

__all__ = [
    "GemvqError", "lib", "exported_names", "header_names",
    "q4k_gemv", "q4k_gemv_multi", "q6k_gemv", "q8_quantize", "q4k_q8_gemv", "swiglu_gemv",
    "lm_head_argmax", "lm_head_argmax_timed", "lm_head_argmax_masked", "lm_head_argmax_noalloc", "lm_head_argmax_ws_bytes", "q4k_q8_isums", "strerror", "tile_geometry", "stream_read",
    "q6k_q8_gemv", "q4k_q8_gemv_from_f32", "q6k_q8_isums", "swiglu_q8_gemv", "swiglu_q8_ws_bytes", "rms_norm_q8", "q4k_q8_gemv_batch", "q6k_q8_gemv_batch", "add_rms_norm_q8",
    "Q4K_BLOCK_BYTES", "Q6K_BLOCK_BYTES", "LIB_PATH", "HEADER_PATH",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgemvq.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "gemvq.h")

Q4K_BLOCK_BYTES = 144
Q6K_BLOCK_BYTES = 210

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_WORKSPACE, ERR_ALIAS, ERR_HIP, ERR_VALUE = range(8)


class GemvqError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn}: status {status}: {message}")
        self.status = status


_lock = threading.Lock()
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SIGS = {
    "q4k_gemv": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P]),
    "q4k_gemv_multi": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int, _P, _I64, _P]),
    "q6k_gemv": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P]),
    "q8_quantize": (ctypes.c_int, [_P, _P, _P, _I64, _P]),
    "q4k_q8_gemv": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _P]),
    "swiglu_gemv": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _P]),
    "q4k_q8_gemv_from_f32": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _P]),
    "q6k_q8_gemv": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _P]),
    "q4k_q8_gemv_batch": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, ctypes.c_int, _P]),
    "q6k_q8_gemv_batch": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, ctypes.c_int, _P]),
    "gemvq_q6k_q8_isums": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P]),
    "swiglu_q8_gemv": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _I64, _I64, _P]),
    "gemvq_swiglu_q8_ws_bytes": (ctypes.c_size_t, [_I64]),
    "rms_norm_q8": (ctypes.c_int, [_P, _P, ctypes.c_float, _P, _P, _P, _I64, _P]),
    "add_rms_norm_q8": (ctypes.c_int, [_P, _P, _P, ctypes.c_float, _P, _P, _P, _P, _I64, _P]),
    "lm_head_argmax": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_size_t, _I64, _I64, _P]),
    "lm_head_argmax_timed": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_size_t, _I64, _I64, _P, _P, _P]),
    "lm_head_argmax_masked": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_size_t, _I64, _I64, _P]),
    "lm_head_argmax_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _P]),
    "gemvq_lm_head_argmax_ws_bytes": (ctypes.c_size_t, [_I64, _I64]),
    "gemvq_q4k_q8_isums": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P]),
    "gemvq_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "gemvq_tile_geometry": (ctypes.c_int, [ctypes.c_int, _I64, _I64, _P]),
    "gemvq_stream_read": (ctypes.c_int, [_P, _I64, ctypes.c_int, ctypes.c_int, _P, _P]),
}


def lib() -> ctypes.CDLL:
    """Load libgemvq.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m gemv_q4k_q6k_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGS.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
        return _lib


def header_names() -> list[str]:
    """Function names declared in include/gemvq.h."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                                 text, flags=re.M)))


def exported_names() -> list[str]:
    return sorted(_SIGS)


(KIND_Q4K, KIND_Q6K, KIND_Q4K_Q8, KIND_SWIGLU, KIND_Q6K_Q8, KIND_SWIGLU_Q8, KIND_Q4K_Q8_BATCH,
 KIND_Q6K_Q8_BATCH) = range(8)


def tile_geometry(kind: int, N: int, K: int) -> dict:
    """Launch geometry the library uses for an N x K matrix (host-only)."""
    out = (ctypes.c_int64 * 11)()
    _check("gemvq_tile_geometry", lib().gemvq_tile_geometry(kind, N, K, ctypes.cast(out, ctypes.c_void_p)))
    return {"waves": out[0], "rows_tile": out[1], "tiles": out[2], "wave_local": out[3],
            "x_in_lds": out[4], "lds_bytes": out[5], "steps": out[6], "wave_unit": out[7],
            "resident": out[8], "phase": out[9], "grid": out[10]}


def stream_read(buf, grid: int, sink, stream=None, threads: int = 1024) -> None:
    """Plain streaming read of a whole device tensor by `grid` workgroups of
    `threads` (256 or 1024) threads (measurement hook)."""
    torch = _torch()
    if not isinstance(buf, torch.Tensor) or buf.device.type != "cuda" or not buf.is_contiguous():
        raise TypeError("buf: expected a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    _check("gemvq_stream_read", lib().gemvq_stream_read(buf.data_ptr(), nbytes - nbytes % 16, int(grid),
                                                         int(threads), sink.data_ptr(), _stream(buf, stream)))


def strerror(status: int) -> str:
    return lib().gemvq_strerror(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise GemvqError(fn, status, strerror(status))


# ------------------------------------------------------------ torch helpers
def _torch():
    import torch
    return torch


def _dev_tensor(t, dtype, numel: int, what: str):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{what}: must be a device tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{what}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{what}: expected {numel} elements, got {t.numel()}")
    return t


def _stream(t, stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _weights(W, N: int, K: int, block: int, what: str = "W"):
    if K % 256:
        raise ValueError("K must be a multiple of 256")
    return _dev_tensor(W, _torch().uint8, N * (K // 256) * block, what)


def _out(out, device, dtype, n: int, what: str):
    torch = _torch()
    if out is None:
        return torch.empty(n, dtype=dtype, device=device)
    return _dev_tensor(out, dtype, n, what)


# ------------------------------------------------------------- entry points
def q4k_gemv(W, x, N: int, K: int, y=None, stream=None):
    """y = W x for a Q4_K matrix W (uint8, N*(K/256)*144 bytes), x float32[K]."""
    torch = _torch()
    _weights(W, N, K, Q4K_BLOCK_BYTES)
    _dev_tensor(x, torch.float32, K, "x")
    y = _out(y, x.device, torch.float32, N, "y")
    _check("q4k_gemv", lib().q4k_gemv(W.data_ptr(), x.data_ptr(), y.data_ptr(), N, K, _stream(x, stream)))
    return y


def q4k_gemv_multi(Ws, Ns, x, K: int, ys=None, residuals=None, stream=None):
    """y_i = W_i x (+ residuals[i]) for up to 4 Q4_K matrices of the same K in
    one launch.  Returns the list of float32 outputs (ys if given).  A
    residual may be its own output (in-place add)."""
    torch = _torch()
    count = len(Ws)
    if count != len(Ns):
        raise ValueError("Ws and Ns differ in length")
    _dev_tensor(x, torch.float32, K, "x")
    for W, N in zip(Ws, Ns):
        _weights(W, N, K, Q4K_BLOCK_BYTES)
    if ys is None:
        ys = [None] * count
    ys = [_out(y, x.device, torch.float32, N, f"y[{i}]") for i, (y, N) in enumerate(zip(ys, Ns))]
    if residuals is not None:
        for i, (r, N) in enumerate(zip(residuals, Ns)):
            if r is not None:
                _dev_tensor(r, torch.float32, N, f"residual[{i}]")
    P = ctypes.c_void_p * count
    w_arr = P(*[W.data_ptr() for W in Ws])
    y_arr = P(*[y.data_ptr() for y in ys])
    n_arr = (ctypes.c_int64 * count)(*Ns)
    r_arr = None if residuals is None else P(*[r.data_ptr() if r is not None else None for r in residuals])
    _check("q4k_gemv_multi", lib().q4k_gemv_multi(ctypes.cast(w_arr, ctypes.c_void_p), ctypes.cast(n_arr, ctypes.c_void_p),
                                                  ctypes.cast(y_arr, ctypes.c_void_p),
                                                  ctypes.cast(r_arr, ctypes.c_void_p) if r_arr is not None else None,
                                                  count, x.data_ptr(), K, _stream(x, stream)))
    return ys


def q6k_gemv(W, x, N: int, K: int, y=None, stream=None):
    """y = W x for a Q6_K matrix W (uint8, N*(K/256)*210 bytes), x float32[K]."""
    torch = _torch()
    _weights(W, N, K, Q6K_BLOCK_BYTES)
    _dev_tensor(x, torch.float32, K, "x")
    y = _out(y, x.device, torch.float32, N, "y")
    _check("q6k_gemv", lib().q6k_gemv(W.data_ptr(), x.data_ptr(), y.data_ptr(), N, K, _stream(x, stream)))
    return y


def q8_quantize(x, xq=None, xd=None, stream=None):
    """x float32[K] -> (int8[K] values, int16[K/32] fp16 scale bits)."""
    torch = _torch()
    K = x.numel()
    _dev_tensor(x, torch.float32, K, "x")
    xq = _out(xq, x.device, torch.int8, K, "xq")
    xd = _out(xd, x.device, torch.int16, K // 32, "xd")
    _check("q8_quantize", lib().q8_quantize(x.data_ptr(), xq.data_ptr(), xd.data_ptr(), K, _stream(x, stream)))
    return xq, xd


def q4k_q8_gemv(W, xq, xd, N: int, K: int, y=None, stream=None):
    """y = W (dequantized Q8 x) with exact int8 dots; xq int8[K], xd int16[K/32]."""
    torch = _torch()
    _weights(W, N, K, Q4K_BLOCK_BYTES)
    _dev_tensor(xq, torch.int8, K, "xq")
    _dev_tensor(xd, torch.int16, K // 32, "xd")
    y = _out(y, xq.device, torch.float32, N, "y")
    _check("q4k_q8_gemv", lib().q4k_q8_gemv(W.data_ptr(), xq.data_ptr(), xd.data_ptr(), y.data_ptr(), N, K,
                                            _stream(xq, stream)))
    return y


def q4k_q8_gemv_from_f32(W, x, N: int, K: int, xq=None, xd=None, y=None, stream=None):
    """q8_quantize(x) then q4k_q8_gemv in one call (one launch where the
    wave-unit kernel runs the shape).  Returns (y, xq, xd)."""
    torch = _torch()
    _weights(W, N, K, Q4K_BLOCK_BYTES)
    _dev_tensor(x, torch.float32, K, "x")
    xq = _out(xq, x.device, torch.int8, K, "xq")
    xd = _out(xd, x.device, torch.int16, K // 32, "xd")
    y = _out(y, x.device, torch.float32, N, "y")
    _check("q4k_q8_gemv_from_f32", lib().q4k_q8_gemv_from_f32(W.data_ptr(), x.data_ptr(), xq.data_ptr(), xd.data_ptr(),
                                                              y.data_ptr(), N, K, _stream(x, stream)))
    return y, xq, xd


def q6k_q8_gemv(W, xq, xd, N: int, K: int, y=None, stream=None):
    """y = W (dequantized Q8 x) for a Q6_K matrix W, exact int8 dots per
    16-element group; xq int8[K], xd int16[K/32]."""
    torch = _torch()
    _weights(W, N, K, Q6K_BLOCK_BYTES)
    _dev_tensor(xq, torch.int8, K, "xq")
    _dev_tensor(xd, torch.int16, K // 32, "xd")
    y = _out(y, xq.device, torch.float32, N, "y")
    _check("q6k_q8_gemv", lib().q6k_q8_gemv(W.data_ptr(), xq.data_ptr(), xd.data_ptr(), y.data_ptr(), N, K,
                                            _stream(xq, stream)))
    return y


def q4k_q8_gemv_batch(W, xq, xd, N: int, K: int, m: int, y=None, stream=None):
    """Y[j] = W xdq_j for m Q8 vectors (xq int8[m*K], xd int16[m*K/32], back
    to back) through one Q4_K matrix; returns float32 [m, N]."""
    return _batch("q4k_q8_gemv_batch", Q4K_BLOCK_BYTES, W, xq, xd, N, K, m, y, stream)


def q6k_q8_gemv_batch(W, xq, xd, N: int, K: int, m: int, y=None, stream=None):
    """As q4k_q8_gemv_batch for a Q6_K matrix."""
    return _batch("q6k_q8_gemv_batch", Q6K_BLOCK_BYTES, W, xq, xd, N, K, m, y, stream)


def _batch(name, block, W, xq, xd, N, K, m, y, stream):
    torch = _torch()
    _weights(W, N, K, block)
    _dev_tensor(xq, torch.int8, m * K, "xq")
    _dev_tensor(xd, torch.int16, m * (K // 32), "xd")
    y = _out(y, xq.device, torch.float32, m * N, "y")
    _check(name, getattr(lib(), name)(W.data_ptr(), xq.data_ptr(), xd.data_ptr(), y.data_ptr(), N, K, m,
                                      _stream(xq, stream)))
    return y.view(m, N)


def swiglu_gemv(Wg, Wu, x, N: int, K: int, h=None, stream=None):
    """h = silu(Wg x) * (Wu x), Wg and Wu Q4_K N x K."""
    torch = _torch()
    _weights(Wg, N, K, Q4K_BLOCK_BYTES, "Wg")
    _weights(Wu, N, K, Q4K_BLOCK_BYTES, "Wu")
    _dev_tensor(x, torch.float32, K, "x")
    h = _out(h, x.device, torch.float32, N, "h")
    _check("swiglu_gemv", lib().swiglu_gemv(Wg.data_ptr(), Wu.data_ptr(), x.data_ptr(), h.data_ptr(), N, K,
                                            _stream(x, stream)))
    return h


def swiglu_q8_ws_bytes(N: int) -> int:
    return int(lib().gemvq_swiglu_q8_ws_bytes(N))


def swiglu_q8_gemv(Wg, Wu, x, N: int, K: int, workspace, hq=None, hd=None, h=None, stream=None):
    """(hq int8[N], hd int16[N/32]): the Q8 encoding of silu(Wg x) * (Wu x),
    written by the GEMV itself (N % 32 == 0).  `h` (float32[N]), if given,
    also receives the f32 product.  `workspace` is a uint8 device tensor of
    at least swiglu_q8_ws_bytes(N) bytes, zero-filled before its first use;
    every call leaves it reusable."""
    torch = _torch()
    _weights(Wg, N, K, Q4K_BLOCK_BYTES, "Wg")
    _weights(Wu, N, K, Q4K_BLOCK_BYTES, "Wu")
    _dev_tensor(x, torch.float32, K, "x")
    if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" or workspace.dtype != torch.uint8:
        raise TypeError("workspace: expected a uint8 device tensor")
    hq = _out(hq, x.device, torch.int8, N, "hq")
    hd = _out(hd, x.device, torch.int16, N // 32, "hd")
    if h is not None:
        _dev_tensor(h, torch.float32, N, "h")
    _check("swiglu_q8_gemv", lib().swiglu_q8_gemv(Wg.data_ptr(), Wu.data_ptr(), x.data_ptr(),
                                                  h.data_ptr() if h is not None else None, hq.data_ptr(),
                                                  hd.data_ptr(), workspace.data_ptr(), workspace.numel(), N, K,
                                                  _stream(x, stream)))
    return hq, hd


def rms_norm_q8(x, w, eps: float, xq=None, xd=None, y=None, stream=None):
    """(xq int8[K], xd int16[K/32]): Q8 encoding of w * x / sqrt(mean(x^2) +
    eps).  `y` (float32[K]), if given, also receives the f32 norm."""
    return _rms(x, None, w, eps, None, xq, xd, y, stream)


def add_rms_norm_q8(x, r, w, eps: float, res=None, xq=None, xd=None, y=None, stream=None):
    """(res, xq, xd): res = x + r (f32; may be x or r itself), then the Q8
    encoding of the RMS norm of res."""
    torch = _torch()
    res = _out(res, x.device, torch.float32, x.numel(), "res")
    xq, xd = _rms(x, r, w, eps, res, xq, xd, y, stream)
    return res, xq, xd


def _rms(x, r, w, eps, res, xq, xd, y, stream):
    torch = _torch()
    K = x.numel()
    _dev_tensor(x, torch.float32, K, "x")
    _dev_tensor(w, torch.float32, K, "w")
    if r is not None:
        _dev_tensor(r, torch.float32, K, "r")
    xq = _out(xq, x.device, torch.int8, K, "xq")
    xd = _out(xd, x.device, torch.int16, K // 32, "xd")
    if y is not None:
        _dev_tensor(y, torch.float32, K, "y")
    yp = y.data_ptr() if y is not None else None
    if r is None:
        _check("rms_norm_q8", lib().rms_norm_q8(x.data_ptr(), w.data_ptr(), float(eps), yp, xq.data_ptr(),
                                                xd.data_ptr(), K, _stream(x, stream)))
    else:
        _check("add_rms_norm_q8", lib().add_rms_norm_q8(x.data_ptr(), r.data_ptr(), w.data_ptr(), float(eps),
                                                        res.data_ptr(), yp, xq.data_ptr(), xd.data_ptr(), K,
                                                        _stream(x, stream)))
    return xq, xd


def lm_head_argmax_ws_bytes(N: int, K: int) -> int:
    return int(lib().gemvq_lm_head_argmax_ws_bytes(N, K))


def _event_handle(ev) -> int:
    """Raw hipEvent_t of a torch.cuda.Event created with enable_timing=True
    (torch creates the handle at the first record, so record it once first)."""
    h = int(ev.cuda_event)
    if h == 0:
        raise ValueError("event has no HIP handle yet: record it once before passing it")
    return h


def lm_head_argmax(W, x, N: int, K: int, workspace, out_idx=None, out_max=None, want_max: bool = False,
                   stream=None):
    """First index of the largest row value of W x (Q6_K W).  Returns the
    int32[1] device tensor holding the index (and the float32[1] maximum if
    want_max or out_max is given).  `workspace` is a uint8 device tensor of at
    least lm_head_argmax_ws_bytes(N, K) bytes, zero-filled before its first use
    (torch.zeros); every call leaves its counters (the first 4096 bytes) zero
    again."""
    return _lm_head(W, x, N, K, workspace, out_idx, out_max, want_max, stream, None)


def lm_head_argmax_timed(W, x, N: int, K: int, workspace, start_event, stop_event, out_idx=None, out_max=None,
                         want_max: bool = False, stream=None):
    """lm_head_argmax that records the kernel's own start and end into two
    torch.cuda.Event(enable_timing=True) objects (each recorded once before),
    so start_event.elapsed_time(stop_event) is the kernel's duration."""
    return _lm_head(W, x, N, K, workspace, out_idx, out_max, want_max, stream,
                    (_event_handle(start_event), _event_handle(stop_event)))


def lm_head_argmax_masked(W, x, mask, N: int, K: int, workspace, out_idx=None, out_max=None,
                          want_max: bool = False, stream=None):
    """lm_head_argmax over the rows the mask allows.  `mask` is an int32 (or
    uint32) device tensor of ceil(N/32) words; bit i % 32 of word i // 32 set
    bans row i."""
    torch = _torch()
    words = (N + 31) // 32
    if (not isinstance(mask, torch.Tensor) or mask.device.type != "cuda" or mask.dtype not in (torch.int32, torch.uint32)
            or mask.numel() < words or not mask.is_contiguous()):
        raise TypeError(f"mask: expected a contiguous int32/uint32 device tensor of at least {words} words")
    return _lm_head(W, x, N, K, workspace, out_idx, out_max, want_max, stream, None, mask)


def lm_head_argmax_noalloc(W, x, N: int, K: int, out_idx=None, out_max=None, want_max: bool = False, stream=None):
    """lm_head_argmax with the library's own per-GPU workspace (no workspace
    argument; the C entry point allocates nothing).  Calls that overlap on one
    GPU race; calls in stream order are safe.  Pass out_idx (and out_max) to
    keep the call free of torch allocations as well."""
    torch = _torch()
    _weights(W, N, K, Q6K_BLOCK_BYTES)
    _dev_tensor(x, torch.float32, K, "x")
    out_idx = _out(out_idx, x.device, torch.int32, 1, "out_idx")
    if want_max and out_max is None:
        out_max = torch.empty(1, dtype=torch.float32, device=x.device)
    if out_max is not None:
        _dev_tensor(out_max, torch.float32, 1, "out_max")
    _check("lm_head_argmax_noalloc", lib().lm_head_argmax_noalloc(
        W.data_ptr(), x.data_ptr(), out_idx.data_ptr(), out_max.data_ptr() if out_max is not None else None,
        N, K, _stream(x, stream)))
    return (out_idx, out_max) if out_max is not None else out_idx


def _lm_head(W, x, N, K, workspace, out_idx, out_max, want_max, stream, events, mask=None):
    torch = _torch()
    _weights(W, N, K, Q6K_BLOCK_BYTES)
    _dev_tensor(x, torch.float32, K, "x")
    if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" or workspace.dtype != torch.uint8:
        raise TypeError("workspace: expected a uint8 device tensor")
    out_idx = _out(out_idx, x.device, torch.int32, 1, "out_idx")
    if want_max and out_max is None:
        out_max = torch.empty(1, dtype=torch.float32, device=x.device)
    if out_max is not None:
        _dev_tensor(out_max, torch.float32, 1, "out_max")
    args = (W.data_ptr(), x.data_ptr(), out_idx.data_ptr(), out_max.data_ptr() if out_max is not None else None,
            workspace.data_ptr(), workspace.numel(), N, K, _stream(x, stream))
    if mask is not None:
        _check("lm_head_argmax_masked", lib().lm_head_argmax_masked(args[0], args[1], mask.data_ptr(), *args[2:]))
    elif events is None:
        _check("lm_head_argmax", lib().lm_head_argmax(*args))
    else:
        _check("lm_head_argmax_timed", lib().lm_head_argmax_timed(*args, *events))
    return (out_idx, out_max) if out_max is not None else out_idx


def q4k_q8_isums(W, xq, N: int, K: int, out=None, stream=None):
    """Exact integer sums isums[n][j] of the Q8 path (test hook)."""
    torch = _torch()
    _weights(W, N, K, Q4K_BLOCK_BYTES)
    _dev_tensor(xq, torch.int8, K, "xq")
    out = _out(out, xq.device, torch.int32, N * (K // 32), "isums")
    _check("gemvq_q4k_q8_isums", lib().gemvq_q4k_q8_isums(W.data_ptr(), xq.data_ptr(), out.data_ptr(), N, K,
                                                          _stream(xq, stream)))
    return out.view(N, K // 32)


def q6k_q8_isums(W, xq, N: int, K: int, out=None, stream=None):
    """Exact integer sums isums[n][g] of the Q6_K x Q8 path, one per
    16-element group (test hook)."""
    torch = _torch()
    _weights(W, N, K, Q6K_BLOCK_BYTES)
    _dev_tensor(xq, torch.int8, K, "xq")
    out = _out(out, xq.device, torch.int32, N * (K // 16), "isums")
    _check("gemvq_q6k_q8_isums", lib().gemvq_q6k_q8_isums(W.data_ptr(), xq.data_ptr(), out.data_ptr(), N, K,
                                                          _stream(xq, stream)))
    return out.view(N, K // 16)
