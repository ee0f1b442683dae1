"""The C-ABI library on the host, with no GPU: it loads, exports every
function include/gemvq.h declares, and rejects bad arguments with the
documented status before any HIP call.

Pointers here are fake integers; every call below is built to be rejected by
the host-side checks, so nothing is ever dereferenced or launched."""
import ctypes
import glob
import os

import pytest

import gemv_q4k_q6k_amd as gq


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0     # counts devices without initialising HIP
    except Exception:
        return False


# Fake pointers must never reach a launch: run these only where no GPU exists.
pytestmark = pytest.mark.skipif(_gpu_visible(), reason="fake-pointer validation tests run on GPU-less hosts only")


def test_library_is_fresh():
    """The built library is newer than every source it is built from."""
    srcs = glob.glob(os.path.join(os.path.dirname(gq.LIB_PATH), "csrc", "*")) + [gq.HEADER_PATH]
    assert os.path.exists(gq.LIB_PATH), "build with python -m gemv_q4k_q6k_amd.build"
    lib_t = os.path.getmtime(gq.LIB_PATH)
    stale = [s for s in srcs if os.path.getmtime(s) > lib_t]
    assert not stale, f"libgemvq.so is older than {stale}; rebuild"

A = 1 << 20          # fake, 256-byte aligned "device" addresses far apart
B = 1 << 30
C = 1 << 34
D = 1 << 38
E = 1 << 42


def _rejected(code, expected):
    assert expected != gq.OK       # never let a test case reach a launch
    assert code == expected, (code, gq.strerror(code))


def test_library_loads_and_exports_header_symbols():
    L = gq.lib()
    names = gq.header_names()
    assert set(names) == set(gq.exported_names())
    for n in names:
        assert hasattr(L, n), n
    for n in ("q4k_gemv", "q6k_gemv", "q8_quantize", "q4k_q8_gemv", "swiglu_gemv", "lm_head_argmax"):
        assert n in names


def test_strerror_and_ws_bytes():
    for s in range(7):
        assert isinstance(gq.strerror(s), str) and gq.strerror(s)
    assert gq.strerror(99) == "unknown status"
    ws = gq.lm_head_argmax_ws_bytes(248_320, 1024)
    assert ws >= 4096 + 8 * 1024 and ws % 256 == 0   # counters, then one 8-byte key per workgroup (up to 1024)


def test_null_pointers():
    L = gq.lib()
    _rejected(L.q4k_gemv(None, B, C, 4, 256, None), gq.ERR_NULL)
    _rejected(L.q4k_gemv(A, None, C, 4, 256, None), gq.ERR_NULL)
    _rejected(L.q4k_gemv(A, B, None, 4, 256, None), gq.ERR_NULL)
    _rejected(L.q6k_gemv(A, B, None, 4, 256, None), gq.ERR_NULL)
    _rejected(L.q8_quantize(A, None, C, 256, None), gq.ERR_NULL)
    _rejected(L.q4k_q8_gemv(A, B, None, D, 4, 256, None), gq.ERR_NULL)
    _rejected(L.swiglu_gemv(A, None, C, D, 4, 256, None), gq.ERR_NULL)
    _rejected(L.lm_head_argmax(A, B, C, None, None, 1 << 20, 4, 256, None), gq.ERR_NULL)
    _rejected(L.lm_head_argmax_timed(A, B, C, None, None, 1 << 20, 4, 256, None, None, None), gq.ERR_NULL)
    _rejected(L.gemvq_q4k_q8_isums(A, B, None, 4, 256, None), gq.ERR_NULL)
    _rejected(L.q6k_q8_gemv(A, B, C, None, 4, 256, None), gq.ERR_NULL)
    _rejected(L.q6k_q8_gemv(None, B, C, D, 4, 256, None), gq.ERR_NULL)
    _rejected(L.gemvq_q6k_q8_isums(A, None, C, 4, 256, None), gq.ERR_NULL)
    _rejected(L.lm_head_argmax_masked(A, B, None, C, D, E, 1 << 20, 4, 256, None), gq.ERR_NULL)


@pytest.mark.parametrize("N,K", [(0, 256), (-1, 256), (4, 0), (4, 255), (4, 300), (4, 128),
                                 (4, 32768 + 256), (1 << 31, 256), (1 << 40, 32768)])
def test_bad_shapes(N, K):
    L = gq.lib()
    _rejected(L.q4k_gemv(A, B, C, N, K, None), gq.ERR_SHAPE)
    _rejected(L.q6k_gemv(A, B, C, N, K, None), gq.ERR_SHAPE)
    _rejected(L.q4k_q8_gemv(A, B, C, D, N, K, None), gq.ERR_SHAPE)
    _rejected(L.swiglu_gemv(A, B, C, D, N, K, None), gq.ERR_SHAPE)
    _rejected(L.lm_head_argmax(A, B, C, D, E, 1 << 20, N, K, None), gq.ERR_SHAPE)
    _rejected(L.lm_head_argmax_timed(A, B, C, D, E, 1 << 20, N, K, None, A, B), gq.ERR_SHAPE)
    _rejected(L.gemvq_q4k_q8_isums(A, B, C, N, K, None), gq.ERR_SHAPE)
    _rejected(L.q6k_q8_gemv(A, B, C, D, N, K, None), gq.ERR_SHAPE)
    _rejected(L.gemvq_q6k_q8_isums(A, B, C, N, K, None), gq.ERR_SHAPE)


def test_q8_bad_shapes():
    L = gq.lib()
    for K in (0, 16, 31, 33, 65536 + 32):
        _rejected(L.q8_quantize(A, B, C, K, None), gq.ERR_SHAPE)


def test_alignment():
    L = gq.lib()
    _rejected(L.q4k_gemv(A + 4, B, C, 4, 256, None), gq.ERR_ALIGN)      # Q4_K weights need 16 B
    _rejected(L.q4k_gemv(A, B + 4, C, 4, 256, None), gq.ERR_ALIGN)      # x needs 16 B
    _rejected(L.q4k_gemv(A, B, C + 2, 4, 256, None), gq.ERR_ALIGN)      # y needs 4 B
    _rejected(L.q6k_gemv(A + 2, B, C, 4, 256, None), gq.ERR_ALIGN)      # Q6_K weights need 4 B
    _rejected(L.q8_quantize(A, B + 8, C, 256, None), gq.ERR_ALIGN)
    _rejected(L.q8_quantize(A, B, C + 2, 256, None), gq.ERR_ALIGN)
    _rejected(L.q4k_q8_gemv(A, B + 1, C, D, 4, 256, None), gq.ERR_ALIGN)
    _rejected(L.swiglu_gemv(A, B + 8, C, D, 4, 256, None), gq.ERR_ALIGN)
    _rejected(L.lm_head_argmax(A, B, C, D, E + 16, 1 << 20, 4, 256, None), gq.ERR_ALIGN)   # workspace 256 B
    _rejected(L.lm_head_argmax(A, B, C + 1, D, E, 1 << 20, 4, 256, None), gq.ERR_ALIGN)
    _rejected(L.lm_head_argmax_timed(A, B, C + 1, D, E, 1 << 20, 4, 256, None, None, None), gq.ERR_ALIGN)
    _rejected(L.gemvq_q4k_q8_isums(A, B, C + 2, 4, 256, None), gq.ERR_ALIGN)
    _rejected(L.q6k_q8_gemv(A + 2, B, C, D, 4, 256, None), gq.ERR_ALIGN)    # Q6_K weights need 4 B
    _rejected(L.q6k_q8_gemv(A, B + 8, C, D, 4, 256, None), gq.ERR_ALIGN)    # xq needs 16 B
    _rejected(L.q6k_q8_gemv(A, B, C + 2, D, 4, 256, None), gq.ERR_ALIGN)    # xd needs 4 B
    _rejected(L.gemvq_q6k_q8_isums(A, B, C + 2, 4, 256, None), gq.ERR_ALIGN)
    _rejected(L.lm_head_argmax_masked(A, B, C + 2, D, None, E, 1 << 20, 4, 256, None), gq.ERR_ALIGN)


def test_workspace_too_small():
    L = gq.lib()
    need = gq.lm_head_argmax_ws_bytes(4, 256)
    _rejected(L.lm_head_argmax(A, B, C, D, E, need - 1, 4, 256, None), gq.ERR_WORKSPACE)
    _rejected(L.lm_head_argmax(A, B, C, None, E, 0, 4, 256, None), gq.ERR_WORKSPACE)
    _rejected(L.lm_head_argmax_timed(A, B, C, D, E, need - 1, 4, 256, None, A, B), gq.ERR_WORKSPACE)


def test_aliasing():
    L = gq.lib()
    N, K = 64, 512
    wbytes = N * (K // 256) * 144
    _rejected(L.q4k_gemv(A, B, A + 64, N, K, None), gq.ERR_ALIAS)               # y inside W
    _rejected(L.q4k_gemv(A, B, B + 4 * (K - 1), N, K, None), gq.ERR_ALIAS)      # y overlaps the end of x
    _rejected(L.q4k_gemv(A, B, A + wbytes - 4, N, K, None), gq.ERR_ALIAS)
    _rejected(L.q6k_gemv(A, B, B, N, K, None), gq.ERR_ALIAS)
    _rejected(L.swiglu_gemv(A, C, B, C + 16, N, K, None), gq.ERR_ALIAS)         # h inside Wu
    _rejected(L.q8_quantize(A, A + 16, C, K, None), gq.ERR_ALIAS)               # xq inside x
    _rejected(L.q8_quantize(A, B, B + 16, K, None), gq.ERR_ALIAS)               # xd inside xq
    _rejected(L.q4k_q8_gemv(A, B, C, C, N, K, None), gq.ERR_ALIAS)              # y over xd
    ws = gq.lm_head_argmax_ws_bytes(N, K)
    _rejected(L.lm_head_argmax(A, B, E + 8, None, E, ws, N, K, None), gq.ERR_ALIAS)   # idx inside ws
    _rejected(L.lm_head_argmax(A, B, C, C, E, ws, N, K, None), gq.ERR_ALIAS)          # max == idx
    _rejected(L.lm_head_argmax(A, B, C, None, A + 256, ws, N, K, None), gq.ERR_ALIAS)  # ws inside W
    _rejected(L.lm_head_argmax_masked(A, B, C, C, None, E, ws, N, K, None), gq.ERR_ALIAS)   # idx over the mask
    _rejected(L.lm_head_argmax_masked(A, B, E + 64, C, None, E, ws, N, K, None), gq.ERR_ALIAS)  # mask inside ws
    _rejected(L.gemvq_q4k_q8_isums(A, B, B, N, K, None), gq.ERR_ALIAS)
    _rejected(L.q6k_q8_gemv(A, B, C, B + 16, N, K, None), gq.ERR_ALIAS)         # y inside xq
    _rejected(L.q6k_q8_gemv(A, B, C, A + 100, N, K, None), gq.ERR_ALIAS)        # y inside W
    _rejected(L.gemvq_q6k_q8_isums(A, B, A, N, K, None), gq.ERR_ALIAS)


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    W = torch.zeros(144, dtype=torch.uint8)
    x = torch.zeros(256, dtype=torch.float32)
    with pytest.raises(ValueError):
        gq.q4k_gemv(W, x, 1, 256)


def _arr(ctype, vals):
    return ctypes.cast((ctype * len(vals))(*vals), ctypes.c_void_p)


def test_multi_rejections():
    L = gq.lib()
    P, I = ctypes.c_void_p, ctypes.c_int64
    W3 = _arr(P, [A, A + (1 << 24), A + (2 << 24)])
    Y3 = _arr(P, [C, C + (1 << 20), C + (2 << 20)])
    N3 = _arr(I, [64, 32, 32])
    _rejected(L.q4k_gemv_multi(None, N3, Y3, None, 3, B, 2560, None), gq.ERR_NULL)
    _rejected(L.q4k_gemv_multi(W3, N3, Y3, None, 3, None, 2560, None), gq.ERR_NULL)
    _rejected(L.q4k_gemv_multi(_arr(P, [A, None, A]), N3, Y3, None, 3, B, 2560, None), gq.ERR_NULL)
    _rejected(L.q4k_gemv_multi(W3, N3, Y3, None, 0, B, 2560, None), gq.ERR_SHAPE)
    _rejected(L.q4k_gemv_multi(W3, N3, Y3, None, 5, B, 2560, None), gq.ERR_SHAPE)
    _rejected(L.q4k_gemv_multi(W3, _arr(I, [64, 0, 32]), Y3, None, 3, B, 2560, None), gq.ERR_SHAPE)
    _rejected(L.q4k_gemv_multi(W3, N3, Y3, None, 3, B, 14336 + 256, None), gq.ERR_SHAPE)   # x too big for LDS
    _rejected(L.q4k_gemv_multi(W3, N3, Y3, None, 3, B + 4, 2560, None), gq.ERR_ALIGN)
    _rejected(L.q4k_gemv_multi(W3, N3, _arr(P, [C, C + 2, C + 4096]), None, 3, B, 2560, None), gq.ERR_ALIGN)
    _rejected(L.q4k_gemv_multi(W3, N3, _arr(P, [C, C + 128, C + 4096]), None, 3, B, 2560, None), gq.ERR_ALIAS)  # y0/y1
    _rejected(L.q4k_gemv_multi(W3, N3, _arr(P, [A + 64, C + 4096, C + 8192]), None, 3, B, 2560, None), gq.ERR_ALIAS)
    R3 = _arr(P, [None, C, None])      # residual of matrix 1 overlaps y[0]
    _rejected(L.q4k_gemv_multi(W3, N3, Y3, R3, 3, B, 2560, None), gq.ERR_ALIAS)


def test_swiglu_q8_rejections():
    L = gq.lib()
    N, K = 64, 512
    ws = gq.swiglu_q8_ws_bytes(N)
    assert ws >= N * 4 + (N // 32) * 4 and gq.swiglu_q8_ws_bytes(33) == 0 and gq.swiglu_q8_ws_bytes(0) == 0
    ok = dict(Wg=A, Wu=B, x=C, h=None, hq=D, hd=D + 4096, ws=E, wsb=ws, N=N, K=K)

    def call(**kw):
        a = dict(ok, **kw)
        return L.swiglu_q8_gemv(a["Wg"], a["Wu"], a["x"], a["h"], a["hq"], a["hd"], a["ws"], a["wsb"],
                                a["N"], a["K"], None)
    _rejected(call(hq=None), gq.ERR_NULL)
    _rejected(call(ws=None), gq.ERR_NULL)
    _rejected(call(N=48), gq.ERR_SHAPE)                    # N % 32 != 0
    _rejected(call(K=300), gq.ERR_SHAPE)
    _rejected(call(wsb=ws - 1), gq.ERR_WORKSPACE)
    _rejected(call(hq=D + 8), gq.ERR_ALIGN)                # hq needs 16 B
    _rejected(call(hd=D + 4096 + 2), gq.ERR_ALIGN)
    _rejected(call(ws=E + 128), gq.ERR_ALIGN)              # workspace 256 B
    _rejected(call(h=C + (1 << 20) + 2), gq.ERR_ALIGN)
    _rejected(call(x=C + 4), gq.ERR_ALIGN)
    _rejected(call(hq=A + 64), gq.ERR_ALIAS)               # hq inside Wg
    _rejected(call(hd=D + 16), gq.ERR_ALIAS)               # hd inside hq
    _rejected(call(h=E + 256), gq.ERR_ALIAS)               # h inside the workspace
    _rejected(call(ws=C), gq.ERR_ALIAS)                    # workspace over x


def test_rms_norm_q8_rejections():
    L = gq.lib()
    K = 256
    _rejected(L.rms_norm_q8(None, B, 1e-5, None, D, D + 4096, K, None), gq.ERR_NULL)
    _rejected(L.rms_norm_q8(A, B, 1e-5, None, None, D + 4096, K, None), gq.ERR_NULL)
    _rejected(L.add_rms_norm_q8(A, None, B, 1e-5, C, None, D, D + 4096, K, None), gq.ERR_NULL)
    _rejected(L.add_rms_norm_q8(A, C, B, 1e-5, None, None, D, D + 4096, K, None), gq.ERR_NULL)
    for bad_k in (0, 16, 33, 32768 + 32):
        _rejected(L.rms_norm_q8(A, B, 1e-5, None, D, D + 4096, bad_k, None), gq.ERR_SHAPE)
    for bad_eps in (-1e-6, float("nan"), float("inf")):
        _rejected(L.rms_norm_q8(A, B, bad_eps, None, D, D + 4096, K, None), gq.ERR_VALUE)
    _rejected(L.rms_norm_q8(A + 2, B, 1e-5, None, D, D + 4096, K, None), gq.ERR_ALIGN)
    _rejected(L.rms_norm_q8(A, B + 4, 1e-5, None, D, D + 4096, K, None), gq.ERR_ALIGN)       # w needs 16 B
    _rejected(L.rms_norm_q8(A, B, 1e-5, E + 8, D, D + 4096, K, None), gq.ERR_ALIGN)          # y needs 16 B
    _rejected(L.add_rms_norm_q8(A, C + 4, B, 1e-5, E, None, D, D + 4096, K, None), gq.ERR_ALIGN)  # r
    _rejected(L.add_rms_norm_q8(A, C, B, 1e-5, E + 4, None, D, D + 4096, K, None), gq.ERR_ALIGN)  # res
    _rejected(L.rms_norm_q8(A, B, 1e-5, None, D + 4, D + 4096, K, None), gq.ERR_ALIGN)   # xq needs 16 B
    _rejected(L.rms_norm_q8(A, B, 1e-5, None, D, D + 4098, K, None), gq.ERR_ALIGN)
    _rejected(L.rms_norm_q8(A, B, 1e-5, A + 64, D, D + 4096, K, None), gq.ERR_ALIAS)     # y over x
    _rejected(L.rms_norm_q8(A, B, 1e-5, None, B + 16, D + 4096, K, None), gq.ERR_ALIAS)  # xq over w
    _rejected(L.rms_norm_q8(A, B, 1e-5, D + 64, D, D + 4096, K, None), gq.ERR_ALIAS)     # y over xq
    # the residual output may be x or r itself, but not a shifted copy of either
    _rejected(L.add_rms_norm_q8(A, C, B, 1e-5, A + 16, None, D, D + 4096, K, None), gq.ERR_ALIAS)
    _rejected(L.add_rms_norm_q8(A, C, B, 1e-5, C - 16, None, D, D + 4096, K, None), gq.ERR_ALIAS)
    _rejected(L.add_rms_norm_q8(A, C, B, 1e-5, B, None, D, D + 4096, K, None), gq.ERR_ALIAS)   # res over w
    # in place is allowed past the alias checks: make the call fail on alignment instead
    _rejected(L.add_rms_norm_q8(A, C, B, 1e-5, A, None, D + 4, D + 4096, K, None), gq.ERR_ALIGN)
    _rejected(L.add_rms_norm_q8(A, C, B, 1e-5, C, None, D + 4, D + 4096, K, None), gq.ERR_ALIGN)


def test_batch_rejections():
    L = gq.lib()
    for fn in (L.q4k_q8_gemv_batch, L.q6k_q8_gemv_batch):
        _rejected(fn(None, B, C, D, 4, 256, 2, None), gq.ERR_NULL)
        _rejected(fn(A, B, C, None, 4, 256, 2, None), gq.ERR_NULL)
        for m in (0, -1, 9):
            _rejected(fn(A, B, C, D, 4, 256, m, None), gq.ERR_SHAPE)
        _rejected(fn(A, B, C, D, 4, 300, 2, None), gq.ERR_SHAPE)
        _rejected(fn(A, B, C, D, (1 << 31) - 1, 256, 2, None), gq.ERR_SHAPE)   # N * m overflows
        _rejected(fn(A, B + 4, C, D, 4, 256, 2, None), gq.ERR_ALIGN)            # xq needs 16 B
        _rejected(fn(A, B, C + 2, D, 4, 256, 2, None), gq.ERR_ALIGN)
        _rejected(fn(A, B, C, D + 2, 4, 256, 2, None), gq.ERR_ALIGN)
        _rejected(fn(A, B, C, B + 256, 4, 256, 2, None), gq.ERR_ALIAS)         # y inside the second vector
        _rejected(fn(A, B, C, C + 16, 4, 256, 2, None), gq.ERR_ALIAS)          # y over the second scales
    _rejected(L.q4k_q8_gemv_batch(A + 4, B, C, D, 4, 256, 2, None), gq.ERR_ALIGN)   # Q4_K weights need 16 B
    _rejected(L.q6k_q8_gemv_batch(A + 2, B, C, D, 4, 256, 2, None), gq.ERR_ALIGN)   # Q6_K weights need 4 B


def test_lm_head_argmax_noalloc_rejections():
    """The no-allocation lm_head entry point checks its arguments like
    lm_head_argmax (no workspace argument), before any HIP call."""
    L = gq.lib()
    _rejected(L.lm_head_argmax_noalloc(None, B, C, None, 4, 256, None), gq.ERR_NULL)
    _rejected(L.lm_head_argmax_noalloc(A, None, C, None, 4, 256, None), gq.ERR_NULL)
    _rejected(L.lm_head_argmax_noalloc(A, B, None, D, 4, 256, None), gq.ERR_NULL)
    _rejected(L.lm_head_argmax_noalloc(A, B, C, None, 0, 256, None), gq.ERR_SHAPE)
    _rejected(L.lm_head_argmax_noalloc(A, B, C, None, 4, 300, None), gq.ERR_SHAPE)
    _rejected(L.lm_head_argmax_noalloc(A, B, C, None, 4, 65536, None), gq.ERR_SHAPE)
    _rejected(L.lm_head_argmax_noalloc(A + 2, B, C, None, 4, 256, None), gq.ERR_ALIGN)
    _rejected(L.lm_head_argmax_noalloc(A, B + 4, C, None, 4, 256, None), gq.ERR_ALIGN)
    _rejected(L.lm_head_argmax_noalloc(A, B, C + 1, None, 4, 256, None), gq.ERR_ALIGN)
    _rejected(L.lm_head_argmax_noalloc(A, B, C, D + 2, 4, 256, None), gq.ERR_ALIGN)
    _rejected(L.lm_head_argmax_noalloc(A, B, A + 64, None, 4, 256, None), gq.ERR_ALIAS)   # idx inside W
    _rejected(L.lm_head_argmax_noalloc(A, B, B + 16, None, 4, 256, None), gq.ERR_ALIAS)   # idx inside x
    _rejected(L.lm_head_argmax_noalloc(A, B, C, C, 4, 256, None), gq.ERR_ALIAS)           # max == idx


def test_stream_read_rejections():
    L = gq.lib()
    _rejected(L.gemvq_stream_read(None, 1024, 256, 1024, C, None), gq.ERR_NULL)
    _rejected(L.gemvq_stream_read(A, 1024, 256, 1024, None, None), gq.ERR_NULL)
    _rejected(L.gemvq_stream_read(A, 0, 256, 1024, C, None), gq.ERR_SHAPE)
    _rejected(L.gemvq_stream_read(A, 1000, 256, 1024, C, None), gq.ERR_SHAPE)
    _rejected(L.gemvq_stream_read(A, 1024, 0, 1024, C, None), gq.ERR_SHAPE)
    _rejected(L.gemvq_stream_read(A, 1024, 256, 512, C, None), gq.ERR_SHAPE)
    _rejected(L.gemvq_stream_read(A, 1024, 256, 0, C, None), gq.ERR_SHAPE)
    _rejected(L.gemvq_stream_read(A + 8, 1024, 256, 1024, C, None), gq.ERR_ALIGN)
    _rejected(L.gemvq_stream_read(A, 1024, 256, 1024, A + 512, None), gq.ERR_ALIAS)


def test_q4k_q8_gemv_from_f32_rejections():
    L = gq.lib()
    N, K = 64, 512
    _rejected(L.q4k_q8_gemv_from_f32(None, B, C, D, E, N, K, None), gq.ERR_NULL)
    _rejected(L.q4k_q8_gemv_from_f32(A, B, None, D, E, N, K, None), gq.ERR_NULL)
    _rejected(L.q4k_q8_gemv_from_f32(A, B, C, D, None, N, K, None), gq.ERR_NULL)
    _rejected(L.q4k_q8_gemv_from_f32(A, B, C, D, E, N, 300, None), gq.ERR_SHAPE)
    _rejected(L.q4k_q8_gemv_from_f32(A + 4, B, C, D, E, N, K, None), gq.ERR_ALIGN)
    _rejected(L.q4k_q8_gemv_from_f32(A, B + 4, C, D, E, N, K, None), gq.ERR_ALIGN)
    _rejected(L.q4k_q8_gemv_from_f32(A, B, C + 8, D, E, N, K, None), gq.ERR_ALIGN)
    _rejected(L.q4k_q8_gemv_from_f32(A, B, C, D + 2, E, N, K, None), gq.ERR_ALIGN)
    _rejected(L.q4k_q8_gemv_from_f32(A, B, C, D, B + 16, N, K, None), gq.ERR_ALIAS)      # y inside x
    _rejected(L.q4k_q8_gemv_from_f32(A, B, A + 256, D, E, N, K, None), gq.ERR_ALIAS)     # xq inside W
    _rejected(L.q4k_q8_gemv_from_f32(A, B, C, C + 16, E, N, K, None), gq.ERR_ALIAS)      # xd inside xq
    _rejected(L.q4k_q8_gemv_from_f32(A, B, C, D, D, N, K, None), gq.ERR_ALIAS)           # y over xd
