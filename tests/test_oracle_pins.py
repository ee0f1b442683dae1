"""Pins of the CPU oracle against things other than itself (CPU only).

Each function of oracle/oracle.c is checked against at least one of: a
closed-form value worked by hand (tests/golden), a library routine (numpy's
float16 conversions, numpy matmul, numpy nanargmax, scipy expit), an
independent test-side encoder (tests/kquant_encode.py), brute force on tiny
inputs, or an invariant of the definition.  The cases are chosen so that a
dropped term, a wrong sign, a wrong index or a transposed operand in the
oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle
from tests.kquant_encode import (f16_bits, pack_q4k, pack_q6k, q4k_matrix_from_fields,
                                 q6k_matrix_from_fields, random_q4k_fields, random_q6k_fields)


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ fp16
def test_fp16_closed_forms():
    table = {0x3C00: 1.0, 0x3800: 0.5, 0xC000: -2.0, 0x7BFF: 65504.0,
             0x0400: 2.0 ** -14, 0x0001: 2.0 ** -24, 0x0000: 0.0}
    for bits, val in table.items():
        assert oracle.fp16_to_f64(bits) == val
    neg0 = oracle.fp16_to_f64(0x8000)
    assert neg0 == 0.0 and math.copysign(1.0, neg0) < 0
    assert oracle.fp16_to_f64(0x7C00) == math.inf
    assert oracle.fp16_to_f64(0xFC00) == -math.inf
    assert math.isnan(oracle.fp16_to_f64(0x7E00))


def test_fp16_decode_exhaustive_vs_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.fp16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_f32_to_fp16_rne_vs_numpy():
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(1000),
        rng.uniform(1e-3, 1e-2, 20000).astype(np.float32),
        (rng.standard_normal(5000) * 1e-6).astype(np.float32),   # subnormal fp16 range
        np.array([0.0, -0.0, 65504.0, 65519.0, 65520.0, 1e6, -1e6, 2.0 ** -24,
                  2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 6.1e-5, np.inf, -np.inf], np.float32),
    ])
    # exact ties of binary16 at several exponents: (2k+1)/2 ulp
    ties = []
    for e in (-24, -20, -14, -10, 0, 5):
        for m in (1, 2, 3, 1023, 2047):
            ties.append(np.float32(m * 2.0 ** e + 2.0 ** (e - 1)))
    vals = np.concatenate([vals, np.array(ties, np.float32)])
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_fp16_bits(v) for v in vals], np.uint16)
    assert np.array_equal(got, ref)
    assert oracle.f32_to_fp16_bits(np.float32(np.nan)) & 0x7C00 == 0x7C00


# ------------------------------------------------------------------ Q4_K
def test_q4k_worked_block(golden_dir):
    g = _golden(golden_dir, "q4k_worked_block.json")
    blk = np.frombuffer(bytes.fromhex(g["bytes_hex"]), np.uint8)
    w = oracle.q4k_decode_block(blk)
    for i, v in g["weights"].items():
        assert w[int(i)] == v, (i, w[int(i)], v)
    assert w.sum() == g["sum_all_ones"]
    y = oracle.q4k_gemv(blk, np.ones(256, np.float32), 1, 256)
    assert y[0] == g["sum_all_ones"]


def test_q4k_scale_packing_exhaustive():
    """Every (sc, m) in [0,63]^2 at every sub-block position survives
    encode (test side) -> decode (oracle)."""
    q = np.zeros(256, int)
    q[::32] = 1                         # weight 32j has q = 1, the rest 0
    one = f16_bits(1.0)                 # d = dmin = 1
    for j in range(8):
        for s in range(64):
            sc = [(j * 7 + 3) % 64] * 8
            mn = [(j * 5 + 11) % 64] * 8
            sc[j] = s
            blk_list = []
            for m in range(64):
                mn_j = list(mn)
                mn_j[j] = m
                blk_list.append((mn_j, pack_q4k(one, one, sc, mn_j, q)))
            for mn_j, blk in blk_list:
                w = oracle.q4k_decode_block(blk)
                # weight 32k has q=1: w = sc_k - m_k; weight 32k+1 has q=0: w = -m_k
                assert np.array_equal(w[1::32], -np.array(mn_j, float))
                assert np.array_equal(w[0::32], np.array(sc, float) - np.array(mn_j, float))


def test_q4k_random_roundtrip():
    rng = np.random.default_rng(1)
    fields = random_q4k_fields(rng, 64)
    blocks, w_ref = q4k_matrix_from_fields(fields, 64, 256)
    for i in range(64):
        assert np.array_equal(oracle.q4k_decode_block(blocks[i]), w_ref[i])


def test_q4k_special_blocks():
    zero = np.zeros(144, np.uint8)
    w = oracle.q4k_decode_block(zero)
    assert np.all(w == 0.0)
    rng = np.random.default_rng(2)
    x = rng.standard_normal(256).astype(np.float32)
    assert oracle.q4k_gemv(zero, x, 1, 256)[0] == 0.0
    # constant block: every q = c, sc = s, m = mu -> y = (d*s*c - dmin*mu) * sum(x)
    for c, s, mu, d, dm in [(15, 63, 63, 0.00999, 0.001), (7, 1, 0, 0.5, 0.25), (0, 5, 9, 0.125, 0.0625)]:
        db, dmb = f16_bits(d), f16_bits(dm)
        blk = pack_q4k(db, dmb, [s] * 8, [mu] * 8, [c] * 256)
        dv = float(np.uint16(db).view(np.float16))
        dmv = float(np.uint16(dmb).view(np.float16))
        wv = dv * s * c - dmv * mu
        assert np.all(oracle.q4k_decode_block(blk) == wv)
        ones = np.ones(256, np.float32)
        assert oracle.q4k_gemv(blk, ones, 1, 256)[0] == pytest.approx(256 * wv, rel=1e-15, abs=1e-12)


# ------------------------------------------------------------------ Q6_K
def test_q6k_worked_block(golden_dir):
    g = _golden(golden_dir, "q6k_worked_block.json")
    blk = np.frombuffer(bytes.fromhex(g["bytes_hex"]), np.uint8)
    w = oracle.q6k_decode_block(blk)
    for i, v in g["weights"].items():
        assert w[int(i)] == v, (i, w[int(i)], v)
    for i in g["negative_zero_indices"]:
        assert w[i] == 0.0 and np.signbit(w[i])
    assert w.sum() == g["sum_all_ones"]
    assert oracle.q6k_gemv(blk, np.ones(256, np.float32), 1, 256)[0] == g["sum_all_ones"]


def test_q6k_random_roundtrip():
    rng = np.random.default_rng(3)
    fields = random_q6k_fields(rng, 64)
    blocks, w_ref = q6k_matrix_from_fields(fields, 64, 256)
    for i in range(64):
        assert np.array_equal(oracle.q6k_decode_block(blocks[i]), w_ref[i])


def test_q6k_every_quant_value_every_position():
    """Each of the 64 quant values at each of the 256 positions decodes to
    d*sc*(q-32) with a distinct scale per 16-group (catches a wrong bit pair,
    nibble or group index)."""
    sc = [g - 8 if g != 8 else 9 for g in range(16)]   # 16 distinct nonzero scales
    for v in range(64):
        q = [(v + 13 * i) % 64 for i in range(256)]
        blk = pack_q6k(f16_bits(1.0), sc, q)
        w = oracle.q6k_decode_block(blk)
        exp = np.array([sc[i // 16] * (q[i] - 32) for i in range(256)], float)
        assert np.array_equal(w, exp)


def test_q6k_zero_quants_closed_form():
    sc = list(range(-8, 8))
    blk = pack_q6k(f16_bits(0.25), sc, [0] * 256)   # ql = qh = 0
    w = oracle.q6k_decode_block(blk)
    assert np.array_equal(w, np.array([-32 * 0.25 * sc[i // 16] for i in range(256)], float))


def test_q6k_block_size_matches_page_figure():
    # qualiaDB resident_decode.rs: 2520 B per 3072-wide Q6_K logits row
    assert 3072 // 256 * oracle.Q6K_BLOCK_BYTES == 2520


# ------------------------------------------------------------------ GEMV
@pytest.mark.parametrize("fmt", ["q4k", "q6k"])
def test_gemv_vs_numpy_matmul(fmt):
    rng = np.random.default_rng(4)
    N, K = 7, 768
    if fmt == "q4k":
        W, Wf = q4k_matrix_from_fields(random_q4k_fields(rng, N * K // 256), N, K)
        gemv = oracle.q4k_gemv
    else:
        W, Wf = q6k_matrix_from_fields(random_q6k_fields(rng, N * K // 256), N, K)
        gemv = oracle.q6k_gemv
    x = rng.standard_normal(K).astype(np.float32)
    y = gemv(W, x, N, K)
    ref = Wf @ x.astype(np.float64)
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13 * np.abs(Wf).sum())
    # one-hot activations extract columns exactly
    for k in (0, 1, 255, 256, 511, 767):
        e = np.zeros(K, np.float32)
        e[k] = 1.0
        assert np.array_equal(gemv(W, e, N, K), Wf[:, k])
    assert np.all(gemv(W, np.zeros(K, np.float32), N, K) == 0.0)
    # linearity: W(2x) = 2 W x exactly (power-of-two scaling)
    assert np.array_equal(gemv(W, 2 * x, N, K), 2 * y)


def test_q6k_gemv_f64x_matches_f32_path():
    rng = np.random.default_rng(5)
    N, K = 5, 512
    W, Wf = q6k_matrix_from_fields(random_q6k_fields(rng, N * K // 256), N, K)
    x = rng.standard_normal(K).astype(np.float32)
    assert np.array_equal(oracle.q6k_gemv_f64x(W, x.astype(np.float64), N, K),
                          oracle.q6k_gemv(W, x, N, K))


# ------------------------------------------------------------------ SwiGLU
def test_swiglu_vs_scipy_expit():
    rng = np.random.default_rng(6)
    N, K = 9, 512
    Wg, Wgf = q4k_matrix_from_fields(random_q4k_fields(rng, N * K // 256), N, K)
    Wu, Wuf = q4k_matrix_from_fields(random_q4k_fields(rng, N * K // 256), N, K)
    x = rng.standard_normal(K).astype(np.float32)
    h, g, u = oracle.swiglu(Wg, Wu, x, N, K)
    g_ref = Wgf @ x.astype(np.float64)
    u_ref = Wuf @ x.astype(np.float64)
    assert np.allclose(g, g_ref, rtol=1e-13, atol=1e-12)
    assert np.allclose(u, u_ref, rtol=1e-13, atol=1e-12)
    assert np.allclose(h, g_ref * u_ref * expit(g_ref), rtol=1e-12, atol=1e-12)
    # gate == up: h = g^2 * sigmoid(g)
    h2, g2, _ = oracle.swiglu(Wg, Wg, x, N, K)
    assert np.allclose(h2, g2 * g2 * expit(g2), rtol=1e-12, atol=1e-12)
    # silu(0) = 0: an all-zero gate row gives h = 0
    Wz = Wg.copy()
    Wz[0] = 0
    h3, g3, _ = oracle.swiglu(Wz, Wu, x, N, K)
    assert g3[0] == 0.0 and h3[0] == 0.0


def test_swiglu_sign_of_exponent():
    """Large positive gate passes through (silu(z) ~ z), large negative is
    suppressed (silu(z) ~ 0): catches e^{+z} in place of e^{-z}."""
    K = 256
    blk_pos = pack_q4k(f16_bits(1.0), f16_bits(0.0), [1] * 8, [0] * 8, [15] * 256)
    ones = np.ones(K, np.float32)
    h, g, u = oracle.swiglu(blk_pos, blk_pos, ones, 1, K)
    assert g[0] == 15 * 256 and h[0] == pytest.approx(g[0] * u[0], rel=1e-12)
    h, g, u = oracle.swiglu(blk_pos, blk_pos, -ones, 1, K)
    assert g[0] == -15 * 256 and abs(h[0]) < 1e-300


# ------------------------------------------------------------------ Q8
def test_q8_worked_blocks(golden_dir):
    g = _golden(golden_dir, "q8_worked_block.json")
    x = np.zeros(64, np.float32)
    for i, v in g["block_a"]["x_nonzero"].items():
        x[int(i)] = v
    q, d = oracle.q8_quantize(x)
    exp = np.zeros(32, np.int8)
    for i, v in g["block_a"]["expected_q_nonzero"].items():
        exp[int(i)] = v
    assert np.array_equal(q[:32], exp)
    assert d[0] == int(g["block_a"]["expected_scale_bits"], 16)
    assert np.all(q[32:] == 0) and d[1] == int(g["block_zero"]["expected_scale_bits"], 16)


def test_q8_invariants_and_numpy():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(32 * 400) * np.repeat(rng.uniform(0.01, 100, 400), 32)).astype(np.float32)
    x[:32] = 0.0
    q, d = oracle.q8_quantize(x)
    xb = x.reshape(-1, 32)
    qb = q.reshape(-1, 32).astype(np.int64)
    amax = np.abs(xb).max(axis=1)
    d32 = (amax / np.float32(127)).astype(np.float32)          # numpy f32 division (IEEE)
    assert np.array_equal(d, d32.astype(np.float16).view(np.uint16))
    assert np.all(np.abs(qb) <= 127)
    nz = amax > 0
    assert np.all(np.abs(qb[nz]).max(axis=1) == 127)
    assert np.all(qb[~nz] == 0)
    t = np.zeros_like(xb)
    t[nz] = (xb[nz] / d32[nz, None]).astype(np.float32)
    # nearest integer, ties away from zero
    frac = np.abs(t.astype(np.float64) - qb)
    assert np.all(frac <= 0.5)
    tie = frac == 0.5
    assert np.all(np.abs(qb[tie]) > np.abs(t[tie]))


def test_q8_rounding_ties_away_from_zero():
    x = np.zeros(32, np.float32)
    x[0] = 127.0
    x[1:9] = [0.5, -0.5, 1.5, -1.5, 2.5, -2.5, 126.5, -126.5]
    q, d = oracle.q8_quantize(x)
    assert list(q[1:9]) == [1, -1, 2, -2, 3, -3, 127, -127]


def test_q4k_q8_worked_dot(golden_dir):
    g = _golden(golden_dir, "q8_worked_block.json")["q4k_dot"]
    blk = np.frombuffer(bytes.fromhex(_golden(golden_dir, "q4k_worked_block.json")["bytes_hex"]), np.uint8)
    x = np.ones(256, np.float32)
    q, d = oracle.q8_quantize(x)
    assert np.all(d == int(g["expected_scale_bits"], 16)) and np.all(q == g["expected_q"])
    isums = oracle.q4k_q8_isums(blk, q, 1, 256)
    assert list(isums[0]) == g["expected_isums"]
    assert int(q[:32].astype(np.int64).sum()) == g["expected_qsum"]
    y = oracle.q4k_q8_gemv(blk, q, d, 1, 256)
    assert y[0] == g["expected_y"]


def test_q4k_q8_vs_numpy():
    rng = np.random.default_rng(9)
    N, K = 6, 1024
    fields = random_q4k_fields(rng, N * K // 256)
    W, Wf = q4k_matrix_from_fields(fields, N, K)
    x = (rng.standard_normal(K) * 3).astype(np.float32)
    q, d = oracle.q8_quantize(x)
    qraw = fields[4].reshape(N, K).astype(np.int64)
    isum_ref = (qraw * q.astype(np.int64)).reshape(N, K // 32, 32).sum(axis=2)
    assert np.array_equal(oracle.q4k_q8_isums(W, q, N, K), isum_ref)
    xdq = np.repeat(d.view(np.float16).astype(np.float64), 32) * q
    y = oracle.q4k_q8_gemv(W, q, d, N, K)
    assert np.allclose(y, Wf @ xdq, rtol=1e-13, atol=1e-12)


# ------------------------------------------------------------------ argmax
def test_argmax_vs_nanargmax_with_ties():
    rng = np.random.default_rng(10)
    for trial in range(300):
        n = int(rng.integers(1, 300))
        v = rng.integers(-5, 5, n).astype(np.float64)     # many exact ties
        if trial % 3 == 0:
            v[rng.integers(0, n, max(1, n // 10))] = np.nan
        if np.all(np.isnan(v)):
            assert oracle.argmax_first(v) == 0
        else:
            assert oracle.argmax_first(v) == int(np.nanargmax(v))
        f = v.astype(np.float32)
        if not np.all(np.isnan(f)):
            assert oracle.argmax_first(f) == int(np.nanargmax(f))


def test_argmax_edges():
    nan, inf = np.nan, np.inf
    assert oracle.argmax_first(np.array([nan, nan])) == 0
    assert oracle.argmax_first(np.array([nan, -inf, -inf])) == 1
    assert oracle.argmax_first(np.array([-0.0, 0.0])) == 0
    assert oracle.argmax_first(np.array([0.0, -0.0])) == 0
    assert oracle.argmax_first(np.array([-1.0, -0.0, 0.0])) == 1
    assert oracle.argmax_first(np.array([1.0, inf, nan, inf])) == 1
    assert oracle.argmax_first(np.array([3.0, 3.0, 3.0], np.float32)) == 0
    assert oracle.argmax_first(np.array([1.0, 2.0, 2.0], np.float32)) == 1


def test_top2_gap():
    assert oracle.top2_gap(np.array([1.0, 5.0, 3.0])) == 2.0
    assert oracle.top2_gap(np.array([5.0, 1.0, 5.0])) == 0.0


# ------------------------------------------------------------ masked argmax
def _np_masked_first_max(v, words, n):
    banned = np.unpackbits(np.asarray(words, np.uint32).view(np.uint8), bitorder="little")[:n].astype(bool)
    allowed = ~banned & ~np.isnan(v)
    if not allowed.any():
        return 0
    m = v[allowed].max()
    return int(np.flatnonzero(allowed & (v == m))[0])


def test_masked_argmax_vs_numpy():
    rng = np.random.default_rng(21)
    for n in (1, 31, 32, 33, 1000, 4097):
        for density in (0.0, 0.3, 0.9, 1.0):
            v = rng.standard_normal(n)
            v[rng.random(n) < 0.05] = np.nan
            if n > 10:
                v[n // 3] = v[2 * n // 3] = 10.0          # a tie
            bits = rng.random(n) < density
            words = np.packbits(np.concatenate([bits, np.zeros((-n) % 32, bool)]), bitorder="little").view(np.uint32)
            for dtype in (np.float64, np.float32):
                vv = v.astype(dtype)
                assert oracle.argmax_first_masked(vv, words) == _np_masked_first_max(vv, words, n), (n, density)


def test_masked_argmax_edges():
    v = np.array([1.0, 7.0, 7.0, 3.0, np.nan, 7.5])
    none = np.zeros(1, np.uint32)
    assert oracle.argmax_first_masked(v, none) == oracle.argmax_first(v) == 5
    assert oracle.argmax_first_masked(v, np.array([1 << 5], np.uint32)) == 1       # best banned: first of the tie
    assert oracle.argmax_first_masked(v, np.array([(1 << 5) | (1 << 1)], np.uint32)) == 2
    assert oracle.argmax_first_masked(v, np.array([0x3F], np.uint32)) == 0          # everything banned
    assert oracle.argmax_first_masked(v, np.array([0xFFFFFFFF], np.uint32)) == 0    # bits past n ignored
    assert oracle.argmax_first_masked(v, np.array([0x2F], np.uint32)) == 0          # only NaN left -> 0


# ------------------------------------------------------------------ Q6_K x Q8
def test_q6k_q8_vs_numpy():
    """Integer sums against the test-side encoder's raw quants, and the GEMV
    against numpy matmul over the dequantized activation."""
    rng = np.random.default_rng(21)
    N, K = 5, 1024
    fields = random_q6k_fields(rng, N * K // 256)
    W, Wf = q6k_matrix_from_fields(fields, N, K)
    x = (rng.standard_normal(K) * 2).astype(np.float32)
    q, d = oracle.q8_quantize(x)
    qraw = fields[2].reshape(N, K).astype(np.int64) - 32
    isum_ref = (qraw * q.astype(np.int64)).reshape(N, K // 16, 16).sum(axis=2)
    assert np.array_equal(oracle.q6k_q8_isums(W, q, N, K), isum_ref)
    xdq = np.repeat(d.view(np.float16).astype(np.float64), 32) * q
    y = oracle.q6k_q8_gemv(W, q, d, N, K)
    assert np.allclose(y, Wf @ xdq, rtol=1e-13, atol=1e-12)
    # the same GEMV through the f64-activation Q6_K path
    assert np.allclose(y, oracle.q6k_gemv_f64x(W, xdq, N, K), rtol=1e-14, atol=1e-12)


def test_q6k_q8_isums_offset_closed_form():
    """All quants 0 give -32 * (group sum of q8), all quants 63 give
    31 * (group sum): catches a missing or doubled -32 offset and a wrong
    group index (every group has a distinct activation sum)."""
    sc = [1] * 16
    xq = np.array([(g + 1) * (1 if i % 2 else 2) for g in range(16) for i in range(16)], np.int8)
    gsum = xq.astype(np.int64).reshape(16, 16).sum(axis=1)
    for v, mult in ((0, -32), (63, 31), (32, 0)):
        blk = pack_q6k(f16_bits(1.0), sc, [v] * 256)
        assert list(oracle.q6k_q8_isums(blk, xq, 1, 256)[0]) == list(mult * gsum)


def test_q6k_q8_worked_block(golden_dir):
    """A constant activation quantizes to 127 with scale fp16(1/127), so the
    Q6_K x Q8 dot of the worked block is its weight sum times 127 * that
    scale."""
    g = _golden(golden_dir, "q6k_worked_block.json")
    blk = np.frombuffer(bytes.fromhex(g["bytes_hex"]), np.uint8)
    q, d = oracle.q8_quantize(np.ones(256, np.float32))
    assert np.all(q == 127) and np.all(d == f16_bits(1.0 / 127.0))
    scale = float(np.array([d[0]], np.uint16).view(np.float16)[0])
    y = oracle.q6k_q8_gemv(blk, q, d, 1, 256)[0]
    assert y == pytest.approx(g["sum_all_ones"] * 127 * scale, rel=1e-15)


# ------------------------------------------------------------------ RMS norm
def test_rms_norm_vs_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(22)
    for K, eps in ((32, 1e-6), (1000, 1e-5), (8192, 0.0), (4096, 0.5)):
        x = (rng.standard_normal(K) * rng.uniform(0.01, 50)).astype(np.float32)
        w = rng.uniform(-2, 2, K).astype(np.float32)
        y = oracle.rms_norm(x, w, eps)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x.astype(np.float64)), (K,),
                                           torch.from_numpy(w.astype(np.float64)),
                                           float(np.float32(eps))).numpy()
        assert np.allclose(y, ref, rtol=1e-13, atol=0)


def test_rms_norm_closed_forms():
    K = 64
    ones = np.ones(K, np.float32)
    # constant vector: y = w * c / sqrt(c^2 + eps)
    for c, eps in ((3.0, 0.0), (0.5, 0.25), (-2.0, 1e-6)):
        y = oracle.rms_norm(np.full(K, c, np.float32), ones, eps)
        e = float(np.float32(eps))
        assert np.allclose(y, c / math.sqrt(c * c + e), rtol=1e-15)
    # eps = 0: unit root mean square, invariant under positive scaling, odd
    rng = np.random.default_rng(23)
    x = rng.standard_normal(K).astype(np.float32)
    y = oracle.rms_norm(x, ones, 0.0)
    assert math.sqrt(float(np.mean(y * y))) == pytest.approx(1.0, rel=1e-14)
    assert np.allclose(oracle.rms_norm(4 * x, ones, 0.0), y, rtol=1e-14)
    assert np.array_equal(oracle.rms_norm(-x, ones, 0.0), -y)
    # the weight multiplies elementwise (a one-hot weight keeps one element)
    w = np.zeros(K, np.float32)
    w[5] = 2.0
    yw = oracle.rms_norm(x, w, 0.0)
    assert yw[5] == pytest.approx(2 * y[5], rel=1e-15) and np.count_nonzero(yw) == 1
    # one-hot x: the only nonzero element becomes sqrt(K) (eps = 0)
    e1 = np.zeros(K, np.float32)
    e1[7] = 5.0
    assert oracle.rms_norm(e1, ones, 0.0)[7] == pytest.approx(math.sqrt(K), rel=1e-15)


def test_add_rms_norm():
    rng = np.random.default_rng(24)
    K = 512
    x = rng.standard_normal(K).astype(np.float32)
    r = rng.standard_normal(K).astype(np.float32)
    w = rng.uniform(0.5, 1.5, K).astype(np.float32)
    res, y = oracle.add_rms_norm(x, r, w, 1e-6)
    assert res.dtype == np.float32 and np.array_equal(res, x + r)   # one f32 rounding per element
    assert np.array_equal(y, oracle.rms_norm(x + r, w, 1e-6))
    # adding zero is the plain norm
    res0, y0 = oracle.add_rms_norm(x, np.zeros(K, np.float32), w, 1e-6)
    assert np.array_equal(res0, x) and np.array_equal(y0, oracle.rms_norm(x, w, 1e-6))


def test_rms_norm_q8_closed_forms():
    K = 256
    ones = np.ones(K, np.float32)
    # constant positive input, eps = 0: y = 1 everywhere -> q = 127, d = fp16(1/127)
    _, y, q, d = oracle.rms_norm_q8(np.full(K, 0.75, np.float32), ones, 0.0)
    assert np.all(y == 1.0) and np.all(q == 127) and np.all(d == f16_bits(1.0 / 127.0))
    # alternating signs: +-127
    alt = np.where(np.arange(K) % 2 == 0, 2.0, -2.0).astype(np.float32)
    _, y, q, d = oracle.rms_norm_q8(alt, ones, 0.0)
    assert np.array_equal(q, np.where(np.arange(K) % 2 == 0, 127, -127).astype(np.int8))
    # with a residual, the returned residual is the f32 sum and the codes are
    # those of the norm of that sum
    rng = np.random.default_rng(25)
    x = rng.standard_normal(K).astype(np.float32)
    r = rng.standard_normal(K).astype(np.float32)
    w = rng.uniform(0.5, 1.5, K).astype(np.float32)
    res, y, q, d = oracle.rms_norm_q8(x, w, 1e-5, r)
    assert np.array_equal(res, x + r)
    qq, dd = oracle.q8_quantize(oracle.rms_norm(x + r, w, 1e-5).astype(np.float32))
    assert np.array_equal(q, qq) and np.array_equal(d, dd)
    # dequantized codes stay within half a step of the normalized value
    step = np.repeat(d.view(np.float16).astype(np.float64), 32)
    # (codes are decided with the f32 scale; the stored fp16 scale is within
    # 2^-11 of it, which moves a code of at most 127 by 127 * 2^-11 steps)
    assert np.all(np.abs(q * step - y) <= (0.5 + 127 * 2.0 ** -11) * step * (1 + 1e-6))


def test_swiglu_q8_properties():
    """The quantized SwiGLU output: h is the plain SwiGLU, codes lie within
    half a step (plus the fp16 scale's rounding) of h, and the largest code
    of every nonzero block is +-127."""
    rng = np.random.default_rng(26)
    N, K = 64, 512
    Wg, _ = q4k_matrix_from_fields(random_q4k_fields(rng, N * K // 256), N, K)
    Wu, _ = q4k_matrix_from_fields(random_q4k_fields(rng, N * K // 256), N, K)
    Wg[40] = Wg[3]
    Wu[40] = Wu[3]
    x = rng.standard_normal(K).astype(np.float32)
    h, q, d = oracle.swiglu_q8(Wg, Wu, x, N, K)
    assert np.array_equal(h, oracle.swiglu(Wg, Wu, x, N, K)[0])
    step = np.repeat(d.view(np.float16).astype(np.float64), 32)
    assert np.all(np.abs(q * step - h) <= (0.5 + 127 * 2.0 ** -11) * step * (1 + 1e-6))
    assert np.all(np.abs(q.astype(np.int64)).reshape(-1, 32).max(axis=1) == 127)
    # rows 3 and 40 are equal by construction and sit in different blocks
    assert h[3] == h[40]


# ------------------------------------------------------------------ batched Q8 GEMV
@pytest.mark.parametrize("fmt", ["q4k", "q6k"])
def test_q8_gemv_batch_vs_numpy(fmt):
    """Y = W Xdq^T for m activation vectors at once, against numpy matmul
    over the independently decoded matrix (catches a transposed operand or a
    vector paired with the wrong scales)."""
    rng = np.random.default_rng(31)
    N, K, m = 6, 768, 5
    if fmt == "q4k":
        W, Wf = q4k_matrix_from_fields(random_q4k_fields(rng, N * K // 256), N, K)
    else:
        W, Wf = q6k_matrix_from_fields(random_q6k_fields(rng, N * K // 256), N, K)
    X = (rng.standard_normal((m, K)) * rng.uniform(0.1, 10, (m, 1))).astype(np.float32)
    qs, ds = zip(*[oracle.q8_quantize(X[j]) for j in range(m)])
    xq, xd = np.stack(qs), np.stack(ds)
    Y = oracle.q8_gemv_batch(fmt, W, xq, xd, N, K, m)
    assert Y.shape == (m, N)
    Xdq = np.repeat(xd.view(np.float16).astype(np.float64), 32, axis=1) * xq
    assert np.allclose(Y, (Wf @ Xdq.T).T, rtol=1e-13, atol=1e-12)
    # m = 1 is the single GEMV; reordering the vectors reorders the outputs
    single = {"q4k": oracle.q4k_q8_gemv, "q6k": oracle.q6k_q8_gemv}[fmt]
    assert np.array_equal(oracle.q8_gemv_batch(fmt, W, xq[:1], xd[:1], N, K, 1)[0], single(W, xq[0], xd[0], N, K))
    perm = [3, 0, 4, 1, 2]
    assert np.array_equal(oracle.q8_gemv_batch(fmt, W, xq[perm], xd[perm], N, K, m), Y[perm])


# ---------------------------------------------------------------------------
# Whole-matrix dequantizers and the multi-output GEMV.  They compose pinned
# block decoders and the pinned GEMV; these pins catch a slip in the
# composition itself: blocks placed in the wrong row or column, a reshape
# that transposes, a residual added to the wrong output or twice.


@pytest.mark.parametrize("N,nb", [(1, 1), (3, 2), (5, 7), (2, 38)])
def test_q4k_dequantize_vs_independent_encoder(N, nb):
    """The matrix the independent encoder builds from random fields (weights
    computed directly from the fields) equals the oracle's dequantization of
    the packed bytes, element for element and in the same N x K layout."""
    rng = np.random.default_rng(900 + 10 * N + nb)
    K = 256 * nb
    raw, w = q4k_matrix_from_fields(random_q4k_fields(rng, N * nb), N, K)
    got = oracle.q4k_dequantize(raw.reshape(-1), N, K)
    assert got.shape == (N, K)
    assert np.array_equal(got, w)


@pytest.mark.parametrize("N,nb", [(1, 1), (3, 2), (5, 7), (2, 38)])
def test_q6k_dequantize_vs_independent_encoder(N, nb):
    rng = np.random.default_rng(950 + 10 * N + nb)
    K = 256 * nb
    raw, w = q6k_matrix_from_fields(random_q6k_fields(rng, N * nb), N, K)
    got = oracle.q6k_dequantize(raw.reshape(-1), N, K)
    assert got.shape == (N, K)
    assert np.array_equal(got, w)


def test_dequantize_block_placement():
    """A block whose weights are all one known value, planted at (row r,
    column block c) of an otherwise all-zero matrix, shows up exactly at
    rows r, columns 256c .. 256c+255 (and nowhere else) -- in both formats,
    on a non-square block grid so a transposed reshape cannot pass."""
    N, nb = 3, 5
    K = 256 * nb
    for r, c in [(0, 0), (1, 3), (2, 4)]:
        # Q4_K: d = 1, every scale 1 and quant 7, min 0 -> every weight 7
        blk = pack_q4k(f16_bits(1.0), f16_bits(0.0), [1] * 8, [0] * 8, [7] * 256)
        W = np.zeros((N, nb, 144), np.uint8)
        W[r, c] = blk
        got = oracle.q4k_dequantize(W.reshape(-1), N, K)
        want = np.zeros((N, K))
        want[r, 256 * c:256 * (c + 1)] = 7.0
        assert np.array_equal(got, want), (r, c)
        # Q6_K: an all-zero block decodes to -32*d*sc = +-0 only with sc = 0;
        # plant d = 0.5, sc = 2, q = 40 -> every weight 0.5*2*8 = 8, and make
        # every other block all zero (quants 0 give -32*d*sc = -0.0 with d = 0)
        blk6 = pack_q6k(f16_bits(0.5), [2] * 16, [40] * 256)
        W6 = np.zeros((N, nb, 210), np.uint8)
        W6[r, c] = blk6
        got6 = oracle.q6k_dequantize(W6.reshape(-1), N, K)
        want6 = np.zeros((N, K))
        want6[r, 256 * c:256 * (c + 1)] = 8.0
        assert np.array_equal(got6, want6), (r, c)


def test_q4k_gemv_multi_composition():
    """y_i = W_i x + r_i: each output is the single-matrix GEMV of its own
    matrix plus its own residual (f32 widened to f64), matrices of different
    row counts, one without a residual."""
    rng = np.random.default_rng(971)
    K = 512
    Ns = [7, 3, 11]
    mats = [q4k_matrix_from_fields(random_q4k_fields(rng, n * K // 256), n, K) for n in Ns]
    x = rng.standard_normal(K).astype(np.float32)
    res = [rng.standard_normal(Ns[0]).astype(np.float32) * 100, None, rng.standard_normal(Ns[2]).astype(np.float32)]
    ys = oracle.q4k_gemv_multi([m[0].reshape(-1) for m in mats], Ns, x, K, res)
    assert [y.shape for y in ys] == [(n,) for n in Ns]
    for (raw, w), n, r, y in zip(mats, Ns, res, ys):
        want = w @ x.astype(np.float64) + (0.0 if r is None else r.astype(np.float64))
        assert np.allclose(y, want, rtol=1e-12, atol=1e-12)
        single = oracle.q4k_gemv(raw.reshape(-1), x, n, K)
        assert np.array_equal(y, single + (0.0 if r is None else r.astype(np.float64)))


def test_q4k_gemv_multi_residual_only_and_one_hot():
    """All-zero matrices give exactly the residual on its own output (and 0
    where none is given); a one-hot x extracts column k of each matrix."""
    rng = np.random.default_rng(972)
    K, Ns = 768, [4, 9]
    zero = [np.zeros(n * K // 256 * 144, np.uint8) for n in Ns]
    r0 = rng.standard_normal(Ns[0]).astype(np.float32)
    ys = oracle.q4k_gemv_multi(zero, Ns, rng.standard_normal(K).astype(np.float32), K, [r0, None])
    assert np.array_equal(ys[0], r0.astype(np.float64))
    assert np.array_equal(ys[1], np.zeros(Ns[1]))
    mats = [q4k_matrix_from_fields(random_q4k_fields(rng, n * K // 256), n, K) for n in Ns]
    for k in (0, 300, K - 1):
        e = np.zeros(K, np.float32)
        e[k] = 1.0
        ys = oracle.q4k_gemv_multi([m[0].reshape(-1) for m in mats], Ns, e, K)
        for (raw, w), y in zip(mats, ys):
            assert np.array_equal(y, w[:, k])
