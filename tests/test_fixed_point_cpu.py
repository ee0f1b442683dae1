"""CPU emulation of the fixed-point activation dot products (no GPU), with an
explicit error bound against the f64 oracle.

Several kernels hold the f32 activation in fixed point: each aligned 64-value
part x_P is scaled by 2^e with e = 22 - E, E the binary exponent of the
part's largest |x| (frexp: max|x| = f * 2^E, 0.5 <= f < 1), and rounded to
an integer X = rint(x * 2^e), |X| <= 2^22.  X is split into a signed high
byte and unsigned middle and low bytes (X = 65536 hi + 256 mid + lo), so a
dot product with small unsigned quants is three exact integer dot products.
The only approximation is the rounding of X: |x - X 2^-e| <= 2^(E-23), which
is at most 2^-22 of the part's largest |x|; the rest is ordinary f32
rounding of the joined sums.  The emulation below follows those steps in
numpy (written from the description above, not from the kernels) and checks,
row by row,

    |y_fx - y| <= sum_k |w_k| 2^-22 pm_k + (4 nb + 40) 2^-24 S,
    S = sum_k (|d sc q_k| + |dmin m| or |d sc 32|) (|x_k| + 2^-22 pm_k),

with y the oracle's f64 GEMV, pm_k the largest |x| of element k's part, and
S the magnitudes the f32 arithmetic works on (the a-priori bound of a chain
of at most 4 nb + 40 f32 roundings).  Inputs: N(0,1) and the wide-range
activation (a 1e4 outlier in every part, tiny and zero parts).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.kquant_encode import q4k_matrix_from_fields, q6k_matrix_from_fields, random_q4k_fields, random_q6k_fields

F32 = np.float32
U = 2.0 ** -24


def fixed_point_parts(x):
    """(X int64 [K], e int [K/64], pm f64 [K]) of the per-part fixed point."""
    x = np.asarray(x, np.float32)
    parts = x.reshape(-1, 64)
    m = np.max(np.abs(parts), axis=1)
    _, E = np.frexp(m.astype(np.float64))
    e = np.where(m > 0, 22 - E, 0).astype(np.int64)
    X = np.rint(parts.astype(np.float64) * np.exp2(e)[:, None]).astype(np.int64)
    assert np.all(np.abs(X) <= 2 ** 22)
    pm = np.repeat(m.astype(np.float64), 64)
    return X.reshape(-1), e, pm


def byte_split(X):
    hi = X >> 16                       # arithmetic shift: signed high byte
    mid = (X >> 8) & 255
    lo = X & 255
    assert np.all((hi >= -128) & (hi <= 127))
    assert np.array_equal(65536 * hi + 256 * mid + lo, X)
    return hi, mid, lo


def f32_sum(v):
    acc = F32(0)
    for t in np.asarray(v, np.float32):
        acc = F32(acc + t)
    return acc


def emulate_q4k(fields, x, N, K):
    """Fixed-point Q4_K GEMV: per part (64 values: sub-blocks 2c and 2c+1),
    exact integer sums of the nibbles against hi/mid/lo, joined in f32,
    scaled by d*sc and 2^-e; the min term from f32 sums of x."""
    d, dmin, sc, mn, q = fields
    nb = K // 256
    X, e, _ = fixed_point_parts(x)
    hi, mid, lo = byte_split(X)
    xf = np.asarray(x, np.float32)
    dv = d.view(np.float16).astype(np.float32)
    mv = dmin.view(np.float16).astype(np.float32)
    y = np.zeros(N, np.float32)
    for n in range(N):
        acc = F32(0)
        for b in range(nb):
            blk = n * nb + b
            for c in range(4):
                P = 4 * b + c
                vals = []
                for j in (2 * c, 2 * c + 1):
                    sl = slice(256 * b + 32 * j, 256 * b + 32 * j + 32)
                    qq = q[blk, 32 * j:32 * j + 32].astype(np.int64)
                    sh = int(np.dot(qq, hi[sl]))
                    smid = int(np.dot(qq, mid[sl])) * 256 + int(np.dot(qq, lo[sl]))
                    vals.append(F32(F32(sh) * F32(65536) + F32(smid)))
                dl, dh = F32(dv[blk] * F32(sc[blk, 2 * c])), F32(dv[blk] * F32(sc[blk, 2 * c + 1]))
                ml, mh = F32(mv[blk] * F32(mn[blk, 2 * c])), F32(mv[blk] * F32(mn[blk, 2 * c + 1]))
                s_lo = f32_sum(xf[256 * b + 64 * c: 256 * b + 64 * c + 32])
                s_hi = f32_sum(xf[256 * b + 64 * c + 32: 256 * b + 64 * c + 64])
                t = F32(np.ldexp(F32(F32(dl * vals[0]) + F32(dh * vals[1])), -int(e[P])))
                t = F32(t - F32(F32(ml * s_lo) + F32(mh * s_hi)))
                acc = F32(acc + t)
        y[n] = acc
    return y


def emulate_q6k(fields, x, N, K):
    """Fixed-point Q6_K GEMV: per 16-value group exact sums of the 6-bit
    quants against hi/mid/lo joined in f32, the -32 offset taken off with the
    group's f32 sum scaled the same way, times the int8 scale; per part
    scaled back by 2^-e and d."""
    d, sc, q = fields
    nb = K // 256
    X, e, _ = fixed_point_parts(x)
    hi, mid, lo = byte_split(X)
    xf = np.asarray(x, np.float32)
    dv = d.view(np.float16).astype(np.float32)
    y = np.zeros(N, np.float32)
    for n in range(N):
        acc = F32(0)
        for b in range(nb):
            blk = n * nb + b
            for P in range(4 * b, 4 * b + 4):          # a part: 64 consecutive values, 4 groups
                t = F32(0)
                for g in range(4 * (P - 4 * b), 4 * (P - 4 * b) + 4):
                    sl = slice(256 * b + 16 * g, 256 * b + 16 * g + 16)
                    qq = q[blk, 16 * g:16 * g + 16].astype(np.int64)
                    sh = int(np.dot(qq, hi[sl]))
                    smid = int(np.dot(qq, mid[sl])) * 256 + int(np.dot(qq, lo[sl]))
                    v = F32(F32(sh) * F32(65536) + F32(smid))
                    off = F32(F32(-32) * F32(np.ldexp(f32_sum(xf[sl]), int(e[P]))))
                    t = F32(t + F32(F32(sc[blk, g]) * F32(v + off)))
                acc = F32(acc + F32(dv[blk] * F32(np.ldexp(t, -int(e[P])))))
        y[n] = acc
    return y


def bound(abs_w, mag, x, nb):
    """Row bound: sum |w| 2^-22 pm + (4 nb + 40) 2^-24 sum mag (|x| + 2^-22 pm)."""
    _, _, pm = fixed_point_parts(x)
    ax = np.abs(np.asarray(x, np.float64))
    return abs_w @ (2.0 ** -22 * pm) + (4 * nb + 40) * U * (mag @ (ax + 2.0 ** -22 * pm))


@pytest.mark.parametrize("wide", [False, True])
@pytest.mark.parametrize("nb", [1, 3])
def test_q4k_fixed_point_within_bound(nb, wide):
    N, K = 6, 256 * nb
    rng = np.random.default_rng(61 + 7 * nb + wide)
    fields = random_q4k_fields(rng, N * nb)
    raw, w = q4k_matrix_from_fields(fields, N, K)
    x = synth.activation_wide_range(rng, K) if wide else synth.activation(rng, K)
    yhat = oracle.q4k_gemv(raw.reshape(-1), x, N, K)
    y = emulate_q4k(fields, x, N, K)
    d, dmin, sc, mn, q = fields
    dv = d.view(np.float16).astype(np.float64)[:, None]
    mv = dmin.view(np.float16).astype(np.float64)[:, None]
    mag = (dv * np.repeat(sc, 32, axis=1) * q + mv * np.repeat(mn, 32, axis=1)).reshape(N, K)
    B = bound(np.abs(w), mag, x, nb)
    err = np.abs(y.astype(np.float64) - yhat)
    assert np.all(err <= B), (err / B).max()
    scale = np.abs(w) @ np.abs(x.astype(np.float64))
    # the bound itself is inside the conditioned bound of the GPU parity tests
    # (1e-4 of sum |w x|), twenty times inside the 2e-3 tolerance
    assert (B / scale).max() <= 1e-4, (B / scale).max()
    assert (err / scale).max() <= 1e-4


@pytest.mark.parametrize("wide", [False, True])
@pytest.mark.parametrize("nb", [1, 3])
def test_q6k_fixed_point_within_bound(nb, wide):
    N, K = 6, 256 * nb
    rng = np.random.default_rng(71 + 7 * nb + wide)
    fields = random_q6k_fields(rng, N * nb)
    raw, w = q6k_matrix_from_fields(fields, N, K)
    x = synth.activation_wide_range(rng, K) if wide else synth.activation(rng, K)
    yhat = oracle.q6k_gemv(raw.reshape(-1), x, N, K)
    y = emulate_q6k(fields, x, N, K)
    d, sc, q = fields
    dv = d.view(np.float16).astype(np.float64)[:, None]
    scw = np.abs(np.repeat(sc, 16, axis=1))
    mag = (dv * scw * (q + 32)).reshape(N, K)
    B = bound(np.abs(w), mag, x, nb)
    err = np.abs(y.astype(np.float64) - yhat)
    assert np.all(err <= B), (err / B).max()
    # the -32 offset is taken off as 32 * sum x, so S (and the a-priori bound)
    # can be far above sum |w x| for a row whose largest |x| meets a weight of
    # quant ~32; the error itself stays inside the GPU tests' conditioned bound
    scale = np.abs(w) @ np.abs(x.astype(np.float64))
    assert (err / scale).max() <= 1e-4, (err / scale).max()


def test_rounding_error_is_at_most_2_pow_minus_22_of_part_max():
    """|x - X 2^-e| <= 2^-22 max|x_P| on every element, and the bound is
    reached within a factor of two (it is not 2^-23 in general)."""
    rng = np.random.default_rng(5)
    x = np.concatenate([synth.activation_wide_range(rng, 4096), synth.activation(rng, 4096)])
    X, e, pm = fixed_point_parts(x)
    back = X.astype(np.float64) * np.exp2(-np.repeat(e, 64))
    err = np.abs(back - x.astype(np.float64))
    nz = pm > 0
    assert np.all(err[nz] <= 2.0 ** -22 * pm[nz])
    assert np.all(err[~nz] == 0)
    assert (err[nz] / pm[nz]).max() > 2.0 ** -23 * 0.9
