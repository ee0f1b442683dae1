"""Test-side encoders for Q4_K / Q6_K super-blocks.

Written independently of ``oracle/oracle.c`` and of the HIP library, from the
layout description (public GGUF K-quant layout, as restated in the oracle's
header): the decoder there walks weights and reads bytes, these encoders walk
bytes and gather weights, so an index slip on either side makes the round-trip
pins fail.  Used only by tests.
"""
from __future__ import annotations

import numpy as np


def pack_q4k(d_bits: int, dmin_bits: int, sc, mn, q) -> np.ndarray:
    """Fields -> 144 bytes.  sc, mn: 8 six-bit values each; q: 256 nibbles in
    weight order (sub-block j holds weights 32j..32j+31)."""
    sc = [int(v) for v in sc]
    mn = [int(v) for v in mn]
    q = [int(v) for v in q]
    assert all(0 <= v < 64 for v in sc + mn) and all(0 <= v < 16 for v in q)
    out = np.zeros(144, np.uint8)
    out[0], out[1] = d_bits & 0xFF, d_bits >> 8
    out[2], out[3] = dmin_bits & 0xFF, dmin_bits >> 8
    s = [0] * 12
    for j in range(4):
        # bytes 0..3: scale j in bits 0-5, top two bits of scale j+4 in bits 6-7
        s[j] = sc[j] | ((sc[j + 4] >> 4) << 6)
        # bytes 4..7: min j in bits 0-5, top two bits of min j+4 in bits 6-7
        s[j + 4] = mn[j] | ((mn[j + 4] >> 4) << 6)
        # bytes 8..11: low four bits of scale j+4 and of min j+4
        s[j + 8] = (sc[j + 4] & 15) | ((mn[j + 4] & 15) << 4)
    out[4:16] = s
    for c in range(4):          # 32-byte chunk c carries sub-blocks 2c (low) and 2c+1 (high)
        for i in range(32):
            out[16 + 32 * c + i] = q[64 * c + i] | (q[64 * c + 32 + i] << 4)
    return out


def pack_q6k(d_bits: int, sc, q) -> np.ndarray:
    """Fields -> 210 bytes.  sc: 16 int8 scales; q: 256 six-bit quants."""
    sc = [int(v) for v in sc]
    q = [int(v) for v in q]
    assert all(-128 <= v < 128 for v in sc) and all(0 <= v < 64 for v in q)
    out = np.zeros(210, np.uint8)
    for half in range(2):
        w = q[128 * half:128 * half + 128]
        for l in range(32):
            # ql byte l: weights l (low nibble) and l+64 (high nibble);
            # ql byte 32+l: weights l+32 (low) and l+96 (high)
            out[64 * half + l] = (w[l] & 15) | ((w[l + 64] & 15) << 4)
            out[64 * half + 32 + l] = (w[l + 32] & 15) | ((w[l + 96] & 15) << 4)
            # qh byte l: top two bits of weights l, l+32, l+64, l+96
            out[128 + 32 * half + l] = ((w[l] >> 4) | ((w[l + 32] >> 4) << 2)
                                        | ((w[l + 64] >> 4) << 4) | ((w[l + 96] >> 4) << 6))
    out[192:208] = np.array(sc, np.int8).view(np.uint8)
    out[208], out[209] = d_bits & 0xFF, d_bits >> 8
    return out


def f16_bits(v: float) -> int:
    return int(np.array([v], np.float16).view(np.uint16)[0])


def random_q4k_fields(rng, nblocks):
    """Random fields for nblocks blocks: (d_bits, dmin_bits, sc, mn, q) arrays."""
    d = rng.uniform(1e-3, 1e-2, nblocks).astype(np.float16)
    dmin = rng.uniform(1e-3, 1e-2, nblocks).astype(np.float16)
    sc = rng.integers(0, 64, (nblocks, 8))
    mn = rng.integers(0, 64, (nblocks, 8))
    q = rng.integers(0, 16, (nblocks, 256))
    return d.view(np.uint16), dmin.view(np.uint16), sc, mn, q


def random_q6k_fields(rng, nblocks):
    d = rng.uniform(1e-3, 1e-2, nblocks).astype(np.float16)
    sc = rng.integers(-32, 32, (nblocks, 16))
    q = rng.integers(0, 64, (nblocks, 256))
    return d.view(np.uint16), sc, q


def q4k_matrix_from_fields(fields, N, K):
    """Pack fields (N*nb blocks, row-major) and return (bytes [N, nb*144],
    f64 weights [N, K] computed directly from the fields)."""
    d, dmin, sc, mn, q = fields
    nb = K // 256
    blocks = np.stack([pack_q4k(int(d[i]), int(dmin[i]), sc[i], mn[i], q[i])
                       for i in range(N * nb)])
    dv = d.view(np.float16).astype(np.float64)[:, None]
    mv = dmin.view(np.float16).astype(np.float64)[:, None]
    scw = np.repeat(sc, 32, axis=1).astype(np.float64)
    mnw = np.repeat(mn, 32, axis=1).astype(np.float64)
    w = dv * scw * q - mv * mnw
    return blocks.reshape(N, nb * 144), w.reshape(N, K)


def q6k_matrix_from_fields(fields, N, K):
    d, sc, q = fields
    nb = K // 256
    blocks = np.stack([pack_q6k(int(d[i]), sc[i], q[i]) for i in range(N * nb)])
    dv = d.view(np.float16).astype(np.float64)[:, None]
    scw = np.repeat(sc, 16, axis=1).astype(np.float64)
    w = dv * scw * (q - 32)
    return blocks.reshape(N, nb * 210), w.reshape(N, K)
