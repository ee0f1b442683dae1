"""Seeded synthetic inputs for the quantized GEMV path.

Shared by the tests, the benchmark and the smoke check; holds none of the
method's arithmetic (no decoding, no dot products, no quantization of
activations).  It only draws random bytes and places them at the byte offsets
of a super-block.  The draw order of every generator is fixed and documented
so that a (generator, seed) pair always gives the same bytes; the tests keep a
checksum per case to catch drift.

Distributions are those of the workloads the method is measured on (GGUF
Q4_K / Q6_K decode shapes):
  Q4_K: fp16 d and dmin ~ U(1e-3, 1e-2); 12 bytes of packed 6-bit
        scales/mins; 128 bytes of 4-bit quants.  The 12 scale bytes are drawn
        as independent uniform bytes: the 16 six-bit fields of the packing use
        each of the 96 bits exactly once, so every scale and every min is an
        independent U{0..63}, and every quant nibble is an independent U{0..15}.
  Q6_K: 128 bytes ql and 64 bytes qh uniform (every 6-bit quant U{0..63}),
        16 int8 scales ~ U{-32..31}, fp16 d ~ U(1e-3, 1e-2).
  x:    f32 ~ N(0, 1); the 70B-class FFN case uses N(0, 2) (variance 2) and
        multiplies round(0.1% of K) distinct entries by 50.
"""
from __future__ import annotations

import numpy as np

Q4K_BLOCK_BYTES = 144
Q6K_BLOCK_BYTES = 210
QK = 256


def rng_for(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def q4k_weights(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    """N x K Q4_K matrix as uint8 [N, K/256*144], rows contiguous.

    Draw order: d, dmin (each f64 U(1e-3,1e-2) over (N, nb), cast to fp16),
    then the scale bytes (N, nb, 12), then the quant bytes (N, nb, 128)."""
    assert K % QK == 0 and N >= 0
    nb = K // QK
    d = rng.uniform(1e-3, 1e-2, (N, nb)).astype(np.float16)
    dmin = rng.uniform(1e-3, 1e-2, (N, nb)).astype(np.float16)
    scales = rng.integers(0, 256, (N, nb, 12), dtype=np.uint8)
    qs = rng.integers(0, 256, (N, nb, 128), dtype=np.uint8)
    blk = np.empty((N, nb, Q4K_BLOCK_BYTES), np.uint8)
    blk[:, :, 0:2] = d.reshape(N, nb, 1).view(np.uint8)
    blk[:, :, 2:4] = dmin.reshape(N, nb, 1).view(np.uint8)
    blk[:, :, 4:16] = scales
    blk[:, :, 16:144] = qs
    return blk.reshape(N, nb * Q4K_BLOCK_BYTES)


def q6k_weights(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    """N x K Q6_K matrix as uint8 [N, K/256*210], rows contiguous.

    Draw order: ql (N, nb, 128), qh (N, nb, 64), scales (N, nb, 16) as
    integers in [-32, 31], d (N, nb) f64 U(1e-3,1e-2) cast to fp16."""
    assert K % QK == 0 and N >= 0
    nb = K // QK
    ql = rng.integers(0, 256, (N, nb, 128), dtype=np.uint8)
    qh = rng.integers(0, 256, (N, nb, 64), dtype=np.uint8)
    sc = rng.integers(-32, 32, (N, nb, 16), dtype=np.int8)
    d = rng.uniform(1e-3, 1e-2, (N, nb)).astype(np.float16)
    blk = np.empty((N, nb, Q6K_BLOCK_BYTES), np.uint8)
    blk[:, :, 0:128] = ql
    blk[:, :, 128:192] = qh
    blk[:, :, 192:208] = sc.view(np.uint8)
    blk[:, :, 208:210] = d.reshape(N, nb, 1).view(np.uint8)
    return blk.reshape(N, nb * Q6K_BLOCK_BYTES)


def activation(rng: np.random.Generator, K: int) -> np.ndarray:
    """x ~ N(0, 1) as f32."""
    return rng.standard_normal(K).astype(np.float32)


def activation_outliers(rng: np.random.Generator, K: int, var: float = 2.0,
                        frac: float = 0.001, mult: float = 50.0) -> np.ndarray:
    """x ~ N(0, var) with round(frac*K) distinct entries multiplied by mult.

    Draw order: the K normals, then the outlier indices (without
    replacement)."""
    x = rng.normal(0.0, np.sqrt(var), K)
    n_out = int(round(frac * K))
    if n_out:
        idx = rng.choice(K, size=n_out, replace=False)
        x[idx] *= mult
    return x.astype(np.float32)


def activation_wide_range(rng: np.random.Generator, K: int) -> np.ndarray:
    """f32[K] with a wide dynamic range inside every aligned 64-value part
    (stress input for kernels that scale each part to a common exponent).

    Draw order: N(0, 1) values (K); per part, one index U{0..63} (K/64) and
    one sign (K/64).  The drawn entry of every part becomes
    sign * 1e4 * (1 + |value|); then every 7th part (part p with p % 7 == 3) is scaled by 1e-6,
    every 13th (p % 13 == 5) by 1e-30 and every 11th (p % 11 == 9) set to zero,
    in that order."""
    assert K % 64 == 0
    x = rng.standard_normal(K)
    parts = K // 64
    idx = rng.integers(0, 64, parts)
    sign = np.where(rng.integers(0, 2, parts) == 0, -1.0, 1.0)
    x = x.reshape(parts, 64)
    rows = np.arange(parts)
    x[rows, idx] = sign * 1e4 * (1.0 + np.abs(x[rows, idx]))
    p = np.arange(parts)
    x[p % 7 == 3] *= 1e-6
    x[p % 13 == 5] *= 1e-30
    x[p % 11 == 9] = 0.0
    return x.reshape(K).astype(np.float32)


def q8_activations(rng: np.random.Generator, m: int, K: int):
    """m Q8 activation vectors drawn directly in their stored form, for the
    int8 GEMVs: (xq int8 [m, K], xd fp16 bits uint16 [m, K/32]).  Values
    ~ U{-127..127}; one position of each 32-element block, drawn uniformly,
    holds +-127 (a block's largest code is +-127 after quantization); scales
    ~ fp16(U(1e-3, 1e-1)).  Draw order: values, the +-127 positions, their
    signs, the scales."""
    assert K % 32 == 0
    q = rng.integers(-127, 128, (m, K)).astype(np.int8)
    nb = K // 32
    pos = rng.integers(0, 32, (m, nb))
    sign = rng.integers(0, 2, (m, nb)) * 2 - 1
    qb = q.reshape(m, nb, 32)
    qb[np.arange(m)[:, None], np.arange(nb)[None, :], pos] = (127 * sign).astype(np.int8)
    d = rng.uniform(1e-3, 1e-1, (m, nb)).astype(np.float16).view(np.uint16)
    return qb.reshape(m, K), d


# ----------------------------------------------------------- workloads
# The five workloads (shapes and distributions) the path is specified on.
C1_Q4K = (1024, 1024)
C2_Q4K = ((4096, 2560), (2560, 9728), (9728, 2560))   # attn, ffn_down, ffn_up
C3_LM_HEAD = (248_320, 1024)                           # Q6_K vocab rows x hidden
C4_SWIGLU = (9728, 2560)                               # gate/up Q4_K; down Q6_K is 2560 x 9728
C5_Q8 = (28_672, 8192)


def c1_inputs(seed: int = 0):
    r = rng_for(seed)
    N, K = C1_Q4K
    return q4k_weights(r, N, K), activation(r, K)


def c2_inputs(index: int, seed: int | None = None):
    """One of the three decode shapes; seed defaults to the shape's index."""
    N, K = C2_Q4K[index]
    r = rng_for(index if seed is None else seed)
    return q4k_weights(r, N, K), activation(r, K)


def c3_inputs(seed: int = 0, N: int | None = None):
    N = C3_LM_HEAD[0] if N is None else N
    K = C3_LM_HEAD[1]
    r = rng_for(seed)
    return q6k_weights(r, N, K), activation(r, K)


def c4_inputs(seed: int = 0):
    """Wg, Wu (Q4_K N x K), Wd (Q6_K K x N), x; drawn in that order."""
    N, K = C4_SWIGLU
    r = rng_for(seed)
    Wg = q4k_weights(r, N, K)
    Wu = q4k_weights(r, N, K)
    Wd = q6k_weights(r, K, N)
    x = activation(r, K)
    return Wg, Wu, Wd, x


def c5_inputs(seed: int = 0):
    N, K = C5_Q8
    r = rng_for(seed)
    return q4k_weights(r, N, K), activation_outliers(r, K)
