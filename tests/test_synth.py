"""Seeded input generators: determinism (checksums) and distributions (CPU)."""
import hashlib

import numpy as np

import synth


def _h(*arrs):
    m = hashlib.sha256()
    for a in arrs:
        m.update(np.ascontiguousarray(a).tobytes())
    return m.hexdigest()[:16]


def test_checksums_fixed():
    # A change in draw order or distribution changes these; update them only
    # together with a stated reason.
    r = synth.rng_for(0)
    assert _h(synth.q4k_weights(r, 64, 512), synth.activation(r, 512)) == "1a80ff6f66e325cb"
    r = synth.rng_for(0)
    assert _h(synth.q6k_weights(r, 64, 512), synth.activation(r, 512)) == "3822445b7cdd00f3"
    r = synth.rng_for(0)
    assert _h(synth.activation_outliers(r, 8192)) == "aed567af945460ea"
    assert _h(*synth.c1_inputs(0)) == "8fd912eb75ae0192"


def test_q4k_layout_and_ranges():
    N, K = 50, 1024
    W = synth.q4k_weights(synth.rng_for(1), N, K)
    assert W.shape == (N, K // 256 * 144) and W.dtype == np.uint8
    blk = W.reshape(N, K // 256, 144)
    d = blk[:, :, 0:2].copy().view(np.float16).astype(np.float64)
    dmin = blk[:, :, 2:4].copy().view(np.float16).astype(np.float64)
    for v in (d, dmin):
        assert v.min() >= 0.00099 and v.max() <= 0.01001
    # the 6-bit fields of uniform bytes are uniform: mean of the low 6 bits ~ 31.5
    assert abs((blk[:, :, 4:8] & 63).mean() - 31.5) < 1.5


def test_q6k_layout_and_ranges():
    N, K = 50, 1024
    W = synth.q6k_weights(synth.rng_for(2), N, K)
    assert W.shape == (N, K // 256 * 210)
    blk = W.reshape(N, K // 256, 210)
    sc = blk[:, :, 192:208].copy().view(np.int8)
    assert sc.min() == -32 and sc.max() == 31
    d = blk[:, :, 208:210].copy().view(np.float16).astype(np.float64)
    assert d.min() >= 0.00099 and d.max() <= 0.01001


def test_activation_outliers():
    x = synth.activation_outliers(synth.rng_for(0), 8192)
    assert x.dtype == np.float32 and x.size == 8192
    big = np.abs(x) > 12.0        # |N(0,2)| > 12 has probability ~1e-17
    assert 1 <= big.sum() <= 8
    assert abs(np.var(x[~big]) - 2.0) < 0.15


def test_shapes_of_workloads():
    assert synth.C3_LM_HEAD == (248_320, 1024)
    assert synth.C3_LM_HEAD[0] * 4 == 993_280   # f32 logits bytes of the unfused path
    assert synth.C5_Q8 == (28_672, 8192)


def test_q8_activations():
    m, K = 5, 1024
    xq, xd = synth.q8_activations(synth.rng_for(3), m, K)
    assert xq.shape == (m, K) and xq.dtype == np.int8 and xd.shape == (m, K // 32) and xd.dtype == np.uint16
    assert xq.min() >= -127                                   # -128 never appears
    # every 32-element block holds a +-127, as a quantized block does
    assert np.all(np.abs(xq.astype(np.int64)).reshape(m, -1, 32).max(axis=2) == 127)
    d = xd.view(np.float16).astype(np.float64)
    assert d.min() >= 0.00099 and d.max() <= 0.1001
    r = synth.rng_for(0)
    assert _h(*synth.q8_activations(r, 3, 512)) == "dc3893e619f8532f"


def test_activation_wide_range():
    """One +-1e4 outlier in each 64-value part, some parts tiny or zero; f32."""
    K = 64 * 100
    a = synth.activation_wide_range(synth.rng_for(5), K)
    b = synth.activation_wide_range(synth.rng_for(5), K)
    assert a.dtype == np.float32 and np.array_equal(a, b)
    parts = a.reshape(-1, 64).astype(np.float64)
    for p, v in enumerate(parts):
        m = np.max(np.abs(v))
        if p % 11 == 9:
            assert m == 0.0
            continue
        scale = (1e-6 if p % 7 == 3 else 1.0) * (1e-30 if p % 13 == 5 else 1.0)
        assert 1e4 * scale <= m * (1 + 1e-6) and m < 1e5 * scale
        assert np.sum(np.abs(v) > 100 * scale) == 1     # exactly one outlier
