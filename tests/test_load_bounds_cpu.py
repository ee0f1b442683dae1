"""Every weight load of the GEMV kernels stays inside the matrix (CPU only).

The kernels' per-lane load windows are emulated here from their address
arithmetic (gemvq_device.h: q4k_load, q6k_load; gemvq_kernels.hip: the tile
fetch) on the launch geometry the library itself reports
(gemvq_tile_geometry), for many shapes.  Q6_K blocks are 210 bytes, so a
block - and a tile - can start 2 bytes past a dword boundary; the loads then
begin 2 bytes before the block, which must never fall before the matrix or
wrap around.  Regression test for an unsigned underflow of that offset.
"""
import numpy as np
import pytest

import gemv_q4k_q6k_amd as gq

W_BASE = 1 << 20          # any dword-aligned matrix address


def lane_table(geo, nb):
    # rows that fit in a wave are processed in units of one wave's rows;
    # otherwise a tile spans the workgroup's waves
    tid = np.arange(64 if geo["wave_local"] else 64 * geo["waves"])
    lr = 4 * nb
    p = tid // lr
    rr = tid - p * lr
    return p, rr >> 2, rr & 3, p < geo["rows_tile"]


def q6k_windows(N, K, tiles_to_check=None):
    """(lowest byte read, one past the highest) over all lanes and tiles."""
    nb = K // 256
    geo = gq.tile_geometry(gq.KIND_Q6K, N, K)
    P, tiles = geo["rows_tile"], geo["tiles"]
    stride = P * nb * 210
    last_rows = N - (tiles - 1) * P
    p, b, u, on = lane_table(geo, nb)
    lane_off = (p * nb + b) * 210
    n, l0 = u >> 1, 16 * (u & 1)
    lo, hi = None, None
    ts = range(tiles) if tiles_to_check is None else tiles_to_check
    for t in ts:
        tile = W_BASE + t * stride
        valid = on & ((t < tiles - 1) | (p < last_rows))
        off = np.where(valid, lane_off, 0)
        lead = tile & 3
        base = tile - lead
        o = off + lead
        sh = o & 3
        al = o - sh
        assert (al >= 0).all()
        starts = [al + 64 * n + l0, al + 64 * n + 32 + l0, al + 128 + 32 * n + l0]
        ends = [s_ + 20 for s_ in starts]                       # dwordx4 + one dword
        ends.append(al + 192 + 8 * n + np.where(sh != 0, 12, 8))  # scale window
        ends.append(o + 210)                                    # d at o + 208, 2 bytes
        l_ = base + min(s_.min() for s_ in starts)
        h_ = base + max(e.max() for e in ends)
        lo = l_ if lo is None else min(lo, l_)
        hi = h_ if hi is None else max(hi, h_)
    return lo, hi, W_BASE + N * nb * 210


def q4k_windows(kind, N, K):
    nb = K // 256
    geo = gq.tile_geometry(kind, N, K)
    P, tiles = geo["rows_tile"], geo["tiles"]
    stride = P * nb * 144
    last_rows = N - (tiles - 1) * P
    if geo["steps"] == 2:
        # one row per tile; lane l takes block l//4, then block 16 + l//4
        lanes = np.arange(64)
        p, b, c, on = np.zeros(64, int), lanes >> 2, lanes & 3, np.ones(64, bool)
        steps = [0, 16]
    else:
        p, b, c, on = lane_table(geo, nb)
        steps = [0]
    lo, hi = None, None
    for t in range(tiles):
        tile = W_BASE + t * stride
        valid = on & ((t < tiles - 1) | (p < last_rows))
        for s16 in steps:
            off = np.where(valid, (p * nb + b + s16) * 144, 0)
            l_ = tile + off.min()
            h_ = tile + max((off + 16).max(), (off + 32 * c + 48).max())
            lo = l_ if lo is None else min(lo, l_)
            hi = h_ if hi is None else max(hi, h_)
    return lo, hi, W_BASE + N * nb * 144


SHAPES = [(N, K) for N in (1, 2, 3, 5, 7, 21, 100, 257) for K in range(256, 10241, 256)]


@pytest.mark.parametrize("N,K", SHAPES)
def test_q6k_loads_in_bounds(N, K):
    lo, hi, end = q6k_windows(N, K)
    assert W_BASE <= lo and hi <= end, (N, K, lo - W_BASE, hi - end)


@pytest.mark.parametrize("N,K", [(248_320, 1024), (2560, 9728), (100, 768), (99_999, 768), (12_345, 3328)])
def test_q6k_loads_in_bounds_large(N, K):
    geo = gq.tile_geometry(gq.KIND_Q6K, N, K)
    tiles = geo["tiles"]
    check = sorted(set(list(range(min(tiles, 64))) + list(range(max(0, tiles - 64), tiles))))
    lo, hi, end = q6k_windows(N, K, check)
    assert W_BASE <= lo and hi <= end


@pytest.mark.parametrize("kind", [gq.KIND_Q4K, gq.KIND_Q4K_Q8, gq.KIND_SWIGLU])
@pytest.mark.parametrize("N,K", [(1, 256), (5, 768), (100, 2560), (257, 9728), (77, 8192), (1, 8192), (3, 32768)])
def test_q4k_loads_in_bounds(kind, N, K):
    lo, hi, end = q4k_windows(kind, N, K)
    assert W_BASE <= lo and hi <= end


def test_geometry_rejects_bad_shapes():
    with pytest.raises(gq.GemvqError):
        gq.tile_geometry(gq.KIND_Q6K, 0, 1024)
    with pytest.raises(gq.GemvqError):
        gq.tile_geometry(gq.KIND_Q4K, 10, 300)


def test_two_step_rows_cover_every_block_once():
    """In a two-step (K = 8192) row every (super-block, quarter) pair is taken
    by exactly one lane and step."""
    geo = gq.tile_geometry(gq.KIND_Q4K_Q8, 28_672, 8192)
    assert geo["wave_local"] == 1 and geo["steps"] == 2 and geo["rows_tile"] == 1 and geo["tiles"] == 28_672
    lanes = np.arange(64)
    pairs = {(int(b) + s16, int(c)) for s16 in (0, 16) for b, c in zip(lanes >> 2, lanes & 3)}
    assert pairs == {(b, c) for b in range(32) for c in range(4)}
