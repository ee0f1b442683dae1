"""Every weight load of the GEMV kernels stays inside the matrix (CPU only).

The kernels' per-lane load windows are emulated here from their address
arithmetic (gemvq_device.h: q4k_load, q6k_load; gemvq_kernels.hip: the fetch
of each kernel) on the launch geometry the library itself reports
(gemvq_tile_geometry), for many shapes.  Two layouts exist:

* rows inside one wave (geometry wave_local = 1; the wave-unit and row-stream
  kernels): a unit of 64/group rows, lane l serving row l // group and
  quarter l % 4 of super-block (l % group) // 4 + 16 * step, in each of
  `steps` steps; lanes past the row's last super-block load the unit's first
  super-block;
* tiles across a workgroup (wave_local = 0): lane t of the workgroup serves
  row t // (4*nb), quarter t % 4 of super-block (t % (4*nb)) // 4.

A lane of a unit or tile past the last row also loads the first super-block
of that unit or tile.  Q6_K blocks are 210 bytes, so a block can start 2
bytes past a dword boundary; its fields are then read at their true
(2-byte aligned) addresses, and every byte read must lie inside the block.
"""
import numpy as np
import pytest

import gemv_q4k_q6k_amd as gq

W_BASE = 1 << 20          # any dword-aligned matrix address


def lane_offsets(geo, nb, B, N):
    """(offsets(t) -> list over steps of per-lane byte offsets within unit or
    tile t, quarter index per lane, base(t) -> byte offset of unit or tile t
    in the matrix)."""
    P, tiles = geo["rows_tile"], geo["tiles"]
    last_rows = N - (tiles - 1) * P
    if geo.get("wave_unit"):
        # wave-unit kernel: fixed lane offsets (lanes past N, only when
        # N < P, read the first super-block); a ragged last unit starts at
        # row N - P
        group = 64 // P
        lane = np.arange(64)
        p, rr = lane // group, lane % group
        b, c = rr >> 2, rr & 3
        shift = last_rows < P and N >= P

        def offsets_w(t):
            return [np.where(p < N, (p * nb + b + 16 * st) * B, 0) for st in range(geo["steps"])]

        def base_w(t):
            return ((N - P) if (shift and t == tiles - 1) else t * P) * nb * B
        return offsets_w, c, base_w
    if geo["wave_local"]:
        group = 64 // P
        lane = np.arange(64)
        p, rr = lane // group, lane % group
        steps = geo["steps"]
    else:
        tid = np.arange(64 * geo["waves"])
        lr = 4 * nb
        p, rr = tid // lr, tid % lr
        steps = 1
    b, c = rr >> 2, rr & 3

    def offsets(t):
        out = []
        for st in range(steps):
            blk = b + 16 * st
            valid = (p < P) & ((t < tiles - 1) | (p < last_rows)) & (blk < nb)
            out.append(np.where(valid, (p * nb + blk) * B, 0))
        return out
    return offsets, c, lambda t: t * P * nb * B


def q6k_windows(N, K, tiles_to_check=None, kind=gq.KIND_Q6K):
    """(lowest byte read, one past the highest, end of the matrix)."""
    nb = K // 256
    geo = gq.tile_geometry(kind, N, K)
    offsets, u, base = lane_offsets(geo, nb, 210, N)
    n, l0 = u >> 1, 16 * (u & 1)
    lo, hi = None, None
    ts = range(geo["tiles"]) if tiles_to_check is None else tiles_to_check
    for t in ts:
        tile = W_BASE + base(t)
        for off in offsets(t):
            blk = tile + off
            assert (blk % 2 == 0).all()
            starts = [blk + 64 * n + l0, blk + 64 * n + 32 + l0, blk + 128 + 32 * n + l0]
            ends = [s_ + 16 for s_ in starts]          # 16-byte loads
            ends.append(blk + 192 + 8 * n + 8)         # scale window
            ends.append(blk + 210)                     # d at 208, 2 bytes
            l_ = min(s_.min() for s_ in starts)
            h_ = max(e.max() for e in ends)
            assert (np.maximum.reduce(ends) <= blk + 210).all()   # inside the lane's own block
            lo = l_ if lo is None else min(lo, l_)
            hi = h_ if hi is None else max(hi, h_)
    return lo, hi, W_BASE + N * nb * 210


def q4k_windows(kind, N, K, tiles_to_check=None):
    nb = K // 256
    geo = gq.tile_geometry(kind, N, K)
    offsets, c, base = lane_offsets(geo, nb, 144, N)
    lo, hi = None, None
    ts = range(geo["tiles"]) if tiles_to_check is None else tiles_to_check
    for t in ts:
        tile = W_BASE + base(t)
        for off in offsets(t):
            l_ = tile + off.min()
            h_ = tile + max((off + 16).max(), (off + 32 * c + 48).max())
            lo = l_ if lo is None else min(lo, l_)
            hi = h_ if hi is None else max(hi, h_)
    return lo, hi, W_BASE + N * nb * 144


def ends_of(geo):
    tiles = geo["tiles"]
    return sorted(set(list(range(min(tiles, 64))) + list(range(max(0, tiles - 64), tiles))))


SHAPES = [(N, K) for N in (1, 2, 3, 5, 7, 21, 100, 257) for K in range(256, 10241, 256)]


@pytest.mark.parametrize("kind", [gq.KIND_Q6K, gq.KIND_Q6K_Q8, gq.KIND_Q6K_Q8_BATCH])
@pytest.mark.parametrize("N,K", SHAPES)
def test_q6k_loads_in_bounds(N, K, kind):
    lo, hi, end = q6k_windows(N, K, kind=kind)
    assert W_BASE <= lo and hi <= end, (N, K, lo - W_BASE, hi - end)


@pytest.mark.parametrize("N,K", [(248_320, 1024), (2560, 9728), (100, 768), (99_999, 768), (12_345, 3328),
                                 (7, 16384), (3, 32768), (1001, 12288)])
@pytest.mark.parametrize("kind", [gq.KIND_Q6K, gq.KIND_Q6K_Q8, gq.KIND_Q6K_Q8_BATCH])
def test_q6k_loads_in_bounds_large(N, K, kind):
    geo = gq.tile_geometry(kind, N, K)
    lo, hi, end = q6k_windows(N, K, ends_of(geo), kind)
    assert W_BASE <= lo and hi <= end


@pytest.mark.parametrize("kind", [gq.KIND_Q4K, gq.KIND_Q4K_Q8, gq.KIND_SWIGLU, gq.KIND_Q4K_Q8_BATCH])
@pytest.mark.parametrize("N,K", [(1, 256), (5, 768), (100, 2560), (257, 9728), (77, 8192), (1, 8192), (3, 32768),
                                 (9, 1280), (33, 4352), (5, 12288), (2, 16384)])
def test_q4k_loads_in_bounds(kind, N, K):
    lo, hi, end = q4k_windows(kind, N, K)
    assert W_BASE <= lo and hi <= end


@pytest.mark.parametrize("N,K", [(32, 256), (96, 1024), (320, 2560), (64, 8192), (32, 32768), (2048, 4352),
                                 (9728, 2560), (4096, 14336)])
def test_swiglu_q8_loads_in_bounds(N, K):
    """The SwiGLU Q8-emission launch (always the tile kernel) at shapes that
    are multiples of 32 rows."""
    geo = gq.tile_geometry(gq.KIND_SWIGLU_Q8, N, K)
    assert geo["wave_local"] == 0
    lo, hi, end = q4k_windows(gq.KIND_SWIGLU_Q8, N, K, ends_of(geo))
    assert W_BASE <= lo and hi <= end


@pytest.mark.parametrize("kind,N,K", [(gq.KIND_Q4K, 9728, 2560), (gq.KIND_SWIGLU, 9728, 2560),
                                      (gq.KIND_Q4K, 2560, 9728), (gq.KIND_Q4K_Q8, 28_672, 8192),
                                      (gq.KIND_Q4K, 28_672, 8192), (gq.KIND_Q4K, 4096, 2560)])
def test_q4k_loads_in_bounds_large(kind, N, K):
    geo = gq.tile_geometry(kind, N, K)
    lo, hi, end = q4k_windows(kind, N, K, ends_of(geo))
    assert W_BASE <= lo and hi <= end


@pytest.mark.parametrize("kind", [gq.KIND_Q4K, gq.KIND_Q6K, gq.KIND_Q4K_Q8, gq.KIND_SWIGLU, gq.KIND_Q6K_Q8,
                                  gq.KIND_Q4K_Q8_BATCH, gq.KIND_Q6K_Q8_BATCH])
@pytest.mark.parametrize("K", [256, 768, 1024, 1280, 2560, 4096, 4352, 8192, 9728, 12288, 16384, 32768])
def test_every_block_quarter_served_once(kind, K):
    """Each (row of a unit or tile, super-block, quarter) is taken by exactly
    one lane and step."""
    nb = K // 256
    geo = gq.tile_geometry(kind, 1000, K)
    P = geo["rows_tile"]
    if geo["wave_local"]:
        group = 64 // P
        lane = np.arange(64)
        p, rr = lane // group, lane % group
        steps = geo["steps"]
    else:
        tid = np.arange(64 * geo["waves"])
        p, rr = tid // (4 * nb), tid % (4 * nb)
        steps = 1
    seen = {}
    for st in range(steps):
        for pp, r_ in zip(p, rr):
            blk = int(r_ >> 2) + 16 * st
            if pp < P and blk < nb:
                key = (int(pp), blk, int(r_ & 3))
                seen[key] = seen.get(key, 0) + 1
    assert set(seen) == {(pp, blk, q) for pp in range(P) for blk in range(nb) for q in range(4)}
    assert set(seen.values()) == {1}


def test_two_step_rows():
    geo = gq.tile_geometry(gq.KIND_Q4K_Q8, 28_672, 8192)
    assert geo["wave_local"] == 1 and geo["steps"] == 2 and geo["rows_tile"] == 1 and geo["tiles"] == 28_672
    # rows of two halves launch 8 waves per CU (each wave walks 14 of the 112 rows a CU gets)
    assert geo["waves"] == 8 and geo["wave_unit"] == 1


def test_geometry_rejects_bad_shapes():
    with pytest.raises(gq.GemvqError):
        gq.tile_geometry(gq.KIND_Q6K, 0, 1024)
    with pytest.raises(gq.GemvqError):
        gq.tile_geometry(gq.KIND_Q4K, 10, 300)
