"""Shapes of the small GPU parity cases, and the kernel path each one takes.

Shared by the GPU parity tests and a CPU test that checks every kernel path
of the library (as reported by its launch geometry) is exercised by at least
one parity case of every kind that can take it.
"""
import gemv_q4k_q6k_amd as gq

# the last entries of each list (tens of MB) reach the tile kernel's ring
# form, which takes more than a CU's share of tiles in flight
SMALL_Q4K = [(1, 256), (5, 256), (1000, 1024), (1001, 1024), (3, 1024), (333, 2560), (77, 8192), (129, 9728), (17, 4352),
             (3, 32768), (70, 512), (130, 2048), (31, 4096), (9, 768), (6000, 2560), (5, 12288), (700, 9728),
             (20000, 2560), (1100, 32768)]
SMALL_Q6K = [(1, 256), (4, 256), (100, 768), (1000, 1024), (1001, 1024), (1003, 1024), (3, 1024), (250, 512), (257, 9728), (33, 1280), (21, 2560),
             (3, 32768), (65, 2048), (5, 16384), (700, 9728), (20000, 2560), (1100, 32768)]
SMALL_SWIGLU = [(1, 256), (100, 1024), (102, 1024), (333, 2560), (50, 8192), (7, 16384), (12000, 2560), (600, 32768)]
SMALL_Q8 = [(1, 256), (1000, 1024), (1003, 1024), (333, 2560), (77, 8192), (50, 9728), (3, 32768), (700, 9728),
            (20000, 2560), (1100, 32768)]
SMALL_Q6K_Q8 = [(1, 256), (100, 768), (1000, 1024), (1001, 1024), (333, 2560), (257, 9728), (3, 32768), (5, 16384),
                (65, 2048), (9, 4352), (20000, 2560), (1100, 32768)]


def kernel_path(kind, N, K):
    """'wave1', 'wave2' (wave-unit kernel), 'rows<S>' (row-stream kernel, S
    steps), 'tile-res' or 'tile-ring' (tile kernel, CU-resident or ring form),
    with '-lds' when the tile kernel stages x in LDS."""
    g = gq.tile_geometry(kind, N, K)
    if not g["wave_local"]:
        return ("tile-res" if g["resident"] else "tile-ring") + ("-lds" if g["x_in_lds"] else "")
    nb = K // 256
    group = 64 // g["rows_tile"]
    if kind == gq.KIND_Q4K_Q8 and g["steps"] == 2:
        return "wave2"
    if g["steps"] == 1 and group == 4 * nb:
        return "wave1"
    return f"rows{g['steps']}"


TILE_PATHS = {"tile-res-lds", "tile-res", "tile-ring-lds", "tile-ring"}
REQUIRED_PATHS = {
    gq.KIND_Q4K: {"wave1", "rows2"} | TILE_PATHS,   # short single-matrix rows run the tile kernel
    gq.KIND_Q6K: {"wave1", "rows1"} | TILE_PATHS,
    gq.KIND_SWIGLU: {"wave1"} | TILE_PATHS,
    gq.KIND_Q4K_Q8: {"wave1", "wave2", "rows1"} | TILE_PATHS,
    gq.KIND_Q6K_Q8: {"wave1", "rows1"} | TILE_PATHS,
}
CASES = {gq.KIND_Q4K: SMALL_Q4K, gq.KIND_Q6K: SMALL_Q6K, gq.KIND_SWIGLU: SMALL_SWIGLU, gq.KIND_Q4K_Q8: SMALL_Q8,
         gq.KIND_Q6K_Q8: SMALL_Q6K_Q8}
