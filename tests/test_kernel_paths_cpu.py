"""Every kernel path the library can launch is taken by at least one small
GPU parity case of each kind that can use it (decided from the library's own
launch geometry, no GPU needed)."""
import pytest

import gemv_q4k_q6k_amd as gq
import parity_shapes as ps


@pytest.mark.parametrize("kind", sorted(ps.CASES))
def test_parity_cases_cover_every_path(kind):
    got = {ps.kernel_path(kind, N, K) for N, K in ps.CASES[kind]}
    assert ps.REQUIRED_PATHS[kind] <= got, ps.REQUIRED_PATHS[kind] - got


@pytest.mark.parametrize("kind,N,K,path", [
    (gq.KIND_Q6K, 248_320, 1024, "wave1"),      # lm_head
    (gq.KIND_Q4K, 4096, 2560, "tile-res-lds"),
    (gq.KIND_Q4K, 9728, 2560, "tile-res-lds"),
    (gq.KIND_Q4K, 2560, 9728, "tile-res-lds"),
    (gq.KIND_SWIGLU, 9728, 2560, "tile-res-lds"),
    (gq.KIND_Q6K, 2560, 9728, "tile-res-lds"),
    (gq.KIND_Q4K_Q8, 28_672, 8192, "wave2"),
    (gq.KIND_Q4K, 28_672, 8192, "rows2"),
    (gq.KIND_Q6K_Q8, 2560, 9728, "tile-res-lds"),
])
def test_workload_paths(kind, N, K, path):
    """The benchmarked workloads run the kernels their parity tests cover."""
    assert ps.kernel_path(kind, N, K) == path


@pytest.mark.parametrize("kind,N,K", [
    (gq.KIND_Q6K, 2560, 9728), (gq.KIND_SWIGLU, 9728, 2560), (gq.KIND_Q4K, 9728, 2560), (gq.KIND_Q4K, 2560, 9728),
    (gq.KIND_SWIGLU_Q8, 9728, 2560), (gq.KIND_Q6K_Q8, 2560, 9728),
])
def test_mid_size_resident_geometry(kind, N, K):
    """The 4B-class FFN and attention shapes run one 12-wave workgroup per CU
    (256 CUs), each with exactly two tiles in flight: N / 256 rows per CU."""
    g = gq.tile_geometry(kind, N, K)
    assert g["resident"] == 1 and g["waves"] == 12 and g["phase"] == 2 and g["grid"] == 256, g
    assert g["rows_tile"] * g["phase"] * g["grid"] == N, g
