"""GPU parity of the permutation call (`moe_permute`) alone, bit-exact against
the oracle's stable counting sort, across the four kernel paths: one wave (at
most 64 slots), one 256-thread workgroup (at most 1024), one 1024-thread
workgroup (at most 4096) and 1024-slot tiles with a scan (more), at each
boundary, with uniform, one-expert and Zipf-skewed expert ids."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _ids(kind, N, E, rng):
    if kind == "uniform":
        return rng.integers(0, E, N)
    if kind == "one":
        return np.full(N, E - 1)
    z = np.minimum(rng.zipf(1.3, N) - 1, E - 1)
    return rng.permutation(E)[z]


@pytest.mark.parametrize("N", [1, 63, 64, 65, 1024, 1025, 4096, 4097, 9000])
@pytest.mark.parametrize("E", [1, 8, 128, 256])
@pytest.mark.parametrize("kind", ["uniform", "one", "zipf"])
def test_permutation_paths(N, E, kind):
    from sparse_moe_amd import binding
    rng = np.random.default_rng(N * 7 + E)
    ids = _ids(kind, N, E, rng).astype(np.int32).reshape(N, 1)
    off_ref, ss_ref, sp_ref = oracle.permute(ids, E)
    print("permute N=%d E=%d %s" % (N, E, kind), flush=True)
    d_ids = torch.from_numpy(ids).cuda()
    off = torch.full((E + 1,), -1, dtype=torch.int32, device="cuda")
    ss = torch.full((N,), -1, dtype=torch.int32, device="cuda")
    sp = torch.full((N,), -1, dtype=torch.int32, device="cuda")
    nws = binding.moe_permute_workspace_bytes(N, 1, E)
    ws = torch.empty((max(nws, 16),), dtype=torch.uint8, device="cuda") if nws else None
    binding.moe_permute(d_ids, E, off, ss, sp, ws=ws)
    torch.cuda.synchronize()
    assert np.array_equal(off.cpu().numpy(), off_ref)
    assert np.array_equal(ss.cpu().numpy(), ss_ref)
    assert np.array_equal(sp.cpu().numpy(), sp_ref)
