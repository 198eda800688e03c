"""hgemm_splitk_noalloc (the split-K GEMM with its partial products in the
library's static device array instead of a caller's workspace) against
hgemm_splitk, through the C ABI.

The two entry points run the same kernels on the same slice plan, so their
results must agree bit for bit; two calls in a row (the second smaller, so
that it reads a region the first left behind) check that nothing of the
previous call leaks into the next.  A problem whose partials exceed the
array is rejected before anything runs.
"""
import numpy as np
import pytest

import oracle
import workloads
from tolerance import check_close

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _case(seed, M, N, K, odt, beta):
    rng = np.random.default_rng(seed)
    A = workloads.uniform_f16(rng, (M, K))
    Bt = workloads.uniform_f16(rng, (N, K))
    C = workloads.uniform_f16(rng, (M, N)).astype(odt)
    return A, Bt, C


@pytest.mark.parametrize("odt", [np.float16, np.float32])
def test_noalloc_equals_splitk_two_calls(hg, odt):
    cases = [(11, 512, 512, 8192, 0, 0.0),       # 16 slices: 16 MiB of partials
             (12, 300, 260, 3000, 4, 0.5)]       # smaller, beta != 0, ragged
    for seed, M, N, K, splits, beta in cases:
        print(f"[noalloc] M={M} N={N} K={K} splits={splits} beta={beta} C={odt.__name__}", flush=True)
        assert hg.splitk_workspace_size(M, N, K, splits) <= hg.NOALLOC_SCRATCH_BYTES
        A, Bt, C = _case(seed, M, N, K, odt, beta)
        Ad, Bd = dev(A), dev(Bt)
        C_ref = dev(C)
        work = torch.empty(hg.splitk_workspace_size(M, N, K, splits), dtype=torch.uint8, device=DEV)
        hg.hgemm_splitk(Ad, Bd, C_ref, 1.25, beta, splits, work)
        C_na = dev(C)
        hg.hgemm_splitk_noalloc(Ad, Bd, C_na, 1.25, beta, splits)
        torch.cuda.synchronize()
        got = C_na.cpu().numpy()
        assert np.array_equal(got, C_ref.cpu().numpy())
        ri, cj = workloads.sample_indices(seed, M, N, 256)
        ref = oracle.hgemm_sampled(A, Bt, ri, cj, 1.25, beta, C)
        check_close(got[ri, cj], ref, K, f"noalloc {M}x{N}x{K}")


def test_noalloc_rejects_problem_beyond_scratch(hg):
    M, N, K, splits = 2048, 2048, 65536, 8          # 128 MiB of partials
    assert hg.splitk_workspace_size(M, N, K, splits) > hg.NOALLOC_SCRATCH_BYTES
    Ad = torch.zeros((M, K), dtype=torch.float16, device=DEV)
    Bd = torch.zeros((N, K), dtype=torch.float16, device=DEV)
    C = torch.full((M, N), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(hg.HgError) as ei:
        hg.hgemm_splitk_noalloc(Ad, Bd, C, 1.0, 0.0, splits)
    assert ei.value.status == hg.ERR_SCRATCH_LIMIT
    assert "scratch" in hg.strerror(hg.ERR_SCRATCH_LIMIT)
    torch.cuda.synchronize()
    assert bool((C == 7.0).all())
