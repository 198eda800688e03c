"""GPU parity of hg_trmm, Out = α·op(A)·B for A lower or upper and op = A or
Aᵀ ("异构计算中高性能TRMM与TRSM的递归算法实现" §2.1 and the §5.1 usage call),
against the fp64 oracle, through the C ABI.  Same rule as the TRMM:
|gpu − ref| <= 1e-3·sqrt(n) + 2^-10·|ref|; integer inputs bit-exact."""
import numpy as np
import pytest

import oracle
import workloads
from tolerance import check_close

pytestmark = pytest.mark.gpu

VARIANTS = [("L", True), ("L", False), ("U", True), ("U", False)]


def _inputs(n, m, seed, uplo, other_fill=0.0):
    rng = np.random.default_rng(seed)
    S = workloads.uniform_f16(rng, (n, n))
    D = workloads.uniform_f16(rng, (n,), 0.5, 1.5)
    B = workloads.uniform_f16(rng, (n, m))
    A = np.tril(S, -1) if uplo == "L" else np.triu(S, 1)
    A[np.arange(n), np.arange(n)] = D
    if other_fill != 0.0:
        A[np.triu_indices(n, 1) if uplo == "L" else np.tril_indices(n, -1)] = other_fill
    return np.ascontiguousarray(A.T), np.ascontiguousarray(B.T)


def run(hg, A_cm, B_cm, alpha, uplo, trans, leaf=256):
    import torch
    dev = torch.device("cuda:0")
    n, m = A_cm.shape[0], B_cm.shape[0]
    print(f"[trmm-variant] n={n} m={m} uplo={uplo} trans={trans} leaf={leaf}", flush=True)
    A = torch.from_numpy(A_cm).to(dev)
    B = torch.from_numpy(B_cm).to(dev)
    Out = torch.full((m, n), float("nan"), dtype=torch.float32, device=dev)
    hg.trmm(A, B, Out, alpha, uplo, trans, leaf)
    torch.cuda.synchronize()
    return Out.cpu().numpy()


def _ref(A_cm, B_cm, alpha, uplo, trans):
    return oracle.trmm(A_cm, B_cm, alpha, oracle.LOWER if uplo == "L" else oracle.UPPER,
                       oracle.TRANS if trans else oracle.NOTRANS)


@pytest.mark.parametrize("uplo,trans", VARIANTS)
@pytest.mark.parametrize("n,m,leaf", [(1, 1, 256), (2, 5, 256), (300, 77, 256), (1000, 50, 100),
                                      (2048, 300, 256), (4096, 256, 256), (777, 64, 64),
                                      # n a multiple of 64 with boundaries off the 64 grid (pieces
                                      # of 160): the per-level schedule on the 16-byte copies of A
                                      (2560, 100, 256)])
def test_parity(hg, uplo, trans, n, m, leaf):
    A_cm, B_cm = _inputs(n, m, n + m, uplo)
    got = run(hg, A_cm, B_cm, -0.75, uplo, trans, leaf)
    check_close(got, _ref(A_cm, B_cm, -0.75, uplo, trans), n, f"{uplo}{'T' if trans else 'N'} n={n} m={m}")


@pytest.mark.parametrize("uplo,trans", VARIANTS)
def test_other_triangle_never_read(hg, uplo, trans):
    n, m = 700, 33
    A0, B_cm = _inputs(n, m, 5, uplo)
    Ax, _ = _inputs(n, m, 5, uplo, np.nan)
    assert np.array_equal(run(hg, A0, B_cm, 1.0, uplo, trans).view(np.uint32),
                          run(hg, Ax, B_cm, 1.0, uplo, trans).view(np.uint32))


@pytest.mark.parametrize("uplo,trans", VARIANTS)
def test_integer_bit_exact(hg, uplo, trans):
    rng = np.random.default_rng(8)
    n, m = 1024, 96
    T = (np.tril if uplo == "L" else np.triu)(workloads.integer_f16(rng, (n, n)))
    B = workloads.integer_f16(rng, (n, m))
    A_cm, B_cm = np.ascontiguousarray(T.T), np.ascontiguousarray(B.T)
    got = run(hg, A_cm, B_cm, 1.0, uplo, trans)
    assert np.array_equal(got.astype(np.float64), _ref(A_cm, B_cm, 1.0, uplo, trans))


def test_lower_trans_is_trmm_lower_trans_bits(hg):
    import torch
    n, m = 2048, 512
    A_cm, B_cm = _inputs(n, m, 9, "L")
    got = run(hg, A_cm, B_cm, 1.25, "L", True)
    dev = torch.device("cuda:0")
    Out = torch.empty((m, n), dtype=torch.float32, device=dev)
    hg.trmm_lower_trans(torch.from_numpy(A_cm).to(dev), torch.from_numpy(B_cm).to(dev), Out, 1.25)
    torch.cuda.synchronize()
    assert np.array_equal(got.view(np.uint32), Out.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("uplo,trans", [("L", False), ("U", False)])
def test_8192_sampled(hg, uplo, trans):
    """n = m = 8192 for the non-transposed variants (the page's usage call is
    lower, non-transposed), 1024 sampled entries."""
    n = m = 8192
    A_cm, B_cm = _inputs(n, m, 11, uplo)
    got = run(hg, A_cm, B_cm, 1.0, uplo, trans)
    ri, cj = workloads.sample_indices(11, n, m)
    ref = oracle.trmm_sampled(A_cm, B_cm, ri, cj, 1.0, oracle.LOWER if uplo == "L" else oracle.UPPER,
                              oracle.TRANS if trans else oracle.NOTRANS)
    check_close(got[cj, ri], ref, n, f"{uplo}N 8192 sampled")


# ---- The one-launch schedule of all four variants (at least two 256×256
# output tiles per CU: m·n >= 2^25).  Upper/transposed and lower/non-transposed
# walk each tile's K from 0 up to its diagonal block (the triangle on the other
# side of the GEMM view); the other two walk down from it.
# (768, 44288, 768): one leaf of 3 tile columns (an odd count) over 173 tile
# rows (odd), so the job list has paired middle-column tiles and a lone one.
ONE_LAUNCH = [(4096, 8192, 256), (2048, 16384, 256), (4096, 8192, 512), (768, 44288, 768)]


@pytest.mark.parametrize("uplo,trans", VARIANTS)
@pytest.mark.parametrize("n,m,leaf", ONE_LAUNCH)
def test_one_launch_sampled(hg, uplo, trans, n, m, leaf):
    A_cm, B_cm = _inputs(n, m, n + m + leaf, uplo)
    got = run(hg, A_cm, B_cm, 0.5, uplo, trans, leaf)
    assert np.isfinite(got).all()
    ri, cj = workloads.sample_indices(n + leaf, n, m)
    ref = oracle.trmm_sampled(A_cm, B_cm, ri, cj, 0.5, oracle.LOWER if uplo == "L" else oracle.UPPER,
                              oracle.TRANS if trans else oracle.NOTRANS)
    check_close(got[cj, ri], ref, n, f"{uplo}{'T' if trans else 'N'} one launch n={n} m={m} leaf={leaf}")


@pytest.mark.parametrize("uplo,trans", VARIANTS)
def test_one_launch_integer_bit_exact(hg, uplo, trans):
    rng = np.random.default_rng(41)
    n, m = 2048, 16384
    T = (np.tril if uplo == "L" else np.triu)(workloads.integer_f16(rng, (n, n)))
    B = workloads.integer_f16(rng, (n, m))
    A_cm, B_cm = np.ascontiguousarray(T.T), np.ascontiguousarray(B.T)
    got = run(hg, A_cm, B_cm, 1.0, uplo, trans)
    ri, cj = workloads.sample_indices(43, n, m, 4096)
    exact = oracle.trmm_sampled(A_cm, B_cm, ri, cj, 1.0, oracle.LOWER if uplo == "L" else oracle.UPPER,
                                oracle.TRANS if trans else oracle.NOTRANS)
    assert np.array_equal(got[cj, ri].astype(np.float64), exact)


@pytest.mark.parametrize("uplo,trans", VARIANTS)
def test_one_launch_other_triangle_never_read(hg, uplo, trans):
    n, m = 4096, 8192
    A0, B_cm = _inputs(n, m, 6, uplo)
    Ax, _ = _inputs(n, m, 6, uplo, np.nan)
    assert np.array_equal(run(hg, A0, B_cm, 1.0, uplo, trans).view(np.uint32),
                          run(hg, Ax, B_cm, 1.0, uplo, trans).view(np.uint32))


# ---- The one-launch schedule on 64×64 tiles (problems with too few 256×256
# tiles for that one: n <= 4096, n <= 8192 with m <= 512, or m·n² <= 2^34;
# boundaries on the 64 grid),
# all four variants, NaN in the triangle that is never read, ragged m.
# The last two have at least two 64×64 tiles per CU (the 5-stage ring), the
# very last with a ragged m.
RING_ONE_LAUNCH = [(2048, 256, 256), (1024, 100, 128), (4096, 64, 256), (2048, 1024, 256),
                   (2048, 1000, 128)]


@pytest.mark.parametrize("uplo,trans", VARIANTS)
@pytest.mark.parametrize("n,m,leaf", RING_ONE_LAUNCH)
def test_ring_one_launch_parity(hg, uplo, trans, n, m, leaf):
    A_cm, B_cm = _inputs(n, m, 3 * n + m + leaf, uplo, np.nan)
    got = run(hg, A_cm, B_cm, -0.75, uplo, trans, leaf)
    A0, _ = _inputs(n, m, 3 * n + m + leaf, uplo)
    check_close(got, _ref(A0, B_cm, -0.75, uplo, trans), n,
                f"{uplo}{'T' if trans else 'N'} ring one launch n={n} m={m} leaf={leaf}")


@pytest.mark.parametrize("uplo,trans", VARIANTS)
def test_ring_one_launch_integer_bit_exact(hg, uplo, trans):
    rng = np.random.default_rng(47)
    n, m = 2048, 192
    T = (np.tril if uplo == "L" else np.triu)(workloads.integer_f16(rng, (n, n)))
    B = workloads.integer_f16(rng, (n, m))
    A_cm, B_cm = np.ascontiguousarray(T.T), np.ascontiguousarray(B.T)
    got = run(hg, A_cm, B_cm, 1.0, uplo, trans)
    assert np.array_equal(got.astype(np.float64), _ref(A_cm, B_cm, 1.0, uplo, trans))


# ---- A with a padded leading dimension.  n a multiple of 64: the variants
# that copy A (all but lower/transposed) take the 16-byte copy kernel when
# lda is a multiple of 8 (pad 8) and the element-wise one otherwise (pad 3);
# n = 2560 runs the per-level schedule (reversing copies for two variants),
# n = 2048 with m = 300 the one-launch schedule on 64×64 tiles.
@pytest.mark.parametrize("uplo,trans", VARIANTS)
@pytest.mark.parametrize("n,m,pad", [(2560, 100, 3), (2560, 100, 8), (2048, 300, 8)])
def test_padded_lda(hg, uplo, trans, n, m, pad):
    import torch
    dev = torch.device("cuda:0")
    A_cm, B_cm = _inputs(n, m, n + m + pad, uplo, other_fill=np.nan)
    Ap = torch.full((n, n + pad), float("nan"), dtype=torch.float16, device=dev)
    Ap[:, :n] = torch.from_numpy(A_cm).to(dev)
    print(f"[trmm-variant] padded lda n={n} m={m} pad={pad} uplo={uplo} trans={trans}", flush=True)
    Out = torch.full((m, n), float("nan"), dtype=torch.float32, device=dev)
    hg.trmm(Ap[:, :n], torch.from_numpy(B_cm).to(dev), Out, 0.75, uplo, trans)
    torch.cuda.synchronize()
    got = Out.cpu().numpy()
    ref = _ref(np.where(np.isnan(A_cm), np.float16(0), A_cm), B_cm, 0.75, uplo, trans)
    check_close(got, ref, n, f"padded lda {uplo}{'T' if trans else 'N'} n={n} pad={pad}")


@pytest.mark.parametrize("uplo,trans", VARIANTS)
def test_one_launch_ragged_tile_rows(hg, uplo, trans):
    """m = 16484 gives 65 tile rows of 256, the last holding 100 rows of Out's
    transpose (columns of B), with 8 tile columns at n = 2048: the 256×256
    one-launch schedule, whose last row of tiles takes the edge epilogue.
    Every entry of B's last 100 columns against the oracle, plus the usual
    1024 samples."""
    n, m = 2048, 16484
    A_cm, B_cm = _inputs(n, m, 61, uplo)
    got = run(hg, A_cm, B_cm, 0.5, uplo, trans)
    assert np.isfinite(got).all()
    u = oracle.LOWER if uplo == "L" else oracle.UPPER
    t = oracle.TRANS if trans else oracle.NOTRANS
    jj, ii = np.meshgrid(np.arange(m - 100, m), np.arange(n), indexing="ij")
    ri, cj = ii.ravel(), jj.ravel()
    ref = oracle.trmm_sampled(A_cm, B_cm, ri, cj, 0.5, u, t)
    check_close(got[cj, ri], ref, n, f"{uplo}{'T' if trans else 'N'} ragged tile row")
    ri, cj = workloads.sample_indices(n + m, n, m)
    ref = oracle.trmm_sampled(A_cm, B_cm, ri, cj, 0.5, u, t)
    check_close(got[cj, ri], ref, n, f"{uplo}{'T' if trans else 'N'} n={n} m={m} sampled")
