"""GPU parity of trsm_lower_trans (X = α·A⁻ᵀ·B, A lower) against the fp64
oracle ("异构计算中高性能TRMM与TRSM的递归算法实现" §2.3), through the C ABI.

Rule (tests/tolerance.py, check_trsm): the residual Aᵀ·X − α·B of the GPU
result within the elementwise bound of the solve's fp16 roundings, and
‖X − X_oracle‖ per column within ‖A⁻¹‖₂ times that bound.  Integer cases whose
every intermediate is exact in fp16 must match the oracle bit for bit.
"""
import numpy as np
import pytest

import oracle
import workloads
from tolerance import check_trsm, trsm_leaves

pytestmark = pytest.mark.gpu


def _inputs(n, m, seed):
    return workloads.trsm_inputs(workloads.TrsmWorkload("t", n, m, 1.0, 256, seed))


def run(hg, A_cm, B_cm, alpha=1.0, leaf=256, pad=0, work_fill=None):
    """Solve on the GPU; A_cm (n, n) and B_cm (m, n) in the column-major
    convention.  `pad` adds columns to every leading dimension.  Out starts
    as NaN (the solve must write every element before reading it)."""
    import torch
    dev = torch.device("cuda:0")
    n, m = A_cm.shape[0], B_cm.shape[0]
    print(f"[trsm] n={n} m={m} alpha={alpha} leaf={leaf} pad={pad}", flush=True)
    A = torch.zeros((n, n + pad), dtype=torch.float16, device=dev)[:, :n]
    A.copy_(torch.from_numpy(A_cm))
    B = torch.zeros((m, n + pad), dtype=torch.float16, device=dev)[:, :n]
    B.copy_(torch.from_numpy(B_cm))
    Out = torch.full((m, n + pad), float("nan"), dtype=torch.float32, device=dev)[:, :n]
    work = None
    if work_fill is not None:
        need = hg.trsm_workspace_size(n, m, leaf)
        work = torch.full((max(need, 1),), work_fill, dtype=torch.uint8, device=dev)
    hg.trsm_lower_trans(A, B, Out, alpha, leaf, work)
    torch.cuda.synchronize()
    return Out.cpu().numpy().astype(np.float64)


SHAPES = [
    (1, 1, 256), (2, 3, 256), (8, 8, 256), (64, 17, 256), (255, 64, 256), (256, 256, 256),
    (257, 100, 256), (300, 77, 256), (512, 513, 256), (777, 128, 64), (1000, 50, 100),
    (1024, 1000, 256), (2048, 256, 256), (200, 40, 16), (130, 70, 33), (1536, 300, 256),
    (512, 31, 256), (1024, 33, 256), (4096, 96, 256),
]


@pytest.mark.parametrize("n,m,leaf", SHAPES)
def test_parity(hg, n, m, leaf):
    A_cm, B_cm = _inputs(n, m, 70 + n + m)
    alpha = -1.25
    X = run(hg, A_cm, B_cm, alpha, leaf)
    ref = oracle.trsm_lower_trans(A_cm, B_cm, alpha)
    check_trsm(X.T, A_cm.T, B_cm.T, alpha, leaf, Xref=ref.T, what=f"n={n} m={m} leaf={leaf}")


@pytest.mark.parametrize("n,m,leaf,pad", [(520, 37, 256, 3), (333, 20, 64, 1), (1024, 64, 256, 8)])
def test_leading_dimensions(hg, n, m, leaf, pad):
    A_cm, B_cm = _inputs(n, m, 5 + pad)
    X = run(hg, A_cm, B_cm, 0.5, leaf, pad=pad)
    ref = oracle.trsm_lower_trans(A_cm, B_cm, 0.5)
    check_trsm(X.T, A_cm.T, B_cm.T, 0.5, leaf, Xref=ref.T, what=f"pad={pad}")


def _integer_case(n, m, leaf, seed, density):
    """Unit lower A with sparse ±1 entries and B in {-1, 0, 1}: X, every leaf
    right-hand side, every leaf inverse and every partial sum are integers of
    magnitude <= 2048, so fp16 and fp32 hold them exactly (checked here)."""
    rng = np.random.default_rng(seed)
    A = np.eye(n)
    low = np.tril_indices(n, -1)
    pick = rng.random(low[0].size) < density
    A[low[0][pick], low[1][pick]] = rng.choice([-1.0, 1.0], pick.sum())
    B = rng.integers(-1, 2, (n, m)).astype(np.float64)
    A_cm = np.ascontiguousarray(A.T.astype(np.float16))
    B_cm = np.ascontiguousarray(B.T.astype(np.float16))
    X = oracle.trsm_lower_trans(A_cm, B_cm).T
    ok = np.abs(X).max() <= 2048
    # |R| <= |B| + Σ|A(k,i)|·|X(k)| bounds every partial sum of every update
    ok &= (np.abs(B) + np.abs(np.tril(A, -1)).T @ np.abs(X)).max() <= 2048
    for o, s in trsm_leaves(n, leaf):
        # A_LL⁻ᵀ (the oracle's solve against the identity): the leaf inverse's entries
        V = oracle.trsm_lower_trans(np.ascontiguousarray(A[o:o + s, o:o + s].T.astype(np.float16)),
                                    np.eye(s, dtype=np.float16))
        ok &= np.abs(V).max() <= 2048 and np.array_equal(V, np.round(V))
    return A_cm, B_cm, X, bool(ok)


@pytest.mark.parametrize("n,m,leaf,seed,density", [(512, 100, 256, 1, 0.004), (700, 33, 64, 2, 0.005),
                                                   (1024, 256, 256, 3, 0.002), (300, 40, 16, 4, 0.01)])
def test_integer_bit_exact(hg, n, m, leaf, seed, density):
    A_cm, B_cm, X, ok = _integer_case(n, m, leaf, seed, density)
    assert ok, "integer case does not stay exact in fp16; pick another seed"
    got = run(hg, A_cm, B_cm, 1.0, leaf)
    assert np.array_equal(got, X.T)


def test_identity_gives_alpha_B(hg):
    n, m = 600, 70
    rng = np.random.default_rng(9)
    B_cm = workloads.uniform_f16(rng, (m, n))
    got = run(hg, np.eye(n, dtype=np.float16), B_cm, 2.0)
    assert np.array_equal(got, 2.0 * B_cm.astype(np.float64))


def test_upper_triangle_never_read(hg):
    n, m = 700, 40
    A_cm, B_cm = _inputs(n, m, 11)
    ref = run(hg, A_cm, B_cm, 1.0)
    A = A_cm.T.copy()
    A[np.triu_indices(n, 1)] = np.nan
    got = run(hg, np.ascontiguousarray(A.T), B_cm, 1.0)
    assert np.array_equal(got, ref)


def test_workspace_contents_ignored_and_deterministic(hg):
    n, m = 900, 64
    A_cm, B_cm = _inputs(n, m, 12)
    a = run(hg, A_cm, B_cm, 1.0, work_fill=0)
    b = run(hg, A_cm, B_cm, 1.0, work_fill=0xFF)      # workspace of NaN patterns
    assert np.array_equal(a, b)


def test_alpha_zero_writes_zeros(hg):
    n, m = 300, 20
    A_cm = np.full((n, n), np.nan, dtype=np.float16)
    B_cm = np.full((m, n), np.nan, dtype=np.float16)
    got = run(hg, A_cm, B_cm, 0.0)
    assert np.array_equal(got, np.zeros((m, n)))


def test_workload_8192_sampled_columns(hg):
    """The 8192×8192 solve at its full size, as the benchmark runs it: 32
    columns (the first, the last and 30 random) against the oracle's fp64
    solve of those columns, and their residuals."""
    w = workloads.TRSM_WORKLOADS["trsm_8192"]
    A_cm, B_cm = workloads.trsm_inputs(w)
    X = run(hg, A_cm, B_cm, w.alpha, w.leaf)
    cols = np.unique(np.concatenate([[0, w.m - 1],
                                     np.random.default_rng(w.seed + 1000).integers(0, w.m, 30)]))
    ref = oracle.trsm_lower_trans_cols(A_cm, B_cm, cols, w.alpha)
    A = A_cm.T.astype(np.float64)
    check_trsm(X[cols].T, A, B_cm[cols].T.astype(np.float64), w.alpha, w.leaf, Xref=ref.T,
               what="trsm_8192")


def test_vector_and_elementwise_paths_agree(hg):
    """n = 1024 with aligned operands (vector loads and stores) against the
    same system with a leading dimension that is not a multiple of 8 (the
    element-wise paths of the leaf step and the GEMM updates): both within
    the rule, and within a few fp16 roundings of each other."""
    n, m = 1024, 200
    A_cm, B_cm = _inputs(n, m, 21)
    vec = run(hg, A_cm, B_cm, 1.0, 256)
    ew = run(hg, A_cm, B_cm, 1.0, 256, pad=3)
    ref = oracle.trsm_lower_trans(A_cm, B_cm, 1.0)
    check_trsm(vec.T, A_cm.T, B_cm.T, 1.0, 256, Xref=ref.T, what="vector paths")
    check_trsm(ew.T, A_cm.T, B_cm.T, 1.0, 256, Xref=ref.T, what="element-wise paths")
    assert np.abs(vec - ew).max() <= 8 * 2.0 ** -11 * np.abs(ref).max()
