"""GPU parity of hg_trmm_inplace, B ← α·op(A)·B with B fp16 and overwritten
("异构计算中高性能TRMM与TRSM的递归算法实现" §2.2), against the fp64 oracle,
through the C ABI.

The product is accumulated in fp32 and rounded to fp16 once (in the
one-launch kernel's epilogue, or by a pass over the fp32 product), so the
fp16 rule of the GEMM holds: |gpu − ref| <= 1e-3·sqrt(n) + 2^-10·|ref|.  Integer inputs give
an exact fp32 product, so B must equal the oracle's product rounded to fp16
(nearest even) bit for bit.
"""
import numpy as np
import pytest

import oracle
import workloads
from tolerance import check_close

pytestmark = pytest.mark.gpu

VARIANTS = [("L", True), ("L", False), ("U", True), ("U", False)]


def _tri(rng, n, uplo):
    S = workloads.uniform_f16(rng, (n, n))
    D = workloads.uniform_f16(rng, (n,), 0.5, 1.5)
    A = np.tril(S, -1) if uplo == "L" else np.triu(S, 1)
    A[np.arange(n), np.arange(n)] = D
    return np.ascontiguousarray(A.T)


def run(hg, A_cm, B_cm, alpha, uplo, trans, leaf=256, pad=0, work_fill=None):
    import torch
    dev = torch.device("cuda:0")
    n, m = A_cm.shape[0], B_cm.shape[0]
    print(f"[trmm-inplace] n={n} m={m} uplo={uplo} trans={trans} leaf={leaf} pad={pad}", flush=True)
    A = torch.from_numpy(A_cm).to(dev)
    B = torch.zeros((m, n + pad), dtype=torch.float16, device=dev)[:, :n]
    B.copy_(torch.from_numpy(B_cm))
    work = None
    if work_fill is not None:
        need = hg.lib.hg_trmm_inplace_workspace_size(0 if uplo == "L" else 1, 1 if trans else 0, n, m)
        work = torch.full((max(need, 1),), work_fill, dtype=torch.uint8, device=dev)
    out = hg.trmm_inplace(A, B, alpha, uplo, trans, leaf, work)
    assert out is B
    torch.cuda.synchronize()
    return B.cpu().numpy()


def _ref(A_cm, B_cm, alpha, uplo, trans):
    return oracle.trmm(A_cm, B_cm, alpha, oracle.LOWER if uplo == "L" else oracle.UPPER,
                       oracle.TRANS if trans else oracle.NOTRANS)


@pytest.mark.parametrize("uplo,trans", VARIANTS)
@pytest.mark.parametrize("n,m,leaf", [(1, 1, 256), (3, 5, 256), (300, 77, 256), (1000, 50, 100),
                                      (2048, 300, 256), (777, 64, 64)])
def test_parity(hg, uplo, trans, n, m, leaf):
    rng = np.random.default_rng(n * 7 + m)
    A_cm = _tri(rng, n, uplo)
    B_cm = workloads.uniform_f16(rng, (m, n))
    got = run(hg, A_cm, B_cm, 0.75, uplo, trans, leaf)
    check_close(got, _ref(A_cm, B_cm, 0.75, uplo, trans), n,
                f"in-place {uplo}{'T' if trans else 'N'} n={n} m={m}")


@pytest.mark.parametrize("uplo,trans", VARIANTS)
def test_integer_bit_exact(hg, uplo, trans):
    rng = np.random.default_rng(31)
    n, m = 1024, 96
    T = (np.tril if uplo == "L" else np.triu)(workloads.integer_f16(rng, (n, n)))
    B = workloads.integer_f16(rng, (n, m))
    A_cm, B_cm = np.ascontiguousarray(T.T), np.ascontiguousarray(B.T)
    ref = _ref(A_cm, B_cm, 1.0, uplo, trans)
    assert np.abs(ref).max() < 65504
    got = run(hg, A_cm, B_cm, 1.0, uplo, trans)
    assert np.array_equal(got.view(np.uint16), ref.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("uplo,trans", VARIANTS)
@pytest.mark.parametrize("n,m,pad", [(1536, 200, 5), (1536, 200, 0), (2048, 1024, 0), (2048, 16384, 0),
                                     (2048, 16484, 0)])
def test_equals_out_of_place_rounded(hg, uplo, trans, n, m, pad):
    """The in-place result is hg_trmm's fp32 result rounded to nearest even,
    bit for bit, with a workspace of NaN patterns.  The out-of-place call
    gets B with the same leading dimension, so both take the same schedule:
    per level when it is padded to an odd value, in one launch otherwise
    (n = 1536, m = 200: 64×64 tiles, one workgroup per CU; n = 2048, m = 1024:
    64×64 tiles, two per CU; n = 2048, m = 16384: 256×256 tiles;
    m = 16484: the last row of 256×256 tiles holds 100 rows, edge epilogue),
    where the in-place form rounds each tile to fp16 in the kernel instead
    of rounding the fp32 product in a second pass."""
    import torch
    rng = np.random.default_rng(5 + n + m + pad)
    A_cm = _tri(rng, n, uplo)
    B_cm = workloads.uniform_f16(rng, (m, n))
    got = run(hg, A_cm, B_cm, -1.25, uplo, trans, pad=pad, work_fill=0xFF)
    dev = torch.device("cuda:0")
    Out = torch.empty((m, n), dtype=torch.float32, device=dev)
    Bd = torch.zeros((m, n + pad), dtype=torch.float16, device=dev)[:, :n]
    Bd.copy_(torch.from_numpy(B_cm))
    hg.trmm(torch.from_numpy(A_cm).to(dev), Bd, Out, -1.25, uplo, trans)
    torch.cuda.synchronize()
    want = Out.cpu().numpy().astype(np.float16)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def test_alpha_zero_writes_zeros(hg):
    n, m = 300, 20
    A_cm = np.full((n, n), np.nan, dtype=np.float16)
    B_cm = np.full((m, n), np.nan, dtype=np.float16)
    got = run(hg, A_cm, B_cm, 0.0, "U", True)
    assert np.array_equal(got.astype(np.float64), np.zeros((m, n)))


def test_8192_sampled(hg):
    """n = m = 8192, lower and not transposed (the page's usage call), 1024
    sampled entries."""
    n = m = 8192
    rng = np.random.default_rng(13)
    A_cm = _tri(rng, n, "L")
    B_cm = workloads.uniform_f16(rng, (m, n))
    got = run(hg, A_cm, B_cm, 1.0, "L", False)
    ri, cj = workloads.sample_indices(13, n, m)
    ref = oracle.trmm_sampled(A_cm, B_cm, ri, cj, 1.0, oracle.LOWER, oracle.NOTRANS)
    check_close(got[cj, ri], ref, n, "in-place 8192 sampled")
