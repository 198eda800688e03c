"""Pass/fail rule shared by the parity tests.

|gpu - ref| <= 1e-3·sqrt(K) + 2^-10·|ref| elementwise, ref in fp64.  The
absolute term covers fp32 accumulation over K terms of size <= 1; the relative
term covers the final rounding to fp16 (at most 2^-11·|ref|).
"""
import numpy as np


def bound(K, ref, rel=2.0 ** -10):
    return 1e-3 * np.sqrt(max(int(K), 1)) + rel * np.abs(ref)


# bf16 output: rounding to bf16 (8-bit significand) is off by at most
# 2^-9·|ref|; the relative term doubles it as the fp16 rule doubles 2^-11.
REL_BF16 = 2.0 ** -8


def check_close(out, ref, K, what="", rel=2.0 ** -10):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert out.shape == ref.shape, (out.shape, ref.shape)
    err = np.abs(out - ref)
    lim = bound(K, ref, rel)
    bad = ~(err <= lim)          # NaN in out counts as a failure
    if bad.any():
        idx = np.argwhere(bad)[:5]
        details = ", ".join(f"{tuple(i)}: got {out[tuple(i)]!r} ref {ref[tuple(i)]!r}" for i in idx)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} entries out of tolerance "
                             f"(max err {np.nanmax(err):.3g}); first: {details}")
    return float(err.max()) if err.size else 0.0


# ---- Triangular solve X = α·A⁻ᵀ·B -----------------------------------------
#
# The solve's result has no closed-form error bound as tight as the GEMM's: its
# fp16 roundings (the right-hand side of each leaf, the inverse of each leaf
# block, the solved rows fed to the updates) propagate through A⁻ᵀ.  The rule
# is the probabilistic rounding-error model of Higham and Mary (SIAM J. Sci.
# Comput. 41(5), 2019): independent rounding errors δ_k, |δ_k| <= u, give
# |Σ_k t_k·δ_k| <= λ·u·‖t‖₂ except with probability <= 2·exp(-λ²/2).  With
# λ = 8 (about 3e-14 per element) the residual r = Aᵀ·X − α·B of the GPU result
# must satisfy, for every row i in leaf I and column j,
#   |r_ij| <= λ·u16·‖(A(k,i)·X(k,j))_{k>i}‖₂         fp16 copies of solved rows
#           + u16·|R_ij|                              leaf right-hand side rounding
#           + λ·u16·sqrt(Σ_{p,l} A(p,i)²·V(l,p)²·R_lj²)  fp16 leaf inverse V = A_II⁻¹
#           + λ·u32·sqrt(n)·‖(A(k,i)·X(k,j))_k‖₂      fp32 accumulation
#           + u16·|α·B_ij|
# where R_I = A_IIᵀ·X_I is the leaf's right-hand side.  From |r| the forward
# error follows rigorously: ‖X_j − X*_j‖₂ <= ‖A⁻¹‖₂·‖r_j‖₂ for every column.
U16 = 2.0 ** -11
U32 = 2.0 ** -24
LAMBDA = 8.0


def trsm_leaves(n, leaf):
    """Leaf blocks (offset, size) of the recursion: split at floor(s/2) until
    s <= leaf ("异构计算中高性能TRMM与TRSM的递归算法实现" §2.1)."""
    out = []

    def rec(o, s):
        if s <= leaf:
            out.append((o, s))
            return
        rec(o, s // 2)
        rec(o + s // 2, s - s // 2)
    if n:
        rec(0, n)
    return out


def trsm_residual_bound(A, B, X, alpha, leaf, lam=LAMBDA):
    """Elementwise bound on |Aᵀ·X − α·B| (see above).  A: (n, n) lower
    triangular fp64; B, X: (n, c) fp64 for any set of c columns."""
    import scipy.linalg
    n = A.shape[0]
    A = np.tril(A)
    A2 = A * A
    X2 = X * X
    full = A2.T @ X2                                   # Σ_k A(k,i)²·X(k,j)²
    strict = np.maximum(full - np.diag(A2)[:, None] * X2, 0.0)
    b = lam * U16 * np.sqrt(strict) + lam * U32 * np.sqrt(max(n, 1)) * np.sqrt(full)
    b += U16 * np.abs(alpha * B)
    for o, s in trsm_leaves(n, leaf):
        AI = A[o:o + s, o:o + s]
        R = AI.T @ X[o:o + s]
        V = scipy.linalg.solve_triangular(AI, np.eye(s), lower=True)
        y = (V * V).T @ (R * R)
        b[o:o + s] += U16 * np.abs(R) + lam * U16 * np.sqrt((AI * AI).T @ y)
    return b


def inv_norm2(A, iters=40):
    """‖A⁻¹‖₂ of a lower triangular A: exact SVD for n <= 2048, else power
    iteration on (AᵀA)⁻¹ (a lower estimate, converged to a few digits here,
    enlarged by 1.25)."""
    import scipy.linalg
    n = A.shape[0]
    if n <= 2048:
        inv = scipy.linalg.solve_triangular(A, np.eye(n), lower=True)
        return float(np.linalg.norm(inv, 2))
    v = np.random.default_rng(0).standard_normal(n)
    lam = 0.0
    for _ in range(iters):
        w = scipy.linalg.solve_triangular(A, v, lower=True, trans="T")
        w = scipy.linalg.solve_triangular(A, w, lower=True)
        lam = np.linalg.norm(w)
        v = w / lam
    return 1.25 * float(np.sqrt(lam))


def check_trsm(X, A, B, alpha, leaf, Xref=None, ainv2=None, what=""):
    """Residual rule elementwise; with Xref (the oracle's solution of the same
    columns), the forward bound per column.  Arrays are logical [row, col]."""
    X = np.asarray(X, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    assert np.isfinite(X).all(), f"{what}: non-finite entries"
    r = np.tril(A).T @ X - alpha * B
    lim = trsm_residual_bound(A, B, X, alpha, leaf)
    bad = ~(np.abs(r) <= lim)
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: residual of {int(bad.sum())} of {bad.size} entries over the "
                             f"bound; first ({i}, {j}): |r| {abs(r[i, j]):.3g} > {lim[i, j]:.3g} "
                             f"(max ratio {np.max(np.abs(r) / lim):.3g})")
    ratio = float(np.max(np.abs(r) / lim)) if r.size else 0.0
    if Xref is not None:
        if ainv2 is None:
            ainv2 = inv_norm2(np.tril(A))
        tol = ainv2 * np.linalg.norm(lim, axis=0)
        err = np.abs(X - Xref)
        badc = ~(err <= tol[None, :])
        if badc.any():
            i, j = np.argwhere(badc)[0]
            raise AssertionError(f"{what}: |X - oracle| over the forward bound at ({i}, {j}): "
                                 f"{err[i, j]:.3g} > {tol[j]:.3g}")
    return ratio
