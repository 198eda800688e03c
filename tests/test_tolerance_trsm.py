"""The triangular-solve tolerance rule, checked on the CPU (no GPU, no HIP).

A numpy model of the solve's arithmetic — every fp16 rounding the library's
solve performs (leaf right-hand sides, leaf-block inverses, the solved rows the
updates read) with fp32 products — must pass the rule with room to spare, and
the same model with a plausible mistake (an update added instead of
subtracted, the wrong leaf block, the leaf inverse untransposed) must fail it.
The model shares nothing with the HIP code; it only exercises the rule.
"""
import numpy as np
import pytest
import scipy.linalg

import oracle
import workloads
from tolerance import check_trsm, trsm_leaves


def f16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def model_solve(A, B, alpha, leaf, mistake=None):
    n, m = B.shape
    out = np.zeros((n, m))
    w = np.zeros((n, m))
    inv = {}
    for o, s in trsm_leaves(n, leaf):
        inv[o] = f16(f32(scipy.linalg.solve_triangular(A[o:o + s, o:o + s], np.eye(s), lower=True)))

    def solve(o, s, touched):
        if s <= leaf:
            rhs = f16(f32(alpha * B[o:o + s] + (out[o:o + s] if touched else 0.0)))
            V = inv[o] if mistake != "untransposed" else inv[o].T
            x = f32(V.T.astype(np.float32) @ rhs.astype(np.float32))
            out[o:o + s] = x
            w[o:o + s] = f16(x)
            return
        h = s // 2
        solve(o + h, s - h, touched)
        lo = o + h if mistake != "wrong_block" else o + h - 1
        upd = f32(A[lo:lo + s - h, o:o + h].T.astype(np.float32) @ w[o + h:o + s].astype(np.float32))
        if mistake == "sign":
            upd = -upd
        out[o:o + h] = f32((out[o:o + h] if touched else 0.0) - upd)
        solve(o, h, True)

    solve(0, n, False)
    return out


def _case(n, m, seed):
    A_cm, B_cm = workloads.trsm_inputs(workloads.TrsmWorkload("t", n, m, 1.0, 256, seed))
    return A_cm.T.astype(np.float64), B_cm.T.astype(np.float64), A_cm, B_cm


@pytest.mark.parametrize("n,m,leaf", [(600, 24, 256), (1000, 16, 100), (300, 9, 33)])
def test_rounding_model_passes_with_margin(n, m, leaf):
    A, B, A_cm, B_cm = _case(n, m, 60 + n)
    X = model_solve(A, B, 1.5, leaf)
    Xref = oracle.trsm_lower_trans(A_cm, B_cm, 1.5).T
    ratio = check_trsm(X, A, B, 1.5, leaf, Xref=Xref, what="model")
    assert ratio < 0.5


@pytest.mark.parametrize("mistake", ["sign", "wrong_block", "untransposed"])
def test_rounding_model_with_a_mistake_fails(mistake):
    A, B, A_cm, B_cm = _case(600, 16, 7)
    X = model_solve(A, B, 1.0, 256, mistake)
    with pytest.raises(AssertionError):
        check_trsm(X, A, B, 1.0, 256, what=mistake)
