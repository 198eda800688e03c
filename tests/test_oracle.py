"""Pins for the fp64 oracle: checks against facts that do not come from the
oracle itself (closed forms, a library routine, brute force, the block
identity of the triangular multiply).  CPU only.

Pages: "Nvidia Tensor Core-MMA PTX编程入门" §4 (HGEMM layouts),
"GPU架构与CUDA" 共享内存与分块 / 混合精度核函数, "异构计算中高性能TRMM与TRSM的
递归算法实现" §2.1–§2.2 (TRMM definition and block recursion).
"""
import itertools

import numpy as np
import pytest

import oracle
import workloads


def _np_gemm(A, Bt, alpha=1.0, beta=0.0, C=None):
    """numpy fp64 matmul as an independent special case of the definition."""
    r = alpha * (A.astype(np.float64) @ Bt.astype(np.float64).T)
    if beta != 0.0:
        r = r + beta * C.astype(np.float64)
    return r


# ---------------------------------------------------------------- decoding
def test_half_decode_matches_numpy_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # sign of zero is kept
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


# ---------------------------------------------------------------- HGEMM pins
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (17, 9, 33), (32, 32, 16), (5, 64, 100)])
def test_hgemm_matches_numpy_matmul(M, N, K):
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    A = workloads.uniform_f16(rng, (M, K))
    Bt = workloads.uniform_f16(rng, (N, K))
    C = workloads.uniform_f16(rng, (M, N))
    for alpha, beta in [(1.0, 0.0), (1.5, 0.5), (-2.0, 1.0)]:
        got = oracle.hgemm(A, Bt, alpha, beta, C)
        ref = _np_gemm(A, Bt, alpha, beta, C)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_hgemm_brute_force_python_loops():
    rng = np.random.default_rng(7)
    M, N, K = 4, 3, 6
    A = workloads.uniform_f16(rng, (M, K))
    Bt = workloads.uniform_f16(rng, (N, K))
    C = workloads.uniform_f16(rng, (M, N)).astype(np.float32)
    got = oracle.hgemm(A, Bt, 0.75, -1.25, C)
    for i in range(M):
        for j in range(N):
            s = 0.0
            for k in range(K):
                s += float(A[i, k]) * float(Bt[j, k])
            assert got[i, j] == pytest.approx(0.75 * s - 1.25 * float(C[i, j]), abs=1e-13)


def test_hgemm_strided_operands():
    """General leading dimensions: a view into a wider buffer gives the same result."""
    rng = np.random.default_rng(11)
    Abig = workloads.uniform_f16(rng, (9, 40))
    Bbig = workloads.uniform_f16(rng, (7, 48))
    Cbig = workloads.uniform_f16(rng, (9, 20))
    A, Bt, C = Abig[:, :33], Bbig[:, :33], Cbig[:, :7]
    got = oracle.hgemm(A, Bt, 1.0, 2.0, C)
    ref = oracle.hgemm(A.copy(), Bt.copy(), 1.0, 2.0, C.copy())
    assert np.array_equal(got, ref)
    np.testing.assert_allclose(got, _np_gemm(A, Bt, 1.0, 2.0, C), rtol=1e-12, atol=1e-12)


def test_identity_gives_A_exactly():
    rng = np.random.default_rng(3)
    A = workloads.uniform_f16(rng, (37, 29))
    I = np.eye(29, dtype=np.float16)        # B = I; its column-major storage is I too
    got = oracle.hgemm(A, I)
    assert np.array_equal(got, A.astype(np.float64))


@pytest.mark.parametrize("K", [1, 256, 1000])
def test_all_ones_give_K(K):
    A = np.ones((6, K), np.float16)
    Bt = np.ones((5, K), np.float16)
    assert np.all(oracle.hgemm(A, Bt) == K)
    C = np.ones((6, 5), np.float16)
    assert np.all(oracle.hgemm(A, Bt, 1.5, 0.5, C) == 1.5 * K + 0.5)


def test_rank_one_outer_product():
    vals = np.array([-2, -1, -0.5, 0.5, 1, 2], np.float16)
    u, v = vals, vals[::-1].copy()
    K = 77
    A = np.repeat(u[:, None], K, axis=1)
    Bt = np.repeat(v[:, None], K, axis=1)
    got = oracle.hgemm(A, Bt)
    assert np.array_equal(got, K * np.outer(u.astype(np.float64), v.astype(np.float64)))


def test_beta_zero_does_not_read_C():
    rng = np.random.default_rng(5)
    A = workloads.uniform_f16(rng, (8, 16))
    Bt = workloads.uniform_f16(rng, (8, 16))
    C = np.full((8, 8), np.nan, np.float16)
    got = oracle.hgemm(A, Bt, 1.0, 0.0, C)
    assert np.isfinite(got).all()
    assert np.array_equal(got, oracle.hgemm(A, Bt))


def test_alpha_zero_does_not_read_A_B():
    A = np.full((4, 9), np.nan, np.float16)
    Bt = np.full((3, 9), np.inf, np.float16)
    C = np.arange(12, dtype=np.float32).reshape(4, 3)
    got = oracle.hgemm(A, Bt, 0.0, 2.0, C)
    assert np.array_equal(got, 2.0 * C.astype(np.float64))


def test_integer_inputs_exact():
    rng = np.random.default_rng(9)
    A = workloads.integer_f16(rng, (20, 300))
    Bt = workloads.integer_f16(rng, (30, 300))
    got = oracle.hgemm(A, Bt)
    exact = A.astype(np.int64) @ Bt.astype(np.int64).T
    assert np.array_equal(got, exact.astype(np.float64))


def test_hgemm_sampled_equals_full():
    rng = np.random.default_rng(12)
    A = workloads.uniform_f16(rng, (50, 70))
    Bt = workloads.uniform_f16(rng, (40, 70))
    C = workloads.uniform_f16(rng, (50, 40))
    full = oracle.hgemm(A, Bt, 1.5, 0.5, C)
    ri, cj = workloads.sample_indices(1, 50, 40, 64)
    got = oracle.hgemm_sampled(A, Bt, ri, cj, 1.5, 0.5, C)
    assert np.array_equal(got, full[ri, cj])


def test_swap_symmetry():
    """(A·B)ᵀ = Bᵀ·Aᵀ: swapping operand roles transposes the result."""
    rng = np.random.default_rng(13)
    A = workloads.uniform_f16(rng, (11, 23))
    Bt = workloads.uniform_f16(rng, (7, 23))
    assert np.array_equal(oracle.hgemm(Bt, A), oracle.hgemm(A, Bt).T)


# ---------------------------------------------------------------- TRMM pins
def _trmm_inputs(n, m, seed, upper_fill=0.0):
    rng = np.random.default_rng(seed)
    S = workloads.uniform_f16(rng, (n, n))
    D = workloads.uniform_f16(rng, (n,), 0.5, 1.5)
    B = workloads.uniform_f16(rng, (n, m))
    A = np.tril(S, -1)
    A[np.arange(n), np.arange(n)] = D
    A[np.triu_indices(n, 1)] = upper_fill
    return A, B     # logical [row, col]


@pytest.mark.parametrize("n,m", [(1, 1), (5, 3), (33, 17), (64, 8)])
def test_trmm_matches_dense_zeroed_upper(n, m):
    A, B = _trmm_inputs(n, m, n + m)
    got = oracle.trmm_lower_trans(np.ascontiguousarray(A.T), np.ascontiguousarray(B.T), 1.25)
    ref = 1.25 * (np.tril(A).astype(np.float64).T @ B.astype(np.float64))
    np.testing.assert_allclose(got.T, ref, rtol=1e-12, atol=1e-12)


def test_trmm_brute_force_python_loops():
    A, B = _trmm_inputs(6, 4, 1)
    got = oracle.trmm_lower_trans(np.ascontiguousarray(A.T), np.ascontiguousarray(B.T), -0.5)
    for i in range(6):
        for j in range(4):
            s = sum(float(A[k, i]) * float(B[k, j]) for k in range(i, 6))
            assert got[j, i] == pytest.approx(-0.5 * s, abs=1e-13)


def test_trmm_upper_triangle_not_referenced():
    A0, B = _trmm_inputs(40, 9, 2, 0.0)
    An, _ = _trmm_inputs(40, 9, 2, np.nan)
    Ab, _ = _trmm_inputs(40, 9, 2, 1e4)
    ref = oracle.trmm_lower_trans(np.ascontiguousarray(A0.T), np.ascontiguousarray(B.T))
    for Ax in (An, Ab):
        got = oracle.trmm_lower_trans(np.ascontiguousarray(Ax.T), np.ascontiguousarray(B.T))
        assert np.array_equal(got, ref)


def test_trmm_identity():
    rng = np.random.default_rng(4)
    B = workloads.uniform_f16(rng, (30, 6))
    I = np.eye(30, dtype=np.float16)
    got = oracle.trmm_lower_trans(I, np.ascontiguousarray(B.T), 2.0)
    assert np.array_equal(got, 2.0 * B.T.astype(np.float64))


def test_trmm_tril_ones_closed_form():
    n, m = 50, 5
    A = np.tril(np.ones((n, n), np.float16))
    B = np.ones((n, m), np.float16)
    got = oracle.trmm_lower_trans(np.ascontiguousarray(A.T), np.ascontiguousarray(B.T), 3.0)
    expect = 3.0 * (n - np.arange(n, dtype=np.float64))
    assert np.array_equal(got, np.tile(expect, (m, 1)))


def test_trmm_block_recursion_identity():
    """With A = [[A11,0],[A21,A22]]: Aᵀ·B = [A11ᵀB1 + A21ᵀB2 ; A22ᵀB2]."""
    n, m, h = 24, 5, 10
    A, B = _trmm_inputs(n, m, 8)
    full = oracle.trmm_lower_trans(np.ascontiguousarray(A.T), np.ascontiguousarray(B.T))
    top = oracle.trmm_lower_trans(np.ascontiguousarray(A[:h, :h].T), np.ascontiguousarray(B[:h].T))
    upd = oracle.hgemm(np.ascontiguousarray(B[h:].T), np.ascontiguousarray(A[h:, :h].T))  # (A21ᵀB2)ᵀ
    bot = oracle.trmm_lower_trans(np.ascontiguousarray(A[h:, h:].T), np.ascontiguousarray(B[h:].T))
    np.testing.assert_allclose(full[:, :h], top + upd, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(full[:, h:], bot, rtol=1e-12, atol=1e-12)


def test_trmm_integer_exact():
    rng = np.random.default_rng(21)
    n, m = 70, 11
    A = np.tril(workloads.integer_f16(rng, (n, n)))
    B = workloads.integer_f16(rng, (n, m))
    got = oracle.trmm_lower_trans(np.ascontiguousarray(A.T), np.ascontiguousarray(B.T))
    exact = A.astype(np.int64).T @ B.astype(np.int64)
    assert np.array_equal(got, exact.T.astype(np.float64))


def test_trmm_sampled_equals_full():
    A, B = _trmm_inputs(45, 13, 6)
    Acm, Bcm = np.ascontiguousarray(A.T), np.ascontiguousarray(B.T)
    full = oracle.trmm_lower_trans(Acm, Bcm, 0.5)
    ri, cj = workloads.sample_indices(4, 45, 13, 100)
    got = oracle.trmm_lower_trans_sampled(Acm, Bcm, ri, cj, 0.5)
    assert np.array_equal(got, full[cj, ri])


def test_empty_shapes():
    A = np.zeros((0, 5), np.float16)
    Bt = np.zeros((3, 5), np.float16)
    assert oracle.hgemm(A, Bt).shape == (0, 3)
    A = np.ones((4, 0), np.float16)
    Bt = np.ones((3, 0), np.float16)
    assert np.array_equal(oracle.hgemm(A, Bt), np.zeros((4, 3)))


# ---- TRSM: X = α·A⁻ᵀ·B, A lower ("异构计算中高性能TRMM与TRSM的递归算法实现" §2.3) ----

def _trsm_inputs(n, m, seed, upper_fill=0.0):
    """Well-conditioned lower A (the TRSM workload recipe) and B, as logical
    [row, col] fp16 arrays; the strict upper triangle holds `upper_fill`."""
    A_cm, B_cm = workloads.trsm_inputs(workloads.TrsmWorkload("t", n, m, 1.0, 256, seed))
    A = A_cm.T.copy()
    if upper_fill != 0.0:
        A[np.triu_indices(n, 1)] = upper_fill
    return A, np.ascontiguousarray(B_cm.T)


def _trsm(A, B, alpha=1.0):
    """oracle.trsm_lower_trans on logical [row, col] arrays; returns X [row, col]."""
    return oracle.trsm_lower_trans(np.ascontiguousarray(A.T), np.ascontiguousarray(B.T), alpha).T


def test_trsm_identity_returns_alpha_B():
    rng = np.random.default_rng(40)
    B = workloads.uniform_f16(rng, (37, 6))
    I = np.eye(37, dtype=np.float16)
    assert np.array_equal(_trsm(I, B, 1.5), 1.5 * B.astype(np.float64))


def test_trsm_diagonal_powers_of_two():
    rng = np.random.default_rng(41)
    n, m = 29, 5
    e = rng.integers(-3, 4, n)
    A = np.diag(np.ldexp(1.0, e)).astype(np.float16)
    B = workloads.uniform_f16(rng, (n, m))
    expect = -0.75 * B.astype(np.float64) / np.ldexp(1.0, e)[:, None]
    assert np.array_equal(_trsm(A, B, -0.75), expect)


@pytest.mark.parametrize("n,m", [(1, 1), (7, 3), (64, 5), (300, 4)])
def test_trsm_matches_scipy_solve_triangular(n, m):
    import scipy.linalg
    A, B = _trsm_inputs(n, m, 42 + n)
    got = _trsm(A, B, 1.25)
    ref = scipy.linalg.solve_triangular(A.astype(np.float64), 1.25 * B.astype(np.float64),
                                        trans="T", lower=True)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12 * max(1.0, np.abs(ref).max()))


def test_trsm_brute_force_inverse():
    A, B = _trsm_inputs(6, 4, 43)
    ref = np.linalg.inv(A.astype(np.float64).T) @ (0.5 * B.astype(np.float64))
    np.testing.assert_allclose(_trsm(A, B, 0.5), ref, rtol=0, atol=1e-13)


def test_trsm_residual_is_zero():
    """The defining equation Aᵀ·X = α·B, evaluated by a matrix product."""
    A, B = _trsm_inputs(500, 9, 44)
    X = _trsm(A, B, 2.0)
    r = A.astype(np.float64).T @ X - 2.0 * B.astype(np.float64)
    assert np.abs(r).max() < 1e-12


def test_trsm_upper_triangle_not_referenced():
    A0, B = _trsm_inputs(40, 7, 45)
    ref = _trsm(A0, B)
    for fill in (np.nan, 1e4):
        Ax, _ = _trsm_inputs(40, 7, 45, fill)
        assert np.array_equal(_trsm(Ax, B), ref)


def test_trsm_undoes_trmm_exactly():
    """Integer unit lower A and integer B: C = Aᵀ·B is exact (oracle TRMM, an
    independent routine), fits fp16 exactly, and the solve returns B."""
    rng = np.random.default_rng(46)
    n, m = 120, 8
    A = np.eye(n)
    low = np.tril_indices(n, -1)
    pick = rng.random(low[0].size) < 0.02
    A[low[0][pick], low[1][pick]] = rng.choice([-1.0, 1.0], pick.sum())
    A = A.astype(np.float16)
    B = workloads.integer_f16(rng, (n, m), -3, 3)
    C = oracle.trmm_lower_trans(np.ascontiguousarray(A.T), np.ascontiguousarray(B.T)).T
    assert np.abs(C).max() <= 2048 and np.array_equal(C, np.round(C))
    X = _trsm(A, C.astype(np.float16))
    assert np.array_equal(X, B.astype(np.float64))


def test_trsm_bidiagonal_closed_form():
    """A = I + subdiagonal a (entries in {-1, 0, 1}): A⁻¹(r, c) is the product
    of -a_k over c <= k < r, so X = α·(A⁻¹)ᵀ·B exactly (integers)."""
    rng = np.random.default_rng(47)
    n, m = 60, 4
    a = rng.integers(-1, 2, n - 1).astype(np.float64)
    A = np.eye(n)
    A[np.arange(1, n), np.arange(n - 1)] = a
    inv = np.zeros((n, n))
    for c in range(n):
        inv[c, c] = 1.0
        for r in range(c + 1, n):
            inv[r, c] = inv[r - 1, c] * -a[r - 1]
    B = workloads.integer_f16(rng, (n, m), -2, 2)
    expect = 3.0 * (inv.T @ B.astype(np.float64))
    assert np.array_equal(_trsm(A.astype(np.float16), B, 3.0), expect)


def test_trsm_cols_equals_full():
    A, B = _trsm_inputs(77, 12, 48)
    Acm, Bcm = np.ascontiguousarray(A.T), np.ascontiguousarray(B.T)
    full = oracle.trsm_lower_trans(Acm, Bcm, -1.5)
    cols = np.array([11, 0, 5, 5, 3])
    assert np.array_equal(oracle.trsm_lower_trans_cols(Acm, Bcm, cols, -1.5), full[cols])


# ---- HGEMM with fused bias and ReLU ("GPU架构与CUDA", 核函数融合) ----

def test_bias_act_matches_numpy():
    rng = np.random.default_rng(50)
    M, N, K = 13, 9, 21
    A = workloads.uniform_f16(rng, (M, K))
    Bt = workloads.uniform_f16(rng, (N, K))
    C = workloads.uniform_f16(rng, (M, N))
    bias = rng.uniform(-2, 2, N).astype(np.float32)
    t = 1.5 * (A.astype(np.float64) @ Bt.astype(np.float64).T) + 0.25 * C.astype(np.float64) \
        + bias.astype(np.float64)
    got = oracle.hgemm_bias_act(A, Bt, 1.5, 0.25, C, bias, oracle.ACT_RELU)
    np.testing.assert_allclose(got, np.maximum(t, 0.0), rtol=1e-13, atol=1e-13)
    got = oracle.hgemm_bias_act(A, Bt, 1.5, 0.25, C, bias, oracle.ACT_NONE)
    np.testing.assert_allclose(got, t, rtol=1e-13, atol=1e-13)


def test_bias_act_brute_force_python_loops():
    rng = np.random.default_rng(51)
    A = workloads.integer_f16(rng, (4, 6))
    Bt = workloads.integer_f16(rng, (5, 6))
    bias = np.array([3.5, -7.0, 0.0, 100.0, -100.0], np.float32)
    got = oracle.hgemm_bias_act(A, Bt, 2.0, 0.0, None, bias, oracle.ACT_RELU)
    for i in range(4):
        for j in range(5):
            t = 2.0 * sum(float(A[i, k]) * float(Bt[j, k]) for k in range(6)) + float(bias[j])
            assert got[i, j] == (0.0 if t < 0 else t)


def test_bias_act_reduces_to_hgemm():
    """No bias and no activation is the plain HGEMM (an independent routine)."""
    rng = np.random.default_rng(52)
    A = workloads.uniform_f16(rng, (17, 33))
    Bt = workloads.uniform_f16(rng, (11, 33))
    C = workloads.uniform_f16(rng, (17, 11)).astype(np.float32)
    assert np.array_equal(oracle.hgemm_bias_act(A, Bt, 0.75, -1.0, C),
                          oracle.hgemm(A, Bt, 0.75, -1.0, C))


def test_bias_only_rows_and_relu_threshold():
    """alpha = 0: every row is the bias (+0 plus the bias: a -0 bias gives +0);
    ReLU zeroes exactly the negative entries, to +0, and a NaN passes
    through."""
    A = np.full((3, 4), np.nan, np.float16)
    Bt = np.full((6, 4), np.nan, np.float16)
    bias = np.array([-1.0, -0.0, 0.0, 1e-30, np.nan, 5.0], np.float32)
    got = oracle.hgemm_bias_act(A, Bt, 0.0, 0.0, None, bias, oracle.ACT_RELU)
    expect = np.array([0.0, 0.0, 0.0, np.float32(1e-30), np.nan, 5.0])
    for row in got:
        assert np.array_equal(row, expect, equal_nan=True)
        assert not np.signbit(row[0]) and not np.signbit(row[1])


# ---- GEMM on bf16 operands ("GPU架构与CUDA", 混合精度核函数) ----

def _bf16_values(bits):
    """numpy's reading of bf16 bit patterns: the upper half of a float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_bf16_decode_matches_numpy_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = _bf16_values(bits)
    got = np.array([oracle.bf16_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (7, 5, 33), (16, 24, 64)])
def test_gemm_bf16_matches_numpy(M, N, K):
    rng = np.random.default_rng(M * N + K)
    A = workloads.uniform_bf16(rng, (M, K))
    Bt = workloads.uniform_bf16(rng, (N, K))
    C32 = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    C16 = workloads.uniform_bf16(rng, (M, N))
    prod = _bf16_values(A) @ _bf16_values(Bt).T
    np.testing.assert_allclose(oracle.gemm_bf16(A, Bt, 1.5, 0.5, C32),
                               1.5 * prod + 0.5 * C32.astype(np.float64), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(oracle.gemm_bf16(A, Bt, -1.0, 2.0, C16, cin_bf16=True),
                               -prod + 2.0 * _bf16_values(C16), rtol=1e-13, atol=1e-13)


def test_gemm_bf16_equals_fp16_routine_on_common_values():
    """Integers in [-4, 4] are exact in both formats: the bf16 routine and the
    fp16 routine (independent decoders and loops) agree exactly."""
    rng = np.random.default_rng(60)
    A16 = workloads.integer_f16(rng, (20, 50))
    B16 = workloads.integer_f16(rng, (15, 50))
    Abf = workloads.to_bf16_bits(A16.astype(np.float32))
    Bbf = workloads.to_bf16_bits(B16.astype(np.float32))
    assert np.array_equal(oracle.gemm_bf16(Abf, Bbf, 2.0), oracle.hgemm(A16, B16, 2.0))


def test_gemm_bf16_sampled_equals_full():
    rng = np.random.default_rng(61)
    A = workloads.uniform_bf16(rng, (40, 70))
    Bt = workloads.uniform_bf16(rng, (30, 70))
    full = oracle.gemm_bf16(A, Bt, 0.75)
    ri, cj = workloads.sample_indices(2, 40, 30, 64)
    assert np.array_equal(oracle.gemm_bf16_sampled(A, Bt, ri, cj, 0.75), full[ri, cj])


# ---- Fused bias and ReLU on bf16 operands, and the fused definition at
# sampled entries ("GPU架构与CUDA", 核函数融合 and 混合精度核函数) ----

def _relu(t):
    return np.where(t < 0, 0.0, t)


def test_bf16_bias_act_matches_numpy():
    rng = np.random.default_rng(53)
    M, N, K = 12, 10, 37
    A = workloads.uniform_bf16(rng, (M, K))
    Bt = workloads.uniform_bf16(rng, (N, K))
    C32 = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    C16 = workloads.uniform_bf16(rng, (M, N))
    bias = rng.uniform(-2, 2, N).astype(np.float32)
    prod = _bf16_values(A) @ _bf16_values(Bt).T
    t = 1.25 * prod + 0.5 * C32.astype(np.float64) + bias.astype(np.float64)
    got = oracle.gemm_bf16_bias_act(A, Bt, 1.25, 0.5, C32, bias, oracle.ACT_RELU)
    np.testing.assert_allclose(got, _relu(t), rtol=1e-13, atol=1e-13)
    got = oracle.gemm_bf16_bias_act(A, Bt, 1.25, 0.5, C32, bias, oracle.ACT_NONE)
    np.testing.assert_allclose(got, t, rtol=1e-13, atol=1e-13)
    t16 = -prod + 2.0 * _bf16_values(C16) + bias.astype(np.float64)
    got = oracle.gemm_bf16_bias_act(A, Bt, -1.0, 2.0, C16, bias, oracle.ACT_RELU, cin_bf16=True)
    np.testing.assert_allclose(got, _relu(t16), rtol=1e-13, atol=1e-13)


def test_bf16_bias_act_brute_force_python_loops():
    rng = np.random.default_rng(54)
    A16 = workloads.integer_f16(rng, (4, 6))
    B16 = workloads.integer_f16(rng, (5, 6))
    A = workloads.to_bf16_bits(A16.astype(np.float32))
    Bt = workloads.to_bf16_bits(B16.astype(np.float32))
    bias = np.array([3.5, -7.0, 0.0, 100.0, -100.0], np.float32)
    got = oracle.gemm_bf16_bias_act(A, Bt, 2.0, 0.0, None, bias, oracle.ACT_RELU)
    for i in range(4):
        for j in range(5):
            t = 2.0 * sum(float(A16[i, k]) * float(B16[j, k]) for k in range(6)) + float(bias[j])
            assert got[i, j] == (0.0 if t < 0 else t)


def test_bf16_bias_act_reduces_to_gemm_bf16():
    """No bias and no activation is the plain bf16 GEMM (an independent
    routine), bit for bit."""
    rng = np.random.default_rng(55)
    A = workloads.uniform_bf16(rng, (17, 33))
    Bt = workloads.uniform_bf16(rng, (11, 33))
    C = rng.uniform(-1, 1, (17, 11)).astype(np.float32)
    assert np.array_equal(oracle.gemm_bf16_bias_act(A, Bt, 0.75, -1.0, C),
                          oracle.gemm_bf16(A, Bt, 0.75, -1.0, C))


def test_bf16_bias_act_alpha_zero_rows_are_the_bias():
    """alpha = 0, beta = 0: A and B (NaN) are not read, every row is act(bias)."""
    A = np.full((3, 4), 0x7fc0, np.uint16)
    Bt = np.full((6, 4), 0x7fc0, np.uint16)
    bias = np.array([-1.0, -0.0, 0.0, 1e-30, np.nan, 5.0], np.float32)
    got = oracle.gemm_bf16_bias_act(A, Bt, 0.0, 0.0, None, bias, oracle.ACT_RELU)
    expect = np.array([0.0, 0.0, 0.0, np.float32(1e-30), np.nan, 5.0])
    for row in got:
        assert np.array_equal(row, expect, equal_nan=True)


@pytest.mark.parametrize("bf16", [False, True])
def test_bias_act_sampled_matches_numpy(bf16):
    """The sampled fused definition against numpy at the sampled entries,
    with beta != 0, a bias and ReLU (fp16 C for fp16 operands, bf16 C for
    bf16 operands)."""
    rng = np.random.default_rng(56 + bf16)
    M, N, K = 40, 30, 70
    if bf16:
        A = workloads.uniform_bf16(rng, (M, K))
        Bt = workloads.uniform_bf16(rng, (N, K))
        C = workloads.uniform_bf16(rng, (M, N))
        av, bv, cv = _bf16_values(A), _bf16_values(Bt), _bf16_values(C)
    else:
        A = workloads.uniform_f16(rng, (M, K))
        Bt = workloads.uniform_f16(rng, (N, K))
        C = workloads.uniform_f16(rng, (M, N))
        av, bv, cv = A.astype(np.float64), Bt.astype(np.float64), C.astype(np.float64)
    bias = rng.uniform(-2, 2, N).astype(np.float32)
    ri, cj = workloads.sample_indices(9, M, N, 200)
    t = -0.75 * (av @ bv.T) + 1.5 * cv + bias.astype(np.float64)[None, :]
    got = oracle.gemm_bias_act_sampled(A, Bt, ri, cj, -0.75, 1.5, C, bias, oracle.ACT_RELU,
                                       bf16=bf16, cin_bf16=bf16)
    np.testing.assert_allclose(got, _relu(t)[ri, cj], rtol=1e-13, atol=1e-13)
    got = oracle.gemm_bias_act_sampled(A, Bt, ri, cj, -0.75, 1.5, C, bias, oracle.ACT_NONE,
                                       bf16=bf16, cin_bf16=bf16)
    np.testing.assert_allclose(got, t[ri, cj], rtol=1e-13, atol=1e-13)


def test_bias_act_sampled_equals_full_routines():
    """Sampled = the full fp16 and bf16 fused routines (each pinned above) at
    the sampled entries; beta = 0 does not read a NaN C."""
    rng = np.random.default_rng(58)
    M, N, K = 33, 45, 50
    A = workloads.uniform_f16(rng, (M, K))
    Bt = workloads.uniform_f16(rng, (N, K))
    C = workloads.uniform_f16(rng, (M, N)).astype(np.float32)
    bias = rng.uniform(-2, 2, N).astype(np.float32)
    ri, cj = workloads.sample_indices(3, M, N, 300)
    full = oracle.hgemm_bias_act(A, Bt, 1.5, 0.5, C, bias, oracle.ACT_RELU)
    assert np.array_equal(oracle.gemm_bias_act_sampled(A, Bt, ri, cj, 1.5, 0.5, C, bias,
                                                       oracle.ACT_RELU), full[ri, cj])
    Ab = workloads.uniform_bf16(rng, (M, K))
    Bb = workloads.uniform_bf16(rng, (N, K))
    full = oracle.gemm_bf16_bias_act(Ab, Bb, 2.0, 0.0, None, bias, oracle.ACT_RELU)
    nanC = np.full((M, N), np.nan, np.float32)
    got = oracle.gemm_bias_act_sampled(Ab, Bb, ri, cj, 2.0, 0.0, nanC, bias, oracle.ACT_RELU,
                                       bf16=True)
    assert np.array_equal(got, full[ri, cj])


# ---- TRMM variants: op(A) = A or Aᵀ, A lower or upper ----

@pytest.mark.parametrize("uplo", [oracle.LOWER, oracle.UPPER])
@pytest.mark.parametrize("trans", [oracle.NOTRANS, oracle.TRANS])
def test_trmm_variants_match_numpy(uplo, trans):
    rng = np.random.default_rng(70 + 2 * uplo + trans)
    n, m = 37, 6
    A = workloads.uniform_f16(rng, (n, n))
    B = workloads.uniform_f16(rng, (n, m))
    T = (np.tril if uplo == oracle.LOWER else np.triu)(A.astype(np.float64))
    op = T.T if trans == oracle.TRANS else T
    got = oracle.trmm(np.ascontiguousarray(A.T), np.ascontiguousarray(B.T), -1.5, uplo, trans)
    np.testing.assert_allclose(got.T, -1.5 * (op @ B.astype(np.float64)), rtol=1e-12, atol=1e-12)


def test_trmm_lower_trans_variant_equals_dedicated_routine():
    A, B = _trmm_inputs(60, 9, 71)
    Acm, Bcm = np.ascontiguousarray(A.T), np.ascontiguousarray(B.T)
    assert np.array_equal(oracle.trmm(Acm, Bcm, 0.5, oracle.LOWER, oracle.TRANS),
                          oracle.trmm_lower_trans(Acm, Bcm, 0.5))


@pytest.mark.parametrize("uplo", [oracle.LOWER, oracle.UPPER])
@pytest.mark.parametrize("trans", [oracle.NOTRANS, oracle.TRANS])
def test_trmm_variants_other_triangle_not_referenced(uplo, trans):
    rng = np.random.default_rng(72)
    n, m = 25, 4
    A = workloads.uniform_f16(rng, (n, n))
    B = workloads.uniform_f16(rng, (n, m))
    other = np.triu_indices(n, 1) if uplo == oracle.LOWER else np.tril_indices(n, -1)
    Ax = A.copy()
    Ax[other] = np.nan
    ref = oracle.trmm(np.ascontiguousarray(A.T), np.ascontiguousarray(B.T), 1.0, uplo, trans)
    got = oracle.trmm(np.ascontiguousarray(Ax.T), np.ascontiguousarray(B.T), 1.0, uplo, trans)
    assert np.array_equal(got, ref)


def test_trmm_upper_notrans_brute_force():
    rng = np.random.default_rng(73)
    A = workloads.integer_f16(rng, (5, 5))
    B = workloads.integer_f16(rng, (5, 3))
    got = oracle.trmm(np.ascontiguousarray(A.T), np.ascontiguousarray(B.T), 2.0, oracle.UPPER,
                      oracle.NOTRANS)
    for i in range(5):
        for j in range(3):
            assert got[j, i] == 2.0 * sum(float(A[i, k]) * float(B[k, j]) for k in range(i, 5))


@pytest.mark.parametrize("uplo", [oracle.LOWER, oracle.UPPER])
@pytest.mark.parametrize("trans", [oracle.NOTRANS, oracle.TRANS])
def test_trmm_variants_sampled_equals_full(uplo, trans):
    rng = np.random.default_rng(74)
    n, m = 45, 13
    A = workloads.uniform_f16(rng, (n, n))
    B = workloads.uniform_f16(rng, (n, m))
    Acm, Bcm = np.ascontiguousarray(A.T), np.ascontiguousarray(B.T)
    full = oracle.trmm(Acm, Bcm, 0.5, uplo, trans)
    ri, cj = workloads.sample_indices(4, n, m, 100)
    assert np.array_equal(oracle.trmm_sampled(Acm, Bcm, ri, cj, 0.5, uplo, trans), full[cj, ri])
