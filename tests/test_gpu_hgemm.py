"""HGEMM parity on the GPU: the HIP path (through the C ABI) against the fp64
oracle, element by element, to |err| <= 1e-3·sqrt(K) + 2^-10·|ref|, plus the
exact pins (identity, all-ones, rank-1, integers, scaling, NaN read rules,
guard bands, determinism).

Problem statement: "Nvidia Tensor Core-MMA PTX编程入门" §4 (layouts);
masking of ragged tiles: "GPU架构与CUDA" 共享内存与分块; fp32 accumulation:
its 混合精度核函数 section.
"""
import itertools

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


def run(hg, A, Bt, C, alpha=1.0, beta=0.0):
    """A, Bt, C numpy; returns the device result as numpy."""
    Cd = dev(C)
    hg.hgemm(dev(A), dev(Bt), Cd, alpha, beta)
    torch.cuda.synchronize()
    return Cd.cpu().numpy()


def rnd(seed, shape, lo=-1.0, hi=1.0):
    return workloads.uniform_f16(np.random.default_rng(seed), shape, lo, hi)


# ------------------------------------------------------------ the workloads
@pytest.mark.parametrize("name", ["hgemm_256", "hgemm_1000_ragged", "hgemm_4096"])
def test_workload_full_parity(hg, name):
    w = workloads.WORKLOADS[name]
    print(f"[case] {name} M={w.M} N={w.N} K={w.K}", flush=True)
    A, Bt, C = workloads.gemm_inputs(w)
    out = run(hg, A, Bt, C, w.alpha, w.beta)
    ref = oracle.hgemm(A, Bt, w.alpha, w.beta, C)
    check_close(out, ref, w.K, name)


def test_workload_8192_sampled_parity(hg):
    """8192³ with fp32 output, in the benchmark's launch configuration; the
    oracle evaluates 1024 sampled entries (4 corners included)."""
    w = workloads.WORKLOADS["hgemm_8192"]
    print(f"[case] hgemm_8192 sampled", flush=True)
    A, Bt, C = workloads.gemm_inputs(w)
    out = run(hg, A, Bt, C, w.alpha, w.beta)
    assert np.isfinite(out).all()
    ri, cj = workloads.sample_indices(w.seed, w.M, w.N)
    ref = oracle.hgemm_sampled(A, Bt, ri, cj, w.alpha, w.beta, C)
    check_close(out[ri, cj], ref, w.K, "hgemm_8192 sampled")
    # property at full size: output statistics match U[-1,1]·U[-1,1] sums,
    # std = sqrt(K)/3 (each product has variance 1/9)
    assert abs(out.std() / (np.sqrt(w.K) / 3) - 1) < 0.01


# ------------------------------------------------------------ brute force
SMALL = list(range(1, 18))
EDGE = [31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]


def _shapes():
    rng = np.random.default_rng(123)
    tiny = list(itertools.product(SMALL, SMALL, SMALL))
    pick = [tiny[i] for i in rng.choice(len(tiny), 150, replace=False)]
    edge = list(itertools.product(EDGE, EDGE, EDGE))
    pick += [edge[i] for i in rng.choice(len(edge), 150, replace=False)]
    return pick


def test_brute_force_small_and_boundary_shapes(hg):
    for t, (M, N, K) in enumerate(_shapes()):
        A = rnd(1000 + t, (M, K))
        Bt = rnd(2000 + t, (N, K))
        C = rnd(3000 + t, (M, N))
        alpha, beta = (1.0, 0.0) if t % 2 else (0.75, -1.5)
        for odt in (np.float16, np.float32):
            Cx = C.astype(odt)
            out = run(hg, A, Bt, Cx, alpha, beta)
            ref = oracle.hgemm(A, Bt, alpha, beta, Cx)
            check_close(out, ref, K, f"M={M} N={N} K={K} out={odt.__name__}")


@pytest.mark.parametrize("M,N,K", [(1500, 1700, 600), (4000, 4100, 1000), (2048, 2048, 136),
                                   (640, 384, 8200)])
def test_tile_families_ragged(hg, M, N, K):
    """Shapes that select each tile family, with ragged M/N edges and K tails."""
    print(f"[case] tile family M={M} N={N} K={K}", flush=True)
    A = rnd(M, (M, K))
    Bt = rnd(N, (N, K))
    C = rnd(K, (M, N)).astype(np.float32)
    out = run(hg, A, Bt, C, 1.25, 0.5)
    ri, cj = workloads.sample_indices(M + N + K, M, N, 4096)
    ref = oracle.hgemm_sampled(A, Bt, ri, cj, 1.25, 0.5, C)
    check_close(out[ri, cj], ref, K, "sampled")
    # full check of the last tile row/column band (the masked edge tiles)
    rows = np.arange(M - 70, M)
    ref_edge = oracle.hgemm(np.ascontiguousarray(A[rows]), Bt, 1.25, 0.5,
                            np.ascontiguousarray(C[rows]))
    check_close(out[rows], ref_edge, K, "last rows")


@pytest.mark.parametrize("K", [8, 40, 96, 256, 1000])
def test_big_tiles_short_k(hg, K):
    """Large M, N (256×256 tiles, the pipelined path) with short K: the
    prefetch ring runs past the end of K on most iterations; repeated so
    that back-to-back workgroups on a CU reuse the same LDS."""
    print(f"[case] big tiles short K={K}", flush=True)
    M, N = 4096, 3840
    A = rnd(K, (M, K))
    Bt = rnd(K + 1, (N, K))
    ri, cj = workloads.sample_indices(K, M, N, 4096)
    ref = oracle.hgemm_sampled(A, Bt, ri, cj)
    Ad, Btd = dev(A), dev(Bt)
    first = None
    for rep in range(3):
        Cd = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        hg.hgemm(Ad, Btd, Cd)
        torch.cuda.synchronize()
        out = Cd.cpu().numpy()
        check_close(out[ri, cj], ref, K, f"K={K} rep {rep}")
        if first is None:
            first = out
        else:
            assert np.array_equal(first.view(np.uint32), out.view(np.uint32))


def test_unaligned_operands(hg):
    """Odd leading dimensions and 2-byte-offset bases take the element-wise
    load path; results still match the oracle."""
    M, N, K = 129, 77, 301
    Abuf = rnd(1, (M, K + 3))
    Bbuf = rnd(2, (N * (K + 5) + 1,))
    Cbuf = np.full((M, N + 3), np.nan, np.float32)
    Ad = dev(Abuf)[:, 1:K + 1]                                  # lda = K+3, odd offset
    Bflat = dev(Bbuf)
    Btd = torch.as_strided(Bflat[1:], (N, K), (K + 5, 1))       # ldb = K+5, misaligned
    Cd = dev(Cbuf)[:, 1:N + 1]                                  # ldc = N+3, misaligned
    hg.hgemm(Ad, Btd, Cd, 1.0, 0.0)
    torch.cuda.synchronize()
    A = Abuf[:, 1:K + 1]
    Bt = np.lib.stride_tricks.as_strided(Bbuf[1:], (N, K), ((K + 5) * 2, 2))
    ref = oracle.hgemm(np.ascontiguousarray(A), np.ascontiguousarray(Bt))
    out = Cd.cpu().numpy()
    check_close(out, ref, K, "unaligned")


# ------------------------------------------------------------ exact pins
@pytest.mark.parametrize("odt", [np.float16, np.float32])
def test_identity_exact(hg, odt):
    A = rnd(5, (300, 260))
    I = np.eye(260, dtype=np.float16)
    out = run(hg, A, I, np.full((300, 260), np.nan, odt))
    assert np.array_equal(out.astype(np.float64), A.astype(np.float64))


@pytest.mark.parametrize("K", [256, 1000, 4096, 8192])
def test_all_ones(hg, K):
    A = np.ones((130, K), np.float16)
    Bt = np.ones((70, K), np.float16)
    out = run(hg, A, Bt, np.zeros((130, 70), np.float32))
    assert np.all(out == K)
    C = np.ones((130, 70), np.float16)
    out = run(hg, A, Bt, C, 1.5, 0.5)
    # fp16 RNE of 1.5K + 0.5: e.g. 1500.5 -> 1500 at K = 1000
    assert np.all(out == np.float16(1.5 * K + 0.5))


def test_rank_one(hg):
    vals = np.array([-2, -1, -0.5, 0.5, 1, 2], np.float16)
    rng = np.random.default_rng(8)
    u = rng.choice(vals, 200)
    v = rng.choice(vals, 150)
    K = 96
    A = np.repeat(u[:, None], K, axis=1)
    Bt = np.repeat(v[:, None], K, axis=1)
    out = run(hg, A, Bt, np.zeros((200, 150), np.float32))
    assert np.array_equal(out, K * np.outer(u.astype(np.float32), v.astype(np.float32)))


@pytest.mark.parametrize("odt", [np.float16, np.float32])
def test_integer_inputs_bit_exact(hg, odt):
    """Integer entries in [-4, 4]: every partial sum is exact in fp32, so the
    output must equal the round-to-nearest-even of the exact value."""
    rng = np.random.default_rng(31)
    M, N, K = 333, 290, 1000
    A = workloads.integer_f16(rng, (M, K))
    Bt = workloads.integer_f16(rng, (N, K))
    out = run(hg, A, Bt, np.zeros((M, N), odt))
    exact = A.astype(np.int64) @ Bt.astype(np.int64).T
    assert np.array_equal(out, exact.astype(odt))


def test_fp16_output_rounds_to_nearest_even(hg):
    """Exact results in (2048, 4096) where fp16 spacing is 2: odd integers sit
    half-way, RNE picks the even mantissa (2051 -> 2052, 2049 -> 2048), while
    truncation would give 2050 / 2048."""
    targets = np.array([2049, 2051, 2053, 2055, 3001, 4093], np.int64)
    K = 1024
    A = np.zeros((len(targets), K), np.float16)
    for r, t in enumerate(targets):
        q, rem = divmod(int(t), 4)
        A[r, :q] = 4
        A[r, q] = rem
    Bt = np.ones((8, K), np.float16)
    out = run(hg, A, Bt, np.zeros((len(targets), 8), np.float16))
    expect = targets.astype(np.float64).astype(np.float16)
    assert np.array_equal(out[:, 0], expect)
    assert out[1, 0] == 2052 and out[0, 0] == 2048


def test_alpha_power_of_two_scaling_exact(hg):
    A = rnd(40, (260, 300))
    Bt = rnd(41, (190, 300))
    base = run(hg, A, Bt, np.zeros((260, 190), np.float32))
    for a in (2.0, 0.5, -4.0):
        out = run(hg, A, Bt, np.zeros((260, 190), np.float32), a)
        assert np.array_equal(out, a * base)


def test_alpha_zero_reads_neither_A_nor_B(hg):
    A = np.full((70, 50), np.nan, np.float16)
    Bt = np.full((60, 50), np.inf, np.float16)
    C = rnd(3, (70, 60)).astype(np.float32)
    out = run(hg, A, Bt, C, 0.0, 2.0)
    assert np.array_equal(out, 2.0 * C)
    out = run(hg, A, Bt, np.full((70, 60), np.nan, np.float32), 0.0, 0.0)
    assert np.array_equal(out, np.zeros((70, 60), np.float32))


def test_K_zero_scales_C(hg):
    Ad = torch.empty((5, 0), dtype=torch.float16, device=DEV)
    Bd = torch.empty((7, 0), dtype=torch.float16, device=DEV)
    C = rnd(4, (5, 7))
    Cd = dev(C)
    hg.hgemm(Ad, Bd, Cd, 1.0, -0.5)
    torch.cuda.synchronize()
    assert np.array_equal(Cd.cpu().numpy(), (np.float32(-0.5) * C.astype(np.float32)).astype(np.float16))


@pytest.mark.parametrize("odt", [np.float16, np.float32])
def test_beta_zero_ignores_nan_C(hg, odt):
    A = rnd(6, (300, 200))
    Bt = rnd(7, (260, 200))
    out = run(hg, A, Bt, np.full((300, 260), np.nan, odt))
    assert np.isfinite(out).all()
    check_close(out, oracle.hgemm(A, Bt), 200, "beta=0 NaN C")


def test_swap_symmetry(hg):
    """hgemm(B as A, A as B) = Cᵀ — checks indexing without the oracle."""
    A = rnd(9, (517, 333))
    Bt = rnd(10, (261, 333))
    c1 = run(hg, A, Bt, np.zeros((517, 261), np.float32))
    c2 = run(hg, Bt, A, np.zeros((261, 517), np.float32))
    check_close(c2, c1.T.astype(np.float64), 333, "swap")


def test_deterministic(hg):
    w = workloads.WORKLOADS["hgemm_1000_ragged"]
    A, Bt, C = workloads.gemm_inputs(w)
    outs = [run(hg, A, Bt, C, w.alpha, w.beta) for _ in range(3)]
    assert all(np.array_equal(outs[0].view(np.uint16), o.view(np.uint16)) for o in outs[1:])


@pytest.mark.parametrize("odt", [np.float16, np.float32])
def test_guard_bands_untouched(hg, odt):
    """Sentinels in the ldc padding and in rows past M survive."""
    M, N, K, pad, extra = 301, 259, 130, 13, 5
    A = rnd(11, (M, K))
    Bt = rnd(12, (N, K))
    sentinel = odt(-12345.0) if odt == np.float32 else np.float16(-1234.0)
    big = np.full((M + extra, N + pad), sentinel, odt)
    bigd = dev(big)
    view = bigd[:M, :N]
    hg.hgemm(dev(A), dev(Bt), view, 1.0, 0.0)
    torch.cuda.synchronize()
    got = bigd.cpu().numpy()
    assert np.all(got[:, N:] == sentinel)
    assert np.all(got[M:, :] == sentinel)
    check_close(got[:M, :N], oracle.hgemm(A, Bt), K, "window")


def test_empty(hg):
    A = torch.empty((0, 8), dtype=torch.float16, device=DEV)
    Bt = torch.empty((4, 8), dtype=torch.float16, device=DEV)
    C = torch.empty((0, 4), dtype=torch.float32, device=DEV)
    hg.hgemm(A, Bt, C)
    A = torch.empty((3, 8), dtype=torch.float16, device=DEV)
    Bt = torch.empty((0, 8), dtype=torch.float16, device=DEV)
    C = torch.empty((3, 0), dtype=torch.float32, device=DEV)
    hg.hgemm(A, Bt, C)
    torch.cuda.synchronize()


@pytest.mark.parametrize("odt", [np.float16, np.float32])
def test_big_tiles_padded_window(hg, odt):
    """256×256-tile kernel (≥ 256 tiles) writing into a window of a larger
    buffer: ldc ≠ N, a nonzero element offset, ragged M and N (interior tiles
    and edge tiles side by side); the padding keeps its sentinels and every
    element of the window matches the oracle."""
    M, N, K, pad = 4096 + 37, 4096 + 64, 192, 12
    print(f"[case] big-tile window M={M} N={N} K={K} ldc={N + pad + 4} {np.dtype(odt).name}", flush=True)
    A = rnd(21, (M, K))
    Bt = rnd(22, (N, K))
    sentinel = odt(-12345.0) if odt == np.float32 else np.float16(-1234.0)
    big = np.full((M + 2, N + pad + 4), sentinel, odt)
    bigd = dev(big)
    view = bigd[1:M + 1, 4:N + 4]            # element offset ldc + 4 (a multiple of 4)
    hg.hgemm(dev(A), dev(Bt), view, 0.5, 0.0)
    torch.cuda.synchronize()
    got = bigd.cpu().numpy()
    assert np.all(got[0] == sentinel) and np.all(got[M + 1] == sentinel)
    assert np.all(got[:, :4] == sentinel) and np.all(got[:, N + 4:] == sentinel)
    check_close(got[1:M + 1, 4:N + 4], 0.5 * oracle.hgemm(A, Bt), K, "window")
