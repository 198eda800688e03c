"""TRMM parity on the GPU: Out = alpha·Aᵀ·B with A lower triangular, by the
recursive blocking of "异构计算中高性能TRMM与TRSM的递归算法实现" §2.1–§2.2
(split at n/2, triangle-masked leaf, A21ᵀ·B2 updates through the GEMM with
beta = 1), against the fp64 oracle to |err| <= 1e-3·sqrt(n) + 2^-10·|ref|,
plus exact pins.

Column-major convention: an n×m column-major matrix is a torch (m, n) tensor
whose row j is column j.
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


def trmm_inputs(n, m, seed, upper_fill=0.0):
    rng = np.random.default_rng(seed)
    S = workloads.uniform_f16(rng, (n, n))
    D = workloads.uniform_f16(rng, (n,), 0.5, 1.5)
    B = workloads.uniform_f16(rng, (n, m))
    A = np.tril(S, -1)
    A[np.arange(n), np.arange(n)] = D
    A[np.triu_indices(n, 1)] = upper_fill
    return np.ascontiguousarray(A.T), np.ascontiguousarray(B.T)


def run(hg, A_cm, B_cm, alpha=1.0, leaf=256, by_level=False):
    m, n = B_cm.shape
    Out = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    fn = hg.trmm_lower_trans_by_level if by_level else hg.trmm_lower_trans
    fn(dev(A_cm), dev(B_cm), Out, alpha, leaf)
    torch.cuda.synchronize()
    return Out.cpu().numpy()


def test_workload_8192(hg):
    """n = m = 8192, leaf 256, in the benchmark's launch configuration:
    1024 sampled entries against the oracle, and the full result against the
    GPU GEMM on the densified (explicitly zero-upper) A — a different kernel
    path (plain tiles, no triangle mask, one K loop per output)."""
    w = workloads.WORKLOADS["trmm_8192"]
    print("[case] trmm_8192", flush=True)
    A_cm, B_cm = workloads.trmm_inputs(w)
    Ad, Bd = dev(A_cm), dev(B_cm)
    Out = torch.full((w.m, w.n), float("nan"), dtype=torch.float32, device=DEV)
    hg.trmm_lower_trans(Ad, Bd, Out, w.alpha, w.leaf)
    dense = torch.zeros((w.m, w.n), dtype=torch.float32, device=DEV)
    hg.hgemm(Bd, Ad, dense, w.alpha, 0.0)      # (Aᵀ·B)ᵀ = Bᵀ·A in the row-major view
    torch.cuda.synchronize()
    out = Out.cpu().numpy()
    ri, cj = workloads.sample_indices(w.seed, w.n, w.m)
    ref = oracle.trmm_lower_trans_sampled(A_cm, B_cm, ri, cj, w.alpha)
    check_close(out[cj, ri], ref, w.n, "trmm_8192 sampled")
    dn = dense.cpu().numpy()
    check_close(out, dn.astype(np.float64), w.n, "trmm_8192 vs dense GEMM")


@pytest.mark.parametrize("n,m", [(1, 1), (1, 7), (255, 1), (255, 256), (257, 7), (257, 256),
                                 (1000, 7), (1000, 256), (513, 100), (2048, 300)])
def test_odd_and_small_shapes_full(hg, n, m):
    print(f"[case] trmm n={n} m={m}", flush=True)
    A_cm, B_cm = trmm_inputs(n, m, n * 7 + m)
    out = run(hg, A_cm, B_cm, 0.75)
    ref = oracle.trmm_lower_trans(A_cm, B_cm, 0.75)
    check_close(out, ref, n, f"n={n} m={m}")


@pytest.mark.parametrize("leaf", [256, 128, 64, 1000, 3])
def test_leaf_invariance(hg, leaf):
    n, m = 1000, 130
    A_cm, B_cm = trmm_inputs(n, m, 77)
    out = run(hg, A_cm, B_cm, 1.0, leaf)
    ref = oracle.trmm_lower_trans(A_cm, B_cm)
    check_close(out, ref, n, f"leaf={leaf}")


def test_identity_exact(hg):
    n, m = 700, 90
    B_cm = workloads.uniform_f16(np.random.default_rng(3), (m, n))
    out = run(hg, np.eye(n, dtype=np.float16), B_cm, 2.0)
    assert np.array_equal(out, 2.0 * B_cm.astype(np.float32))


def test_tril_ones_closed_form(hg):
    n, m = 1100, 40
    A = np.tril(np.ones((n, n), np.float16))
    out = run(hg, np.ascontiguousarray(A.T), np.ones((m, n), np.float16), 0.5)
    expect = 0.5 * (n - np.arange(n, dtype=np.float32))
    assert np.array_equal(out, np.tile(expect, (m, 1)))


@pytest.mark.parametrize("fill", [np.nan, 1e4, -np.inf])
def test_upper_triangle_never_read(hg, fill):
    n, m = 777, 64
    A0, B_cm = trmm_inputs(n, m, 5, 0.0)
    Ax, _ = trmm_inputs(n, m, 5, fill)
    base = run(hg, A0, B_cm)
    got = run(hg, Ax, B_cm)
    assert np.array_equal(base.view(np.uint32), got.view(np.uint32))


def test_integer_bit_exact(hg):
    rng = np.random.default_rng(17)
    n, m = 1500, 120
    A = np.tril(workloads.integer_f16(rng, (n, n)))
    B = workloads.integer_f16(rng, (n, m))
    out = run(hg, np.ascontiguousarray(A.T), np.ascontiguousarray(B.T))
    exact = A.astype(np.int64).T @ B.astype(np.int64)
    assert np.array_equal(out, exact.T.astype(np.float32))


def test_alpha_zero_gives_zeros_without_reading(hg):
    n, m = 300, 20
    A = np.full((n, n), np.nan, np.float16)
    B = np.full((m, n), np.nan, np.float16)
    out = run(hg, A, B, 0.0)
    assert np.array_equal(out, np.zeros((m, n), np.float32))


def test_strided_operands(hg):
    """Leading dimensions larger than n; Out's padding stays untouched."""
    n, m, pad = 600, 50, 24
    A_cm, B_cm = trmm_inputs(n, m, 9)
    Ab = np.zeros((n, n + pad), np.float16)
    Ab[:, :n] = A_cm
    Bb = np.zeros((m, n + pad), np.float16)
    Bb[:, :n] = B_cm
    Ob = torch.full((m, n + pad), -7.0, dtype=torch.float32, device=DEV)
    hg.trmm_lower_trans(dev(Ab)[:, :n], dev(Bb)[:, :n], Ob[:, :n], 1.0, 128)
    torch.cuda.synchronize()
    got = Ob.cpu().numpy()
    assert np.all(got[:, n:] == -7.0)
    check_close(got[:, :n], oracle.trmm_lower_trans(A_cm, B_cm), n, "strided")


def test_deterministic(hg):
    A_cm, B_cm = trmm_inputs(1030, 200, 2)
    a = run(hg, A_cm, B_cm)
    b = run(hg, A_cm, B_cm)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ---- the one-launch schedule against the level-by-level one and the oracle.
# The one-launch schedule runs on 256×256 tiles when the recursion's
# boundaries fall on the 256 grid and there are at least two such output
# tiles per CU (m·n >= 512·256²: the shapes below with m·n of 2^25), and on
# 64×64 tiles when the boundaries fall on the 64 grid (3072: pieces of 192);
# 2560 and 2500 (boundaries off the 64 grid: pieces of 160 and 156) run level
# by level in both calls, so there the two calls run the same launches and
# must agree bit for bit.  The
# one-launch schedule adds a tile's updates in its fp32 accumulators, the
# level-by-level one rounds Out to fp32 after each update, so the two differ
# only by fp32 rounding: each is within (K/32 + depth + 2)·6·2^-24 of
# Σ|terms| of the exact value (one rounding per MFMA step of 32 products,
# counted with a tree of depth 5 inside the step, and one per update).
U32 = 2.0 ** -24


def _fp32_bound(A_cm, B_cm, ri, cj, alpha, n, leaf):
    depth = max(1, int(np.ceil(np.log2(max(n / leaf, 1)))) + 1)
    mag = oracle.trmm_lower_trans_sampled(np.abs(A_cm), np.abs(B_cm), ri, cj, abs(alpha))
    return (n / 32 + depth + 2) * 6 * U32 * mag


@pytest.mark.parametrize("n,m,leaf,one_launch", [(4096, 8192, 256, True), (2048, 16384, 256, True),
                                                 (4096, 8192, 512, True), (8192, 4096, 256, True),
                                                 (3072, 64, 256, True), (2560, 100, 256, False),
                                                 (2500, 64, 256, False),
                                                 # 64×64 one launch, two workgroups per CU
                                                 (3072, 3072, 256, True), (2048, 1024, 128, True),
                                                 (8192, 300, 256, True)])
def test_schedules_agree(hg, n, m, leaf, one_launch):
    print(f"[case] trmm schedules n={n} m={m} leaf={leaf}", flush=True)
    A_cm, B_cm = trmm_inputs(n, m, n + 3 * m + leaf)
    one = run(hg, A_cm, B_cm, 1.25, leaf)
    lev = run(hg, A_cm, B_cm, 1.25, leaf, by_level=True)
    if not one_launch:
        assert np.array_equal(one.view(np.uint32), lev.view(np.uint32))
    if n * m <= 2 ** 20:
        ref = oracle.trmm_lower_trans(A_cm, B_cm, 1.25)
        check_close(one, ref, n, f"n={n} m={m} leaf={leaf}")
        check_close(lev, ref, n, f"n={n} m={m} leaf={leaf} by level")
        return
    ri, cj = workloads.sample_indices(n + m, n, m)
    ref = oracle.trmm_lower_trans_sampled(A_cm, B_cm, ri, cj, 1.25)
    check_close(one[cj, ri], ref, n, f"n={n} m={m} leaf={leaf} sampled")
    check_close(lev[cj, ri], ref, n, f"n={n} m={m} leaf={leaf} sampled, by level")
    lim = _fp32_bound(A_cm, B_cm, ri, cj, 1.25, n, leaf)
    for name, got in (("one launch", one), ("by level", lev)):
        err = np.abs(got[cj, ri] - ref)
        assert (err <= lim).all(), f"{name}: fp32 accumulation error {err.max():.3g} over the bound"


def test_one_launch_odd_tile_columns(hg):
    """n = 768 with leaf >= n is a single leaf of 3 tile columns (the only way
    an odd count of 256-wide columns reaches the one-launch schedule), and
    m = 44288 gives 173 tile rows: the middle column's tiles pair up by rows
    and the last forms a job of its own.  A single leaf is one K loop per tile
    in both schedules; the one-launch schedule walks it upward in tile
    columns 0 (the long tile of each pair) and 1 (the middle column), as the
    level-by-level one does, so there the two agree bit for bit, and
    downward in column 2 (the short tile), where they differ by fp32
    rounding only.  Sampled entries against the oracle and its fp32 bound."""
    n, m = 768, 44288
    A_cm, B_cm = trmm_inputs(n, m, 29)
    one = run(hg, A_cm, B_cm, 1.5, 768)
    lev = run(hg, A_cm, B_cm, 1.5, 768, by_level=True)
    assert np.array_equal(one[:, :512].view(np.uint32), lev[:, :512].view(np.uint32))
    ri, cj = workloads.sample_indices(31, n, m, 4096)
    ref = oracle.trmm_lower_trans_sampled(A_cm, B_cm, ri, cj, 1.5)
    check_close(one[cj, ri], ref, n, "n=768 m=44288 one launch")
    lim = _fp32_bound(A_cm, B_cm, ri, cj, 1.5, n, 768)
    assert (np.abs(one[cj, ri] - ref) <= lim).all()


def test_one_launch_integer_bit_exact(hg):
    rng = np.random.default_rng(23)
    n, m = 2048, 16384
    A = np.tril(workloads.integer_f16(rng, (n, n)))
    B = workloads.integer_f16(rng, (n, m))
    A_cm, B_cm = np.ascontiguousarray(A.T), np.ascontiguousarray(B.T)
    out = run(hg, A_cm, B_cm)
    ri, cj = workloads.sample_indices(7, n, m, 4096)
    exact = oracle.trmm_lower_trans_sampled(A_cm, B_cm, ri, cj)      # integers, exact in fp64
    assert np.array_equal(out[cj, ri].astype(np.float64), exact)


@pytest.mark.parametrize("fill", [np.nan, -np.inf])
def test_one_launch_upper_triangle_never_read(hg, fill):
    n, m = 4096, 8192
    A0, B_cm = trmm_inputs(n, m, 8, 0.0)
    Ax, _ = trmm_inputs(n, m, 8, fill)
    base = run(hg, A0, B_cm)
    got = run(hg, Ax, B_cm)
    assert np.array_equal(base.view(np.uint32), got.view(np.uint32))


def test_one_launch_tril_ones_closed_form(hg):
    n, m = 2048, 16384
    A = np.tril(np.ones((n, n), np.float16))
    out = run(hg, np.ascontiguousarray(A.T), np.ones((m, n), np.float16), 0.5)
    expect = 0.5 * (n - np.arange(n, dtype=np.float32))
    assert np.array_equal(out, np.tile(expect, (m, 1)))


@pytest.mark.parametrize("n,m", [(4096, 256), (8192, 256), (4096, 1024)])
def test_skinny_b(hg, n, m):
    """Skinny right-hand sides ("异构计算中高性能TRMM与TRSM的递归算法实现" §5.1
    uses n = 4096, m = 256): level-by-level launches, against the oracle in full."""
    A_cm, B_cm = trmm_inputs(n, m, n + m)
    out = run(hg, A_cm, B_cm, 0.75)
    check_close(out, oracle.trmm_lower_trans(A_cm, B_cm, 0.75), n, f"skinny n={n} m={m}")


# ---- the per-level schedule spread over several streams
# (hg_trmm_lower_trans_streams): every launch runs the kernel of its
# phase's batched launch, so the bits equal the level-by-level entry point's.
@pytest.mark.parametrize("n,m,leaf,nstreams", [(4096, 256, 256, 4), (2048, 1000, 256, 2),
                                               (1000, 300, 100, 3), (8192, 512, 256, 8),
                                               (600, 70, 128, 1)])
def test_streams_equal_by_level(hg, n, m, leaf, nstreams):
    print(f"[case] trmm streams n={n} m={m} leaf={leaf} streams={nstreams}", flush=True)
    A_cm, B_cm = trmm_inputs(n, m, n + m + nstreams)
    lev = run(hg, A_cm, B_cm, 0.75, leaf, by_level=True)
    streams = [torch.cuda.current_stream()] + [torch.cuda.Stream() for _ in range(nstreams - 1)]
    Out = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    hg.trmm_lower_trans_streams(dev(A_cm), dev(B_cm), Out, streams, 0.75, leaf)
    torch.cuda.synchronize()
    got = Out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), lev.view(np.uint32))


def test_streams_join_onto_first_stream(hg):
    """Work queued on streams[0] after the call sees the finished product
    (the final join), also when streams[0] is not the current stream."""
    n, m, leaf = 2048, 512, 256
    print(f"[case] trmm streams join n={n} m={m}", flush=True)
    A_cm, B_cm = trmm_inputs(n, m, 77)
    lev = run(hg, A_cm, B_cm, 1.0, leaf, by_level=True)
    s0, s1, s2 = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    Ad, Bd = dev(A_cm), dev(B_cm)
    Out = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    with torch.cuda.stream(s0):
        hg.trmm_lower_trans_streams(Ad, Bd, Out, [s0, s1, s2], 1.0, leaf)
        copy = Out.clone()          # queued on s0 right behind the product
    torch.cuda.synchronize()
    assert np.array_equal(copy.cpu().numpy().view(np.uint32), lev.view(np.uint32))
