"""The 256×256 fast kernel's 16-bit-C paths, exact pins at shapes that select
it, and fp16 overflow on every kernel family, through the C ABI.

A problem with at least 256 tiles of 256×256 runs the fast kernel; these
tests pin what the smaller shapes of the other files never reach there:
  * a 16-bit C that is read (beta != 0): its C_in loads, the epilogue's LDS
    staging with the 16-bit swizzle, fp16 and bf16, with and without a K
    tail and ragged edges, checked element by element against the oracle;
  * integer inputs (every partial sum exact in fp32): bit-exact, fp16 and
    fp32 C, beta = 0 and beta != 0;
  * round-to-nearest-even of the output ("Nvidia Tensor Core-MMA PTX编程入门"
    §4 writes C in fp16; the rounding mode is the IEEE default) on exact
    values half-way between two fp16 (or bf16) numbers, spread over the
    whole big-tile problem;
  * overflow: an exact value at or beyond the fp16 rounding threshold 65520
    becomes ±inf, one just below it the largest finite 65504, on the fast,
    ring and general kernels and the split-K reduction.
Layouts and tolerance as the other GPU parity tests ("GPU架构与CUDA",
共享内存与分块 and 混合精度核函数).
"""
import numpy as np
import pytest

import oracle
import workloads
from tolerance import REL_BF16, check_close

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def bf16_host(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_values(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def run_f16(hg, A, Bt, C, alpha, beta):
    M, K = A.shape
    print(f"[fast] hgemm M={M} N={Bt.shape[0]} K={K} C={C.dtype} alpha={alpha} beta={beta}", flush=True)
    Cd = dev(C)
    hg.hgemm(dev(A), dev(Bt), Cd, alpha, beta)
    torch.cuda.synchronize()
    return Cd.cpu().numpy()


# ---------------------------------------------------------- 16-bit C read
@pytest.mark.parametrize("M,N,K", [(4096, 4096, 512), (4133, 4133, 1000), (4096, 4352, 64)])
def test_f16_c_beta_parity(hg, M, N, K):
    """fp16 C read and written by the fast kernel (alpha = 1.5, beta = 0.5),
    every element against the oracle."""
    rng = np.random.default_rng(M + 3 * N + K)
    A = workloads.uniform_f16(rng, (M, K))
    Bt = workloads.uniform_f16(rng, (N, K))
    C = workloads.uniform_f16(rng, (M, N))
    out = run_f16(hg, A, Bt, C, 1.5, 0.5)
    ref = oracle.hgemm(A, Bt, 1.5, 0.5, C)
    check_close(out, ref, K, f"fp16 C beta {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 512), (4133, 4133, 1000)])
def test_bf16_c_beta_parity(hg, M, N, K):
    """bf16 operands and a bf16 C read by the fast kernel (hgemm_bf16)."""
    rng = np.random.default_rng(M + 5 * N + K)
    A = workloads.uniform_bf16(rng, (M, K))
    Bt = workloads.uniform_bf16(rng, (N, K))
    C = workloads.uniform_bf16(rng, (M, N))
    print(f"[fast] hgemm_bf16 M={M} N={N} K={K} bf16 C beta=0.5", flush=True)
    Cd = bf16_dev(C)
    hg.hgemm_bf16(bf16_dev(A), bf16_dev(Bt), Cd, 1.5, 0.5)
    torch.cuda.synchronize()
    out = bf16_values(bf16_host(Cd))
    ref = oracle.gemm_bf16(A, Bt, 1.5, 0.5, C, cin_bf16=True)
    check_close(out, ref, K, f"bf16 C beta {M}x{N}x{K}", rel=REL_BF16)


# ---------------------------------------------------------- integer inputs
@pytest.mark.parametrize("odt", [np.float16, np.float32])
@pytest.mark.parametrize("beta", [0.0, 0.5])
def test_integer_bit_exact_big_tiles(hg, odt, beta):
    """Integers in [-4, 4] at 4096×4096×512 (fast kernel): every partial sum
    and beta·C_in is exact in fp32, so the output is the exact value rounded
    to nearest even, bit for bit."""
    rng = np.random.default_rng(77 + int(beta * 2) + (odt is np.float16))
    M = N = 4096
    K = 512
    A = workloads.integer_f16(rng, (M, K))
    Bt = workloads.integer_f16(rng, (N, K))
    C = workloads.integer_f16(rng, (M, N)).astype(odt)
    out = run_f16(hg, A, Bt, C, 1.0, beta)
    exact = oracle.hgemm(A, Bt, 1.0, beta, C if beta else None)
    assert np.array_equal(out, exact.astype(odt))


# ---------------------------------------------------------- rounding mode
def _target_rows(targets, K, unit):
    """fp16 rows whose sum against a column of ones is exactly the target:
    `unit` in the first t // unit entries, the remainder in the next."""
    A = np.zeros((len(targets), K), np.float16)
    for r, t in enumerate(targets):
        q, rem = divmod(int(abs(t)), unit)
        s = 1 if t >= 0 else -1
        A[r, :q] = s * unit
        A[r, q] = s * rem
    return A


def test_f16_rne_halfway_big_tiles(hg):
    """Every row of a 4096×4096 fp16-C problem sums to an odd integer in
    (2048, 4096), where fp16 spacing is 2: each output lies half-way between
    two fp16 values and must round to the even one (2049 -> 2048,
    2051 -> 2052); truncation or round-half-up would differ on every other
    row.  Columns alternate +1 / -1 so both signs are covered."""
    M = N = 4096
    K = 1024
    targets = 2049 + 2 * (np.arange(M) % 1000)
    A = _target_rows(targets, K, 4)
    sign = np.where(np.arange(N) % 2 == 0, 1.0, -1.0)
    Bt = np.repeat(sign[:, None], K, axis=1).astype(np.float16)
    for beta in (0.0, 1.0):
        C = np.zeros((M, N), np.float16)
        out = run_f16(hg, A, Bt, C, 1.0, beta)
        expect = np.outer(targets.astype(np.float64), sign).astype(np.float16)
        assert np.array_equal(out, expect)
    assert out[0, 0] == 2048 and out[1, 0] == 2052 and out[1, 1] == -2052


def test_bf16_rne_halfway_big_tiles(hg):
    """The same pin for bf16 C: odd integers in (256, 512), where bf16
    spacing is 2, round to the even neighbour."""
    M = N = 4096
    K = 256
    targets = 257 + 2 * (np.arange(M) % 120)
    rows = np.zeros((M, K), np.float32)
    for r, t in enumerate(targets):
        q, rem = divmod(int(t), 2)
        rows[r, :q] = 2
        rows[r, q] = rem
    A = workloads.to_bf16_bits(rows)
    Bt = workloads.to_bf16_bits(np.ones((N, K), np.float32))
    print(f"[fast] bf16 halfway M={M} N={N} K={K}", flush=True)
    Cd = torch.zeros((M, N), dtype=torch.bfloat16, device=DEV)
    hg.hgemm_bf16(bf16_dev(A), bf16_dev(Bt), Cd)
    torch.cuda.synchronize()
    got = bf16_host(Cd)
    expect = workloads.to_bf16_bits(np.repeat(targets.astype(np.float32)[:, None], N, axis=1))
    assert np.array_equal(got, expect)
    assert bf16_values(got[:2, :1]).ravel().tolist() == [256.0, 260.0]


# ---------------------------------------------------------- fp16 overflow
# Exact row sums around the fp16 overflow threshold: 65504 is the largest
# finite fp16, 65520 lies half-way to 65536 (= 2^16, not representable), so
# round-to-nearest-even sends it and everything above to +inf.
OVF_TARGETS = np.array([65504, 65519, 65520, 65536, 70000, -65519, -65520, -70000, 1000, -1000])


def _overflow_problem(M, N, K):
    reps = -(-M // len(OVF_TARGETS))
    targets = np.tile(OVF_TARGETS, reps)[:M]
    A = _target_rows(targets, K, 16)
    scale = np.where(np.arange(N) % 3 == 2, -1.0, 1.0)      # columns +1, +1, -1, ...
    Bt = np.repeat(scale[:, None], K, axis=1).astype(np.float16)
    with np.errstate(over="ignore"):     # the targets past 65519 round to ±inf on purpose
        expect = np.outer(targets.astype(np.float64), scale).astype(np.float16)
    return A, Bt, expect


@pytest.mark.parametrize("M,N,K,beta,path", [
    (4096, 4096, 4608, 0.0, "fast"),
    (4096, 4096, 4608, 1.0, "fast, C read"),
    (1000, 1000, 4608, 0.0, "ring"),
    (300, 260, 4608, 0.5, "ring, C read"),
    (200, 130, 4601, 0.0, "general (K not a multiple of 8)"),
])
def test_f16_overflow_to_inf(hg, M, N, K, beta, path):
    A, Bt, expect = _overflow_problem(M, N, K)
    out = run_f16(hg, A, Bt, np.zeros((M, N), np.float16), 1.0, beta)
    assert np.array_equal(out, expect), path
    assert np.isposinf(out).any() and np.isneginf(out).any()
    assert (out == np.float16(65504)).any() and (out == np.float16(-65504)).any()
    # the oracle agrees with the constructed targets at a few entries
    ri, cj = workloads.sample_indices(K, M, N, 64)
    ref = oracle.hgemm_sampled(A, Bt, ri, cj)
    with np.errstate(over="ignore"):
        assert np.array_equal(ref.astype(np.float16), expect[ri, cj])


def test_f16_overflow_splitk_reduction(hg):
    """The split-K reduction rounds its fp32 sum to fp16 the same way."""
    M, N, K = 512, 512, 8192
    A, Bt, expect = _overflow_problem(M, N, K)
    Ad, Bd = dev(A), dev(Bt)
    Cd = torch.zeros((M, N), dtype=torch.float16, device=DEV)
    work = torch.empty(hg.splitk_workspace_size(M, N, K, 0), dtype=torch.uint8, device=DEV)
    print(f"[fast] split-K overflow M={M} N={N} K={K}", flush=True)
    hg.hgemm_splitk(Ad, Bd, Cd, 1.0, 0.0, 0, work)
    torch.cuda.synchronize()
    assert np.array_equal(Cd.cpu().numpy(), expect)
