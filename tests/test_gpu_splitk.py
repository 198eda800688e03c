"""GPU parity of hgemm_splitk (C = alpha·A·B + beta·C with K cut into
slices summed in fp32; the tiled product of "GPU架构与CUDA" 共享内存与分块 with
its K loop partitioned) against the fp64 oracle, through the C ABI.

Same rule as the HGEMM: |gpu − ref| <= 1e-3·sqrt(K) + 2^-10·|ref|; integer
inputs bit-exact (every partial sum is an integer below 2^24).
"""
import numpy as np
import pytest

import oracle
import workloads
from tolerance import check_close

pytestmark = pytest.mark.gpu


def run(hg, A, Bt, C0, alpha, beta, out, splits, fn="splitk"):
    import torch
    dev = torch.device("cuda:0")
    M, K = A.shape
    N = Bt.shape[0]
    print(f"[splitk] M={M} N={N} K={K} out={out} alpha={alpha} beta={beta} splits={splits} fn={fn}",
          flush=True)
    Ad = torch.from_numpy(A).to(dev)
    Bd = torch.from_numpy(Bt).to(dev)
    Cd = torch.from_numpy(C0.astype(np.float16 if out == "f16" else np.float32)).to(dev)
    if fn == "splitk":
        hg.hgemm_splitk(Ad, Bd, Cd, alpha, beta, splits)
    else:
        hg.hgemm(Ad, Bd, Cd, alpha, beta)
    torch.cuda.synchronize()
    return Cd.cpu().numpy()


CASES = [
    # M, N, K, out, beta, splits
    (512, 512, 65536, "f32", 0.0, 0),
    (512, 512, 65536, "f16", 0.5, 16),
    (300, 257, 10000, "f16", 0.5, 0),       # ragged M, N and last slice
    (1024, 768, 20480, "f32", 1.0, 5),
    (200, 100, 4099, "f32", 0.5, 6),        # K not a multiple of 8: element-wise kernel
    (64, 64, 96, "f32", 0.0, 32),           # K too short for more than one slice
]


@pytest.mark.parametrize("M,N,K,out,beta,splits", CASES)
def test_parity(hg, M, N, K, out, beta, splits):
    rng = np.random.default_rng(M + N + K + splits)
    A = workloads.uniform_f16(rng, (M, K))
    Bt = workloads.uniform_f16(rng, (N, K))
    C0 = workloads.uniform_f16(rng, (M, N))
    got = run(hg, A, Bt, C0, 1.25, beta, out, splits)
    cin = C0.astype(np.float16 if out == "f16" else np.float32)
    ref = oracle.hgemm(A, Bt, 1.25, beta, cin if beta else None)
    check_close(got, ref, K, f"splitk {M}x{N}x{K} {out} splits={splits}")


def test_integer_bit_exact(hg):
    rng = np.random.default_rng(17)
    M, N, K = 512, 256, 16384
    A = workloads.integer_f16(rng, (M, K))
    Bt = workloads.integer_f16(rng, (N, K))
    C0 = workloads.integer_f16(rng, (M, N))
    got = run(hg, A, Bt, C0, 1.0, 2.0, "f32", 8)
    ref = oracle.hgemm(A, Bt, 1.0, 2.0, C0.astype(np.float32))
    assert np.array_equal(got.astype(np.float64), ref)


@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (0.75, 0.5)])
def test_one_slice_is_hgemm(hg, alpha, beta):
    """One slice: the same products as hgemm, stored in fp32 and finished by
    the reduction.  fp32 C is hgemm's bit for bit.  For a 16-bit C with beta
    the compiler forms fp16(fma(alpha, acc, beta·c)) either with one rounding
    (v_fma_mix) or as an fp32 fma and a conversion, element by element as it
    schedules them, so the two calls agree within one fp16 ulp there."""
    rng = np.random.default_rng(5)
    M, N, K = 512, 512, 8192
    A = workloads.uniform_f16(rng, (M, K))
    Bt = workloads.uniform_f16(rng, (N, K))
    C0 = workloads.uniform_f16(rng, (M, N))
    a = run(hg, A, Bt, C0, alpha, beta, "f32", 1)
    b = run(hg, A, Bt, C0, alpha, beta, "f32", 0, fn="hgemm")
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    a = run(hg, A, Bt, C0, alpha, beta, "f16", 1).astype(np.float64)
    b = run(hg, A, Bt, C0, alpha, beta, "f16", 0, fn="hgemm").astype(np.float64)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(b), 2.0 ** -14))) - 10)
    assert (np.abs(a - b) <= ulp).all()
    if beta == 0.0:
        assert np.array_equal(a, b)


def test_deterministic(hg):
    rng = np.random.default_rng(6)
    M, N, K = 256, 384, 32768
    A = workloads.uniform_f16(rng, (M, K))
    Bt = workloads.uniform_f16(rng, (N, K))
    C0 = np.zeros((M, N), np.float16)
    a = run(hg, A, Bt, C0, 1.0, 0.0, "f32", 0)
    b = run(hg, A, Bt, C0, 1.0, 0.0, "f32", 0)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_alpha_zero_scales_c(hg):
    rng = np.random.default_rng(7)
    M, N, K = 70, 90, 4096
    A = np.full((M, K), np.nan, np.float16)
    Bt = np.full((N, K), np.nan, np.float16)
    C0 = workloads.uniform_f16(rng, (M, N))
    got = run(hg, A, Bt, C0, 0.0, 1.5, "f32", 4)
    assert np.array_equal(got, (1.5 * C0.astype(np.float32)).astype(np.float32))
