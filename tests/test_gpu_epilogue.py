"""GPU parity of hgemm_bias_act, C = act(α·A·B + β·C + bias) in one launch
("GPU架构与CUDA", section 核函数融合), against the fp64 oracle, through the C ABI.

Same rule as the HGEMM: |gpu − ref| <= 1e-3·sqrt(K) + 2^-10·|ref| (the bias
add and the ReLU are exact or one fp32 rounding); integer inputs with an
integer bias are bit-exact.  Shapes cover the three kernel families (256×256
fast tiles, 64/128 ring tiles, the general element-wise path) and the
alpha = 0 quick return.
"""
import numpy as np
import pytest

import oracle
import workloads
from tolerance import check_close

pytestmark = pytest.mark.gpu


def _dev():
    import torch
    return torch.device("cuda:0")


def run(hg, A, Bt, C0, bias, relu, alpha, beta, out_dtype, lda_pad=0):
    import torch
    dev = _dev()
    M, K = A.shape
    N = Bt.shape[0]
    print(f"[epi] M={M} N={N} K={K} relu={relu} bias={bias is not None} alpha={alpha} "
          f"beta={beta} out={out_dtype} pad={lda_pad}", flush=True)
    Ad = torch.zeros((M, K + lda_pad), dtype=torch.float16, device=dev)[:, :K]
    Ad.copy_(torch.from_numpy(A))
    Bd = torch.from_numpy(Bt).to(dev)
    tdt = torch.float16 if out_dtype == "f16" else torch.float32
    Cd = torch.from_numpy(C0.astype(np.float16 if out_dtype == "f16" else np.float32)).to(dev)
    bd = None if bias is None else torch.from_numpy(bias).to(dev)
    assert Cd.dtype == tdt
    hg.hgemm_bias_act(Ad, Bd, Cd, bd, relu, alpha, beta)
    torch.cuda.synchronize()
    return Cd.cpu().numpy()


CASES = [
    # M, N, K, out, beta, path
    (4096, 4096, 256, "f16", 0.0),      # 256x256 fast tiles
    (4096, 4096, 200, "f32", 0.5),      # fast, K not a multiple of 64
    (1000, 1000, 1000, "f16", 0.5),     # ring (64x64), ragged edges
    (1536, 1024, 512, "f32", 0.0),      # ring (128x128)
    (300, 257, 64, "f32", 1.0),         # ring, N not a multiple of 4
    (200, 130, 33, "f16", 0.0),         # general path: K not a multiple of 8
    (4096, 4096, 512, "f16", 0.5),      # fast, 16-bit C read (beta != 0)
    (4133, 4133, 1000, "f16", 0.5),     # fast, 16-bit C read, ragged edges, K tail
]


@pytest.mark.parametrize("M,N,K,out,beta", CASES)
@pytest.mark.parametrize("relu", [False, True])
def test_parity(hg, M, N, K, out, beta, relu):
    rng = np.random.default_rng(M + N + K + int(relu))
    A = workloads.uniform_f16(rng, (M, K))
    Bt = workloads.uniform_f16(rng, (N, K))
    C0 = workloads.uniform_f16(rng, (M, N))
    bias = rng.uniform(-2, 2, N).astype(np.float32)
    got = run(hg, A, Bt, C0, bias, relu, 1.25, beta, out)
    cin = C0.astype(np.float16 if out == "f16" else np.float32)
    ref = oracle.hgemm_bias_act(A, Bt, 1.25, beta, cin if beta else None, bias,
                                oracle.ACT_RELU if relu else oracle.ACT_NONE)
    check_close(got, ref, K, f"bias_act {M}x{N}x{K} {out} relu={relu}")
    if relu:
        assert (got >= 0).all()


def test_unaligned_lda_general_path(hg):
    rng = np.random.default_rng(3)
    M, N, K = 130, 96, 64
    A = workloads.uniform_f16(rng, (M, K))
    Bt = workloads.uniform_f16(rng, (N, K))
    C0 = np.zeros((M, N), np.float16)
    bias = rng.uniform(-1, 1, N).astype(np.float32)
    got = run(hg, A, Bt, C0, bias, True, 1.0, 0.0, "f32", lda_pad=3)
    ref = oracle.hgemm_bias_act(A, Bt, 1.0, 0.0, None, bias, oracle.ACT_RELU)
    check_close(got, ref, K, "unaligned lda")


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 512), (1000, 1000, 1000), (77, 50, 24)])
def test_integer_bit_exact(hg, M, N, K):
    rng = np.random.default_rng(K)
    A = workloads.integer_f16(rng, (M, K))
    Bt = workloads.integer_f16(rng, (N, K))
    C0 = workloads.integer_f16(rng, (M, N))
    bias = rng.integers(-40, 41, N).astype(np.float32)
    got = run(hg, A, Bt, C0, bias, True, 1.0, 2.0, "f32")
    ref = oracle.hgemm_bias_act(A, Bt, 1.0, 2.0, C0.astype(np.float32), bias, oracle.ACT_RELU)
    assert np.array_equal(got.astype(np.float64), ref)


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 256), (1000, 1000, 1000)])
def test_no_epilogue_equals_hgemm_bits(hg, M, N, K):
    import torch
    rng = np.random.default_rng(9)
    A = workloads.uniform_f16(rng, (M, K))
    Bt = workloads.uniform_f16(rng, (N, K))
    C0 = workloads.uniform_f16(rng, (M, N))
    got = run(hg, A, Bt, C0, None, False, 0.75, 0.5, "f16")
    dev = _dev()
    Cd = torch.from_numpy(C0).to(dev)
    hg.hgemm(torch.from_numpy(A).to(dev), torch.from_numpy(Bt).to(dev), Cd, 0.75, 0.5)
    torch.cuda.synchronize()
    assert np.array_equal(got.view(np.uint16), Cd.cpu().numpy().view(np.uint16))


def test_alpha_zero_bias_and_relu(hg):
    """alpha = 0 reads neither A nor B (NaN there): C = relu(beta·C + bias)."""
    rng = np.random.default_rng(11)
    M, N, K = 70, 90, 32
    A = np.full((M, K), np.nan, np.float16)
    Bt = np.full((N, K), np.nan, np.float16)
    C0 = workloads.uniform_f16(rng, (M, N))
    bias = rng.uniform(-1, 1, N).astype(np.float32)
    got = run(hg, A, Bt, C0, bias, True, 0.0, 1.5, "f32")
    ref = oracle.hgemm_bias_act(A, Bt, 0.0, 1.5, C0.astype(np.float32), bias, oracle.ACT_RELU)
    check_close(got, ref, 1, "alpha = 0")


def test_workload_8192_sampled(hg):
    """The 8192³ shape as the benchmark runs it (fp16 out, bias, ReLU): 1024
    sampled entries against the oracle's fused definition at those entries."""
    w = workloads.WORKLOADS["hgemm_8192"]
    A, Bt, _ = workloads.gemm_inputs(w)
    rng = np.random.default_rng(w.seed + 7)
    bias = rng.uniform(-1, 1, w.N).astype(np.float32)
    C0 = np.zeros((w.M, w.N), np.float16)
    got = run(hg, A, Bt, C0, bias, True, 1.0, 0.0, "f16")
    ri, cj = workloads.sample_indices(w.seed, w.M, w.N)
    ref = oracle.gemm_bias_act_sampled(A, Bt, ri, cj, 1.0, 0.0, None, bias, oracle.ACT_RELU)
    check_close(got[ri, cj], ref, w.K, "bias_act 8192 sampled")
