"""GPU parity of hgemm_bf16 (bf16 A and B, fp32 accumulation, bf16 or fp32 C;
"GPU架构与CUDA", section 混合精度核函数) against the fp64 oracle, through the
C ABI.

Rule: |gpu − ref| <= 1e-3·sqrt(K) + rel·|ref| with rel = 2^-10 for fp32 C and
2^-8 for bf16 C (its rounding); integer inputs are bit-exact.  Shapes cover
the 256×256 fast tiles, the ring tiles and the general path.
"""
import numpy as np
import pytest

import oracle
import workloads
from tolerance import REL_BF16, check_close

pytestmark = pytest.mark.gpu


def _bf16_tensor(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def run(hg, A, Bt, C0, alpha, beta, out, lda_pad=0):
    """A, Bt, C0 (when out == 'bf16') are bf16 bit patterns; C0 float32 otherwise."""
    import torch
    dev = torch.device("cuda:0")
    M, K = A.shape
    N = Bt.shape[0]
    print(f"[bf16] M={M} N={N} K={K} alpha={alpha} beta={beta} out={out} pad={lda_pad}", flush=True)
    Ad = torch.zeros((M, K + lda_pad), dtype=torch.bfloat16, device=dev)[:, :K]
    Ad.copy_(_bf16_tensor(A, dev))
    Bd = _bf16_tensor(Bt, dev)
    Cd = _bf16_tensor(C0, dev) if out == "bf16" else torch.from_numpy(C0).to(dev)
    hg.hgemm_bf16(Ad, Bd, Cd, alpha, beta)
    torch.cuda.synchronize()
    if out == "bf16":
        bits = Cd.view(torch.int16).cpu().numpy().view(np.uint16)
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return Cd.cpu().numpy().astype(np.float64)


CASES = [
    (4096, 4096, 256, "bf16", 0.0),
    (4096, 4096, 200, "f32", 0.5),
    (1000, 1000, 1000, "bf16", 0.5),
    (1536, 1024, 512, "f32", 0.0),
    (300, 257, 64, "f32", 1.0),
    (200, 130, 33, "bf16", 0.0),
    (4096, 4096, 512, "bf16", 0.5),     # fast kernel, 16-bit C read (beta != 0)
    (4133, 4133, 1000, "bf16", 0.5),    # fast kernel, 16-bit C read, ragged edges, K tail
]


@pytest.mark.parametrize("M,N,K,out,beta", CASES)
def test_parity(hg, M, N, K, out, beta):
    rng = np.random.default_rng(M + N + K)
    A = workloads.uniform_bf16(rng, (M, K))
    Bt = workloads.uniform_bf16(rng, (N, K))
    if out == "bf16":
        C0 = workloads.uniform_bf16(rng, (M, N))
    else:
        C0 = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    got = run(hg, A, Bt, C0, 1.25, beta, out)
    ref = oracle.gemm_bf16(A, Bt, 1.25, beta, C0 if beta else None, cin_bf16=(out == "bf16"))
    check_close(got, ref, K, f"bf16 {M}x{N}x{K} {out}", rel=REL_BF16 if out == "bf16" else 2.0 ** -10)


def test_unaligned_lda_general_path(hg):
    rng = np.random.default_rng(5)
    M, N, K = 130, 96, 64
    A = workloads.uniform_bf16(rng, (M, K))
    Bt = workloads.uniform_bf16(rng, (N, K))
    C0 = np.zeros((M, N), np.float32)
    got = run(hg, A, Bt, C0, 1.0, 0.0, "f32", lda_pad=3)
    check_close(got, oracle.gemm_bf16(A, Bt), K, "bf16 unaligned lda")


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 512), (1000, 1000, 1000), (77, 50, 24)])
def test_integer_bit_exact(hg, M, N, K):
    rng = np.random.default_rng(K + 1)
    A = workloads.to_bf16_bits(rng.integers(-4, 5, (M, K)).astype(np.float32))
    Bt = workloads.to_bf16_bits(rng.integers(-4, 5, (N, K)).astype(np.float32))
    C0 = rng.integers(-4, 5, (M, N)).astype(np.float32)
    got = run(hg, A, Bt, C0, 1.0, 2.0, "f32")
    assert np.array_equal(got, oracle.gemm_bf16(A, Bt, 1.0, 2.0, C0))


def test_alpha_zero_reads_neither_operand(hg):
    rng = np.random.default_rng(6)
    M, N, K = 64, 72, 16
    A = np.full((M, K), 0x7FC0, np.uint16)          # NaN patterns
    Bt = np.full((N, K), 0x7FC0, np.uint16)
    C0 = workloads.uniform_bf16(rng, (M, N))
    got = run(hg, A, Bt, C0, 0.0, 0.5, "bf16")
    ref = oracle.gemm_bf16(A, Bt, 0.0, 0.5, C0, cin_bf16=True)
    assert np.array_equal(got, ref)


def test_8192_sampled(hg):
    """8192³ with bf16 operands (the HGEMM workload's shape, values drawn
    the same way and rounded to bf16), fp32 C: 1024 sampled entries."""
    w = workloads.WORKLOADS["hgemm_8192"]
    rng = np.random.default_rng(w.seed)
    A = workloads.uniform_bf16(rng, (w.M, w.K))
    Bt = workloads.uniform_bf16(rng, (w.N, w.K))
    got = run(hg, A, Bt, np.zeros((w.M, w.N), np.float32), 1.0, 0.0, "f32")
    ri, cj = workloads.sample_indices(w.seed, w.M, w.N)
    check_close(got[ri, cj], oracle.gemm_bf16_sampled(A, Bt, ri, cj), w.K, "bf16 8192 sampled")


# ---- bf16 operands with the fused bias and ReLU (hgemm_bf16_bias_act):
# C = act(alpha·A·B + beta·C + bias) in one launch, against the oracle's
# fused bf16 definition.
def run_epi(hg, A, Bt, C0, bias, relu, alpha, beta, out):
    import torch
    dev = torch.device("cuda:0")
    M, K = A.shape
    N = Bt.shape[0]
    print(f"[bf16-epi] M={M} N={N} K={K} relu={relu} beta={beta} out={out}", flush=True)
    Ad = _bf16_tensor(A, dev)
    Bd = _bf16_tensor(Bt, dev)
    Cd = _bf16_tensor(C0, dev) if out == "bf16" else torch.from_numpy(C0).to(dev)
    bd = torch.from_numpy(bias).to(dev)
    hg.hgemm_bias_act(Ad, Bd, Cd, bd, relu, alpha, beta)
    torch.cuda.synchronize()
    if out == "bf16":
        bits = Cd.view(torch.int16).cpu().numpy().view(np.uint16)
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return Cd.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("M,N,K,out,beta", CASES)
@pytest.mark.parametrize("relu", [False, True])
def test_bias_act_parity(hg, M, N, K, out, beta, relu):
    rng = np.random.default_rng(M + N + K + 7 * relu)
    A = workloads.uniform_bf16(rng, (M, K))
    Bt = workloads.uniform_bf16(rng, (N, K))
    C0 = workloads.uniform_bf16(rng, (M, N)) if out == "bf16" else rng.uniform(-1, 1, (M, N)).astype(np.float32)
    bias = rng.uniform(-2, 2, N).astype(np.float32)
    got = run_epi(hg, A, Bt, C0, bias, relu, 1.25, beta, out)
    ref = oracle.gemm_bf16_bias_act(A, Bt, 1.25, beta, C0 if beta else None, bias,
                                    oracle.ACT_RELU if relu else oracle.ACT_NONE, cin_bf16=(out == "bf16"))
    check_close(got, ref, K, f"bf16 bias {M}x{N}x{K} {out} relu={relu}",
                rel=REL_BF16 if out == "bf16" else 2.0 ** -10)
    if relu:
        assert (got >= 0).all()


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 512), (1000, 1000, 1000), (77, 50, 24)])
def test_bias_act_integer_bit_exact(hg, M, N, K):
    rng = np.random.default_rng(K + 3)
    A = workloads.to_bf16_bits(rng.integers(-4, 5, (M, K)).astype(np.float32))
    Bt = workloads.to_bf16_bits(rng.integers(-4, 5, (N, K)).astype(np.float32))
    C0 = rng.integers(-4, 5, (M, N)).astype(np.float32)
    bias = rng.integers(-40, 41, N).astype(np.float32)
    got = run_epi(hg, A, Bt, C0, bias, True, 1.0, 2.0, "f32")
    assert np.array_equal(got, oracle.gemm_bf16_bias_act(A, Bt, 1.0, 2.0, C0, bias, oracle.ACT_RELU))
