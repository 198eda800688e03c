"""GPU parity of hgemm_layout (A row- or column-major, B column- or
row-major; "GPU架构与CUDA"'s matmul stores B row-major) against the fp64 oracle,
through the C ABI.  The oracle's definition does not depend on storage, so the
test hands it the same matrices re-laid in its own layout (numpy transposes:
storage only, no arithmetic).  Same rule as the HGEMM; the product must also be
bit-identical to hgemm on operands transposed beforehand (same kernels)."""
import numpy as np
import pytest

import oracle
import workloads
from tolerance import check_close

pytestmark = pytest.mark.gpu

LAYOUTS = [(False, False), (True, False), (False, True), (True, True)]   # (A col-major, B row-major)


def run(hg, A_store, B_store, M, N, C0, a_col, b_row, alpha, beta, out):
    import torch
    dev = torch.device("cuda:0")
    print(f"[layout] M={M} N={N} a_col={a_col} b_row={b_row} out={out}", flush=True)
    A = torch.from_numpy(A_store).to(dev)
    B = torch.from_numpy(B_store).to(dev)
    C = torch.from_numpy(C0.astype(np.float16 if out == "f16" else np.float32)).to(dev)
    hg.hgemm_layout(A, B, C, a_col, b_row, alpha, beta)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def _case(M, N, K, seed):
    rng = np.random.default_rng(seed)
    A = workloads.uniform_f16(rng, (M, K))        # logical A, M×K
    Bt = workloads.uniform_f16(rng, (N, K))       # logical Bᵀ, N×K (B is K×N)
    C0 = workloads.uniform_f16(rng, (M, N))
    return A, Bt, C0


def _stores(A, Bt, a_col, b_row):
    A_store = np.ascontiguousarray(A.T) if a_col else A          # column-major M×K = (K, M) array
    B_store = np.ascontiguousarray(Bt.T) if b_row else Bt        # row-major K×N = (K, N) array
    return A_store, B_store


@pytest.mark.parametrize("a_col,b_row", LAYOUTS)
@pytest.mark.parametrize("M,N,K,out,beta", [(256, 256, 256, "f16", 0.0), (1000, 1000, 1000, "f16", 0.5),
                                            (4096, 4096, 512, "f32", 0.0), (300, 257, 33, "f32", 1.0)])
def test_parity(hg, a_col, b_row, M, N, K, out, beta):
    A, Bt, C0 = _case(M, N, K, M + K)
    A_store, B_store = _stores(A, Bt, a_col, b_row)
    got = run(hg, A_store, B_store, M, N, C0, a_col, b_row, 1.5, beta, out)
    cin = C0.astype(np.float16 if out == "f16" else np.float32)
    check_close(got, oracle.hgemm(A, Bt, 1.5, beta, cin if beta else None), K,
                f"layout a_col={a_col} b_row={b_row} {M}x{N}x{K}")


@pytest.mark.parametrize("a_col,b_row", LAYOUTS[1:])
def test_bit_identical_to_hgemm_on_transposed_operands(hg, a_col, b_row):
    import torch
    M, N, K = 2048, 1536, 768
    A, Bt, C0 = _case(M, N, K, 3)
    A_store, B_store = _stores(A, Bt, a_col, b_row)
    got = run(hg, A_store, B_store, M, N, C0, a_col, b_row, 1.0, 0.0, "f32")
    dev = torch.device("cuda:0")
    C = torch.empty((M, N), dtype=torch.float32, device=dev)
    hg.hgemm(torch.from_numpy(A).to(dev), torch.from_numpy(Bt).to(dev), C)
    torch.cuda.synchronize()
    assert np.array_equal(got.view(np.uint32), C.cpu().numpy().view(np.uint32))


def test_row_major_b_8192_sampled(hg):
    """8192³ with the page's row-major B, fp32 C, 1024 sampled entries."""
    w = workloads.WORKLOADS["hgemm_8192"]
    A, Bt, _ = workloads.gemm_inputs(w)
    got = run(hg, A, np.ascontiguousarray(Bt.T), w.M, w.N, np.zeros((w.M, w.N), np.float32), False, True,
              1.0, 0.0, "f32")
    ri, cj = workloads.sample_indices(w.seed, w.M, w.N)
    check_close(got[ri, cj], oracle.hgemm_sampled(A, Bt, ri, cj), w.K, "row-major B 8192 sampled")
