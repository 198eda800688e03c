"""Seeded synthetic inputs for the HGEMM and TRMM workloads.

This module draws random numbers and lays them out; it holds none of the
method's arithmetic.  Both the HIP path (through the tests and ``bench.py``)
and the fp64 oracle consume exactly the fp16 bytes produced here.

Recipe: ``rng = numpy.random.default_rng(seed)`` (PCG64); every real-valued
draw is ``rng.uniform(lo, hi, shape)`` in float64, rounded to float16 with
``astype`` (round to nearest even), drawn in the order listed in ``WORKLOADS``.

Layouts (the HGEMM problem statement of "Nvidia Tensor Core-MMA PTX编程入门"
§4): A is M×K row-major, B is K×N column-major, which is handed over as its
(N, K) row-major transpose ``Bt``; C is M×N row-major.  TRMM matrices are
column-major ("异构计算中高性能TRMM与TRSM的递归算法实现" works on Julia arrays,
which are column-major): a column-major n×m matrix is handed over as an
(m, n) row-major array whose row j is column j.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class GemmWorkload:
    name: str
    M: int
    N: int
    K: int
    alpha: float
    beta: float
    out_dtype: str          # "f16" or "f32"
    seed: int
    note: str = ""

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K


@dataclass(frozen=True)
class TrmmWorkload:
    name: str
    n: int
    m: int
    alpha: float
    leaf: int
    seed: int
    out_dtype: str = "f32"
    note: str = ""

    @property
    def flops(self) -> float:
        # Σ_i 2·(n-i)·m multiply-adds over the triangle = n(n+1)m
        return float(self.n) * (self.n + 1) * self.m


WORKLOADS = {
    "hgemm_256": GemmWorkload("hgemm_256", 256, 256, 256, 1.0, 0.0, "f16", 0,
                              "A, Bt U[-1,1]; C pre-filled with NaN (beta = 0 must not read it)"),
    "hgemm_1000_ragged": GemmWorkload("hgemm_1000_ragged", 1000, 1000, 1000, 1.5, 0.5,
                                      "f16", 1, "A, Bt, C0 U[-1,1]; not tile multiples"),
    "hgemm_4096": GemmWorkload("hgemm_4096", 4096, 4096, 4096, 1.0, 0.0, "f16", 2),
    "hgemm_8192": GemmWorkload("hgemm_8192", 8192, 8192, 8192, 1.0, 0.0, "f32", 3),
    "trmm_8192": TrmmWorkload("trmm_8192", 8192, 8192, 1.0, 256, 4, "f32",
                              "A lower: strict lower U[-1,1], diagonal U[0.5,1.5], upper 0"),
}


@dataclass(frozen=True)
class TrsmWorkload:
    name: str
    n: int
    m: int
    alpha: float
    leaf: int
    seed: int
    note: str = ""

    @property
    def flops(self) -> float:
        # back substitution: Σ_i 2·(n-1-i)·m multiply-adds plus n·m divisions ≈ n²·m
        return float(self.n) * self.n * self.m


# The triangular solve X = α·A⁻ᵀ·B ("异构计算中高性能TRMM与TRSM的递归算法实现"
# §2.3, timed there at 8192×8192).  A lower triangular matrix with O(1) random
# off-diagonal entries has a condition number that grows exponentially with n,
# so the strict lower part is scaled by 1/sqrt(n) and the diagonal drawn from
# [1, 2]: the 2-norm condition number stays near 3 at every n.
TRSM_WORKLOADS = {
    "trsm_8192": TrsmWorkload("trsm_8192", 8192, 8192, 1.0, 256, 5,
                              "A lower: strict lower U[-1,1]/sqrt(n), diagonal U[1,2], upper 0; B U[-1,1]"),
}


def uniform_f16(rng: np.random.Generator, shape, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    return rng.uniform(lo, hi, shape).astype(np.float16)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round values to bfloat16 (via float32, round to nearest even on the
    dropped 16 bits; NaN kept quiet) and return the bit patterns as uint16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    r = np.where(nan, (u >> 16) | 0x40, r)
    return r.astype(np.uint16)


def uniform_bf16(rng: np.random.Generator, shape, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    """uniform[lo, hi) in float64, rounded to bf16; returns bit patterns (uint16)."""
    return to_bf16_bits(rng.uniform(lo, hi, shape))


def integer_f16(rng: np.random.Generator, shape, lo: int = -4, hi: int = 4) -> np.ndarray:
    """Integers drawn uniformly from [lo, hi], stored as fp16 (exact)."""
    return rng.integers(lo, hi + 1, size=shape).astype(np.float16)


def gemm_inputs(w: GemmWorkload):
    """Return (A (M,K) f16, Bt (N,K) f16, Cin (M,N) or None) for a workload.

    Draw order: A, Bt, then C0 when beta != 0.  For beta == 0 the C buffer is
    filled with NaN so that an implementation that reads it is caught.
    """
    rng = np.random.default_rng(w.seed)
    A = uniform_f16(rng, (w.M, w.K))
    Bt = uniform_f16(rng, (w.N, w.K))
    odt = np.float16 if w.out_dtype == "f16" else np.float32
    if w.beta != 0.0:
        C = uniform_f16(rng, (w.M, w.N)).astype(odt)
    else:
        C = np.full((w.M, w.N), np.nan, dtype=odt)
    return A, Bt, C


def trmm_inputs(w: TrmmWorkload):
    """Return (A_cm (n,n) f16, B_cm (m,n) f16) in the column-major convention.

    Draw order: S (n,n) U[-1,1], D (n,) U[0.5,1.5], B (n,m) U[-1,1], all
    indexed logically [row, column].  A = strict-lower part of S plus diag(D);
    its upper triangle is exactly zero.
    """
    rng = np.random.default_rng(w.seed)
    n, m = w.n, w.m
    S = uniform_f16(rng, (n, n))
    D = uniform_f16(rng, (n,), 0.5, 1.5)
    B = uniform_f16(rng, (n, m))
    A = np.tril(S, -1)
    A[np.arange(n), np.arange(n)] = D
    del S
    A_cm = np.ascontiguousarray(A.T)   # row c of A_cm = column c of A
    del A
    B_cm = np.ascontiguousarray(B.T)   # row j of B_cm = column j of B
    return A_cm, B_cm


def trsm_inputs(w: TrsmWorkload):
    """Return (A_cm (n,n) f16, B_cm (m,n) f16) in the column-major convention.

    Draw order: S (n,n) U[-1,1], D (n,) U[1,2], B (n,m) U[-1,1], all indexed
    logically [row, column].  A = strict-lower part of S·(1/sqrt(n)), rounded
    to fp16, plus diag(D); its upper triangle is exactly zero.
    """
    rng = np.random.default_rng(w.seed)
    n, m = w.n, w.m
    S = (rng.uniform(-1.0, 1.0, (n, n)) * (1.0 / np.sqrt(n))).astype(np.float16)
    D = uniform_f16(rng, (n,), 1.0, 2.0)
    B = uniform_f16(rng, (n, m))
    A = np.tril(S, -1)
    A[np.arange(n), np.arange(n)] = D
    del S
    A_cm = np.ascontiguousarray(A.T)
    del A
    B_cm = np.ascontiguousarray(B.T)
    return A_cm, B_cm


def sample_indices(seed: int, rows: int, cols: int, count: int = 1024):
    """(count-4) uniform random (i, j) from default_rng(seed + 1000) plus the 4 corners."""
    rng = np.random.default_rng(seed + 1000)
    ri = rng.integers(0, rows, size=count - 4)
    cj = rng.integers(0, cols, size=count - 4)
    ri = np.concatenate([ri, [0, 0, rows - 1, rows - 1]]).astype(np.int64)
    cj = np.concatenate([cj, [0, cols - 1, 0, cols - 1]]).astype(np.int64)
    return ri, cj


def sha256(x: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(x).tobytes()).hexdigest()
