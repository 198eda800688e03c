"""fp64 CPU oracle for half-precision GEMM and lower-triangular transposed TRMM.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The
product library never calls it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over output
rows); this module only marshals numpy arrays to it through ctypes and builds
``liboracle.so`` with gcc when it is missing.

Pages followed (cited by title and section):
  * "Nvidia Tensor Core-MMA PTX编程入门" §4: HGEMM C = A·B, A M×K row-major,
    B K×N column-major, C M×N row-major, fp16 operands.
  * "GPU架构与CUDA", 共享内存与分块 (masked tiled matmul), 混合精度核函数
    (fp16 inputs, wider accumulation) and 核函数融合 (matmul + bias + ReLU).
  * "异构计算中高性能TRMM与TRSM的递归算法实现" §2.1–§2.2: B <- α·Aᵀ·B with A
    lower triangular; §2.3: the triangular solve, here X = α·A⁻ᵀ·B.

Every function here is pinned by ``tests/test_oracle.py`` against closed forms,
brute force and library routines (see that file's docstrings).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# A different build of oracle.c (the pin-strength test compiles deliberately
# broken copies) can be loaded instead through this variable.
_LIB = os.environ.get("ORACLE_LIB_PATH") or os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

F16 = 0
F32 = 1


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so (gcc -O2 -fopenmp, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build()
            lib = ctypes.CDLL(_LIB)
            i64, f64, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
            lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
            lib.oracle_half_to_double.restype = f64
            lib.oracle_hgemm.argtypes = [i64, i64, i64, f64, vp, i64, vp, i64,
                                         f64, vp, i64, ctypes.c_int, vp, i64]
            lib.oracle_hgemm.restype = None
            lib.oracle_hgemm_sampled.argtypes = [i64, f64, vp, i64, vp, i64, f64,
                                                 vp, i64, ctypes.c_int, i64, vp,
                                                 vp, vp]
            lib.oracle_hgemm_sampled.restype = None
            lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
            lib.oracle_bf16_to_double.restype = f64
            lib.oracle_gemm_bf16.argtypes = [i64, i64, i64, f64, vp, i64, vp, i64,
                                             f64, vp, i64, ctypes.c_int, vp, i64]
            lib.oracle_gemm_bf16.restype = None
            lib.oracle_gemm_bf16_sampled.argtypes = [i64, f64, vp, i64, vp, i64, i64,
                                                     vp, vp, vp]
            lib.oracle_gemm_bf16_sampled.restype = None
            lib.oracle_hgemm_bias_act.argtypes = [i64, i64, i64, f64, vp, i64, vp, i64,
                                                  f64, vp, i64, ctypes.c_int, vp,
                                                  ctypes.c_int, vp, i64]
            lib.oracle_hgemm_bias_act.restype = None
            lib.oracle_trmm_lower_trans.argtypes = [i64, i64, f64, vp, i64, vp,
                                                    i64, vp, i64]
            lib.oracle_trmm_lower_trans.restype = None
            lib.oracle_trmm_lower_trans_sampled.argtypes = [i64, f64, vp, i64,
                                                            vp, i64, i64, vp,
                                                            vp, vp]
            lib.oracle_trmm_lower_trans_sampled.restype = None
            lib.oracle_trmm.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, f64, vp, i64,
                                        vp, i64, vp, i64]
            lib.oracle_trmm.restype = None
            lib.oracle_trmm_sampled.argtypes = [ctypes.c_int, ctypes.c_int, i64, f64, vp, i64,
                                                vp, i64, i64, vp, vp, vp]
            lib.oracle_trmm_sampled.restype = None
            lib.oracle_trsm_lower_trans.argtypes = [i64, i64, f64, vp, i64, vp,
                                                    i64, vp, i64]
            lib.oracle_trsm_lower_trans.restype = None
            lib.oracle_trsm_lower_trans_cols.argtypes = [i64, f64, vp, i64, vp, i64,
                                                         i64, vp, vp, i64]
            lib.oracle_trsm_lower_trans_cols.restype = None
            lib.oracle_num_threads.argtypes = []
            lib.oracle_num_threads.restype = ctypes.c_int
            lib.oracle_gemm_bf16_bias_act.argtypes = [i64, i64, i64, f64, vp, i64, vp, i64,
                                                      f64, vp, i64, ctypes.c_int, vp,
                                                      ctypes.c_int, vp, i64]
            lib.oracle_gemm_bf16_bias_act.restype = None
            lib.oracle_gemm_bias_act_sampled.argtypes = [ctypes.c_int, i64, f64, vp, i64, vp,
                                                         i64, f64, vp, i64, ctypes.c_int, vp,
                                                         ctypes.c_int, i64, vp, vp, vp]
            lib.oracle_gemm_bias_act_sampled.restype = None
            lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
            lib.oracle_set_num_threads.restype = None
            _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f16_2d(x: np.ndarray, name: str) -> np.ndarray:
    if x.dtype != np.float16 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D float16 array")
    if x.size and x.shape[1] > 1 and x.strides[1] != 2:
        raise ValueError(f"{name} must have unit stride along its last axis")
    return x


def _ld(x: np.ndarray) -> int:
    return max(1, x.strides[0] // x.itemsize) if x.shape[0] > 1 else max(1, x.shape[1])


def half_to_double(bits: int) -> float:
    """Decode one binary16 bit pattern (the oracle's own decoder)."""
    return _load().oracle_half_to_double(bits)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return _load().oracle_num_threads()


def hgemm(A: np.ndarray, Bt: np.ndarray, alpha: float = 1.0, beta: float = 0.0,
          Cin: np.ndarray | None = None) -> np.ndarray:
    """fp64 reference of α·A·B + β·C_in.

    ``A`` is (M, K) fp16 row-major; ``Bt`` is (N, K) fp16, i.e. B (K×N)
    stored column-major; ``Cin`` is (M, N) fp16 or fp32, read only when
    ``beta != 0``.  Returns the (M, N) fp64 result.
    """
    lib = _load()
    _f16_2d(A, "A")
    _f16_2d(Bt, "Bt")
    M, K = A.shape
    N, K2 = Bt.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    ref = np.empty((M, N), dtype=np.float64)
    cin_dtype, cptr, ldc = F16, None, max(1, N)
    if beta != 0.0:
        if Cin is None or Cin.shape != (M, N) or Cin.strides[1] != Cin.itemsize:
            raise ValueError("Cin of shape (M, N) with unit column stride needed when beta != 0")
        if Cin.dtype == np.float16:
            cin_dtype = F16
        elif Cin.dtype == np.float32:
            cin_dtype = F32
        else:
            raise TypeError("Cin must be float16 or float32")
        cptr, ldc = _ptr(Cin), _ld(Cin)
    if M and N:
        lib.oracle_hgemm(M, N, K, float(alpha), _ptr(A), _ld(A), _ptr(Bt), _ld(Bt),
                         float(beta), cptr, ldc, cin_dtype, _ptr(ref), N)
    return ref


ACT_NONE = 0
ACT_RELU = 1
BF16 = 2


def bf16_to_double(bits: int) -> float:
    """Decode one bfloat16 bit pattern (the oracle's own decoder)."""
    return _load().oracle_bf16_to_double(bits)


def _bf16_2d(x: np.ndarray, name: str) -> np.ndarray:
    if x.dtype != np.uint16 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D uint16 array of bf16 bit patterns")
    if x.size and x.shape[1] > 1 and x.strides[1] != 2:
        raise ValueError(f"{name} must have unit stride along its last axis")
    return x


def gemm_bf16(A: np.ndarray, Bt: np.ndarray, alpha: float = 1.0, beta: float = 0.0,
              Cin: np.ndarray | None = None, cin_bf16: bool = False) -> np.ndarray:
    """fp64 reference of α·A·B + β·C_in with bf16 operands.

    ``A`` (M, K) and ``Bt`` (N, K) are uint16 arrays of bf16 bit patterns in
    the layouts of ``hgemm``; ``Cin`` (M, N) is float32, or bf16 bit patterns
    (uint16) when ``cin_bf16``.  Returns the (M, N) fp64 result.
    """
    lib = _load()
    _bf16_2d(A, "A")
    _bf16_2d(Bt, "Bt")
    M, K = A.shape
    N, K2 = Bt.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    ref = np.empty((M, N), dtype=np.float64)
    cin_dtype, cptr, ldc = F32, None, max(1, N)
    if beta != 0.0:
        if Cin is None or Cin.shape != (M, N) or Cin.strides[1] != Cin.itemsize:
            raise ValueError("Cin of shape (M, N) with unit column stride needed when beta != 0")
        if cin_bf16:
            if Cin.dtype != np.uint16:
                raise TypeError("bf16 Cin must be uint16 bit patterns")
            cin_dtype = BF16
        elif Cin.dtype != np.float32:
            raise TypeError("Cin must be float32 (or bf16 bit patterns with cin_bf16)")
        cptr, ldc = _ptr(Cin), _ld(Cin)
    if M and N:
        lib.oracle_gemm_bf16(M, N, K, float(alpha), _ptr(A), _ld(A), _ptr(Bt), _ld(Bt),
                             float(beta), cptr, ldc, cin_dtype, _ptr(ref), N)
    return ref


def gemm_bf16_sampled(A: np.ndarray, Bt: np.ndarray, rows: np.ndarray, cols: np.ndarray,
                      alpha: float = 1.0) -> np.ndarray:
    """``gemm_bf16`` (β = 0) at entries (rows[s], cols[s])."""
    lib = _load()
    _bf16_2d(A, "A")
    _bf16_2d(Bt, "Bt")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= A.shape[0] or
                      cols.min() < 0 or cols.max() >= Bt.shape[0]):
        raise IndexError("sample index out of range")
    ref = np.empty(rows.shape, dtype=np.float64)
    lib.oracle_gemm_bf16_sampled(A.shape[1], float(alpha), _ptr(A), _ld(A), _ptr(Bt), _ld(Bt),
                                 rows.size, _ptr(rows), _ptr(cols), _ptr(ref))
    return ref


def hgemm_bias_act(A: np.ndarray, Bt: np.ndarray, alpha: float = 1.0, beta: float = 0.0,
                   Cin: np.ndarray | None = None, bias: np.ndarray | None = None,
                   act: int = ACT_NONE) -> np.ndarray:
    """fp64 reference of act(α·A·B + β·C_in + bias), bias a float32 vector of
    length N added to every row (None: no bias), act ACT_NONE or ACT_RELU
    (t < 0 → +0; NaN passes through).  Layouts as in ``hgemm``."""
    lib = _load()
    _f16_2d(A, "A")
    _f16_2d(Bt, "Bt")
    M, K = A.shape
    N, K2 = Bt.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    if act not in (ACT_NONE, ACT_RELU):
        raise ValueError("act must be ACT_NONE or ACT_RELU")
    bptr = None
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        if bias.shape != (N,):
            raise ValueError("bias must have shape (N,)")
        bptr = _ptr(bias)
    ref = np.empty((M, N), dtype=np.float64)
    cin_dtype, cptr, ldc = F16, None, max(1, N)
    if beta != 0.0:
        if Cin is None or Cin.shape != (M, N) or Cin.strides[1] != Cin.itemsize:
            raise ValueError("Cin of shape (M, N) with unit column stride needed when beta != 0")
        cin_dtype = F16 if Cin.dtype == np.float16 else F32
        cptr, ldc = _ptr(Cin), _ld(Cin)
    if M and N:
        lib.oracle_hgemm_bias_act(M, N, K, float(alpha), _ptr(A), _ld(A), _ptr(Bt), _ld(Bt),
                                  float(beta), cptr, ldc, cin_dtype, bptr, int(act), _ptr(ref), N)
    return ref


def gemm_bf16_bias_act(A: np.ndarray, Bt: np.ndarray, alpha: float = 1.0, beta: float = 0.0,
                       Cin: np.ndarray | None = None, bias: np.ndarray | None = None,
                       act: int = ACT_NONE, cin_bf16: bool = False) -> np.ndarray:
    """fp64 reference of act(α·A·B + β·C_in + bias) with bf16 operands.

    ``A`` (M, K) and ``Bt`` (N, K) are uint16 arrays of bf16 bit patterns in
    the layouts of ``hgemm``; ``Cin`` (M, N) is float32, or bf16 bit patterns
    when ``cin_bf16``, read only when ``beta != 0``; ``bias`` a float32
    vector of length N (None: no bias); ``act`` ACT_NONE or ACT_RELU."""
    lib = _load()
    _bf16_2d(A, "A")
    _bf16_2d(Bt, "Bt")
    M, K = A.shape
    N, K2 = Bt.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    if act not in (ACT_NONE, ACT_RELU):
        raise ValueError("act must be ACT_NONE or ACT_RELU")
    bptr = None
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        if bias.shape != (N,):
            raise ValueError("bias must have shape (N,)")
        bptr = _ptr(bias)
    ref = np.empty((M, N), dtype=np.float64)
    cin_dtype, cptr, ldc = F32, None, max(1, N)
    if beta != 0.0:
        cin_dtype, cptr, ldc = _cin_args(Cin, (M, N), cin_bf16)
    if M and N:
        lib.oracle_gemm_bf16_bias_act(M, N, K, float(alpha), _ptr(A), _ld(A), _ptr(Bt), _ld(Bt),
                                      float(beta), cptr, ldc, cin_dtype, bptr, int(act),
                                      _ptr(ref), N)
    return ref


def _cin_args(Cin, shape, cin_bf16):
    """(cin_dtype, pointer, ldc) of an incoming C: fp16, fp32, or bf16 bit
    patterns (uint16) when ``cin_bf16``."""
    if Cin is None or Cin.shape != shape or (Cin.size and Cin.strides[1] != Cin.itemsize):
        raise ValueError("Cin of shape (M, N) with unit column stride needed when beta != 0")
    if cin_bf16:
        if Cin.dtype != np.uint16:
            raise TypeError("bf16 Cin must be uint16 bit patterns")
        return BF16, _ptr(Cin), _ld(Cin)
    if Cin.dtype == np.float16:
        return F16, _ptr(Cin), _ld(Cin)
    if Cin.dtype == np.float32:
        return F32, _ptr(Cin), _ld(Cin)
    raise TypeError("Cin must be float16 or float32 (or bf16 bit patterns with cin_bf16)")


def gemm_bias_act_sampled(A: np.ndarray, Bt: np.ndarray, rows: np.ndarray, cols: np.ndarray,
                          alpha: float = 1.0, beta: float = 0.0, Cin: np.ndarray | None = None,
                          bias: np.ndarray | None = None, act: int = ACT_NONE,
                          bf16: bool = False, cin_bf16: bool = False) -> np.ndarray:
    """act(α·A·B + β·C_in + bias) evaluated only at entries (rows[s], cols[s]).

    ``A``/``Bt`` are fp16 arrays, or uint16 bf16 bit patterns when ``bf16``;
    ``Cin`` as in ``gemm_bf16_bias_act`` (fp16 or fp32 for fp16 operands)."""
    lib = _load()
    if bf16:
        _bf16_2d(A, "A")
        _bf16_2d(Bt, "Bt")
    else:
        _f16_2d(A, "A")
        _f16_2d(Bt, "Bt")
    if A.shape[1] != Bt.shape[1]:
        raise ValueError("inner dimensions differ")
    if act not in (ACT_NONE, ACT_RELU):
        raise ValueError("act must be ACT_NONE or ACT_RELU")
    N = Bt.shape[0]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows and cols differ in length")
    if rows.size and (rows.min() < 0 or rows.max() >= A.shape[0] or
                      cols.min() < 0 or cols.max() >= N):
        raise IndexError("sample index out of range")
    bptr = None
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        if bias.shape != (N,):
            raise ValueError("bias must have shape (N,)")
        bptr = _ptr(bias)
    cin_dtype, cptr, ldc = F16, None, 1
    if beta != 0.0:
        cin_dtype, cptr, ldc = _cin_args(Cin, (A.shape[0], N), cin_bf16)
    ref = np.empty(rows.shape, dtype=np.float64)
    lib.oracle_gemm_bias_act_sampled(BF16 if bf16 else F16, A.shape[1], float(alpha), _ptr(A), _ld(A),
                                     _ptr(Bt), _ld(Bt), float(beta), cptr, ldc, cin_dtype, bptr,
                                     int(act), rows.size, _ptr(rows), _ptr(cols), _ptr(ref))
    return ref


def set_num_threads(n: int) -> None:
    """Threads the oracle's parallel loops use from now on (n >= 1)."""
    _load().oracle_set_num_threads(int(n))


def hgemm_sampled(A: np.ndarray, Bt: np.ndarray, rows: np.ndarray, cols: np.ndarray,
                  alpha: float = 1.0, beta: float = 0.0,
                  Cin: np.ndarray | None = None) -> np.ndarray:
    """The ``hgemm`` definition evaluated only at entries (rows[s], cols[s])."""
    lib = _load()
    _f16_2d(A, "A")
    _f16_2d(Bt, "Bt")
    K = A.shape[1]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows and cols differ in length")
    if rows.size and (rows.min() < 0 or rows.max() >= A.shape[0] or
                      cols.min() < 0 or cols.max() >= Bt.shape[0]):
        raise IndexError("sample index out of range")
    ref = np.empty(rows.shape, dtype=np.float64)
    cin_dtype, cptr, ldc = F16, None, 1
    if beta != 0.0:
        cin_dtype = F16 if Cin.dtype == np.float16 else F32
        cptr, ldc = _ptr(Cin), _ld(Cin)
    lib.oracle_hgemm_sampled(K, float(alpha), _ptr(A), _ld(A), _ptr(Bt), _ld(Bt),
                             float(beta), cptr, ldc, cin_dtype, rows.size,
                             _ptr(rows), _ptr(cols), _ptr(ref))
    return ref


def trmm_lower_trans(A_cm: np.ndarray, B_cm: np.ndarray, alpha: float = 1.0) -> np.ndarray:
    """fp64 reference of Out = α·Aᵀ·B, A lower triangular (strict upper unread).

    Column-major matrices are passed as their row-major transposes: ``A_cm``
    is an (n, n) fp16 array whose row c holds column c of A; ``B_cm`` is an
    (m, n) fp16 array whose row j holds column j of B.  Returns Out in the
    same convention, an (m, n) fp64 array whose row j is column j of Out.
    """
    lib = _load()
    _f16_2d(A_cm, "A_cm")
    _f16_2d(B_cm, "B_cm")
    n = A_cm.shape[0]
    if A_cm.shape != (n, n) or B_cm.shape[1] != n:
        raise ValueError("shape mismatch")
    m = B_cm.shape[0]
    ref = np.empty((m, n), dtype=np.float64)
    if n and m:
        lib.oracle_trmm_lower_trans(n, m, float(alpha), _ptr(A_cm), _ld(A_cm),
                                    _ptr(B_cm), _ld(B_cm), _ptr(ref), n)
    return ref


def trmm_lower_trans_sampled(A_cm: np.ndarray, B_cm: np.ndarray, rows: np.ndarray,
                             cols: np.ndarray, alpha: float = 1.0) -> np.ndarray:
    """``trmm_lower_trans`` at entries (row i, column j) = (rows[s], cols[s])."""
    lib = _load()
    _f16_2d(A_cm, "A_cm")
    _f16_2d(B_cm, "B_cm")
    n = A_cm.shape[0]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= n or
                      cols.min() < 0 or cols.max() >= B_cm.shape[0]):
        raise IndexError("sample index out of range")
    ref = np.empty(rows.shape, dtype=np.float64)
    lib.oracle_trmm_lower_trans_sampled(n, float(alpha), _ptr(A_cm), _ld(A_cm),
                                        _ptr(B_cm), _ld(B_cm), rows.size,
                                        _ptr(rows), _ptr(cols), _ptr(ref))
    return ref


LOWER, UPPER = 0, 1
NOTRANS, TRANS = 0, 1


def trmm(A_cm: np.ndarray, B_cm: np.ndarray, alpha: float = 1.0, uplo: int = LOWER,
         trans: int = TRANS) -> np.ndarray:
    """fp64 reference of Out = α·op(A)·B, A triangular (uplo LOWER or UPPER;
    only that triangle read), op = transpose when trans == TRANS.  Same
    column-major convention as ``trmm_lower_trans``."""
    lib = _load()
    _f16_2d(A_cm, "A_cm")
    _f16_2d(B_cm, "B_cm")
    n = A_cm.shape[0]
    if A_cm.shape != (n, n) or B_cm.shape[1] != n:
        raise ValueError("shape mismatch")
    if uplo not in (LOWER, UPPER) or trans not in (NOTRANS, TRANS):
        raise ValueError("uplo / trans out of range")
    m = B_cm.shape[0]
    ref = np.empty((m, n), dtype=np.float64)
    if n and m:
        lib.oracle_trmm(int(uplo), int(trans), n, m, float(alpha), _ptr(A_cm), _ld(A_cm),
                        _ptr(B_cm), _ld(B_cm), _ptr(ref), n)
    return ref


def trmm_sampled(A_cm: np.ndarray, B_cm: np.ndarray, rows: np.ndarray, cols: np.ndarray,
                 alpha: float = 1.0, uplo: int = LOWER, trans: int = TRANS) -> np.ndarray:
    """``trmm`` at entries (row i, column j) = (rows[s], cols[s])."""
    lib = _load()
    _f16_2d(A_cm, "A_cm")
    _f16_2d(B_cm, "B_cm")
    n = A_cm.shape[0]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= n or
                      cols.min() < 0 or cols.max() >= B_cm.shape[0]):
        raise IndexError("sample index out of range")
    ref = np.empty(rows.shape, dtype=np.float64)
    lib.oracle_trmm_sampled(int(uplo), int(trans), n, float(alpha), _ptr(A_cm), _ld(A_cm),
                            _ptr(B_cm), _ld(B_cm), rows.size, _ptr(rows), _ptr(cols), _ptr(ref))
    return ref


def trsm_lower_trans(A_cm: np.ndarray, B_cm: np.ndarray, alpha: float = 1.0) -> np.ndarray:
    """fp64 reference of X = α·A⁻ᵀ·B (the X with Aᵀ·X = α·B), A lower
    triangular (strict upper unread), by back substitution per column.

    Same convention as ``trmm_lower_trans``: ``A_cm`` (n, n) fp16 whose row c
    is column c of A, ``B_cm`` (m, n) fp16 whose row j is column j of B.
    Returns X as an (m, n) fp64 array whose row j is column j of X.
    """
    lib = _load()
    _f16_2d(A_cm, "A_cm")
    _f16_2d(B_cm, "B_cm")
    n = A_cm.shape[0]
    if A_cm.shape != (n, n) or B_cm.shape[1] != n:
        raise ValueError("shape mismatch")
    m = B_cm.shape[0]
    ref = np.empty((m, n), dtype=np.float64)
    if n and m:
        lib.oracle_trsm_lower_trans(n, m, float(alpha), _ptr(A_cm), _ld(A_cm),
                                    _ptr(B_cm), _ld(B_cm), _ptr(ref), n)
    return ref


def trsm_lower_trans_cols(A_cm: np.ndarray, B_cm: np.ndarray, cols: np.ndarray,
                          alpha: float = 1.0) -> np.ndarray:
    """``trsm_lower_trans`` for the listed columns of B only: row s of the
    (len(cols), n) result is column cols[s] of X."""
    lib = _load()
    _f16_2d(A_cm, "A_cm")
    _f16_2d(B_cm, "B_cm")
    n = A_cm.shape[0]
    if A_cm.shape != (n, n) or B_cm.shape[1] != n:
        raise ValueError("shape mismatch")
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if cols.size and (cols.min() < 0 or cols.max() >= B_cm.shape[0]):
        raise IndexError("column index out of range")
    ref = np.empty((cols.size, n), dtype=np.float64)
    if n and cols.size:
        lib.oracle_trsm_lower_trans_cols(n, float(alpha), _ptr(A_cm), _ld(A_cm),
                                         _ptr(B_cm), _ld(B_cm), cols.size, _ptr(cols),
                                         _ptr(ref), n)
    return ref
