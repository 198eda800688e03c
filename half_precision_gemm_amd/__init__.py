"""Python binding of libhgemm.so, the MI355X (gfx950) half-precision GEMM and
recursive TRMM library whose C ABI is declared in include/hgemm.h.

Argument marshalling only: every step of the computation runs in the
library's HIP kernels.  PyTorch supplies device memory and the current
stream.  There is no fallback: if the library is missing or fails to load,
importing this package raises.

    hgemm(A, Bt, C, alpha=1.0, beta=0.0)
        C = alpha·A·B + beta·C.  A: (M, K) float16, row-major.  Bt: (N, K)
        float16, which is B (K×N) stored column-major.  C: (M, N) float16 or
        float32, row-major.  Each needs unit stride along its last axis; row
        strides become lda / ldb / ldc.

    hgemm_bf16(A, Bt, C, alpha=1.0, beta=0.0)
        hgemm with bfloat16 A and Bt; C bfloat16 or float32.

    hgemm_layout(A, B, C, a_col_major=False, b_row_major=False, alpha, beta, work)
        hgemm with A column-major and/or B row-major (transposed into a
        workspace first).

    hgemm_bias_act(A, Bt, C, bias=None, relu=False, alpha=1.0, beta=0.0)
        C = act(alpha·A·B + beta·C + bias) in one launch, bias a float32
        device vector of length N added to every row, act ReLU or none;
        float16 or bfloat16 operands.

    hgemm_splitk(A, Bt, C, alpha=1.0, beta=0.0, splits=0, work=None)
        hgemm with K cut into slices run side by side (few output tiles,
        long K); partial products summed in order in fp32.

    hgemm_splitk_noalloc(A, Bt, C, alpha=1.0, beta=0.0, splits=0)
        the same with the partials in the library's static device array (no
        workspace, nothing allocated; calls overlapping on one GPU race).

    trmm(A, B, Out, alpha=1.0, uplo="L", trans=True, leaf=256, work=None)
        Out = alpha·op(A)·B for every triangle / transposition.

    trmm_inplace(A, B, alpha=1.0, uplo="L", trans=True, leaf=256, work=None)
        B = alpha·op(A)·B with B float16, overwritten (the product formed in
        fp32 and rounded once).

    trmm_lower_trans(A, B, Out, alpha=1.0, leaf=256)
    trmm_lower_trans_by_level(A, B, Out, alpha=1.0, leaf=256)
        Out = alpha·Aᵀ·B with A lower triangular (strict upper never read);
        the second schedules it one launch per recursion level.
        Column-major matrices are passed as their row-major transposes:
        A is an (n, n) float16 tensor whose row c is column c of A; B is
        (m, n) float16 whose row j is column j of B; Out is (m, n) float32
        in the same convention.

    trsm_lower_trans(A, B, Out, alpha=1.0, leaf=256, work=None)
        Out = alpha·A⁻ᵀ·B (the X with Aᵀ·X = alpha·B), A lower triangular,
        same conventions as trmm_lower_trans.  `work` is a device uint8
        tensor of at least trsm_workspace_size(n, m, leaf) bytes; when None
        one is allocated with torch for the call.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhgemm.so")

HG_F16 = 0
HG_F32 = 1
HG_BF16 = 2

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                      "or python half_precision_gemm_amd/build.py")

# PyTorch ships its own HIP runtime and loads it under a name the dynamic
# loader does not match against the system copy the library was linked with.
# Loading the library first would put two HIP runtimes in the process, and
# the library's launches would then go through one that does not own the
# tensors' memory or streams.  Importing torch first makes the library bind
# to torch's runtime (same soname), so there is exactly one.
import torch  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)
_i64, _f32, _vp, _int = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_int
lib.hgemm.argtypes = [_i64, _i64, _i64, _f32, _vp, _i64, _vp, _i64, _f32, _vp, _i64, _int, _vp]
lib.hgemm.restype = _int
lib.hgemm_bias_act.argtypes = [_i64, _i64, _i64, _f32, _vp, _i64, _vp, _i64, _f32, _vp, _i64, _int,
                               _vp, _int, _vp]
lib.hgemm_bias_act.restype = _int
lib.hgemm_layout.argtypes = [_int, _int, _i64, _i64, _i64, _f32, _vp, _i64, _vp, _i64, _f32, _vp,
                             _i64, _int, _vp, _i64, _vp]
lib.hgemm_layout.restype = _int
lib.hg_hgemm_layout_workspace_size.argtypes = [_int, _int, _i64, _i64, _i64]
lib.hg_hgemm_layout_workspace_size.restype = _i64
lib.hgemm_bf16.argtypes = lib.hgemm.argtypes
lib.hgemm_bf16.restype = _int
lib.trmm_lower_trans.argtypes = [_i64, _i64, _f32, _vp, _i64, _vp, _i64, _vp, _i64, _int, _i64,
                                 _vp]
lib.trmm_lower_trans.restype = _int
lib.hg_trmm.argtypes = [_int, _int, _i64, _i64, _f32, _vp, _i64, _vp, _i64, _vp, _i64, _int, _i64,
                        _vp, _i64, _vp]
lib.hg_trmm.restype = _int
lib.hg_trmm_workspace_size.argtypes = [_int, _int, _i64, _i64]
lib.hg_trmm_workspace_size.restype = _i64
lib.hgemm_bf16_bias_act.argtypes = lib.hgemm_bias_act.argtypes
lib.hgemm_bf16_bias_act.restype = _int
lib.hgemm_splitk.argtypes = [_i64, _i64, _i64, _f32, _vp, _i64, _vp, _i64, _f32, _vp, _i64, _int, _int, _vp,
                             _i64, _vp]
lib.hgemm_splitk.restype = _int
lib.hgemm_splitk_noalloc.argtypes = [_i64, _i64, _i64, _f32, _vp, _i64, _vp, _i64, _f32, _vp, _i64, _int,
                                     _int, _vp]
lib.hgemm_splitk_noalloc.restype = _int
lib.hg_hgemm_splitk_workspace_size.argtypes = [_i64, _i64, _i64, _int]
lib.hg_hgemm_splitk_workspace_size.restype = _i64
lib.hg_trmm_inplace.argtypes = [_int, _int, _i64, _i64, _f32, _vp, _i64, _vp, _i64, _i64, _vp, _i64,
                                _vp]
lib.hg_trmm_inplace.restype = _int
lib.hg_trmm_inplace_workspace_size.argtypes = [_int, _int, _i64, _i64]
lib.hg_trmm_inplace_workspace_size.restype = _i64
lib.hg_trmm_lower_trans_by_level.argtypes = lib.trmm_lower_trans.argtypes
lib.hg_trmm_lower_trans_streams.argtypes = [_i64, _i64, _f32, _vp, _i64, _vp, _i64, _vp, _i64, _int, _i64,
                                            ctypes.POINTER(_vp), _int]
lib.hg_trmm_lower_trans_streams.restype = _int
lib.hg_trmm_lower_trans_by_level.restype = _int
lib.trsm_lower_trans.argtypes = [_i64, _i64, _f32, _vp, _i64, _vp, _i64, _vp, _i64, _int, _i64,
                                 _vp, _i64, _vp]
lib.trsm_lower_trans.restype = _int
lib.hg_trsm_workspace_size.argtypes = [_i64, _i64, _i64]
lib.hg_trsm_workspace_size.restype = _i64
lib.hg_strerror.argtypes = [_int]
lib.hg_strerror.restype = ctypes.c_char_p
lib.hg_trmm_plan.argtypes = [_i64, _i64, ctypes.POINTER(_i64), _i64]
lib.hg_trmm_plan.restype = _i64

EXPORTS = ("hgemm", "hgemm_bias_act", "hgemm_bf16", "trmm_lower_trans", "hg_trmm_lower_trans_by_level",
           "hg_strerror", "hg_trmm_plan", "trsm_lower_trans", "hg_trsm_workspace_size", "hg_trmm",
           "hg_trmm_workspace_size", "hgemm_layout", "hg_hgemm_layout_workspace_size",
           "hg_trmm_inplace", "hg_trmm_inplace_workspace_size", "hgemm_splitk", "hgemm_bf16_bias_act",
           "hg_trmm_lower_trans_streams",
           "hg_hgemm_splitk_workspace_size", "hgemm_splitk_noalloc")

ROW_MAJOR = 0
COL_MAJOR = 1

ACT_NONE = 0
ACT_RELU = 1


class HgError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed with status {status}: "
                         f"{lib.hg_strerror(status).decode()}")


def strerror(status: int) -> str:
    return lib.hg_strerror(status).decode()


# The current stream's raw handle of a device: torch's getter of the raw
# pointer when it has one (it skips building a Stream object, which costs
# more than the rest of a small call's marshalling), else the public API.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(t):
    if _raw_stream is not None:
        return _raw_stream(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


def _check_matrix(t, name, dtypes):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    shape = t.shape
    if len(shape) != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if shape[0] and shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} needs unit stride along its last axis")


def _ld(t) -> int:
    return max(1, t.stride(0)) if t.shape[0] > 1 else max(1, t.shape[1])


def hgemm(A, Bt, C, alpha: float = 1.0, beta: float = 0.0):
    """C = alpha·A·B + beta·C on the current stream; returns C."""
    import torch
    _check_matrix(A, "A", (torch.float16,))
    _check_matrix(Bt, "Bt", (torch.float16,))
    _check_matrix(C, "C", (torch.float16, torch.float32))
    M, K = A.shape
    N = Bt.shape[0]
    if Bt.shape[1] != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, Bt {tuple(Bt.shape)}, "
                         f"C {tuple(C.shape)}")
    out_dtype = HG_F16 if C.dtype == torch.float16 else HG_F32
    st = lib.hgemm(M, N, K, float(alpha), A.data_ptr() or None, _ld(A), Bt.data_ptr() or None,
                   _ld(Bt), float(beta), C.data_ptr() or None, _ld(C), out_dtype,
                   _stream_handle(C))
    if st != 0:
        raise HgError("hgemm", st)
    return C


def hgemm_splitk(A, Bt, C, alpha: float = 1.0, beta: float = 0.0, splits: int = 0, work=None):
    """hgemm with K split into `splits` slices (0: chosen from the shape and
    the device) summed in order in fp32; `work`: device uint8 tensor of at
    least splitk_workspace_size(M, N, K, splits) bytes (allocated with torch
    when None).  Returns C."""
    import torch
    _check_matrix(A, "A", (torch.float16,))
    _check_matrix(Bt, "Bt", (torch.float16,))
    _check_matrix(C, "C", (torch.float16, torch.float32))
    M, K = A.shape
    N = Bt.shape[0]
    if Bt.shape[1] != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, Bt {tuple(Bt.shape)}, "
                         f"C {tuple(C.shape)}")
    need = lib.hg_hgemm_splitk_workspace_size(M, N, K, int(splits))
    if need < 0:
        raise HgError("hg_hgemm_splitk_workspace_size", int(need))
    if work is None:
        work = torch.empty(max(need, 1), dtype=torch.uint8, device=C.device)
    out_dtype = HG_F16 if C.dtype == torch.float16 else HG_F32
    st = lib.hgemm_splitk(M, N, K, float(alpha), A.data_ptr() or None, _ld(A), Bt.data_ptr() or None,
                          _ld(Bt), float(beta), C.data_ptr() or None, _ld(C), out_dtype, int(splits),
                          work.data_ptr(), work.numel() * work.element_size(), _stream_handle(C))
    if st != 0:
        raise HgError("hgemm_splitk", st)
    return C


def hgemm_splitk_noalloc(A, Bt, C, alpha: float = 1.0, beta: float = 0.0, splits: int = 0):
    """hgemm_splitk with its fp32 partials in the library's static device
    array (HG_NOALLOC_SCRATCH_BYTES per GPU): no workspace, nothing allocated.
    Calls that overlap on one GPU race on that array.  Returns C."""
    import torch
    _check_matrix(A, "A", (torch.float16,))
    _check_matrix(Bt, "Bt", (torch.float16,))
    _check_matrix(C, "C", (torch.float16, torch.float32))
    M, K = A.shape
    N = Bt.shape[0]
    if Bt.shape[1] != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, Bt {tuple(Bt.shape)}, "
                         f"C {tuple(C.shape)}")
    out_dtype = HG_F16 if C.dtype == torch.float16 else HG_F32
    st = lib.hgemm_splitk_noalloc(M, N, K, float(alpha), A.data_ptr() or None, _ld(A),
                                  Bt.data_ptr() or None, _ld(Bt), float(beta), C.data_ptr() or None,
                                  _ld(C), out_dtype, int(splits), _stream_handle(C))
    if st != 0:
        raise HgError("hgemm_splitk_noalloc", st)
    return C


NOALLOC_SCRATCH_BYTES = 32 << 20
ERR_SCRATCH_LIMIT = -100


def splitk_workspace_size(M: int, N: int, K: int, splits: int = 0) -> int:
    """Bytes of workspace hgemm_splitk needs on the current device."""
    need = lib.hg_hgemm_splitk_workspace_size(M, N, K, int(splits))
    if need < 0:
        raise HgError("hg_hgemm_splitk_workspace_size", int(need))
    return int(need)


def hgemm_layout(A, B, C, a_col_major: bool = False, b_row_major: bool = False,
                 alpha: float = 1.0, beta: float = 0.0, work=None):
    """C = alpha·A·B + beta·C with A given M×K row-major (a (M, K) tensor) or
    column-major (a (K, M) tensor holding Aᵀ), and B given K×N column-major
    (an (N, K) tensor, hgemm's Bt) or row-major (a (K, N) tensor).  C is
    (M, N).  `work`: device uint8 tensor of at least
    hgemm_layout_workspace_size(...) bytes (allocated with torch when None)."""
    import torch
    _check_matrix(A, "A", (torch.float16,))
    _check_matrix(B, "B", (torch.float16,))
    _check_matrix(C, "C", (torch.float16, torch.float32))
    M, N = C.shape
    K = A.shape[0] if a_col_major else A.shape[1]
    if (A.shape[1] if a_col_major else A.shape[0]) != M:
        raise ValueError(f"A {tuple(A.shape)} does not match C {tuple(C.shape)}")
    if tuple(B.shape) != ((K, N) if b_row_major else (N, K)):
        raise ValueError(f"B {tuple(B.shape)} does not match K={K}, N={N}")
    al, bl = (COL_MAJOR if a_col_major else ROW_MAJOR), (ROW_MAJOR if b_row_major else COL_MAJOR)
    need = lib.hg_hgemm_layout_workspace_size(al, bl, M, N, K)
    if need < 0:
        raise HgError("hg_hgemm_layout_workspace_size", int(need))
    if work is None and need > 0:
        work = torch.empty(need, dtype=torch.uint8, device=C.device)
    wptr = work.data_ptr() if work is not None else None
    wbytes = work.numel() * work.element_size() if work is not None else 0
    out_dtype = HG_F16 if C.dtype == torch.float16 else HG_F32
    st = lib.hgemm_layout(al, bl, M, N, K, float(alpha), A.data_ptr() or None, _ld(A),
                          B.data_ptr() or None, _ld(B), float(beta), C.data_ptr() or None, _ld(C),
                          out_dtype, wptr, wbytes, _stream_handle(C))
    if st != 0:
        raise HgError("hgemm_layout", st)
    return C


def hgemm_bf16(A, Bt, C, alpha: float = 1.0, beta: float = 0.0):
    """C = alpha·A·B + beta·C with bf16 A and Bt (layouts as hgemm), C bf16 or
    float32; returns C."""
    import torch
    _check_matrix(A, "A", (torch.bfloat16,))
    _check_matrix(Bt, "Bt", (torch.bfloat16,))
    _check_matrix(C, "C", (torch.bfloat16, torch.float32))
    M, K = A.shape
    N = Bt.shape[0]
    if Bt.shape[1] != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, Bt {tuple(Bt.shape)}, "
                         f"C {tuple(C.shape)}")
    out_dtype = HG_BF16 if C.dtype == torch.bfloat16 else HG_F32
    st = lib.hgemm_bf16(M, N, K, float(alpha), A.data_ptr() or None, _ld(A), Bt.data_ptr() or None,
                        _ld(Bt), float(beta), C.data_ptr() or None, _ld(C), out_dtype,
                        _stream_handle(C))
    if st != 0:
        raise HgError("hgemm_bf16", st)
    return C


def hgemm_bias_act(A, Bt, C, bias=None, relu: bool = False, alpha: float = 1.0,
                   beta: float = 0.0):
    """C = act(alpha·A·B + beta·C + bias) in one launch; bias a float32 device
    vector of length N (or None), act ReLU when `relu`.  A and Bt float16 (C
    float16 or float32) or both bfloat16 (C bfloat16 or float32).  Returns C."""
    import torch
    _check_matrix(A, "A", (torch.float16, torch.bfloat16))
    _check_matrix(Bt, "Bt", (A.dtype,))
    bf = A.dtype == torch.bfloat16
    _check_matrix(C, "C", (torch.bfloat16 if bf else torch.float16, torch.float32))
    M, K = A.shape
    N = Bt.shape[0]
    if Bt.shape[1] != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, Bt {tuple(Bt.shape)}, "
                         f"C {tuple(C.shape)}")
    bptr = None
    if bias is not None:
        if not (isinstance(bias, torch.Tensor) and bias.is_cuda and bias.dtype == torch.float32
                and bias.dim() == 1 and bias.shape[0] == N and bias.is_contiguous()):
            raise ValueError("bias must be a contiguous float32 device vector of length N")
        bptr = bias.data_ptr() or None
    out_dtype = HG_F32 if C.dtype == torch.float32 else (HG_BF16 if bf else HG_F16)
    fn = lib.hgemm_bf16_bias_act if bf else lib.hgemm_bias_act
    st = fn(M, N, K, float(alpha), A.data_ptr() or None, _ld(A), Bt.data_ptr() or None, _ld(Bt),
            float(beta), C.data_ptr() or None, _ld(C), out_dtype, bptr, ACT_RELU if relu else ACT_NONE,
            _stream_handle(C))
    if st != 0:
        raise HgError("hgemm_bf16_bias_act" if bf else "hgemm_bias_act", st)
    return C


def trmm_lower_trans(A, B, Out, alpha: float = 1.0, leaf: int = 256):
    """Out = alpha·Aᵀ·B (A lower triangular) on the current stream; returns Out."""
    return _trmm(lib.trmm_lower_trans, "trmm_lower_trans", A, B, Out, alpha, leaf)


def trmm_lower_trans_by_level(A, B, Out, alpha: float = 1.0, leaf: int = 256):
    """trmm_lower_trans scheduled as one batched launch per recursion level
    (same result up to fp32 rounding); see hg_trmm_lower_trans_by_level."""
    return _trmm(lib.hg_trmm_lower_trans_by_level, "hg_trmm_lower_trans_by_level", A, B, Out,
                 alpha, leaf)


def trmm_lower_trans_streams(A, B, Out, streams, alpha: float = 1.0, leaf: int = 256):
    """trmm_lower_trans_by_level with each phase's launches spread over the
    torch streams in `streams` (1 to 8; the first is where the result is
    ordered); the same bits as trmm_lower_trans_by_level.  Returns Out."""
    import torch
    _check_matrix(A, "A", (torch.float16,))
    _check_matrix(B, "B", (torch.float16,))
    _check_matrix(Out, "Out", (torch.float32,))
    n = A.shape[0]
    m = B.shape[0]
    if tuple(A.shape) != (n, n) or B.shape[1] != n or tuple(Out.shape) != (m, n):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, Out {tuple(Out.shape)}")
    arr = (ctypes.c_void_p * len(streams))(*[ctypes.c_void_p(st.cuda_stream) for st in streams])
    st = lib.hg_trmm_lower_trans_streams(n, m, float(alpha), A.data_ptr() or None, _ld(A),
                                         B.data_ptr() or None, _ld(B), Out.data_ptr() or None, _ld(Out),
                                         HG_F32, int(leaf), arr, len(streams))
    if st != 0:
        raise HgError("hg_trmm_lower_trans_streams", st)
    return Out


def _trmm(fn, fname, A, B, Out, alpha, leaf):
    import torch
    _check_matrix(A, "A", (torch.float16,))
    _check_matrix(B, "B", (torch.float16,))
    _check_matrix(Out, "Out", (torch.float32,))
    n = A.shape[0]
    m = B.shape[0]
    if tuple(A.shape) != (n, n) or B.shape[1] != n or tuple(Out.shape) != (m, n):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, "
                         f"Out {tuple(Out.shape)}")
    st = fn(n, m, float(alpha), A.data_ptr() or None, _ld(A), B.data_ptr() or None, _ld(B),
            Out.data_ptr() or None, _ld(Out), HG_F32, int(leaf), _stream_handle(Out))
    if st != 0:
        raise HgError(fname, st)
    return Out


def trsm_workspace_size(n: int, m: int, leaf: int = 256) -> int:
    """Bytes of device workspace trsm_lower_trans needs (hg_trsm_workspace_size)."""
    sz = lib.hg_trsm_workspace_size(n, m, leaf)
    if sz < 0:
        raise HgError("hg_trsm_workspace_size", int(sz))
    return int(sz)


def trsm_lower_trans(A, B, Out, alpha: float = 1.0, leaf: int = 256, work=None):
    """Out = alpha·A⁻ᵀ·B (A lower triangular) on the current stream; returns Out."""
    import torch
    _check_matrix(A, "A", (torch.float16,))
    _check_matrix(B, "B", (torch.float16,))
    _check_matrix(Out, "Out", (torch.float32,))
    n = A.shape[0]
    m = B.shape[0]
    if tuple(A.shape) != (n, n) or B.shape[1] != n or tuple(Out.shape) != (m, n):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, "
                         f"Out {tuple(Out.shape)}")
    need = trsm_workspace_size(n, m, leaf) if int(leaf) <= 256 else 0
    if work is None:
        work = torch.empty(max(need, 1), dtype=torch.uint8, device=Out.device)
    elif not (isinstance(work, torch.Tensor) and work.is_cuda and work.is_contiguous()):
        raise ValueError("work must be a contiguous device tensor")
    st = lib.trsm_lower_trans(n, m, float(alpha), A.data_ptr() or None, _ld(A),
                              B.data_ptr() or None, _ld(B), Out.data_ptr() or None, _ld(Out),
                              HG_F32, int(leaf), work.data_ptr() or None,
                              work.numel() * work.element_size(), _stream_handle(Out))
    if st != 0:
        raise HgError("trsm_lower_trans", st)
    return Out


def trmm(A, B, Out, alpha: float = 1.0, uplo: str = "L", trans: bool = True, leaf: int = 256,
         work=None):
    """Out = alpha·op(A)·B, A lower (uplo "L") or upper ("U") triangular, op
    the transpose when `trans`; conventions as trmm_lower_trans.  `work` is a
    device uint8 tensor of at least trmm_workspace_size(...) bytes (allocated
    with torch for the call when None)."""
    import torch
    _check_matrix(A, "A", (torch.float16,))
    _check_matrix(B, "B", (torch.float16,))
    _check_matrix(Out, "Out", (torch.float32,))
    n = A.shape[0]
    m = B.shape[0]
    if tuple(A.shape) != (n, n) or B.shape[1] != n or tuple(Out.shape) != (m, n):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, "
                         f"Out {tuple(Out.shape)}")
    if uplo not in ("L", "U"):
        raise ValueError("uplo must be 'L' or 'U'")
    u = 0 if uplo == "L" else 1
    t = 1 if trans else 0
    need = trmm_workspace_size(n, m, uplo, trans)
    if work is None and need > 0:
        work = torch.empty(need, dtype=torch.uint8, device=Out.device)
    wptr = work.data_ptr() if work is not None else None
    wbytes = work.numel() * work.element_size() if work is not None else 0
    st = lib.hg_trmm(u, t, n, m, float(alpha), A.data_ptr() or None, _ld(A), B.data_ptr() or None,
                     _ld(B), Out.data_ptr() or None, _ld(Out), HG_F32, int(leaf), wptr, wbytes,
                     _stream_handle(Out))
    if st != 0:
        raise HgError("hg_trmm", st)
    return Out


def trmm_inplace(A, B, alpha: float = 1.0, uplo: str = "L", trans: bool = True, leaf: int = 256,
                 work=None):
    """B ← alpha·op(A)·B with B a float16 (m, n) tensor in the column-major
    convention, overwritten with the product rounded to fp16; returns B."""
    import torch
    _check_matrix(A, "A", (torch.float16,))
    _check_matrix(B, "B", (torch.float16,))
    n = A.shape[0]
    m = B.shape[0]
    if tuple(A.shape) != (n, n) or B.shape[1] != n:
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}")
    if uplo not in ("L", "U"):
        raise ValueError("uplo must be 'L' or 'U'")
    u, t = (0 if uplo == "L" else 1), (1 if trans else 0)
    need = lib.hg_trmm_inplace_workspace_size(u, t, n, m)
    if need < 0:
        raise HgError("hg_trmm_inplace_workspace_size", int(need))
    if work is None:
        work = torch.empty(max(need, 1), dtype=torch.uint8, device=B.device)
    st = lib.hg_trmm_inplace(u, t, n, m, float(alpha), A.data_ptr() or None, _ld(A),
                             B.data_ptr() or None, _ld(B), int(leaf), work.data_ptr(),
                             work.numel() * work.element_size(), _stream_handle(B))
    if st != 0:
        raise HgError("hg_trmm_inplace", st)
    return B


def trmm_workspace_size(n: int, m: int, uplo: str = "L", trans: bool = True) -> int:
    sz = lib.hg_trmm_workspace_size(0 if uplo == "L" else 1, 1 if trans else 0, n, m)
    if sz < 0:
        raise HgError("hg_trmm_workspace_size", int(sz))
    return int(sz)


def trmm_plan(n: int, leaf: int = 256):
    """The recursion trmm_lower_trans runs: list of (kind, offset, size, depth),
    kind 0 = leaf, 1 = update (see hg_trmm_plan in include/hgemm.h)."""
    cnt = lib.hg_trmm_plan(n, leaf, None, 0)
    if cnt < 0:
        raise HgError("hg_trmm_plan", int(cnt))
    buf = (_i64 * (4 * cnt))()
    lib.hg_trmm_plan(n, leaf, buf, cnt)
    return [tuple(buf[4 * i:4 * i + 4]) for i in range(cnt)]
