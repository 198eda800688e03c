"""Host-side checks of the C ABI (CPU only, no kernel launches).

Every call here returns before the library touches the HIP runtime:
argument validation (BLAS xerbla-style negative status = position of the
first bad argument), quick returns, status strings and the TRMM recursion
plan of "异构计算中高性能TRMM与TRSM的递归算法实现" §2.1–§2.2.  Pointer
arguments are fake addresses that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hgemm.h")


@pytest.fixture(scope="module")
def lib(hg):
    return hg.lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|int64_t|char|void)\s*\*?\s*(\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["hg_hgemm_layout_workspace_size", "hg_hgemm_splitk_workspace_size",
                                    "hg_strerror", "hg_trmm",
                                    "hg_trmm_inplace", "hg_trmm_inplace_workspace_size",
                                    "hg_trmm_lower_trans_by_level", "hg_trmm_lower_trans_streams",
                                    "hg_trmm_plan",
                                    "hg_trmm_workspace_size", "hg_trsm_workspace_size", "hgemm",
                                    "hgemm_bf16", "hgemm_bf16_bias_act", "hgemm_bias_act", "hgemm_layout",
                                    "hgemm_splitk", "hgemm_splitk_noalloc",
                                    "trmm_lower_trans", "trsm_lower_trans"]


def test_library_exports_every_declared_symbol(hg):
    lib = ctypes.CDLL(hg.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"libhgemm.so does not export {name}"
    assert set(hg.EXPORTS) == set(declared_functions())


P = 0x10000      # fake device addresses, never dereferenced on these paths
Q = 0x20000000
R = 0x40000000


def gemm(lib, M=4, N=4, K=4, alpha=1.0, A=P, lda=None, B=Q, ldb=None, beta=0.0, C=R, ldc=None,
         dt=0):
    lda = max(1, K) if lda is None else lda
    ldb = max(1, K) if ldb is None else ldb
    ldc = max(1, N) if ldc is None else ldc
    return lib.hgemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), -1), (dict(N=-1), -2), (dict(K=-1), -3),
    (dict(M=2 ** 31), -1), (dict(N=2 ** 31), -2), (dict(K=2 ** 31), -3),
    (dict(K=8, lda=7), -6), (dict(K=0, lda=0), -6),
    (dict(K=8, ldb=7), -8), (dict(N=8, ldc=7), -11),
    (dict(dt=2), -12), (dict(dt=-1), -12),
    (dict(C=None), -10), (dict(A=None), -5), (dict(B=None), -7),
])
def test_hgemm_argument_errors(lib, kw, code):
    assert gemm(lib, **kw) == code


def bias_act(lib, M=4, N=4, K=4, A=P, B=Q, C=R, bias=None, act=1, dt=1):
    return lib.hgemm_bias_act(M, N, K, 1.0, A, max(1, K), B, max(1, K), 0.0, C, max(1, N), dt,
                              bias, act, None)


def test_hgemm_bias_act_argument_errors(lib):
    assert bias_act(lib, act=2) == -14
    assert bias_act(lib, act=-1) == -14
    assert bias_act(lib, M=-1) == -1
    assert bias_act(lib, dt=5) == -12
    assert bias_act(lib, C=None) == -10
    assert bias_act(lib, A=None) == -5
    assert bias_act(lib, bias=R + 8) == -13          # bias inside C
    assert bias_act(lib, C=P + 8) == -10             # C overlaps A
    assert bias_act(lib, M=0, A=None, B=None, C=None) == 0


def test_hgemm_bf16_output_types(lib):
    """bf16 operands take HG_BF16 or HG_F32 output; HG_F16 is rejected, and
    the fp16 entry point rejects HG_BF16."""
    args = (4, 4, 4, 1.0, P, 4, Q, 4, 0.0, R, 4)
    assert lib.hgemm_bf16(*args, 0, None) == -12
    assert lib.hgemm_bf16(*args, 3, None) == -12
    assert lib.hgemm(*args, 2, None) == -12
    assert lib.hgemm_bf16(0, 4, 4, 1.0, None, 4, None, 4, 0.0, None, 4, 2, None) == 0


def test_hgemm_first_bad_argument_wins(lib):
    assert gemm(lib, M=-1, N=-1, dt=7) == -1
    assert gemm(lib, K=8, lda=1, ldb=1) == -6


def test_hgemm_quick_return_touches_nothing(lib):
    # M == 0 or N == 0: success without looking at any pointer
    assert gemm(lib, M=0, A=None, B=None, C=None) == 0
    assert gemm(lib, N=0, A=None, B=None, C=None, ldc=1) == 0


def test_hgemm_overlap_rejected(lib):
    # C (fp16 4×4, ld 4) starting inside A's extent
    assert gemm(lib, A=P, C=P + 8) == -10
    assert gemm(lib, B=Q, C=Q + 30) == -10
    # alpha == 0 does not read A, so no overlap with A is checked there;
    # that path launches, so it is covered by the GPU tests instead


@pytest.mark.parametrize("args,code", [
    ((-1, 4, 1.0, P, 4, Q, 4, R, 4, 1, 256), -1),
    ((4, -1, 1.0, P, 4, Q, 4, R, 4, 1, 256), -2),
    ((8, 4, 1.0, P, 7, Q, 8, R, 8, 1, 256), -5),
    ((8, 4, 1.0, P, 8, Q, 7, R, 8, 1, 256), -7),
    ((8, 4, 1.0, P, 8, Q, 8, R, 7, 1, 256), -9),
    ((8, 4, 1.0, P, 8, Q, 8, R, 8, 0, 256), -10),     # fp16 Out is not supported
    ((8, 4, 1.0, P, 8, Q, 8, None, 8, 1, 256), -8),
    ((8, 4, 1.0, None, 8, Q, 8, R, 8, 1, 256), -4),
    ((8, 4, 1.0, P, 8, None, 8, R, 8, 1, 256), -6),
    ((8, 4, 1.0, P, 8, Q, 8, Q + 16, 8, 1, 256), -8),  # Out overlaps B
    ((0, 4, 1.0, None, 1, None, 1, None, 1, 1, 256), 0),
    ((8, 0, 1.0, None, 8, None, 8, None, 8, 1, 256), 0),
])
def test_trmm_argument_errors(lib, args, code):
    assert lib.trmm_lower_trans(*args, None) == code


W = 0x60000000   # fake workspace address


def _trsm_need(lib, n, m, leaf):
    return lib.hg_trsm_workspace_size(n, m, leaf)


@pytest.mark.parametrize("args,code", [
    ((-1, 4, 1.0, P, 8, Q, 8, R, 8, 1, 256, W, 1 << 30), -1),
    ((8, -1, 1.0, P, 8, Q, 8, R, 8, 1, 256, W, 1 << 30), -2),
    ((2 ** 31, 4, 1.0, P, 2 ** 31, Q, 2 ** 31, R, 2 ** 31, 1, 256, W, 1 << 30), -1),
    ((8, 4, 1.0, P, 7, Q, 8, R, 8, 1, 256, W, 1 << 30), -5),
    ((8, 4, 1.0, P, 8, Q, 7, R, 8, 1, 256, W, 1 << 30), -7),
    ((8, 4, 1.0, P, 8, Q, 8, R, 7, 1, 256, W, 1 << 30), -9),
    ((8, 4, 1.0, P, 8, Q, 8, R, 8, 0, 256, W, 1 << 30), -10),
    ((8, 4, 1.0, P, 8, Q, 8, R, 8, 1, 257, W, 1 << 30), -11),
    ((8, 4, 1.0, P, 8, Q, 8, None, 8, 1, 256, W, 1 << 30), -8),
    ((8, 4, 1.0, None, 8, Q, 8, R, 8, 1, 256, W, 1 << 30), -4),
    ((8, 4, 1.0, P, 8, None, 8, R, 8, 1, 256, W, 1 << 30), -6),
    ((8, 4, 1.0, P, 8, Q, 8, Q + 16, 8, 1, 256, W, 1 << 30), -8),   # Out overlaps B
    ((8, 4, 1.0, P, 8, Q, 8, R, 8, 1, 256, None, 1 << 30), -12),
    ((8, 4, 1.0, P, 8, Q, 8, R, 8, 1, 256, W + 8, 1 << 30), -12),    # misaligned
    ((8, 4, 1.0, P, 8, Q, 8, R, 8, 1, 256, R + 64, 1 << 30), -12),   # overlaps Out
    ((8, 4, 1.0, P, 8, Q, 8, R, 8, 1, 256, W, 16), -13),             # too small
    ((0, 4, 1.0, None, 1, None, 1, None, 1, 1, 256, None, 0), 0),
    ((8, 0, 1.0, None, 8, None, 8, None, 8, 1, 256, None, 0), 0),
])
def test_trsm_argument_errors(lib, args, code):
    assert lib.trsm_lower_trans(*args, None) == code


@pytest.mark.parametrize("n,m,leaf", [(8192, 8192, 256), (1000, 77, 256), (300, 5, 100), (13, 3, 1),
                                      (257, 9, 0)])
def test_trsm_workspace_size(lib, n, m, leaf):
    """Leaf inverses (ld×ld fp16 blocks, ld = largest leaf rounded up to 8)
    plus the fp16 copy of X (ldw = n rounded up to 8), each 256-byte padded."""
    L = 256 if leaf <= 0 else leaf
    leaves = []

    def rec(o, s):
        if s <= L:
            leaves.append(s)
            return
        rec(o, s // 2)
        rec(o + s // 2, s - s // 2)
    rec(0, n)
    ld = -(-max(leaves) // 8) * 8
    up = lambda x: -(-x // 256) * 256
    expect = up(len(leaves) * ld * ld * 2) + up(-(-n // 8) * 8 * m * 2)
    assert _trsm_need(lib, n, m, leaf) == expect


def test_trsm_workspace_size_errors(lib):
    assert _trsm_need(lib, -1, 4, 256) == -1
    assert _trsm_need(lib, 4, -1, 256) == -2
    assert _trsm_need(lib, 4, 4, 300) == -3
    assert _trsm_need(lib, 0, 4, 256) == 0 and _trsm_need(lib, 4, 0, 256) == 0


@pytest.mark.parametrize("args,code", [
    ((2, 1, 8, 4, 1.0, P, 8, Q, 8, R, 8, 1, 256, W, 1 << 30), -1),
    ((0, 2, 8, 4, 1.0, P, 8, Q, 8, R, 8, 1, 256, W, 1 << 30), -2),
    ((0, 0, -1, 4, 1.0, P, 8, Q, 8, R, 8, 1, 256, W, 1 << 30), -3),
    ((0, 0, 8, -1, 1.0, P, 8, Q, 8, R, 8, 1, 256, W, 1 << 30), -4),
    ((0, 0, 8, 4, 1.0, P, 7, Q, 8, R, 8, 1, 256, W, 1 << 30), -7),
    ((0, 0, 8, 4, 1.0, P, 8, Q, 7, R, 8, 1, 256, W, 1 << 30), -9),
    ((0, 0, 8, 4, 1.0, P, 8, Q, 8, R, 7, 1, 256, W, 1 << 30), -11),
    ((0, 0, 8, 4, 1.0, P, 8, Q, 8, R, 8, 0, 256, W, 1 << 30), -12),
    ((0, 0, 8, 4, 1.0, P, 8, Q, 8, None, 8, 1, 256, W, 1 << 30), -10),
    ((0, 0, 8, 4, 1.0, None, 8, Q, 8, R, 8, 1, 256, W, 1 << 30), -6),
    ((0, 0, 8, 4, 1.0, P, 8, None, 8, R, 8, 1, 256, W, 1 << 30), -8),
    ((0, 0, 8, 4, 1.0, P, 8, Q, 8, R, 8, 1, 256, None, 1 << 30), -14),
    ((1, 1, 8, 4, 1.0, P, 8, Q, 8, R, 8, 1, 256, W + 4, 1 << 30), -14),
    ((1, 0, 8, 4, 1.0, P, 8, Q, 8, R, 8, 1, 256, W, 8), -15),
    ((0, 0, 0, 4, 1.0, None, 1, None, 1, None, 1, 1, 256, None, 0), 0),
])
def test_hg_trmm_argument_errors(lib, args, code):
    assert lib.hg_trmm(*args, None) == code


def test_hg_trmm_workspace_size(lib):
    up = lambda x: -(-x // 256) * 256
    ldl = -(-1000 // 8) * 8
    assert lib.hg_trmm_workspace_size(0, 1, 1000, 77) == 0                   # lower, trans
    assert lib.hg_trmm_workspace_size(1, 0, 1000, 77) == up(ldl * 1000 * 2)  # upper, notrans
    both = up(ldl * 1000 * 2) + up(ldl * 77 * 2)
    assert lib.hg_trmm_workspace_size(1, 1, 1000, 77) == both               # upper, trans
    assert lib.hg_trmm_workspace_size(0, 0, 1000, 77) == both               # lower, notrans
    assert lib.hg_trmm_workspace_size(2, 0, 4, 4) == -1
    assert lib.hg_trmm_workspace_size(0, 2, 4, 4) == -2
    assert lib.hg_trmm_workspace_size(0, 0, -1, 4) == -3
    assert lib.hg_trmm_workspace_size(0, 0, 4, -1) == -4


def test_hgemm_layout_argument_errors(lib):
    L = lambda *a: lib.hgemm_layout(*a, None)
    assert L(2, 1, 4, 4, 4, 1.0, P, 4, Q, 4, 0.0, R, 4, 1, W, 1 << 20) == -1
    assert L(0, 2, 4, 4, 4, 1.0, P, 4, Q, 4, 0.0, R, 4, 1, W, 1 << 20) == -2
    assert L(0, 1, -1, 4, 4, 1.0, P, 4, Q, 4, 0.0, R, 4, 1, W, 1 << 20) == -3
    assert L(1, 1, 8, 4, 2, 1.0, P, 2, Q, 2, 0.0, R, 4, 1, W, 1 << 20) == -8    # col-major A: lda >= M
    assert L(0, 0, 4, 8, 2, 1.0, P, 2, Q, 2, 0.0, R, 8, 1, W, 1 << 20) == -10   # row-major B: ldb >= N
    assert L(0, 1, 4, 4, 4, 1.0, P, 4, Q, 4, 0.0, R, 4, 3, W, 1 << 20) == -14
    assert L(0, 1, 4, 4, 4, 1.0, P, 4, Q, 4, 0.0, None, 4, 1, W, 1 << 20) == -12
    assert L(0, 0, 4, 4, 4, 1.0, None, 4, Q, 4, 0.0, R, 4, 1, W, 1 << 20) == -7
    assert L(0, 0, 4, 4, 4, 1.0, P, 4, Q, 4, 0.0, R, 4, 1, None, 1 << 20) == -15
    assert L(0, 0, 4, 4, 4, 1.0, P, 4, Q, 4, 0.0, R, 4, 1, W, 8) == -16
    assert L(1, 1, 0, 4, 4, 1.0, None, 4, None, 4, 0.0, None, 4, 1, None, 0) == 0


def test_hgemm_layout_workspace_size(lib):
    up = lambda x: -(-x // 256) * 256
    ldk = -(-100 // 8) * 8
    assert lib.hg_hgemm_layout_workspace_size(0, 1, 30, 40, 100) == 0
    assert lib.hg_hgemm_layout_workspace_size(1, 1, 30, 40, 100) == up(30 * ldk * 2)
    assert lib.hg_hgemm_layout_workspace_size(0, 0, 30, 40, 100) == up(40 * ldk * 2)
    assert lib.hg_hgemm_layout_workspace_size(1, 0, 30, 40, 100) == up(30 * ldk * 2) + up(40 * ldk * 2)
    assert lib.hg_hgemm_layout_workspace_size(3, 0, 1, 1, 1) == -1


def test_hg_trmm_inplace_arguments(lib):
    up = lambda x: -(-x // 256) * 256
    assert lib.hg_trmm_inplace_workspace_size(0, 1, 1000, 77) == up(1000 * 77 * 4)
    assert lib.hg_trmm_inplace_workspace_size(1, 0, 1000, 77) == \
        up(1000 * 77 * 4) + lib.hg_trmm_workspace_size(1, 0, 1000, 77)
    assert lib.hg_trmm_inplace_workspace_size(5, 0, 10, 10) == -1
    I = lambda *a: lib.hg_trmm_inplace(*a, None)
    assert I(3, 1, 8, 4, 1.0, P, 8, Q, 8, 256, W, 1 << 20) == -1
    assert I(0, 1, 8, 4, 1.0, P, 7, Q, 8, 256, W, 1 << 20) == -7
    assert I(0, 1, 8, 4, 1.0, P, 8, Q, 7, 256, W, 1 << 20) == -9
    assert I(0, 1, 8, 4, 1.0, P, 8, None, 8, 256, W, 1 << 20) == -8
    assert I(0, 1, 8, 4, 1.0, P, 8, P + 16, 8, 256, W, 1 << 20) == -8     # B overlaps A
    assert I(0, 1, 8, 4, 1.0, P, 8, Q, 8, 256, None, 1 << 20) == -11
    assert I(0, 1, 8, 4, 1.0, P, 8, Q, 8, 256, W, 16) == -12
    assert I(0, 1, 0, 4, 1.0, None, 1, None, 1, 256, None, 0) == 0


def test_strerror(hg):
    assert hg.strerror(0) == "success"
    assert "argument 14" in hg.strerror(-14)
    assert "argument 6" in hg.strerror(-6)
    assert hg.strerror(-99) == "unknown status"
    assert isinstance(hg.strerror(1000 + 1), str)


# ------------------------------------------------------------ recursion plan
def test_plan_n8192_leaf256(hg):
    plan = hg.trmm_plan(8192, 256)
    leaves = [p for p in plan if p[0] == 0]
    upd = [p for p in plan if p[0] == 1]
    assert len(leaves) == 32 and len(upd) == 31
    assert all(p[2] == 256 for p in leaves)
    assert sorted({p[3] for p in upd}) == [0, 1, 2, 3, 4]          # five levels
    # flop share of the GEMM updates: each update is h·(s-h)·m multiply-adds
    # against n(n+1)m/2 for the whole triangle -> 96.9 % at n=8192, leaf 256
    # (the page claims "more than 90 %" in §2.2 and ">= 70 %" in §2.1)
    n = 8192
    gemm_macs = sum((p[2] // 2) * (p[2] - p[2] // 2) for p in upd)
    share = gemm_macs / (n * (n + 1) / 2)
    assert share == pytest.approx(0.969, abs=5e-4)
    assert share > 0.9


@pytest.mark.parametrize("n,leaf", [(1, 256), (255, 256), (257, 256), (1000, 256), (1000, 64),
                                    (4097, 128), (13, 1), (8192, 8192)])
def test_plan_structure(hg, n, leaf):
    plan = hg.trmm_plan(n, leaf)
    # leaves tile [0, n) in order, each of size <= leaf
    leaves = [(p[1], p[2]) for p in plan if p[0] == 0]
    pos = 0
    for o, s in leaves:
        assert o == pos and 1 <= s <= max(leaf, 1)
        pos += s
    assert pos == n
    # every update block has s > leaf, splits at floor(s/2), and covers the
    # strictly-lower part below its top half exactly once overall
    covered = 0
    for kind, o, s, d in plan:
        if kind == 1:
            assert s > leaf and 0 <= o and o + s <= n
            h = s // 2
            covered += h * (s - h)
    covered += sum(s * (s + 1) // 2 for _, s in leaves)
    assert covered == n * (n + 1) // 2      # every (k >= i) pair exactly once


@pytest.mark.parametrize("n,leaf", [(8192, 256), (1000, 64), (777, 16)])
def test_plan_batched_order_matches_recursion(hg, n, leaf):
    """Running all leaves, then updates deepest level first, gives every row
    the same sequence of contributions as the depth-first recursion: along the
    recursion order, the updates touching any one row have strictly
    decreasing depth, and updates of one depth touch disjoint rows."""
    plan = hg.trmm_plan(n, leaf)
    seen = {}
    by_depth = {}
    for kind, o, s, d in plan:
        if kind != 1:
            continue
        h = s // 2
        for r in range(o, o + h):           # every row of Out1
            if r in seen:
                assert d < seen[r][-1]
            seen.setdefault(r, []).append(d)
        by_depth.setdefault(d, []).append((o, o + h))
    for d, iv in by_depth.items():
        iv.sort()
        for (a0, a1), (b0, b1) in zip(iv, iv[1:]):
            assert a1 <= b0


def test_plan_errors(hg):
    assert hg.lib.hg_trmm_plan(-1, 256, None, 0) == -1
    assert hg.lib.hg_trmm_plan(10, 256, None, 5) == -2
    assert hg.trmm_plan(0) == []
    assert hg.trmm_plan(10, 0) == [(0, 0, 10, 0)]     # leaf <= 0 means 256


def test_one_hip_runtime_in_the_process():
    """Importing the binding loads torch before the library, so the library
    binds to torch's HIP runtime and the process maps a single one."""
    import subprocess
    import sys
    code = ("import half_precision_gemm_amd\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "libs = {l.split()[-1] for l in maps if 'libamdhip64' in l}\n"
            "print(len(libs))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip().splitlines()[-1] == "1"


def test_hgemm_splitk_workspace_and_arguments(lib):
    up = lambda x: -(-x // 256) * 256
    # explicit splits: Ks = ceil(K / s) rounded up to 64, S = ceil(K / Ks)
    assert lib.hg_hgemm_splitk_workspace_size(512, 512, 65536, 8) == up(8 * 512 * 512 * 4)
    assert lib.hg_hgemm_splitk_workspace_size(100, 60, 1000, 3) == up(3 * 100 * 60 * 4)
    assert lib.hg_hgemm_splitk_workspace_size(100, 60, 100, 32) == up(100 * 60 * 4)       # slices >= 64 columns
    assert lib.hg_hgemm_splitk_workspace_size(100, 60, 200, 32) == up(2 * 100 * 60 * 4)   # 3 asked: 128 + 72
    assert lib.hg_hgemm_splitk_workspace_size(100, 60, 10, 4) == up(100 * 60 * 4)         # one slice
    assert lib.hg_hgemm_splitk_workspace_size(0, 60, 10, 4) == 0
    assert lib.hg_hgemm_splitk_workspace_size(-1, 60, 10, 4) == -1
    assert lib.hg_hgemm_splitk_workspace_size(4, 4, 4, 33) == -4
    assert lib.hg_hgemm_splitk_workspace_size(4, 4, 4, -1) == -4
    S = lambda *a: lib.hgemm_splitk(*a, None)
    assert S(4, 4, 4, 1.0, P, 4, Q, 4, 0.0, R, 4, 1, 33, W, 1 << 20) == -13
    assert S(4, 4, 4, 1.0, P, 4, Q, 4, 0.0, R, 4, 2, 2, W, 1 << 20) == -12
    assert S(4, 4, 4, 1.0, P, 3, Q, 4, 0.0, R, 4, 1, 2, W, 1 << 20) == -6
    assert S(4, 4, 4, 1.0, P, 4, Q, 4, 0.0, R, 3, 1, 2, W, 1 << 20) == -11
    assert S(4, 4, 4, 1.0, P, 4, Q, 4, 0.0, R, 4, 1, 2, None, 1 << 20) == -14
    assert S(4, 4, 4, 1.0, P, 4, Q, 4, 0.0, R, 4, 1, 2, W, 16) == -15
    assert S(4, 4, 4, 1.0, P, 4, Q, 4, 0.0, R, 4, 1, 2, R, 1 << 20) == -14        # work overlaps C
    assert S(0, 4, 4, 1.0, None, 4, None, 4, 0.0, None, 4, 1, 2, None, 0) == 0


def test_trmm_streams_arguments(lib):
    import ctypes
    arr = (ctypes.c_void_p * 2)(None, None)
    T = lambda ns, streams=arr: lib.hg_trmm_lower_trans_streams(8, 4, 1.0, P, 8, Q, 8, R, 8, 1, 256, streams, ns)
    assert T(0) == -13
    assert T(9) == -13
    assert T(2, None) == -12
    assert lib.hg_trmm_lower_trans_streams(8, 4, 1.0, P, 8, Q, 8, R, 8, 2, 256, arr, 2) == -10   # fp16 Out
    assert lib.hg_trmm_lower_trans_streams(0, 4, 1.0, None, 1, None, 1, None, 1, 1, 256, arr, 2) == 0
