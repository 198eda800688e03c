// hg_api.cpp — host side of the C ABI declared in include/hgemm.h: argument
// validation (BLAS xerbla-style status codes), quick returns, kernel
// selection, and the recursive TRMM and TRSM drivers of
// "异构计算中高性能TRMM与TRSM的递归算法实现" §2.1–§2.3.
#include "hgemm.h"

#include <stdint.h>

#include <algorithm>
#include <utility>
#include <vector>

#include "hg_internal.h"

namespace {

constexpr int64_t kI32Max = 0x7fffffff;

struct Extent {
    uintptr_t lo, hi;  // [lo, hi) in bytes; empty when lo == hi
};

Extent extent(const void *p, int64_t rows, int64_t ld, int64_t cols, int64_t esize)
{
    if (rows <= 0 || cols <= 0 || p == nullptr)
        return {0, 0};
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return {lo, lo + (uintptr_t)(((rows - 1) * ld + cols) * esize)};
}

bool overlap(const Extent &a, const Extent &b)
{
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

int hip_status(hipError_t e) { return e == hipSuccess ? HG_OK : HG_ERR_HIP_BASE + (int)e; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Recursion of the TRMM driver, depth first: for a diagonal block (o, s),
// s <= leaf is a leaf; otherwise with h = floor(s/2): recurse on (o, h),
// update rows o..o+h-1 from the block below the diagonal, recurse on
// (o+h, s-h).
struct Node {
    int64_t kind, o, s, depth;
};

void plan_rec(int64_t o, int64_t s, int64_t leaf, int64_t depth, std::vector<Node> &out)
{
    if (s <= leaf) {
        out.push_back({0, o, s, depth});
        return;
    }
    const int64_t h = s / 2;
    plan_rec(o, h, leaf, depth + 1, out);
    out.push_back({1, o, s, depth});
    plan_rec(o + h, s - h, leaf, depth + 1, out);
}

// Whether a TRMM of n×n A and n×m B too small for the 256×256 one-launch
// schedule runs in one launch of 64×64 tiles rather than level by level.
// In one launch the tiles of the first column walk all n/64 K stages, and
// 64×64 tiles move more bytes per flop than the per-level launches' larger
// tiles, but with two or more tiles per CU two workgroups share each CU.
// Measured back to back (one box, HIP events), one launch against level by
// level: n = 4096, m = 2048 67 / 84 us, n = m = 4096 129 / 150, n = m = 3072
// 68 / 118, n = 2048, m = 8192 79 / 104, n = 8192, m = 256 50 / 59, n = 8192,
// m = 512 87 / 93, n = 6144, m = 512 60 / 85, n = 16384, m = 64 77 / 118;
// but n = 8192, m = 1024 150 / 122, n = 8192, m = 2048 225 / 230 and
// n = 12288, m = 128 100 / 77 (there the tiles of the first column, which
// walk all n/64 stages, set the time); n = 6144, m = 256 55 / 52 and
// n = 16384, m = 128 111 / 119 are close either way (n = m = 2048 and
// n = 4096, m = 1024 were one launch before: 23 and 43 us).  So: n <= 4096,
// or n <= 8192 with m <= 512, or the work m·n² at most 2^34.
bool ring_fused_wanted(int64_t m, int64_t n)
{
    return n <= 4096 || (n <= 8192 && m <= 512) ||
           (double)m * (double)n * (double)n <= 17179869184.0;
}

// The one-launch TRMM in the row-major view of the column-major operands
// (C = Outᵀ, M = m; its A is Bᵀ; its B is the triangle T, N = K = n): T
// lower walked down from each tile's diagonal block, or (tri_up) T upper
// walked from K = 0 up to it.
hg::GemmParams one_launch_params(const void *T, int64_t ldt, const void *B, int64_t ldb, void *Out,
                                 int64_t ldo, int64_t m, int64_t n, float alpha, int64_t leaf, bool tri_up)
{
    hg::GemmParams p{};
    p.A = static_cast<const _Float16 *>(B);
    p.B = static_cast<const _Float16 *>(T);
    p.C = Out;
    p.lda = ldb;
    p.ldb = ldt;
    p.ldc = ldo;
    p.M = (int32_t)m;
    p.alpha = alpha;
    p.beta = 1.0f;
    p.leaf = (int32_t)std::min<int64_t>(leaf <= 0 ? 256 : leaf, kI32Max);
    p.tri_up = tri_up ? 1 : 0;
    p.nbatch = 1;
    p.e[0] = {0, 0, 0, (int32_t)n, (int32_t)n};
    return p;
}

// Which one-launch kernel runs p: 1 the 256×256 tiles, 2 the 64×64 tiles,
// 0 none (the per-level launches run instead).
int one_launch_kind(const hg::GemmParams &p, int64_t m, int64_t n)
{
    if (hg::trmm_fused_ok(p))
        return 1;
    if (ring_fused_wanted(m, n) && hg::trmm_ring_fused_ok(p))
        return 2;
    return 0;
}

hipError_t launch_one_launch(const hg::GemmParams &p, int kind, bool out_f16, hipStream_t s)
{
    return kind == 1 ? hg::launch_trmm_fused(p, s, out_f16) : hg::launch_trmm_fused_ring(p, s, out_f16);
}

hg::Tile choose_batched_tile(int64_t M, int64_t maxN, int64_t nbatch)
{
    const int64_t big = ((M + 255) / 256) * ((maxN + 255) / 256) * nbatch;
    if (big >= 256)
        return hg::Tile::Big;
    const int64_t mid = ((M + 127) / 128) * ((maxN + 127) / 128) * nbatch;
    if (mid >= 128)
        return hg::Tile::Mid;
    return hg::Tile::Small;
}

}  // namespace

extern "C" {

const char *hg_strerror(int status)
{
    if (status == HG_OK)
        return "success";
    if (status >= HG_ERR_HIP_BASE)
        return hipGetErrorString(static_cast<hipError_t>(status - HG_ERR_HIP_BASE));
    switch (status) {
    case -1: return "invalid argument 1";
    case -2: return "invalid argument 2";
    case -3: return "invalid argument 3";
    case -4: return "invalid argument 4";
    case -5: return "invalid argument 5";
    case -6: return "invalid argument 6";
    case -7: return "invalid argument 7";
    case -8: return "invalid argument 8";
    case -9: return "invalid argument 9";
    case -10: return "invalid argument 10";
    case -11: return "invalid argument 11";
    case -12: return "invalid argument 12";
    case -13: return "invalid argument 13";
    case -14: return "invalid argument 14";
    case -15: return "invalid argument 15";
    case -16: return "invalid argument 16";
    case -17: return "invalid argument 17";
    case HG_ERR_SCRATCH_LIMIT:
        return "problem needs more scratch than the static array holds (HG_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
    }
}

}  // extern "C"

namespace {

// hgemm, hgemm_bias_act and hgemm_bf16: the plain call is bias == nullptr,
// act == 0, fp16 operands; bf16 operands take out_dtype HG_BF16 or HG_F32.
int hgemm_impl(int64_t M, int64_t N, int64_t K, float alpha, const void *A, int64_t lda,
               const void *B, int64_t ldb, float beta, void *C, int64_t ldc, int out_dtype,
               const float *bias, int act, void *stream, bool in_bf16 = false)
{
    if (M < 0 || M > kI32Max)
        return -1;
    if (N < 0 || N > kI32Max)
        return -2;
    if (K < 0 || K > kI32Max)
        return -3;
    if (lda < std::max<int64_t>(1, K))
        return -6;
    if (ldb < std::max<int64_t>(1, K))
        return -8;
    if (ldc < std::max<int64_t>(1, N))
        return -11;
    if (in_bf16 ? (out_dtype != HG_BF16 && out_dtype != HG_F32)
                : (out_dtype != HG_F16 && out_dtype != HG_F32))
        return -12;
    if (act != HG_ACT_NONE && act != HG_ACT_RELU)
        return -14;
    if (M == 0 || N == 0)
        return HG_OK;
    if (C == nullptr)
        return -10;
    const bool out_f16 = out_dtype == HG_F16 || out_dtype == HG_BF16;   // 16-bit C
    const int64_t esize = out_f16 ? 2 : 4;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Extent ec = extent(C, M, ldc, N, esize);
    if (bias != nullptr && overlap(ec, extent(bias, 1, N, N, 4)))
        return -13;
    if (alpha == 0.0f || K == 0)
        return hip_status(hg::launch_scale(C, ldc, M, N, beta, out_f16, s, bias, act, in_bf16));
    if (A == nullptr)
        return -5;
    if (B == nullptr)
        return -7;
    if (overlap(ec, extent(A, M, lda, K, 2)) || overlap(ec, extent(B, N, ldb, K, 2)))
        return -10;

    hg::GemmParams p{};
    p.A = static_cast<const _Float16 *>(A);
    p.B = static_cast<const _Float16 *>(B);
    p.C = C;
    p.lda = lda;
    p.ldb = ldb;
    p.ldc = ldc;
    p.M = (int32_t)M;
    p.nbatch = 1;
    p.alpha = alpha;
    p.beta = beta;
    p.bias = bias;
    p.act = act;
    p.e[0] = {0, 0, 0, (int32_t)N, (int32_t)K};
    hg::LaunchOpts o{};
    o.out_f16 = out_f16;
    o.beta_read = beta != 0.0f;
    o.tri = false;
    o.vec = aligned16(A) && aligned16(B) && lda % 8 == 0 && ldb % 8 == 0;
    o.epi = bias != nullptr || act != HG_ACT_NONE;
    o.in_bf16 = in_bf16;
    o.tile = hg::choose_tile(M, N, K);
    return hip_status(hg::launch_gemm(p, o, s));
}

}  // namespace

extern "C" {

int hgemm(int64_t M, int64_t N, int64_t K, float alpha, const void *A, int64_t lda, const void *B,
          int64_t ldb, float beta, void *C, int64_t ldc, int out_dtype, void *stream)
{
    return hgemm_impl(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, out_dtype, nullptr,
                      HG_ACT_NONE, stream);
}

int hgemm_bias_act(int64_t M, int64_t N, int64_t K, float alpha, const void *A, int64_t lda,
                   const void *B, int64_t ldb, float beta, void *C, int64_t ldc, int out_dtype,
                   const float *bias, int act, void *stream)
{
    return hgemm_impl(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, out_dtype, bias, act, stream);
}

int hgemm_bf16_bias_act(int64_t M, int64_t N, int64_t K, float alpha, const void *A, int64_t lda,
                        const void *B, int64_t ldb, float beta, void *C, int64_t ldc, int out_dtype,
                        const float *bias, int act, void *stream)
{
    return hgemm_impl(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, out_dtype, bias, act, stream, true);
}

int hgemm_bf16(int64_t M, int64_t N, int64_t K, float alpha, const void *A, int64_t lda,
               const void *B, int64_t ldb, float beta, void *C, int64_t ldc, int out_dtype,
               void *stream)
{
    return hgemm_impl(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, out_dtype, nullptr,
                      HG_ACT_NONE, stream, true);
}

int64_t hg_trmm_plan(int64_t n, int64_t leaf, int64_t *nodes, int64_t cap)
{
    if (n < 0)
        return -1;
    if (nodes == nullptr && cap > 0)
        return -2;
    if (leaf <= 0)
        leaf = 256;
    std::vector<Node> v;
    if (n > 0)
        plan_rec(0, n, leaf, 0, v);
    for (int64_t i = 0; i < (int64_t)v.size() && i < cap; ++i) {
        nodes[4 * i + 0] = v[i].kind;
        nodes[4 * i + 1] = v[i].o;
        nodes[4 * i + 2] = v[i].s;
        nodes[4 * i + 3] = v[i].depth;
    }
    return (int64_t)v.size();
}

}  // extern "C"

namespace {

// Both TRMM entry points: `fused` allows the one-launch schedule (each
// output tile walks its own leaf and updates, adding the updates in its
// accumulators); without
// it, or when the recursion's boundaries do not fall on tile edges, one
// batched launch per recursion level.
// With `streams` (nstreams > 1, fused off) the per-level schedule puts each
// leaf and each update of a level on its own stream, round-robin, with the
// streams joined between levels (hg_trmm_lower_trans_streams).
int trmm_impl(int64_t n, int64_t m, float alpha, const void *A, int64_t lda, const void *B,
              int64_t ldb, void *Out, int64_t ldo, int out_dtype, int64_t leaf, void *stream,
              bool fused, const hipStream_t *streams = nullptr, int nstreams = 0)
{
    if (n < 0 || n > kI32Max)
        return -1;
    if (m < 0 || m > kI32Max)
        return -2;
    if (lda < std::max<int64_t>(1, n))
        return -5;
    if (ldb < std::max<int64_t>(1, n))
        return -7;
    if (ldo < std::max<int64_t>(1, n))
        return -9;
    if (out_dtype != HG_F32)
        return -10;
    if (n == 0 || m == 0)
        return HG_OK;
    if (Out == nullptr)
        return -8;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (leaf <= 0)
        leaf = 256;
    // Out (column-major n×m) seen as row-major m×n with leading dimension ldo.
    if (alpha == 0.0f)
        return hip_status(hg::launch_scale(Out, ldo, m, n, 0.0f, false, s));
    if (A == nullptr)
        return -4;
    if (B == nullptr)
        return -6;
    const Extent eo = extent(Out, m, ldo, n, 4);
    if (overlap(eo, extent(A, n, lda, n, 2)) || overlap(eo, extent(B, m, ldb, n, 2)))
        return -8;

    std::vector<Node> plan;
    plan_rec(0, n, leaf, 0, plan);
    int64_t max_depth = 0;
    for (const Node &x : plan)
        max_depth = std::max(max_depth, x.depth);

    // Every GEMM here is in the row-major view of the column-major operands:
    //   C'(j, i) = Out(o+i, j)             C' = Out + o,        ldc = ldo
    //   A'(j, k) = B(o+h+k, j)  (M'=m)     A' = B + o+h,        lda' = ldb
    //   B'(i, k) = A(o+h+k, o+i) (N'×K')   B' = A + o·lda+o+h,  ldb' = lda
    // i.e. Out1ᵀ += alpha·B2ᵀ·A21, the transpose of Out1 += alpha·A21ᵀ·B2.
    hg::GemmParams base{};
    base.A = static_cast<const _Float16 *>(B);
    base.B = static_cast<const _Float16 *>(A);
    base.C = Out;
    base.lda = ldb;
    base.ldb = lda;
    base.ldc = ldo;
    base.M = (int32_t)m;
    base.alpha = alpha;
    const bool base_vec = aligned16(A) && aligned16(B) && lda % 8 == 0 && ldb % 8 == 0;

    if (fused) {
        const hg::GemmParams p = one_launch_params(A, lda, B, ldb, Out, ldo, m, n, alpha, leaf, false);
        const int kind = one_launch_kind(p, m, n);
        if (kind != 0)
            return hip_status(launch_one_launch(p, kind, false, s));
    }

    // Several streams: events to join them between levels (every stream
    // waits for the others' work so far); the first stream is the caller's.
    std::vector<hipEvent_t> evs;
    auto cleanup = [&]() {
        for (hipEvent_t e : evs)
            (void)hipEventDestroy(e);
        evs.clear();
    };
    auto join = [&]() -> int {
        for (int i = 0; i < nstreams; ++i) {
            const hipError_t e = hipEventRecord(evs[i], streams[i]);
            if (e != hipSuccess)
                return hip_status(e);
        }
        for (int i = 0; i < nstreams; ++i)
            for (int k = 0; k < nstreams; ++k) {
                if (k == i)
                    continue;
                const hipError_t e = hipStreamWaitEvent(streams[i], evs[k], 0);
                if (e != hipSuccess)
                    return hip_status(e);
            }
        return HG_OK;
    };
    if (nstreams > 1) {
        for (int i = 0; i < nstreams; ++i) {
            hipEvent_t e;
            const hipError_t err = hipEventCreateWithFlags(&e, hipEventDisableTiming);
            if (err != hipSuccess) {
                cleanup();
                return hip_status(err);
            }
            evs.push_back(e);
        }
        // the other streams start after the caller's stream's earlier work
        const int stj = join();
        if (stj != HG_OK) {
            cleanup();
            return stj;
        }
    }
    int rr = 0;   // next stream, round-robin

    auto run_batch = [&](const std::vector<hg::BatchEntry> &ents, bool tri, float beta) -> int {
        for (size_t first = 0; first < ents.size(); first += hg::kMaxBatch) {
            hg::GemmParams p = base;
            p.beta = beta;
            const size_t cnt = std::min<size_t>(hg::kMaxBatch, ents.size() - first);
            p.nbatch = (int32_t)cnt;
            bool vec = base_vec;
            int64_t maxN = 0;
            for (size_t i = 0; i < cnt; ++i) {
                p.e[i] = ents[first + i];
                vec = vec && p.e[i].a_off % 8 == 0 && p.e[i].b_off % 8 == 0;
                maxN = std::max<int64_t>(maxN, p.e[i].N);
            }
            hg::LaunchOpts o{};
            o.out_f16 = false;
            o.beta_read = beta != 0.0f;
            o.tri = tri;
            o.vec = vec;
            o.tile = choose_batched_tile(m, maxN, (int64_t)cnt);
            if (nstreams > 1) {
                // each entry alone, with the tile family of the whole batch:
                // the same kernel computes every tile as in the batched launch
                for (size_t i = 0; i < cnt; ++i) {
                    hg::GemmParams q = p;
                    q.nbatch = 1;
                    q.e[0] = p.e[i];
                    const hipError_t e = hg::launch_gemm(q, o, streams[rr++ % nstreams]);
                    if (e != hipSuccess)
                        return hip_status(e);
                }
                continue;
            }
            const hipError_t e = hg::launch_gemm(p, o, s);
            if (e != hipSuccess)
                return hip_status(e);
        }
        return nstreams > 1 ? join() : HG_OK;
    };

    // Leaves: Out(o+i, j) = alpha·Σ_{k>=i} A(o+k, o+i)·B(o+k, j), written once.
    std::vector<hg::BatchEntry> ents;
    for (const Node &x : plan)
        if (x.kind == 0)
            ents.push_back({x.o, x.o * lda + x.o, x.o, (int32_t)x.s, (int32_t)x.s});
    int st = run_batch(ents, true, 0.0f);
    if (st != HG_OK) {
        cleanup();
        return st;
    }
    // Updates, deepest level first; within a level they write disjoint rows.
    for (int64_t d = max_depth; d >= 0; --d) {
        ents.clear();
        for (const Node &x : plan) {
            if (x.kind != 1 || x.depth != d)
                continue;
            const int64_t h = x.s / 2;
            ents.push_back({x.o + h, x.o * lda + x.o + h, x.o, (int32_t)h, (int32_t)(x.s - h)});
        }
        if (ents.empty())
            continue;
        st = run_batch(ents, false, 1.0f);
        if (st != HG_OK) {
            cleanup();
            return st;
        }
    }
    cleanup();
    return HG_OK;
}

}  // namespace

extern "C" {

int trmm_lower_trans(int64_t n, int64_t m, float alpha, const void *A, int64_t lda, const void *B,
                     int64_t ldb, void *Out, int64_t ldo, int out_dtype, int64_t leaf,
                     void *stream)
{
    return trmm_impl(n, m, alpha, A, lda, B, ldb, Out, ldo, out_dtype, leaf, stream, true);
}

int hg_trmm_lower_trans_by_level(int64_t n, int64_t m, float alpha, const void *A, int64_t lda,
                                 const void *B, int64_t ldb, void *Out, int64_t ldo, int out_dtype,
                                 int64_t leaf, void *stream)
{
    return trmm_impl(n, m, alpha, A, lda, B, ldb, Out, ldo, out_dtype, leaf, stream, false);
}

int hg_trmm_lower_trans_streams(int64_t n, int64_t m, float alpha, const void *A, int64_t lda,
                                const void *B, int64_t ldb, void *Out, int64_t ldo, int out_dtype,
                                int64_t leaf, void *const *streams, int nstreams)
{
    if (nstreams < 1 || nstreams > 8)
        return -13;
    if (streams == nullptr)
        return -12;
    hipStream_t ss[8];
    for (int i = 0; i < nstreams; ++i)
        ss[i] = static_cast<hipStream_t>(streams[i]);
    return trmm_impl(n, m, alpha, A, lda, B, ldb, Out, ldo, out_dtype, leaf, ss[0], false, ss, nstreams);
}

}  // extern "C"

namespace {

// ---- Recursive TRSM, X = alpha·A⁻ᵀ·B ("异构计算中高性能TRMM与TRSM的递归算法实现"
// §2.1, §2.3).  With A = [[A11, 0], [A21, A22]] split at h = floor(s/2),
// Aᵀ·X = alpha·B reads
//   A22ᵀ·X2 = alpha·B2                        (solve the lower half first)
//   A11ᵀ·X1 = alpha·B1 − A21ᵀ·X2               (GEMM update, then solve)
// down to leaves of at most `leaf` rows.

void trsm_leaves(int64_t o, int64_t s, int64_t leaf, std::vector<std::pair<int64_t, int64_t>> &out)
{
    if (s <= leaf) {
        out.push_back({o, s});
        return;
    }
    const int64_t h = s / 2;
    trsm_leaves(o, h, leaf, out);
    trsm_leaves(o + h, s - h, leaf, out);
}

// Workspace: the leaf inverses (fp16 ld×ld blocks, in ascending leaf
// order), then W, the fp16 copy of X (n×m column-major, ldw = n rounded up
// to 8), each part 256-byte aligned.
struct TrsmLayout {
    std::vector<std::pair<int64_t, int64_t>> leaves;
    int32_t ld = 0;
    int64_t v_bytes = 0;
    int64_t ldw = 0;
    int64_t total = 0;
};

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

TrsmLayout trsm_layout(int64_t n, int64_t m, int64_t leaf)
{
    TrsmLayout L;
    if (n == 0 || m == 0)
        return L;
    trsm_leaves(0, n, leaf, L.leaves);
    int64_t smax = 0;
    for (const auto &x : L.leaves)
        smax = std::max(smax, x.second);
    L.ld = (int32_t)round_up(smax, 8);
    L.v_bytes = round_up((int64_t)L.leaves.size() * L.ld * L.ld * 2, 256);
    L.ldw = round_up(n, 8);
    L.total = L.v_bytes + round_up(L.ldw * m * 2, 256);
    return L;
}

struct TrsmRun {
    const _Float16 *A, *B;
    int64_t lda, ldb, ldo, ldw, m;
    float *Out;
    _Float16 *V, *W;
    int32_t ld;
    float alpha;
    const std::vector<std::pair<int64_t, int64_t>> *leaves;
    int64_t leaf;
    hipStream_t stream;

    // sb > 0: the leaf also applies the update of the node (o, s + sb) whose
    // lower half [o+s, o+s+sb) is already solved (see TrsmLeafParams).
    int leaf_step(int64_t o, int64_t s, bool touched, int64_t sb = 0) const
    {
        const auto it = std::lower_bound(leaves->begin(), leaves->end(), std::make_pair(o, (int64_t)0));
        const int64_t idx = it - leaves->begin();
        hg::TrsmLeafParams p{};
        p.B = B;
        p.ldb = ldb;
        p.Out = Out;
        p.ldo = ldo;
        p.W = W;
        p.ldw = ldw;
        p.V = V + idx * ld * ld;
        p.ldv = ld;
        p.s = (int32_t)s;
        p.o = o;
        p.m = (int32_t)m;
        p.alpha = alpha;
        p.touched = touched ? 1 : 0;
        p.A = static_cast<const _Float16 *>(A);
        p.lda = lda;
        p.sb = (int32_t)sb;
        const bool vec = leaf_vec(o, s);
        return hip_status(hg::launch_trsm_leaf(p, vec, stream));
    }

    bool leaf_vec(int64_t o, int64_t s) const
    {
        return aligned16(B) && aligned16(Out) && aligned16(W) && o % 8 == 0 && s % 8 == 0 &&
               ldb % 8 == 0 && ldo % 4 == 0 && ldw % 4 == 0;
    }

    // The deepest nodes (both halves leaves) run as the lower leaf, then the
    // upper leaf with the node's update fused in, when the vector paths and
    // the fused update's alignment allow it.
    bool fuse_ok(int64_t o, int64_t s) const
    {
        const int64_t h = s / 2;
        return s > leaf && h <= leaf && s - h <= leaf && leaf_vec(o, h) && (s - h) % 8 == 0 &&
               aligned16(A) && lda % 8 == 0 && ldw % 8 == 0;
    }

    // Rows o..o+h-1 of the right-hand side: S = beta·S − A21ᵀ·X2 with
    // A21 = A[o+h:o+s, o:o+h] and X2 from W, in the row-major view
    //   C'(i, j) = Out(o+j, i),  A'(i, k) = W(o+h+k, i),  B'(j, k) = A(o+h+k, o+j).
    int update(int64_t o, int64_t s, bool touched) const
    {
        const int64_t h = s / 2;
        hg::GemmParams p{};
        p.A = W;
        p.B = A;
        p.C = Out;
        p.lda = ldw;
        p.ldb = lda;
        p.ldc = ldo;
        p.M = (int32_t)m;
        p.nbatch = 1;
        p.alpha = -1.0f;
        p.beta = touched ? 1.0f : 0.0f;
        p.e[0] = {o + h, (o + h) + o * lda, o, (int32_t)h, (int32_t)(s - h)};
        hg::LaunchOpts op{};
        op.out_f16 = false;
        op.beta_read = touched;
        op.tri = false;
        op.vec = aligned16(W) && aligned16(A) && ldw % 8 == 0 && lda % 8 == 0 &&
                 p.e[0].a_off % 8 == 0 && p.e[0].b_off % 8 == 0;
        op.tile = hg::choose_tile(m, h, s - h);
        return hip_status(hg::launch_gemm(p, op, stream));
    }

    // `touched`: some update has already written rows o..o+s-1 of Out.
    int solve(int64_t o, int64_t s, bool touched) const
    {
        if (s <= leaf)
            return leaf_step(o, s, touched);
        const int64_t h = s / 2;
        if (fuse_ok(o, s)) {
            const int st = leaf_step(o + h, s - h, touched);
            return st == HG_OK ? leaf_step(o, h, touched, s - h) : st;
        }
        int st = solve(o + h, s - h, touched);
        if (st == HG_OK)
            st = update(o, s, touched);
        if (st == HG_OK)
            st = solve(o, h, true);
        return st;
    }
};

}  // namespace

extern "C" {

int64_t hg_trsm_workspace_size(int64_t n, int64_t m, int64_t leaf)
{
    if (n < 0)
        return -1;
    if (m < 0)
        return -2;
    if (leaf <= 0)
        leaf = 256;
    if (leaf > hg::kTrsmLeafMax)
        return -3;
    return trsm_layout(n, m, leaf).total;
}

int trsm_lower_trans(int64_t n, int64_t m, float alpha, const void *A, int64_t lda, const void *B,
                     int64_t ldb, void *Out, int64_t ldo, int out_dtype, int64_t leaf, void *work,
                     int64_t work_bytes, void *stream)
{
    if (n < 0 || n > kI32Max)
        return -1;
    if (m < 0 || m > kI32Max)
        return -2;
    if (lda < std::max<int64_t>(1, n))
        return -5;
    if (ldb < std::max<int64_t>(1, n))
        return -7;
    if (ldo < std::max<int64_t>(1, n))
        return -9;
    if (out_dtype != HG_F32)
        return -10;
    if (leaf <= 0)
        leaf = 256;
    if (leaf > hg::kTrsmLeafMax)
        return -11;
    if (n == 0 || m == 0)
        return HG_OK;
    if (Out == nullptr)
        return -8;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (alpha == 0.0f)
        return hip_status(hg::launch_scale(Out, ldo, m, n, 0.0f, false, st));
    if (A == nullptr)
        return -4;
    if (B == nullptr)
        return -6;
    const Extent eo = extent(Out, m, ldo, n, 4);
    const Extent ea = extent(A, n, lda, n, 2);
    const Extent eb = extent(B, m, ldb, n, 2);
    if (overlap(eo, ea) || overlap(eo, eb))
        return -8;
    const TrsmLayout L = trsm_layout(n, m, leaf);
    if (work == nullptr || !aligned16(work))
        return -12;
    if (work_bytes < L.total)
        return -13;
    const Extent ew = {reinterpret_cast<uintptr_t>(work), reinterpret_cast<uintptr_t>(work) + (uintptr_t)L.total};
    if (overlap(ew, eo) || overlap(ew, ea) || overlap(ew, eb))
        return -12;

    TrsmRun r{};
    r.A = static_cast<const _Float16 *>(A);
    r.B = static_cast<const _Float16 *>(B);
    r.lda = lda;
    r.ldb = ldb;
    r.ldo = ldo;
    r.ldw = L.ldw;
    r.m = m;
    r.Out = static_cast<float *>(Out);
    r.V = static_cast<_Float16 *>(work);
    r.W = reinterpret_cast<_Float16 *>(static_cast<unsigned char *>(work) + L.v_bytes);
    r.ld = L.ld;
    r.alpha = alpha;
    r.leaves = &L.leaves;
    r.leaf = leaf;
    r.stream = st;

    // Every leaf's inverse first (they depend on A only).
    for (size_t first = 0; first < L.leaves.size(); first += hg::kTrsmInvBatch) {
        hg::TrsmInvParams p{};
        p.A = r.A;
        p.lda = lda;
        p.V = r.V;
        p.ld = L.ld;
        p.nleaf = (int32_t)std::min<size_t>(hg::kTrsmInvBatch, L.leaves.size() - first);
        for (int i = 0; i < p.nleaf; ++i) {
            p.o[i] = L.leaves[first + i].first;
            p.s[i] = (int32_t)L.leaves[first + i].second;
            p.voff[i] = (int64_t)(first + i) * L.ld * L.ld;
        }
        const int s = hip_status(hg::launch_trsm_inv(p, st));
        if (s != HG_OK)
            return s;
    }
    return r.solve(0, n, false);
}

}  // extern "C"

namespace {

// Workspace of hg_trmm: L (ldl×n fp16, ldl = n rounded up to 8), then the
// row-reversed B (ldl×m fp16) when the variant reverses rows; 256-byte
// aligned parts.
struct TrmmVariant {
    int mode = 0;         // index map of A (0: none)
    bool reverse = false; // B and Out rows reversed
    int64_t ldl = 0, l_bytes = 0, total = 0;
};

TrmmVariant trmm_variant(int uplo, int trans, int64_t n, int64_t m)
{
    TrmmVariant v;
    if (uplo == HG_LOWER && trans == HG_TRANS)
        return v;
    v.mode = uplo == HG_UPPER ? (trans == HG_NOTRANS ? 1 : 2) : 3;
    v.reverse = v.mode != 1;
    v.ldl = round_up(std::max<int64_t>(n, 1), 8);
    v.l_bytes = round_up(v.ldl * n * 2, 256);
    v.total = v.l_bytes + (v.reverse ? round_up(v.ldl * m * 2, 256) : 0);
    return v;
}

}  // namespace

extern "C" {

int64_t hg_trmm_workspace_size(int uplo, int trans, int64_t n, int64_t m)
{
    if (uplo != HG_LOWER && uplo != HG_UPPER)
        return -1;
    if (trans != HG_NOTRANS && trans != HG_TRANS)
        return -2;
    if (n < 0)
        return -3;
    if (m < 0)
        return -4;
    if (n == 0 || m == 0)
        return 0;
    return trmm_variant(uplo, trans, n, m).total;
}

int hg_trmm(int uplo, int trans, int64_t n, int64_t m, float alpha, const void *A, int64_t lda,
            const void *B, int64_t ldb, void *Out, int64_t ldo, int out_dtype, int64_t leaf,
            void *work, int64_t work_bytes, void *stream)
{
    if (uplo != HG_LOWER && uplo != HG_UPPER)
        return -1;
    if (trans != HG_NOTRANS && trans != HG_TRANS)
        return -2;
    if (n < 0 || n > kI32Max)
        return -3;
    if (m < 0 || m > kI32Max)
        return -4;
    if (lda < std::max<int64_t>(1, n))
        return -7;
    if (ldb < std::max<int64_t>(1, n))
        return -9;
    if (ldo < std::max<int64_t>(1, n))
        return -11;
    if (out_dtype != HG_F32)
        return -12;
    if (n == 0 || m == 0)
        return HG_OK;
    if (Out == nullptr)
        return -10;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (alpha == 0.0f)
        return hip_status(hg::launch_scale(Out, ldo, m, n, 0.0f, false, s));
    if (A == nullptr)
        return -6;
    if (B == nullptr)
        return -8;
    const Extent eo = extent(Out, m, ldo, n, 4);
    const Extent ea = extent(A, n, lda, n, 2);
    const Extent eb = extent(B, m, ldb, n, 2);
    if (overlap(eo, ea) || overlap(eo, eb))
        return -10;
    const TrmmVariant v = trmm_variant(uplo, trans, n, m);
    if (v.mode == 0)
        return trmm_impl(n, m, alpha, A, lda, B, ldb, Out, ldo, out_dtype, leaf, stream, true);
    if (work == nullptr || !aligned16(work))
        return -14;
    if (work_bytes < v.total)
        return -15;
    const Extent ew = {reinterpret_cast<uintptr_t>(work), reinterpret_cast<uintptr_t>(work) + (uintptr_t)v.total};
    if (overlap(ew, eo) || overlap(ew, ea) || overlap(ew, eb))
        return -14;
    _Float16 *L = static_cast<_Float16 *>(work);
    // Upper/transposed (L = A) and lower/non-transposed (L = Aᵀ, upper) are,
    // in the GEMM view, the lower-transposed product with the triangle on the
    // other side: the one-launch schedule walks each tile's K from 0 to its
    // diagonal block (tri_up), with no row reversal of B or Out.
    if ((uplo == HG_UPPER && trans == HG_TRANS) || (uplo == HG_LOWER && trans == HG_NOTRANS)) {
        const bool copy = uplo == HG_LOWER;
        const hg::GemmParams p = one_launch_params(copy ? static_cast<const void *>(L) : A, copy ? v.ldl : lda,
                                                   B, ldb, Out, ldo, m, n, alpha, leaf, true);
        const int kind = one_launch_kind(p, m, n);
        if (kind != 0) {
            if (copy) {
                const int st = hip_status(hg::launch_tri_xform(4, static_cast<const _Float16 *>(A), lda, L, v.ldl, n, s));
                if (st != HG_OK)
                    return st;
            }
            return hip_status(launch_one_launch(p, kind, false, s));
        }
    }
    int st = hip_status(hg::launch_tri_xform(v.mode, static_cast<const _Float16 *>(A), lda, L, v.ldl, n, s));
    if (st != HG_OK)
        return st;
    const void *Bin = B;
    int64_t ldbin = ldb;
    if (v.reverse) {
        _Float16 *Bp = reinterpret_cast<_Float16 *>(static_cast<unsigned char *>(work) + v.l_bytes);
        st = hip_status(hg::launch_row_reverse_copy(static_cast<const _Float16 *>(B), ldb, Bp, v.ldl, n, m, s));
        if (st != HG_OK)
            return st;
        Bin = Bp;
        ldbin = v.ldl;
    }
    st = trmm_impl(n, m, alpha, L, v.ldl, Bin, ldbin, Out, ldo, out_dtype, leaf, stream, true);
    if (st != HG_OK)
        return st;
    if (v.reverse)
        st = hip_status(hg::launch_row_reverse_inplace(static_cast<float *>(Out), ldo, n, m, s));
    return st;
}

}  // extern "C"

namespace {

// Workspace of hgemm_layout: A in the native row-major M×K form when it is
// given column-major, then B in the native N×K (K-contiguous) form when it
// is given row-major; ld = K rounded up to 8, parts 256-byte aligned.
struct GemmLayout {
    int64_t ldk = 0, a_bytes = 0, b_bytes = 0;
};

GemmLayout gemm_layout(int a_layout, int b_layout, int64_t M, int64_t N, int64_t K)
{
    GemmLayout g;
    g.ldk = round_up(std::max<int64_t>(K, 1), 8);
    g.a_bytes = a_layout == HG_COL_MAJOR ? round_up(M * g.ldk * 2, 256) : 0;
    g.b_bytes = b_layout == HG_ROW_MAJOR ? round_up(N * g.ldk * 2, 256) : 0;
    return g;
}

}  // namespace

extern "C" {

int64_t hg_hgemm_layout_workspace_size(int a_layout, int b_layout, int64_t M, int64_t N, int64_t K)
{
    if (a_layout != HG_ROW_MAJOR && a_layout != HG_COL_MAJOR)
        return -1;
    if (b_layout != HG_ROW_MAJOR && b_layout != HG_COL_MAJOR)
        return -2;
    if (M < 0 || N < 0 || K < 0)
        return -3;
    if (M == 0 || N == 0 || K == 0)
        return 0;
    const GemmLayout g = gemm_layout(a_layout, b_layout, M, N, K);
    return g.a_bytes + g.b_bytes;
}

int hgemm_layout(int a_layout, int b_layout, int64_t M, int64_t N, int64_t K, float alpha,
                 const void *A, int64_t lda, const void *B, int64_t ldb, float beta, void *C,
                 int64_t ldc, int out_dtype, void *work, int64_t work_bytes, void *stream)
{
    if (a_layout != HG_ROW_MAJOR && a_layout != HG_COL_MAJOR)
        return -1;
    if (b_layout != HG_ROW_MAJOR && b_layout != HG_COL_MAJOR)
        return -2;
    if (M < 0 || M > kI32Max)
        return -3;
    if (N < 0 || N > kI32Max)
        return -4;
    if (K < 0 || K > kI32Max)
        return -5;
    // A is M×K: row-major needs lda >= K, column-major lda >= M; B is K×N:
    // column-major needs ldb >= K, row-major ldb >= N.
    if (lda < std::max<int64_t>(1, a_layout == HG_ROW_MAJOR ? K : M))
        return -8;
    if (ldb < std::max<int64_t>(1, b_layout == HG_COL_MAJOR ? K : N))
        return -10;
    if (ldc < std::max<int64_t>(1, N))
        return -13;
    if (out_dtype != HG_F16 && out_dtype != HG_F32)
        return -14;
    if (M == 0 || N == 0)
        return HG_OK;
    if (C == nullptr)
        return -12;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool native_a = a_layout == HG_ROW_MAJOR, native_b = b_layout == HG_COL_MAJOR;
    const bool reads = alpha != 0.0f && K != 0;
    if (reads && A == nullptr)
        return -7;
    if (reads && B == nullptr)
        return -9;
    const int64_t esize = out_dtype == HG_F16 ? 2 : 4;
    const Extent ec = extent(C, M, ldc, N, esize);
    const Extent ea = native_a ? extent(A, M, lda, K, 2) : extent(A, K, lda, M, 2);
    const Extent eb = native_b ? extent(B, N, ldb, K, 2) : extent(B, K, ldb, N, 2);
    if (reads && (overlap(ec, ea) || overlap(ec, eb)))
        return -12;
    // Native layouts (and the quick returns, which read neither operand) are
    // hgemm itself; every argument it checks has been checked above.
    if ((native_a && native_b) || !reads)
        return hgemm_impl(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, out_dtype, nullptr,
                          HG_ACT_NONE, stream);
    const GemmLayout g = gemm_layout(a_layout, b_layout, M, N, K);
    if (work == nullptr || !aligned16(work))
        return -15;
    if (work_bytes < g.a_bytes + g.b_bytes)
        return -16;
    const Extent ew = {reinterpret_cast<uintptr_t>(work),
                       reinterpret_cast<uintptr_t>(work) + (uintptr_t)(g.a_bytes + g.b_bytes)};
    if (overlap(ew, ec) || overlap(ew, ea) || overlap(ew, eb))
        return -15;
    const void *An = A;
    int64_t ldan = lda;
    const void *Bn = B;
    int64_t ldbn = ldb;
    unsigned char *wp = static_cast<unsigned char *>(work);
    if (!native_a) {
        // A column-major M×K is Aᵀ row-major K×M: transpose it to M×K row-major.
        _Float16 *Ap = reinterpret_cast<_Float16 *>(wp);
        const int st = hip_status(hg::launch_transpose(static_cast<const _Float16 *>(A), lda, Ap, g.ldk, K, M, s));
        if (st != HG_OK)
            return st;
        An = Ap;
        ldan = g.ldk;
    }
    if (!native_b) {
        // B row-major K×N: transpose it to N×K row-major (K-contiguous columns).
        _Float16 *Bp = reinterpret_cast<_Float16 *>(wp + g.a_bytes);
        const int st = hip_status(hg::launch_transpose(static_cast<const _Float16 *>(B), ldb, Bp, g.ldk, K, N, s));
        if (st != HG_OK)
            return st;
        Bn = Bp;
        ldbn = g.ldk;
    }
    return hgemm_impl(M, N, K, alpha, An, ldan, Bn, ldbn, beta, C, ldc, out_dtype, nullptr,
                      HG_ACT_NONE, stream);
}

}  // extern "C"

extern "C" {

int64_t hg_trmm_inplace_workspace_size(int uplo, int trans, int64_t n, int64_t m)
{
    const int64_t v = hg_trmm_workspace_size(uplo, trans, n, m);
    if (v < 0 || n == 0 || m == 0)
        return v;
    return round_up(round_up(n, 8) * m * 4, 256) + v;
}

int hg_trmm_inplace(int uplo, int trans, int64_t n, int64_t m, float alpha, const void *A, int64_t lda,
                    void *B, int64_t ldb, int64_t leaf, void *work, int64_t work_bytes, void *stream)
{
    if (uplo != HG_LOWER && uplo != HG_UPPER)
        return -1;
    if (trans != HG_NOTRANS && trans != HG_TRANS)
        return -2;
    if (n < 0 || n > kI32Max)
        return -3;
    if (m < 0 || m > kI32Max)
        return -4;
    if (lda < std::max<int64_t>(1, n))
        return -7;
    if (ldb < std::max<int64_t>(1, n))
        return -9;
    if (n == 0 || m == 0)
        return HG_OK;
    if (B == nullptr)
        return -8;
    if (alpha != 0.0f && A == nullptr)
        return -6;
    const int64_t ldx = round_up(n, 8);
    const int64_t x_bytes = round_up(ldx * m * 4, 256);
    const int64_t need = x_bytes + hg_trmm_workspace_size(uplo, trans, n, m);
    if (work == nullptr || !aligned16(work))
        return -11;
    if (work_bytes < need)
        return -12;
    const Extent ew = {reinterpret_cast<uintptr_t>(work), reinterpret_cast<uintptr_t>(work) + (uintptr_t)need};
    if (overlap(ew, extent(B, m, ldb, n, 2)) || (A && overlap(ew, extent(A, n, lda, n, 2))))
        return -11;
    if (A && overlap(extent(B, m, ldb, n, 2), extent(A, n, lda, n, 2)))
        return -8;
    float *X = static_cast<float *>(work);
    unsigned char *vwork = static_cast<unsigned char *>(work) + x_bytes;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // When the variant runs in one launch, its tiles round alpha·acc to fp16
    // themselves (the rounding the fp32 route below applies to the same fp32
    // value) into the workspace's first ldx·m·2 bytes, and one copy moves the
    // product into B: at n = m = 8192, 384 MiB less traffic than writing the
    // fp32 product and rounding it in a second pass.  The variants map onto
    // the one-launch kernel as hg_trmm's do: lower/trans on A, upper/trans
    // with tri_up on A, lower/notrans with tri_up on an upper copy of Aᵀ,
    // upper/notrans on the lower copy L = Aᵀ.
    if (alpha != 0.0f) {
        const TrmmVariant v = trmm_variant(uplo, trans, n, m);
        _Float16 *L = reinterpret_cast<_Float16 *>(vwork);
        const bool up = (uplo == HG_UPPER) == (trans == HG_TRANS);
        const int copy_mode = trans == HG_TRANS ? 0 : (uplo == HG_LOWER ? 4 : 1);
        _Float16 *Y = static_cast<_Float16 *>(work);
        const hg::GemmParams p = one_launch_params(copy_mode ? static_cast<const void *>(L) : A,
                                                   copy_mode ? v.ldl : lda, B, ldb, Y, ldx, m, n, alpha, leaf, up);
        const int kind = one_launch_kind(p, m, n);
        if (kind != 0) {
            int st = HG_OK;
            if (copy_mode)
                st = hip_status(hg::launch_tri_xform(copy_mode, static_cast<const _Float16 *>(A), lda, L, v.ldl, n, s));
            if (st == HG_OK)
                st = hip_status(launch_one_launch(p, kind, true, s));
            if (st == HG_OK)
                st = hip_status(hipMemcpy2DAsync(B, (size_t)ldb * 2, Y, (size_t)ldx * 2, (size_t)n * 2, (size_t)m,
                                                 hipMemcpyDeviceToDevice, s));
            return st;
        }
    }
    int st = hg_trmm(uplo, trans, n, m, alpha, A, lda, B, ldb, X, ldx, HG_F32, leaf, vwork,
                     work_bytes - x_bytes, stream);
    if (st != HG_OK)
        return st;   // a HIP error: the arguments were checked above
    return hip_status(hg::launch_f32_to_f16(X, ldx, static_cast<_Float16 *>(B), ldb, n, m, s));
}

}  // extern "C"

namespace {

// ---- Split-K: K cut into S slices of Ks (a multiple of 64) columns; the
// slices run as one batched GEMM into fp32 partials (alpha = 1, beta = 0),
// then one reduction kernel sums them in slice order and applies alpha,
// beta and the output conversion.
struct SplitK {
    int64_t S = 1, Ks = 0, bytes = 0;
};

int device_cus()
{
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    return n;
}

// splits > 0: that many slices (at most 32, each at least 64 columns of K);
// 0: enough slices to give every CU a 128×128 tile, each slice at least 256
// columns of K.
SplitK splitk_plan(int64_t M, int64_t N, int64_t K, int splits)
{
    SplitK p;
    int64_t want = splits;
    if (splits == 0) {
        const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
        want = std::max<int64_t>(1, device_cus() / std::max<int64_t>(tiles, 1));
        want = std::min<int64_t>(want, std::max<int64_t>(1, K / 256));
    }
    want = std::max<int64_t>(1, std::min<int64_t>({want, 32, std::max<int64_t>(1, K / 64)}));
    p.Ks = round_up((K + want - 1) / want, 64);
    p.S = std::max<int64_t>(1, (K + p.Ks - 1) / p.Ks);
    p.bytes = round_up(p.S * M * N * 4, 256);
    return p;
}

}  // namespace

extern "C" {

int64_t hg_hgemm_splitk_workspace_size(int64_t M, int64_t N, int64_t K, int splits)
{
    if (M < 0 || M > kI32Max)
        return -1;
    if (N < 0 || N > kI32Max)
        return -2;
    if (K < 0 || K > kI32Max)
        return -3;
    if (splits < 0 || splits > 32)
        return -4;
    if (M == 0 || N == 0 || K == 0)
        return 0;
    return splitk_plan(M, N, K, splits).bytes;
}

int hgemm_splitk(int64_t M, int64_t N, int64_t K, float alpha, const void *A, int64_t lda, const void *B,
                 int64_t ldb, float beta, void *C, int64_t ldc, int out_dtype, int splits, void *work,
                 int64_t work_bytes, void *stream)
{
    if (M < 0 || M > kI32Max)
        return -1;
    if (N < 0 || N > kI32Max)
        return -2;
    if (K < 0 || K > kI32Max)
        return -3;
    if (lda < std::max<int64_t>(1, K))
        return -6;
    if (ldb < std::max<int64_t>(1, K))
        return -8;
    if (ldc < std::max<int64_t>(1, N))
        return -11;
    if (out_dtype != HG_F16 && out_dtype != HG_F32)
        return -12;
    if (splits < 0 || splits > 32)
        return -13;
    if (M == 0 || N == 0)
        return HG_OK;
    if (C == nullptr)
        return -10;
    const bool out_f16 = out_dtype == HG_F16;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Extent ec = extent(C, M, ldc, N, out_f16 ? 2 : 4);
    if (alpha == 0.0f || K == 0)
        return hip_status(hg::launch_scale(C, ldc, M, N, beta, out_f16, s));
    if (A == nullptr)
        return -5;
    if (B == nullptr)
        return -7;
    const Extent ea = extent(A, M, lda, K, 2), eb = extent(B, N, ldb, K, 2);
    if (overlap(ec, ea) || overlap(ec, eb))
        return -10;
    const SplitK plan = splitk_plan(M, N, K, splits);
    if (work == nullptr || !aligned16(work))
        return -14;
    if (work_bytes < plan.bytes)
        return -15;
    const Extent ew = {reinterpret_cast<uintptr_t>(work), reinterpret_cast<uintptr_t>(work) + (uintptr_t)plan.bytes};
    if (overlap(ew, ec) || overlap(ew, ea) || overlap(ew, eb))
        return -14;
    float *P = static_cast<float *>(work);
    hg::GemmParams p{};
    p.A = static_cast<const _Float16 *>(A);
    p.B = static_cast<const _Float16 *>(B);
    p.C = P;
    p.lda = lda;
    p.ldb = ldb;
    p.ldc = N;
    p.M = (int32_t)M;
    p.alpha = 1.0f;
    p.beta = 0.0f;
    p.nbatch = (int32_t)plan.S;
    bool vec = aligned16(A) && aligned16(B) && lda % 8 == 0 && ldb % 8 == 0;
    for (int64_t q = 0; q < plan.S; ++q) {
        const int64_t k0 = q * plan.Ks;
        p.e[q] = {k0, k0, q * M * N, (int32_t)N, (int32_t)std::min(plan.Ks, K - k0)};
    }
    hg::LaunchOpts o{};
    o.out_f16 = false;
    o.beta_read = false;
    o.tri = false;
    o.vec = vec;
    o.tile = choose_batched_tile(M, N, plan.S);
    int st = hip_status(hg::launch_gemm(p, o, s));
    if (st != HG_OK)
        return st;
    return hip_status(hg::launch_splitk_reduce(P, M * N, (int)plan.S, M, N, alpha, beta, C, ldc, out_f16, s));
}

}  // extern "C"
