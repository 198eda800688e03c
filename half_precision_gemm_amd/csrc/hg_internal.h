// Internal interface between the host API (hg_api.cpp) and the gfx950
// kernels (hg_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace hg {

// One GEMM of a batched launch.  All GEMMs of a launch share M, lda, ldb,
// ldc, alpha, beta and the base pointers; each has its own element offsets
// and its own N and K.  The TRMM driver uses this to run every leaf, or every
// update of one recursion level, in a single launch.
struct BatchEntry {
    int64_t a_off;   // element offset into A (row-major M×K operand)
    int64_t b_off;   // element offset into B (N×K operand, K contiguous)
    int64_t c_off;   // element offset into C (row-major M×N)
    int32_t N;
    int32_t K;
};

constexpr int kMaxBatch = 32;

struct GemmParams {
    const _Float16 *A;
    const _Float16 *B;
    void *C;
    int64_t lda, ldb, ldc;
    int32_t M;
    int32_t nbatch;
    float alpha, beta;
    int32_t leaf;    // recursive TRMM in one launch: the recursion's leaf size
    int32_t tri_up;  // recursive TRMM in one launch: B element (j, k) counts for
                     // k <= j (an upper-triangular operand in the GEMM view)
                     // instead of k >= j
    const float *bias;   // fused epilogue: per-column bias (nullptr: none)
    int32_t act;         // fused epilogue: 0 identity, 1 ReLU
    BatchEntry e[kMaxBatch];
};

// Fused epilogue of hgemm_bias_act: t + bias, then the activation.  A missing
// bias is passed as -0, which leaves every t unchanged (also ±0); ReLU maps
// t < 0 to +0 and lets NaN through.
__device__ __forceinline__ float epi_apply(float t, float bias, int act)
{
    t += bias;
    return (act == 1 && t < 0.0f) ? 0.0f : t;
}

// v as an fp32 value the compiler cannot see through: a product rounded to
// fp32 here and then converted to a 16-bit type is rounded twice, as when an
// fp32 result is stored and converted later, instead of being fused with the
// conversion into one rounding (v_fma_mix).
__device__ __forceinline__ float opaque_f32(float v)
{
    __asm__("" : "+v"(v));
    return v;
}

// Compute units of the current device (queried once per device).
int cu_count();

// Kernel families the launcher can pick.
enum class Tile { Big, Mid, Small };

struct LaunchOpts {
    bool out_f16;     // C element type
    bool beta_read;   // beta != 0: read C
    bool tri;         // TRMM leaf: B operand element (j, k) is zero for k < j
    bool vec;         // 16-byte aligned operands: vector loads
    bool epi;         // fused bias / activation (p.bias, p.act)
    bool in_bf16;     // A and B (and a 16-bit C) are bf16 instead of fp16
    Tile tile;
};

// Validated arguments in, kernels launched on `stream`; returns hipError_t.
hipError_t launch_gemm(const GemmParams &p, const LaunchOpts &o, hipStream_t stream);

// 256×256 direct-to-LDS pipelined kernel (hg_fast.hip): usable when the
// operands allow 16-byte buffer loads and K % 8 == 0 (TRI: fp32 output
// written once).
bool fast_path_ok(const GemmParams &p, const LaunchOpts &o);
hipError_t launch_gemm_fast(const GemmParams &p, const LaunchOpts &o, hipStream_t stream);

// 64×64 / 128×128 tiles with a deep ring of direct buffer→LDS stages
// (hg_ring.hip), for the Small and Mid tile families when the operands
// allow 16-byte buffer loads and K % 8 == 0 (with the triangle mask: fp32
// output written once, fp16 operands, no epilogue extras).
bool ring_path_ok(const GemmParams &p, const LaunchOpts &o);
hipError_t launch_gemm_ring(const GemmParams &p, const LaunchOpts &o, hipStream_t stream);

// Recursive TRMM (Out = alpha·Aᵀ·B, A lower) in one launch, in the GEMM view
// C = Outᵀ (M = m, N = K = n; p.A = B, p.B = A, p.C = Out, p.e[0] = {0, 0,
// 0, n, n}, p.leaf): every output tile walks its leaf and then the recursion's
// updates that touch it, deepest first, in one persistent workgroup, the
// updates accumulated in registers (one store per tile).
// With p.tri_up the GEMM view's B element (j, k) counts for k <= j: a tile
// walks K from 0 to its own diagonal block (the outermost update first, the
// leaf last).
// trmm_fused_ok: the operands suit the fast path, every recursion boundary
// falls on a 256-column tile edge, and there are at least two output tiles
// per CU.
// With out_f16 the tiles are written as fp16 (alpha·acc rounded once to
// nearest even) instead of fp32; p.C points to fp16 elements then.
bool trmm_fused_ok(const GemmParams &p);
hipError_t launch_trmm_fused(const GemmParams &p, hipStream_t stream, bool out_f16 = false);
// The same one-launch recursion on 64×64 tiles (hg_ring.hip), one workgroup
// per tile, for right-hand sides too narrow to give every CU two 256×256
// tiles: every recursion boundary on a 64-column tile edge, leaf >= 64.
bool trmm_ring_fused_ok(const GemmParams &p);
hipError_t launch_trmm_fused_ring(const GemmParams &p, hipStream_t stream, bool out_f16 = false);

// Recursive triangular solve X = alpha·A⁻ᵀ·B (hg_trsm.hip).  Leaves are at
// most kTrsmLeafMax rows; their inverses V_L = A_LL⁻¹ are stored in fp16 as
// full ld×ld column-major blocks (zeros above the diagonal and outside the
// leaf), block l at V + voff[l].
constexpr int kTrsmLeafMax = 256;
constexpr int kTrsmInvBatch = 64;

struct TrsmInvParams {
    const _Float16 *A;     // n×n column-major, lower triangle read
    int64_t lda;
    _Float16 *V;           // workspace
    int32_t ld;            // leading dimension (and size) of every V block, multiple of 8
    int32_t nleaf;         // leaves in this launch (<= kTrsmInvBatch)
    int64_t o[kTrsmInvBatch];     // leaf offsets (first row/column in A)
    int64_t voff[kTrsmInvBatch];  // element offset of each V block
    int32_t s[kTrsmInvBatch];     // leaf sizes (<= ld)
};

// One leaf of the solve, rows o..o+s-1 of X:
//   R = fp16(alpha·B + S) (S = Out rows, the updates so far, when `touched`),
//   X = V_Lᵀ·R with fp32 accumulation, Out = X (fp32), W = fp16(X).
struct TrsmLeafParams {
    const _Float16 *B;     // n×m column-major right-hand side
    int64_t ldb;
    float *Out;            // n×m column-major fp32 result / running update sums
    int64_t ldo;
    _Float16 *W;           // n×m column-major fp16 copy of X (operand of the updates)
    int64_t ldw;
    const _Float16 *V;     // this leaf's inverse block
    int32_t ldv;
    int32_t s;             // leaf size, 1..kTrsmLeafMax
    int64_t o;             // leaf offset
    int32_t m;             // columns of B
    float alpha;
    int32_t touched;       // nonzero: add S = Out rows to alpha·B
    // Fused update of the recursion node whose upper half is this leaf
    // (sb > 0, vec only): S -= A21ᵀ·X2 first, A21 = A[o+s : o+s+sb, o : o+s],
    // X2 = W rows o+s .. o+s+sb-1 (the lower half, already solved).
    const _Float16 *A;
    int64_t lda;
    int32_t sb;
};

hipError_t launch_trsm_inv(const TrsmInvParams &p, hipStream_t stream);
// vec: B, Out, W 16-byte aligned, o % 8 == 0, s % 8 == 0, ldb % 8 == 0,
// ldo % 4 == 0, ldw % 4 == 0 (vector loads and stores); a fused update
// (sb > 0) also needs vec, A 16-byte aligned, lda % 8 == 0, ldw % 8 == 0 and
// sb % 8 == 0.
hipError_t launch_trsm_leaf(const TrsmLeafParams &p, bool vec, hipStream_t stream);

// TRMM variants (hg_xform.hip): L = map(A) on L's lower triangle (mode 1:
// A(c, r), 2: A(n-1-r, n-1-c), 3: A(n-1-c, n-1-r)), or mode 4: A(c, r) on
// L's upper triangle; B's rows reversed into
// Bp; Out's rows reversed in place.
hipError_t launch_tri_xform(int mode, const _Float16 *A, int64_t lda, _Float16 *L, int64_t ldl,
                            int64_t n, hipStream_t stream);
hipError_t launch_row_reverse_copy(const _Float16 *B, int64_t ldb, _Float16 *Bp, int64_t ldp, int64_t n,
                                   int64_t m, hipStream_t stream);
hipError_t launch_row_reverse_inplace(float *Out, int64_t ldo, int64_t n, int64_t m, hipStream_t stream);
// Split-K: C = alpha·Σ_s P_s + beta·C over S fp32 partials (M×N row-major,
// ld N, `slice` elements apart), in slice order.
hipError_t launch_splitk_reduce(const float *P, int64_t slice, int S, int64_t M, int64_t N, float alpha,
                                float beta, void *C, int64_t ldc, bool out_f16, hipStream_t stream);
// B = fp16(X) (nearest even), column-major n×m.
hipError_t launch_f32_to_f16(const float *X, int64_t ldx, _Float16 *B, int64_t ldb, int64_t n, int64_t m,
                             hipStream_t stream);
// D = Sᵀ, S rows×cols row-major (lds), D cols×rows row-major (ldd), fp16.
hipError_t launch_transpose(const _Float16 *S, int64_t lds, _Float16 *D, int64_t ldd, int64_t rows,
                            int64_t cols, hipStream_t stream);

// C = beta·C over an M×N window (beta == 0 writes zeros without reading);
// with `bias` or `act`, C = act(beta·C + bias[j]) (the alpha = 0 / K = 0
// case of the fused epilogue).
hipError_t launch_scale(void *C, int64_t ldc, int64_t M, int64_t N, float beta,
                        bool out_f16, hipStream_t stream, const float *bias = nullptr,
                        int act = 0, bool bf16 = false);

// Tile family the launcher would choose for a single M×N GEMM.
Tile choose_tile(int64_t M, int64_t N, int64_t K);

}  // namespace hg
