// hg_trsm.hip — gfx950 kernels of the recursive triangular solve
// X = alpha·A⁻ᵀ·B with A lower triangular ("异构计算中高性能TRMM与TRSM的递归算法实现"
// §2.1 blocking, §2.3 triangular solve).
//
// The host driver (hg_api.cpp) runs the recursion: for a diagonal block of
// size s > leaf split at h = floor(s/2), solve the lower half first, update
// the upper half's right-hand side with the GEMM kernels (alpha = -1), then
// solve the upper half.  This file holds the two pieces the GEMM kernels do
// not cover:
//
//   * trsm_inv_kernel — the inverse V_L = A_LL⁻¹ of every leaf's diagonal
//     block, in fp32 by block forward substitution, stored as fp16.  It
//     depends on A only, so all leaves are inverted up front in one launch.
//   * trsm_leaf_kernel — the leaf step X_L = V_Lᵀ·R_L as a matrix-core
//     product (v_mfma_f32_32x32x16_f16, fp32 accumulation), where
//     R_L = fp16(alpha·B_L + S_L) and S_L holds the sum of the updates already
//     applied to these rows.  It writes X_L in fp32 and an fp16 copy that the
//     updates above it take as their GEMM operand.
//
// The page solves each leaf by column-parallel substitution with a light
// synchronisation after every row.  On the matrix cores a 256-row leaf is
// instead one small GEMM against the precomputed inverse: every one of the
// m columns of B is independent, as in the page's scheme, and the
// row-by-row dependence moves into the inversion, which is done once per
// leaf instead of once per column.
#include "hg_internal.h"

typedef int32_t hg_trsm_i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer load of 16 bytes per lane (LLVM intrinsic).  An offset past the
// resource's range returns zeros without a memory request.
extern "C" __device__ hg_trsm_i32x4 hg_trsm_buffer_load_b128(hg_trsm_i32x4 rsrc, int voffset, int soffset,
                                                            int aux) __asm("llvm.amdgcn.raw.buffer.load.v4i32");

namespace hg {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));

// ---- Diagonal block inverses -------------------------------------------------
//
// Workgroup (leaf l, column block J) computes columns c0 = 32·J .. c0+31 of
// V = A_LL⁻¹ (lower triangular) over 32-row blocks I = J, J+1, …:
//   T = E_IJ − Σ_{K=J}^{I−1} A_IK·V_KJ      (E = identity)
//   V_IJ = D_I·T,  D_I = A_II⁻¹
// The D_I of all its blocks are computed first, together (one forward
// substitution per thread), so that the block-by-block sweep holds no
// serial substitution, only products.  All arithmetic is fp32; the block is written as fp16, each element exactly
// once: the computed lower part, zeros above the diagonal, outside the leaf
// and in the padding up to ld, so that the leaf kernel needs no masks.
constexpr int kInvCols = 32;

__global__ void __launch_bounds__(256) trsm_inv_kernel(const TrsmInvParams p)
{
    // This column block of V, transposed: vt[c][r] = V(r, c0 + c).  Row
    // stride 260 floats keeps every row 16-byte aligned for float4 reads.
    constexpr int VT = kTrsmLeafMax + 4;
    constexpr int NDB = kTrsmLeafMax / kInvCols;       // diagonal blocks per leaf (8)
    constexpr int DT = kInvCols + 4;
    __shared__ __attribute__((aligned(16))) float vt[kInvCols][VT];
    __shared__ __attribute__((aligned(16))) float as[kInvCols][VT];   // A row panel of block I
    // D_I = A_II⁻¹ of the diagonal blocks I = J, J+1, …: dd[I - J][r][k].
    __shared__ __attribute__((aligned(16))) float dd[NDB][kInvCols][DT];
    // Per-wave partial sums of T.
    __shared__ float red[4][kInvCols][kInvCols + 1];

    const int nj = (p.ld + kInvCols - 1) / kInvCols;
    const int l = blockIdx.x / nj;
    const int J = blockIdx.x - l * nj;
    const int ld = p.ld;
    const int s = p.s[l];
    const int64_t o = p.o[l];
    const _Float16 *__restrict__ A = p.A;
    const int64_t lda = p.lda;
    _Float16 *__restrict__ V = p.V + p.voff[l];
    const int t = threadIdx.x;
    const int c0 = J * kInvCols;
    const int ncol = min(kInvCols, ld - c0);
    const int nrb = (ld + kInvCols - 1) / kInvCols;   // row blocks of the ld×ld block
    const int nb = (s + kInvCols - 1) / kInvCols;     // row blocks holding leaf rows

    // Rows [r0, r0+32) of this column block: zeros, or the values in vt.
    auto store_rows = [&](int r0, bool zero) {
        for (int idx = t; idx < kInvCols * ncol; idx += 256) {
            const int rr = idx % kInvCols, c = idx / kInvCols;
            const int r = r0 + rr, col = c0 + c;
            if (r >= ld)
                continue;
            const bool inside = !zero && r < s && col < s && r >= col;
            V[r + (int64_t)col * ld] = (_Float16)(inside ? vt[c][r] : 0.0f);
        }
    };

    if (c0 >= s) {
        for (int I = 0; I < nrb; ++I)
            store_rows(I * kInvCols, true);
        return;
    }
    for (int I = 0; I < J; ++I)
        store_rows(I * kInvCols, true);

    const int c = t % kInvCols;   // column of the block this thread works on
    const int g = t / kInvCols;   // row group: rows g, g+8, g+16, g+24 of a block
    const int lane = t & 63, wave = t >> 6;
    // A panel of block I: rows r0..r0+31, columns c0..r0+31 (the diagonal
    // block last), at most 32×256 values, 32 per thread: thread t takes row
    // r0 + t mod 32 of columns c0 + t/32 + 8u.  All 32 loads of a panel are
    // issued together, and the next block's panel is requested before this
    // block's arithmetic, so each panel costs one memory round trip that
    // overlaps the previous block's work.
    constexpr int kPanelPerT = kInvCols * kTrsmLeafMax / 256;
    _Float16 pa[kPanelPerT];
    auto load_panel = [&](int I) {
        const int r = I * kInvCols + c;
        const int ka = I * kInvCols + kInvCols - c0;
#pragma unroll
        for (int u = 0; u < kPanelPerT; ++u) {
            const int kk = g + 8 * u;
            const int k = c0 + kk;
            pa[u] = (kk < ka && r < s && k <= r) ? A[(o + r) + (o + k) * lda] : (_Float16)0.0f;
        }
    };
    if (J < nb)
        load_panel(J);

    // Inverses of the diagonal blocks, all at once: thread t solves
    // A_II·d = e_c for block I = J + t/32, column c = t mod 32, by forward
    // substitution (fp32, coefficients from LDS); rows past the leaf get a
    // unit diagonal, so d stays finite there (those rows are stored as zeros).
    {
        const int ndb = nb - J;
#pragma unroll
        for (int u = 0; u < kPanelPerT; ++u) {
            const int idx = t + 256 * u;
            const int bi = idx / (kInvCols * kInvCols);
            const int kk = (idx / kInvCols) % kInvCols, rr = idx % kInvCols;
            if (bi < ndb) {
                const int r = (J + bi) * kInvCols + rr, k = (J + bi) * kInvCols + kk;
                float a = 0.0f;
                if (r < s && k <= r)
                    a = (float)A[(o + r) + (o + k) * lda];
                else if (r >= s && k == r)
                    a = 1.0f;
                dd[bi][rr][kk] = a;
            }
        }
        __syncthreads();
        const int bi = t / kInvCols;
        float y[kInvCols];
        if (bi < ndb) {
#pragma unroll
            for (int rr = 0; rr < kInvCols; ++rr) {
                float acc = rr == c ? 1.0f : 0.0f;
#pragma unroll
                for (int kk = 0; kk < rr; ++kk)
                    acc = __builtin_fmaf(-dd[bi][rr][kk], y[kk], acc);
                y[rr] = acc / dd[bi][rr][rr];
            }
        }
        __syncthreads();
        if (bi < ndb) {
#pragma unroll
            for (int rr = 0; rr < kInvCols; ++rr)
                dd[bi][rr][c] = y[rr];
        }
        __syncthreads();
    }

    for (int I = J; I < nb; ++I) {
        const int r0 = I * kInvCols;
        const int ka = r0 + kInvCols - c0;
#pragma unroll
        for (int u = 0; u < kPanelPerT; ++u) {
            const int kk = g + 8 * u;
            if (kk < ka)
                as[c][c0 + kk] = (float)pa[u];
        }
        __syncthreads();
        if (I + 1 < nb)
            load_panel(I + 1);
        // T for rows of block I, into vt (those rows are not read yet).  The
        // sum over k in [c0, r0) runs on the matrix cores in fp32
        // (v_mfma_f32_32x32x2_f32), split evenly over the four waves (a
        // multiple of 8 k each); in group k0 .. k0+7, step m takes
        // k = k0 + 4·(lane div 32) + m from both operands, so each lane
        // reads one float4 of its A row (as) and one of its V column (vt).
        // The four partial 32×32 sums meet in LDS.
        {
            const int kw = (r0 - c0) / 4;
            const int kb = c0 + wave * kw;
            const int h = lane >> 5, li = lane & 31;
            floatx16 acc = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
            for (int k0 = kb; k0 < kb + kw; k0 += 8) {
                const float4 a = *reinterpret_cast<const float4 *>(&as[li][k0 + 4 * h]);
                const float4 v = *reinterpret_cast<const float4 *>(&vt[li][k0 + 4 * h]);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, v.x, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, v.y, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, v.z, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, v.w, acc, 0, 0, 0);
            }
            // Lane holds column li, rows 8·(v div 4) + 4h + v mod 4.
#pragma unroll
            for (int v = 0; v < 16; ++v)
                red[wave][8 * (v >> 2) + 4 * h + (v & 3)][li] = acc[v];
            __syncthreads();
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int i = g + 8 * q;
                const float sum = (red[0][i][c] + red[1][i][c]) + (red[2][i][c] + red[3][i][c]);
                vt[c][r0 + i] = (r0 + i == c0 + c ? 1.0f : 0.0f) - sum;
            }
        }
        __syncthreads();
        // V_IJ = D_I·T: the thread's four rows of column c, T's column read
        // as float4 from vt, D's rows from dd; written back over T once every
        // thread has read it.
        {
            const float(*D)[DT] = dd[I - J];
            float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < kInvCols; kk += 4) {
                const float4 v = *reinterpret_cast<const float4 *>(&vt[c][r0 + kk]);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 d = *reinterpret_cast<const float4 *>(&D[g + 8 * q][kk]);
                    acc[q] = __builtin_fmaf(d.x, v.x, acc[q]);
                    acc[q] = __builtin_fmaf(d.y, v.y, acc[q]);
                    acc[q] = __builtin_fmaf(d.z, v.z, acc[q]);
                    acc[q] = __builtin_fmaf(d.w, v.w, acc[q]);
                }
            }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < 4; ++q)
                vt[c][r0 + g + 8 * q] = acc[q];
        }
        __syncthreads();
        store_rows(r0, false);
    }
    for (int I = nb; I < nrb; ++I)
        store_rows(I * kInvCols, true);
}

// ---- Leaf step ---------------------------------------------------------------
//
// GEMM view: C(i, j) = Σ_k R(i, k)·V(k, j) with i over the m columns of B and
// j, k over the s leaf rows; C(i, j) is X(o+j, i).  One workgroup owns 32
// consecutive i and all j < 256, so the rows of Out it reads as S (columns k
// of its own i) are exactly the ones it overwrites, after its last read.
// The whole K range fits in LDS (R: 32×256, V: 256×256 fp16, 144 KB), so
// every load is issued up front — one global round trip — then one barrier
// and the products.  V(k, j) = 0 for k < j: a 16-wide k step whose k are all
// below a 32-row j block is not loaded (and enters the product as zero).
// Wave w owns the j blocks [32w, 32w+32) and [224-32w, 256-32w).
constexpr int LBM = 32, LBN = 256, LBK = 256;
constexpr int LKC = LBK / 8;                 // 16-byte chunks per LDS row
constexpr int LDS_R = LBM * LBK * 2;         // 16 KB
constexpr int LDS_V = LBN * LBK * 2;         // 128 KB
constexpr int R_PER_T = LBM * LKC / 256;     // 4
constexpr int V_PER_T = LBN * LKC / 256;     // 32
constexpr int XLD = LBN + 4;                 // padded fp32 row of a staged 32×256 result

// 16-byte chunk kc of row `row` in a 32-chunk row: XOR-swizzled so that the
// fragment reads of 32 consecutive rows at one kc hit distinct bank groups.
__device__ __forceinline__ int lds_chunk(int row, int kc) { return row * LKC + (kc ^ (row & 31)); }

// Buffer resource over `bytes` bytes from `base` (no stride; the offset of a
// load is checked against `bytes`).
__device__ __forceinline__ hg_trsm_i32x4 buffer_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    hg_trsm_i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;
    return r;
}

// Chunk kc (8 consecutive k) of V row j is read by the MFMA k step kc/2 of
// j block j/32, which runs when that step reaches the block: 16·(kc/2) + 16
// > 32·(j/32).
__device__ __forceinline__ bool v_chunk_used(int j, int kc) { return 8 * (kc & ~1) + 16 > (j & ~31); }

template <bool VEC>
__global__ void __launch_bounds__(256, 1) trsm_leaf_kernel(const TrsmLeafParams p)
{
    __shared__ __attribute__((aligned(16))) unsigned char smem[LDS_R + LDS_V];
    unsigned char *Rs = smem;
    unsigned char *Vs = smem + LDS_R;

    const int m0 = blockIdx.x * LBM;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int s = p.s;
    const int M = p.m;
    const int64_t o = p.o;
    const float alpha = p.alpha;
    const bool touched = p.touched != 0;
    const hg_trsm_i32x4 vrs = buffer_rsrc(p.V, (uint32_t)p.ldv * (uint32_t)p.ldv * 2u);

    // R(i, k..k+7) = fp16(alpha·B(o+k.., i) + S(o+k.., i)), zero past the
    // leaf or past the last column of B.
    auto load_r = [&](int i, int k) -> uint4 {
        half8 h;
        if (i >= M || k >= s)
            return make_uint4(0u, 0u, 0u, 0u);
        const _Float16 *bp = p.B + (o + k) + (int64_t)i * p.ldb;
        const float *sp = p.Out + (o + k) + (int64_t)i * p.ldo;
        if (VEC && k + 8 <= s) {
            const half8 b = *reinterpret_cast<const half8 *>(bp);
            if (touched) {
                const floatx4 s0 = *reinterpret_cast<const floatx4 *>(sp);
                const floatx4 s1 = *reinterpret_cast<const floatx4 *>(sp + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h[e] = (_Float16)__builtin_fmaf(alpha, (float)b[e], s0[e]);
                    h[e + 4] = (_Float16)__builtin_fmaf(alpha, (float)b[e + 4], s1[e]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    h[e] = (_Float16)(alpha * (float)b[e]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float v = 0.0f;
                if (k + e < s) {
                    v = alpha * (float)bp[e];
                    if (touched)
                        v = __builtin_fmaf(alpha, (float)bp[e], sp[e]);
                }
                h[e] = (_Float16)v;
            }
        }
        return __builtin_bit_cast(uint4, h);
    };

    // All loads first.  Thread t takes chunk column t mod 32 of rows
    // t/32 + 8u: R rows u < 4, V rows t/32 + 8·((u + rot) mod 32).  Every
    // workgroup reads the same V; the rotation makes the workgroups of one
    // XCD (consecutive workgroups go to different XCDs, so those of one XCD
    // are 8 apart) request different lines (different L2 channels) instead
    // of queueing on the same ones.
    const int lkc = t & 31;
    const int lrow = t >> 5;
    const int rot = (blockIdx.x >> 3) & (V_PER_T - 1);
    auto vrow = [&](int u) { return lrow + 8 * ((u + rot) & (V_PER_T - 1)); };
    uint4 ra[R_PER_T];
    uint4 rv[V_PER_T];
    bool vok[V_PER_T];
    if (VEC && p.sb > 0) {
        // Fused update of the deepest recursion node above this leaf:
        // S <- S − A21ᵀ·X2 for the leaf's rows, A21 = A[o+s : o+s+sb, o : o+s]
        // and X2 the lower half's solved rows (fp16, from W).  Its operands
        // are staged in LDS first (A21ᵀ in V's area, X2 in R's), the
        // inverse's loads are issued before its products so that they are in
        // flight meanwhile, and its 32×s result meets B and S in fp32 through
        // LDS: S_new = S − U (or −U on rows no update has touched yet), the
        // arithmetic of the separate beta = 1 GEMM, then R = fp16(alpha·B + S_new).
        const int sb = p.sb;
        const int k = lkc * 8;
        const int64_t ob = o + s;                  // first row of the lower half
        uint4 ru[V_PER_T];
        uint4 rx[R_PER_T];
        half8 bv[R_PER_T];
        floatx4 sv[2 * R_PER_T];
        bool rok[R_PER_T];
        const int64_t bdummy = o + (int64_t)m0 * p.ldb;
        const int64_t sdummy = o + (int64_t)m0 * p.ldo;
        const int64_t wdummy = ob + (int64_t)m0 * p.ldw;
        const int64_t adummy = ob + o * p.lda;
#pragma unroll
        for (int u = 0; u < R_PER_T; ++u) {
            const int i = m0 + lrow + 8 * u;
            rok[u] = i < M && k < s;
            bv[u] = *reinterpret_cast<const half8 *>(p.B + (rok[u] ? (o + k) + (int64_t)i * p.ldb : bdummy));
            const bool xok = i < M && k < sb;
            const uint4 x = *reinterpret_cast<const uint4 *>(p.W + (xok ? (ob + k) + (int64_t)i * p.ldw : wdummy));
            const uint32_t keep = xok ? 0xffffffffu : 0u;
            rx[u] = make_uint4(x.x & keep, x.y & keep, x.z & keep, x.w & keep);
        }
        if (touched) {
#pragma unroll
            for (int u = 0; u < R_PER_T; ++u) {
                const int i = m0 + lrow + 8 * u;
                const float *sp = p.Out + (rok[u] ? (o + k) + (int64_t)i * p.ldo : sdummy);
                sv[2 * u] = *reinterpret_cast<const floatx4 *>(sp);
                sv[2 * u + 1] = *reinterpret_cast<const floatx4 *>(sp + 4);
            }
        }
#pragma unroll
        for (int u = 0; u < V_PER_T; ++u) {
            const int j = vrow(u);
            const bool aok = j < s && k < sb;
            const uint4 a = *reinterpret_cast<const uint4 *>(p.A + (aok ? (ob + k) + (o + j) * p.lda : adummy));
            const uint32_t keep = aok ? 0xffffffffu : 0u;
            ru[u] = make_uint4(a.x & keep, a.y & keep, a.z & keep, a.w & keep);
        }
#pragma unroll
        for (int u = 0; u < R_PER_T; ++u)
            *reinterpret_cast<uint4 *>(Rs + lds_chunk(lrow + 8 * u, lkc) * 16) = rx[u];
#pragma unroll
        for (int u = 0; u < V_PER_T; ++u)
            *reinterpret_cast<uint4 *>(Vs + lds_chunk(vrow(u), lkc) * 16) = ru[u];
        __syncthreads();
#pragma unroll
        for (int u = 0; u < V_PER_T; ++u) {
            const int j = vrow(u);
            vok[u] = j < s && k < s && v_chunk_used(j, lkc);
            // unused chunks: an out-of-range offset, so no memory request
            const uint32_t voff = vok[u] ? (uint32_t)(j * p.ldv + k) * 2u : 0x80000000u;
            rv[u] = __builtin_bit_cast(uint4, hg_trsm_buffer_load_b128(vrs, (int)voff, 0, 0));
        }
        // U(i, j) = Σ_k' X2(i, k')·A21(k', j), the fragments of the leaf
        // product below with A21ᵀ in place of the inverse (every chunk of
        // both operands was written, zeros past sb and s).
        {
            const int frow = lane & 31;
            const int fkc = lane >> 5;
            const int jbs[2] = {wave, 7 - wave};
            floatx16 uacc[2];
#pragma unroll
            for (int b = 0; b < 2; ++b)
                uacc[b] = floatx16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int st = 0; st < LBK / 16; ++st) {
                const int kc = 2 * st + fkc;
                const half8 af = *reinterpret_cast<const half8 *>(Rs + lds_chunk(frow, kc) * 16);
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const half8 bf = *reinterpret_cast<const half8 *>(Vs + lds_chunk(32 * jbs[b] + frow, kc) * 16);
                    uacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf, af, uacc[b], 0, 0, 0);
                }
            }
            __syncthreads();                       // every wave is past its reads of Rs, Vs
            float *Us = reinterpret_cast<float *>(Vs);
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *reinterpret_cast<floatx4 *>(Us + frow * XLD + 32 * jbs[b] + 8 * g + 4 * fkc) =
                        floatx4{uacc[b][4 * g + 0], uacc[b][4 * g + 1], uacc[b][4 * g + 2], uacc[b][4 * g + 3]};
            __syncthreads();
#pragma unroll
            for (int u = 0; u < R_PER_T; ++u) {
                const float *ur = Us + (lrow + 8 * u) * XLD + k;
                const floatx4 u0 = *reinterpret_cast<const floatx4 *>(ur);
                const floatx4 u1 = *reinterpret_cast<const floatx4 *>(ur + 4);
                half8 h;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float uv = e < 4 ? u0[e] : u1[e - 4];
                    const float sn = touched ? __builtin_fmaf(-1.0f, uv, sv[2 * u + e / 4][e % 4]) : -uv;
                    h[e] = rok[u] ? (_Float16)__builtin_fmaf(alpha, (float)bv[u][e], sn) : (_Float16)0.0f;
                }
                ra[u] = __builtin_bit_cast(uint4, h);
            }
        }
#pragma unroll
        for (int u = 0; u < V_PER_T; ++u) {
            const uint32_t keep = vok[u] ? 0xffffffffu : 0u;
            rv[u] = make_uint4(rv[u].x & keep, rv[u].y & keep, rv[u].z & keep, rv[u].w & keep);
        }
        __syncthreads();                           // U read by every thread before V overwrites it
    } else if constexpr (VEC) {
        // Branch-free: every load is issued from a valid address (the real
        // chunk, or a chunk known to be in range) and masked afterwards, so
        // all of them are in flight together.  VEC implies s % 8 == 0: no
        // chunk is partial.
        const int k = lkc * 8;
        half8 bv[R_PER_T];
        floatx4 sv[2 * R_PER_T];
        bool rok[R_PER_T];
        const int64_t bdummy = o + (int64_t)m0 * p.ldb;
        const int64_t sdummy = o + (int64_t)m0 * p.ldo;
#pragma unroll
        for (int u = 0; u < R_PER_T; ++u) {
            const int i = m0 + lrow + 8 * u;
            rok[u] = i < M && k < s;
            bv[u] = *reinterpret_cast<const half8 *>(
                p.B + (rok[u] ? (o + k) + (int64_t)i * p.ldb : bdummy));
        }
        if (touched) {
#pragma unroll
            for (int u = 0; u < R_PER_T; ++u) {
                const int i = m0 + lrow + 8 * u;
                const float *sp = p.Out + (rok[u] ? (o + k) + (int64_t)i * p.ldo : sdummy);
                sv[2 * u] = *reinterpret_cast<const floatx4 *>(sp);
                sv[2 * u + 1] = *reinterpret_cast<const floatx4 *>(sp + 4);
            }
        }
#pragma unroll
        for (int u = 0; u < V_PER_T; ++u) {
            const int j = vrow(u);
            vok[u] = j < s && k < s && v_chunk_used(j, lkc);
            // unused chunks: an out-of-range offset, so no memory request
            const uint32_t voff = vok[u] ? (uint32_t)(j * p.ldv + k) * 2u : 0x80000000u;
            rv[u] = __builtin_bit_cast(uint4, hg_trsm_buffer_load_b128(vrs, (int)voff, 0, 0));
        }
#pragma unroll
        for (int u = 0; u < R_PER_T; ++u) {
            half8 h;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float b = alpha * (float)bv[u][e];
                const float v = touched ? __builtin_fmaf(alpha, (float)bv[u][e], sv[2 * u + e / 4][e % 4]) : b;
                h[e] = rok[u] ? (_Float16)v : (_Float16)0.0f;
            }
            ra[u] = __builtin_bit_cast(uint4, h);
        }
#pragma unroll
        for (int u = 0; u < V_PER_T; ++u) {
            const uint32_t keep = vok[u] ? 0xffffffffu : 0u;
            rv[u] = make_uint4(rv[u].x & keep, rv[u].y & keep, rv[u].z & keep, rv[u].w & keep);
        }
    } else {
#pragma unroll
        for (int u = 0; u < R_PER_T; ++u)
            ra[u] = load_r(m0 + lrow + 8 * u, lkc * 8);
#pragma unroll
        for (int u = 0; u < V_PER_T; ++u) {
            const int j = vrow(u);
            rv[u] = make_uint4(0u, 0u, 0u, 0u);
            if (j < s && lkc * 8 < s && v_chunk_used(j, lkc))
                rv[u] = *reinterpret_cast<const uint4 *>(p.V + (int64_t)j * p.ldv + lkc * 8);
        }
    }
#pragma unroll
    for (int u = 0; u < R_PER_T; ++u)
        *reinterpret_cast<uint4 *>(Rs + lds_chunk(lrow + 8 * u, lkc) * 16) = ra[u];
#pragma unroll
    for (int u = 0; u < V_PER_T; ++u) {
        const int j = vrow(u);
        if (v_chunk_used(j, lkc))
            *reinterpret_cast<uint4 *>(Vs + lds_chunk(j, lkc) * 16) = rv[u];
    }
    __syncthreads();

    // Fragments: lane l supplies row (l mod 32) of a 32-row block and the 8
    // consecutive k from 8·(l div 32) of the current 16-wide k step, for both
    // operands; the V fragment goes first, so each 32×32 result is Cᵀ.
    // Wave w owns the 32-row j blocks w and 7 - w: block jb needs the k steps
    // st >= 2·jb (V(k, j) = 0 for k < j), 18 steps per wave in all.  The
    // loop runs every step with no branch, so the fragment reads can be
    // issued ahead of the products; a V chunk that was not loaded (k below
    // the block, or past the leaf) enters as zero.
    const int frow = lane & 31;
    const int fkc = lane >> 5;
    const int jbs[2] = {wave, 7 - wave};
    floatx16 acc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
        acc[b] = floatx16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int st = 0; st < LBK / 16; ++st) {
        const int kc = 2 * st + fkc;
        const half8 af = *reinterpret_cast<const half8 *>(Rs + lds_chunk(frow, kc) * 16);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int jb = jbs[b];
            const uint4 raw = *reinterpret_cast<const uint4 *>(Vs + lds_chunk(32 * jb + frow, kc) * 16);
            const uint32_t keep = st >= 2 * jb && 8 * kc < s ? 0xffffffffu : 0u;
            const half8 bf = __builtin_bit_cast(
                half8, make_uint4(raw.x & keep, raw.y & keep, raw.z & keep, raw.w & keep));
            acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf, af, acc[b], 0, 0, 0);
        }
    }

    // Epilogue, staged through LDS (the inverse's area, free once every wave
    // is past its last MFMA): block b of this wave holds C(i, j..j+3) for
    // i = m0 + (lane mod 32) and, in register group g,
    // j = 32·jb + 8g + 4·(lane div 32) for its row block jb.  Written to LDS
    // as rows i of 256 fp32, then each store instruction writes one column i of X: 64
    // lanes × 4 rows = the column's 1 KiB of fp32 and 512 B of fp16, whole
    // cache lines (scattered 16-byte pieces tripled the written bytes).
    float *Xs = reinterpret_cast<float *>(Vs);
    __syncthreads();
    {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int j = 32 * jbs[b] + 8 * g + 4 * fkc;
                *reinterpret_cast<floatx4 *>(Xs + frow * XLD + j) =
                    floatx4{acc[b][4 * g + 0], acc[b][4 * g + 1], acc[b][4 * g + 2], acc[b][4 * g + 3]};
            }
    }
    __syncthreads();
    const int j = 4 * lane;                      // rows j..j+3 of each column
#pragma unroll
    for (int c = 0; c < LBM / 4; ++c) {
        const int il = wave + 4 * c;
        const int i = m0 + il;
        if (i >= M || j >= s)
            continue;
        const floatx4 v = *reinterpret_cast<const floatx4 *>(Xs + il * XLD + j);
        float *orow = p.Out + o + (int64_t)i * p.ldo;
        _Float16 *wrow = p.W + o + (int64_t)i * p.ldw;
        if (VEC && j + 4 <= s) {
            *reinterpret_cast<floatx4 *>(orow + j) = v;
            *reinterpret_cast<halfx4 *>(wrow + j) =
                halfx4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (j + e < s) {
                    orow[j + e] = v[e];
                    wrow[j + e] = (_Float16)v[e];
                }
        }
    }
}

}  // namespace

hipError_t launch_trsm_inv(const TrsmInvParams &p, hipStream_t stream)
{
    if (p.nleaf <= 0)
        return hipSuccess;
    if (p.nleaf > kTrsmInvBatch || p.ld <= 0 || p.ld > kTrsmLeafMax || p.ld % 8 != 0)
        return hipErrorInvalidValue;
    for (int l = 0; l < p.nleaf; ++l)
        if (p.s[l] <= 0 || p.s[l] > p.ld)
            return hipErrorInvalidValue;
    const int nj = (p.ld + kInvCols - 1) / kInvCols;
    hipLaunchKernelGGL(trsm_inv_kernel, dim3((unsigned)(p.nleaf * nj)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_trsm_leaf(const TrsmLeafParams &p, bool vec, hipStream_t stream)
{
    if (p.m <= 0)
        return hipSuccess;
    if (p.s <= 0 || p.s > kTrsmLeafMax || p.s > p.ldv || p.ldv % 8 != 0)
        return hipErrorInvalidValue;
    if (p.sb < 0 || p.sb > kTrsmLeafMax ||
        (p.sb > 0 && (!vec || p.A == nullptr || reinterpret_cast<uintptr_t>(p.A) % 16 != 0 ||
                      p.lda % 8 != 0 || p.ldw % 8 != 0 || p.sb % 8 != 0)))
        return hipErrorInvalidValue;
    const unsigned grid = (unsigned)((p.m + LBM - 1) / LBM);
    if (vec)
        hipLaunchKernelGGL(trsm_leaf_kernel<true>, dim3(grid), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(trsm_leaf_kernel<false>, dim3(grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace hg
