// hg_kernels.hip — gfx950 (CDNA4) kernels for the half-precision GEMM and the
// triangle-masked TRMM leaf.
//
// Computation: C = alpha·A·B + beta·C with A (M×K) row-major, B (K×N)
// column-major, C (M×N) row-major, fp16 operands and fp32 accumulation — the
// HGEMM of "Nvidia Tensor Core-MMA PTX编程入门" §4, with the masked tiles and
// guarded stores of the tiled matmul in "GPU架构与CUDA" (共享内存与分块) and
// the fp16-in/fp32-accumulate contract of its 混合精度核函数 section.
//
// Both operands are K-contiguous, so every 16-byte global load carries eight
// consecutive k of one row of A or one column of B, and every MFMA operand
// fragment is one 16-byte LDS read (no transposes anywhere).
//
// Structure of one workgroup (4 waves, 2×2):
//   * owns a BM×BN macro-tile of C; waves own (BM/2)×(BN/2) sub-tiles made of
//     32×32 blocks, each accumulated by v_mfma_f32_32x32x16_f16;
//   * K is walked in BK = 64 slices staged in LDS, double-buffered: the
//     global loads of slice t+1 are in flight while slice t is multiplied,
//     one barrier per slice;
//   * LDS rows are 128 bytes (64 halves); the 16-byte chunk index is XOR-
//     swizzled with the row so that the 16-byte fragment reads of 8
//     consecutive rows fall in distinct banks (the LDS counterpart of the
//     padded (32, 33) shared array in "异构计算中高性能TRMM与TRSM的递归算法实现"
//     §3.2);
//   * the MFMA is issued with the B fragment as its first operand, so the
//     32×32 result block is Cᵀ: every lane then holds four consecutive
//     columns of one C row and the epilogue stores 16 bytes (fp32) or 8 bytes
//     (fp16) per lane;
//   * interior tiles take unmasked loads and stores; edge tiles and the K
//     tail zero-fill out-of-range operand elements and guard every store.
//
// Workgroup→tile order: consecutive workgroup ids are spread round-robin over
// the 8 XCDs (each with its own L2), so ids are first regrouped per XCD, then
// each XCD's range is walked in bands of 4 tile rows, column by column, so the
// tiles resident on one XCD at a time share A row panels and B column panels.
#include "hg_internal.h"

namespace hg {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// v_mfma_f32_32x32x16 on 16-byte fragments of fp16 or bf16 values.
template <bool BF16>
__device__ __forceinline__ floatx16 mfma_32x32x16(const half8 &a, const half8 &b, const floatx16 &c)
{
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int THREADS = WM * WN * 64;
    static constexpr int WTM = BM / WM;      // wave sub-tile rows
    static constexpr int WTN = BN / WN;      // wave sub-tile columns
    static constexpr int TM = WTM / 32;      // 32×32 MFMA blocks per wave, M
    static constexpr int TN = WTN / 32;      // 32×32 MFMA blocks per wave, N
    static constexpr int KC = BK / 8;        // 16-byte chunks per LDS row
    static constexpr int RSTEP = THREADS / KC;       // rows covered per load round
    static constexpr int A_PER_T = BM * KC / THREADS;
    static constexpr int B_PER_T = BN * KC / THREADS;
    static constexpr int LDS_A = BM * BK * 2;        // bytes per stage
    static constexpr int LDS_B = BN * BK * 2;
    static constexpr int LDS_STAGE = LDS_A + LDS_B;
    static_assert(BK == 64, "LDS swizzle assumes 8 chunks per row");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be 32-aligned");
    static_assert(A_PER_T * THREADS == BM * KC && B_PER_T * THREADS == BN * KC, "");
    static_assert(RSTEP % 8 == 0, "row step must keep the swizzle phase");
};

using CfgBig = Cfg<256, 256, 64, 2, 2>;
using CfgMid = Cfg<128, 128, 64, 2, 2>;
using CfgSmall = Cfg<64, 64, 64, 2, 2>;

__device__ __forceinline__ int lds_chunk(int row, int kc) { return row * 8 + (kc ^ (row & 7)); }

__device__ __forceinline__ uint4 ld16(const _Float16 *p)
{
    return *reinterpret_cast<const uint4 *>(p);
}

// Elements k..k+7 of one operand row (rowp points at element 0 of the row).
// Elements with index >= K, and for a TRI operand those with index < diag,
// read as +0; an out-of-range row (row_ok false) reads as all zeros.  Nothing
// outside the valid region is dereferenced.
template <bool VEC, bool TRI>
__device__ __forceinline__ uint4 load_chunk_masked(const _Float16 *rowp, int k, int K, bool row_ok,
                                                   int diag)
{
    uint4 z = make_uint4(0u, 0u, 0u, 0u);
    if (!row_ok || k >= K || (TRI && k + 8 <= diag))
        return z;
    if (VEC && k + 8 <= K && (!TRI || k >= diag))
        return ld16(rowp + k);
    const uint16_t *q = reinterpret_cast<const uint16_t *>(rowp);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int kk = k + e;
        const bool ok = kk < K && (!TRI || kk >= diag);
        const uint32_t h = ok ? q[kk] : 0u;
        w[e >> 1] |= h << (16 * (e & 1));
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Workgroup id → (batch, tile row, tile column); see the header comment.
__device__ __forceinline__ void map_tile(int wg, int total, int tiles_m, int tiles_n, int &batch,
                                         int &tm, int &tn)
{
    const int per = total >> 3, rem = total & 7;
    const int x = wg & 7;
    const int q = x * per + min(x, rem) + (wg >> 3);
    const int per_batch = tiles_m * tiles_n;
    batch = q / per_batch;
    const int l = q - batch * per_batch;
    constexpr int G = 4;
    const int band = l / (G * tiles_n);
    const int first = band * G;
    const int gsz = min(tiles_m - first, G);
    const int r = l - band * G * tiles_n;
    tm = first + r % gsz;
    tn = r / gsz;
}

template <class CF, bool OUT_F16, bool BETA, bool TRI, bool VEC, bool IN_BF16>
__global__ void __launch_bounds__(CF::THREADS, 1)
hgemm_kernel(const GemmParams p, int tiles_m, int tiles_n, int total, int cvec)
{
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * CF::LDS_STAGE];

    int batch, tm, tn;
    map_tile(blockIdx.x, total, tiles_m, tiles_n, batch, tm, tn);
    const int M = p.M;
    const int N = p.e[batch].N;
    const int K = p.e[batch].K;
    const int m0 = tm * CF::BM;
    const int n0 = tn * CF::BN;
    if (m0 >= M || n0 >= N)
        return;  // whole workgroup: a ragged batch entry narrower than the grid
    const _Float16 *__restrict__ A = p.A + p.e[batch].a_off;
    const _Float16 *__restrict__ B = p.B + p.e[batch].b_off;
    const int64_t lda = p.lda, ldb = p.ldb;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int wm = wave / CF::WN;
    const int wn = wave % CF::WN;

    // Global→register staging: thread t loads chunk column lkc of rows
    // lrow + i·RSTEP (8 consecutive threads cover one 128-byte row segment).
    const int lkc = t % CF::KC;
    const int lrow = t / CF::KC;
    const bool full_m = m0 + CF::BM <= M;
    const bool full_n = n0 + CF::BN <= N;

    uint4 ra[CF::A_PER_T];
    uint4 rb[CF::B_PER_T];

    auto gload = [&](int kt) {
        const int kb = kt * CF::BK + lkc * 8;
        const bool kfull = (kt + 1) * CF::BK <= K;
        if (VEC && full_m && kfull) {
#pragma unroll
            for (int i = 0; i < CF::A_PER_T; ++i)
                ra[i] = ld16(A + (int64_t)(m0 + lrow + i * CF::RSTEP) * lda + kb);
        } else {
#pragma unroll
            for (int i = 0; i < CF::A_PER_T; ++i) {
                const int row = m0 + lrow + i * CF::RSTEP;
                ra[i] = load_chunk_masked<VEC, false>(A + (int64_t)row * lda, kb, K, row < M, 0);
            }
        }
        const bool tri_stage = TRI && (kt * CF::BK < n0 + CF::BN);
        if (VEC && full_n && kfull && !tri_stage) {
#pragma unroll
            for (int i = 0; i < CF::B_PER_T; ++i)
                rb[i] = ld16(B + (int64_t)(n0 + lrow + i * CF::RSTEP) * ldb + kb);
        } else {
#pragma unroll
            for (int i = 0; i < CF::B_PER_T; ++i) {
                const int row = n0 + lrow + i * CF::RSTEP;
                rb[i] = load_chunk_masked<VEC, TRI>(B + (int64_t)row * ldb, kb, K, row < N, row);
            }
        }
    };

    auto sstore = [&](int buf) {
        unsigned char *As = smem + buf * CF::LDS_STAGE;
        unsigned char *Bs = As + CF::LDS_A;
#pragma unroll
        for (int i = 0; i < CF::A_PER_T; ++i)
            *reinterpret_cast<uint4 *>(As + lds_chunk(lrow + i * CF::RSTEP, lkc) * 16) = ra[i];
#pragma unroll
        for (int i = 0; i < CF::B_PER_T; ++i)
            *reinterpret_cast<uint4 *>(Bs + lds_chunk(lrow + i * CF::RSTEP, lkc) * 16) = rb[i];
    };

    floatx16 acc[CF::TM][CF::TN];
#pragma unroll
    for (int i = 0; i < CF::TM; ++i)
#pragma unroll
        for (int j = 0; j < CF::TN; ++j)
            acc[i][j] = floatx16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

    // MFMA operand fragments: lane l supplies row (l mod 32) of its 32-row
    // block and the 8 consecutive k starting at 8·(l div 32) of the current
    // 16-wide k step.  The same (lane, element) → k assignment is used for
    // both operands, so the contraction pairs matching k.
    const int frow = lane & 31;
    const int fkc = lane >> 5;
    auto compute = [&](int buf) {
        const unsigned char *As = smem + buf * CF::LDS_STAGE;
        const unsigned char *Bs = As + CF::LDS_A;
#pragma unroll
        for (int s = 0; s < CF::BK / 16; ++s) {
            half8 af[CF::TM], bf[CF::TN];
            const int kc = 2 * s + fkc;
#pragma unroll
            for (int i = 0; i < CF::TM; ++i) {
                const int row = wm * CF::WTM + i * 32 + frow;
                af[i] = *reinterpret_cast<const half8 *>(As + lds_chunk(row, kc) * 16);
            }
#pragma unroll
            for (int j = 0; j < CF::TN; ++j) {
                const int row = wn * CF::WTN + j * 32 + frow;
                bf[j] = *reinterpret_cast<const half8 *>(Bs + lds_chunk(row, kc) * 16);
            }
#pragma unroll
            for (int i = 0; i < CF::TM; ++i)
#pragma unroll
                for (int j = 0; j < CF::TN; ++j)
                    acc[i][j] = mfma_32x32x16<IN_BF16>(bf[j], af[i], acc[i][j]);
        }
    };

    // TRI operand: columns j < k only, so k slices wholly before the tile's
    // first column contribute nothing and are skipped.
    const int kt0 = TRI ? n0 / CF::BK : 0;
    const int kt1 = (K + CF::BK - 1) / CF::BK;

    gload(kt0);
    sstore(0);
    __syncthreads();
    for (int kt = kt0; kt < kt1; ++kt) {
        const int buf = (kt - kt0) & 1;
        const bool more = kt + 1 < kt1;
        if (more)
            gload(kt + 1);
        compute(buf);
        if (more)
            sstore(buf ^ 1);
        __syncthreads();
    }

    // Epilogue.  Result block (i, j) of this wave is Cᵀ for rows
    // m0 + wm·WTM + 32i + (lane mod 32) and, for register group g (4 values),
    // columns n0 + wn·WTN + 32j + 8g + 4·(lane div 32) + 0..3.
    const float alpha = p.alpha;
    const float beta = p.beta;
    const int64_t ldc = p.ldc;
    const bool full = full_m && full_n;
    const bool epi = p.bias != nullptr || p.act != 0;
    // 16-bit C has the input's type (fp16 or bf16).
    typedef typename std::conditional<IN_BF16, __bf16, _Float16>::type e16;
    typedef typename std::conditional<IN_BF16, bf16x4, halfx4>::type vec16;
#pragma unroll
    for (int i = 0; i < CF::TM; ++i) {
        const int row = m0 + wm * CF::WTM + i * 32 + frow;
#pragma unroll
        for (int j = 0; j < CF::TN; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = n0 + wn * CF::WTN + j * 32 + 8 * g + 4 * fkc;
                floatx4 v = {acc[i][j][4 * g + 0], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                             acc[i][j][4 * g + 3]};
                const int64_t off = p.e[batch].c_off + (int64_t)row * ldc + col;
                if (full && cvec) {
                    if (OUT_F16) {
                        vec16 *cp = reinterpret_cast<vec16 *>(static_cast<e16 *>(p.C) + off);
                        floatx4 r;
                        if (BETA) {
                            const vec16 c = *cp;
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                r[e] = __builtin_fmaf(alpha, v[e], beta * (float)c[e]);
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                r[e] = alpha * v[e];
                        }
                        if (epi) {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                r[e] = epi_apply(r[e], p.bias ? p.bias[col + e] : -0.0f, p.act);
                        }
                        vec16 h;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            h[e] = (e16)r[e];
                        *cp = h;
                    } else {
                        floatx4 *cp = reinterpret_cast<floatx4 *>(static_cast<float *>(p.C) + off);
                        floatx4 r;
                        if (BETA) {
                            const floatx4 c = *cp;
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                r[e] = __builtin_fmaf(alpha, v[e], beta * c[e]);
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                r[e] = alpha * v[e];
                        }
                        if (epi) {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                r[e] = epi_apply(r[e], p.bias ? p.bias[col + e] : -0.0f, p.act);
                        }
                        *cp = r;
                    }
                } else if (row < M) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (col + e < N) {
                            const float b = epi && p.bias ? p.bias[col + e] : -0.0f;
                            if (OUT_F16) {
                                e16 *cp = static_cast<e16 *>(p.C) + off + e;
                                float r = BETA ? __builtin_fmaf(alpha, v[e], beta * (float)*cp)
                                               : alpha * v[e];
                                if (epi)
                                    r = epi_apply(r, b, p.act);
                                *cp = (e16)r;
                            } else {
                                float *cp = static_cast<float *>(p.C) + off + e;
                                float r = BETA ? __builtin_fmaf(alpha, v[e], beta * *cp)
                                               : alpha * v[e];
                                if (epi)
                                    r = epi_apply(r, b, p.act);
                                *cp = r;
                            }
                        }
                    }
                }
            }
        }
    }
}

// C = beta·C over the M×N window; beta == 0 writes zeros without reading C.
template <bool OUT_F16, bool BF16>
__global__ void __launch_bounds__(256) scale_kernel(void *C, int64_t ldc, int64_t M, int64_t N,
                                                    float beta, const float *bias, int act)
{
    typedef typename std::conditional<BF16, __bf16, _Float16>::type e16;
    const int64_t total = M * N;
    const bool epi = bias != nullptr || act != 0;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = idx / N, j = idx - i * N;
        if (OUT_F16) {
            e16 *cp = static_cast<e16 *>(C) + i * ldc + j;
            float t = beta == 0.0f ? 0.0f : beta * (float)*cp;
            if (epi)
                t = epi_apply(t, bias ? bias[j] : -0.0f, act);
            *cp = (e16)t;
        } else {
            float *cp = static_cast<float *>(C) + i * ldc + j;
            float t = beta == 0.0f ? 0.0f : beta * *cp;
            if (epi)
                t = epi_apply(t, bias ? bias[j] : -0.0f, act);
            *cp = t;
        }
    }
}

template <class CF, bool OUT_F16, bool BETA, bool TRI, bool VEC, bool IN_BF16 = false>
hipError_t launch_cfg(const GemmParams &p, hipStream_t stream)
{
    int maxN = 0;
    for (int b = 0; b < p.nbatch; ++b)
        maxN = p.e[b].N > maxN ? p.e[b].N : maxN;
    const int tiles_m = (p.M + CF::BM - 1) / CF::BM;
    const int tiles_n = (maxN + CF::BN - 1) / CF::BN;
    const int64_t total64 = (int64_t)tiles_m * tiles_n * p.nbatch;
    if (total64 <= 0)
        return hipSuccess;
    if (total64 > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    // Vector C access needs every 4-element group 16-byte (fp32) or 8-byte
    // (fp16) aligned: aligned base, ldc and offsets multiples of 4.
    const uintptr_t align = OUT_F16 ? 8 : 16;
    int cvec = (reinterpret_cast<uintptr_t>(p.C) % align == 0) && (p.ldc % 4 == 0);
    for (int b = 0; b < p.nbatch; ++b)
        cvec = cvec && (p.e[b].c_off % 4 == 0);
    hipLaunchKernelGGL((hgemm_kernel<CF, OUT_F16, BETA, TRI, VEC, IN_BF16>), dim3((unsigned)total64),
                       dim3(CF::THREADS), 0, stream, p, tiles_m, tiles_n, (int)total64, cvec);
    return hipGetLastError();
}

template <class CF>
hipError_t launch_tile(const GemmParams &p, const LaunchOpts &o, hipStream_t s)
{
    if (o.tri) {
        // TRMM leaves: fp32 output written once (beta = 0).
        if (o.out_f16 || o.beta_read)
            return hipErrorInvalidValue;
        return o.vec ? launch_cfg<CF, false, false, true, true>(p, s)
                     : launch_cfg<CF, false, false, true, false>(p, s);
    }
    if (o.in_bf16) {
        if (o.out_f16)
            return o.beta_read ? (o.vec ? launch_cfg<CF, true, true, false, true, true>(p, s)
                                        : launch_cfg<CF, true, true, false, false, true>(p, s))
                               : (o.vec ? launch_cfg<CF, true, false, false, true, true>(p, s)
                                        : launch_cfg<CF, true, false, false, false, true>(p, s));
        return o.beta_read ? (o.vec ? launch_cfg<CF, false, true, false, true, true>(p, s)
                                    : launch_cfg<CF, false, true, false, false, true>(p, s))
                           : (o.vec ? launch_cfg<CF, false, false, false, true, true>(p, s)
                                    : launch_cfg<CF, false, false, false, false, true>(p, s));
    }
    if (o.out_f16) {
        if (o.beta_read)
            return o.vec ? launch_cfg<CF, true, true, false, true>(p, s)
                         : launch_cfg<CF, true, true, false, false>(p, s);
        return o.vec ? launch_cfg<CF, true, false, false, true>(p, s)
                     : launch_cfg<CF, true, false, false, false>(p, s);
    }
    if (o.beta_read)
        return o.vec ? launch_cfg<CF, false, true, false, true>(p, s)
                     : launch_cfg<CF, false, true, false, false>(p, s);
    return o.vec ? launch_cfg<CF, false, false, false, true>(p, s)
                 : launch_cfg<CF, false, false, false, false>(p, s);
}

}  // namespace

Tile choose_tile(int64_t M, int64_t N, int64_t K)
{
    (void)K;
    // Prefer the largest tile that still gives at least one workgroup per CU
    // (256 CUs); small problems drop to smaller tiles for occupancy.
    const int64_t big = ((M + 255) / 256) * ((N + 255) / 256);
    if (big >= 256)
        return Tile::Big;
    const int64_t mid = ((M + 127) / 128) * ((N + 127) / 128);
    if (mid >= 128)
        return Tile::Mid;
    return Tile::Small;
}

hipError_t launch_gemm(const GemmParams &p, const LaunchOpts &o, hipStream_t stream)
{
    switch (o.tile) {
    case Tile::Big:
        if (fast_path_ok(p, o))
            return launch_gemm_fast(p, o, stream);
        return launch_tile<CfgBig>(p, o, stream);
    case Tile::Mid:
        if (ring_path_ok(p, o))
            return launch_gemm_ring(p, o, stream);
        return launch_tile<CfgMid>(p, o, stream);
    default:
        if (ring_path_ok(p, o))
            return launch_gemm_ring(p, o, stream);
        return launch_tile<CfgSmall>(p, o, stream);
    }
}

hipError_t launch_scale(void *C, int64_t ldc, int64_t M, int64_t N, float beta, bool out_f16,
                        hipStream_t stream, const float *bias, int act, bool bf16)
{
    const int64_t total = M * N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    if (blocks < 1)
        return hipSuccess;
    if (out_f16 && bf16)
        hipLaunchKernelGGL((scale_kernel<true, true>), dim3((unsigned)blocks), dim3(256), 0, stream, C,
                           ldc, M, N, beta, bias, act);
    else if (out_f16)
        hipLaunchKernelGGL((scale_kernel<true, false>), dim3((unsigned)blocks), dim3(256), 0, stream, C,
                           ldc, M, N, beta, bias, act);
    else
        hipLaunchKernelGGL((scale_kernel<false, false>), dim3((unsigned)blocks), dim3(256), 0, stream, C,
                           ldc, M, N, beta, bias, act);
    return hipGetLastError();
}

}  // namespace hg
