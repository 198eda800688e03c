// hg_xform.hip — the index maps that turn every TRMM variant of
// "异构计算中高性能TRMM与TRSM的递归算法实现" (§2.1 shows the lower and the upper
// blocking; §5.1 calls the lower, non-transposed product) into the lower
// transposed one the recursive driver runs.
//
// With P the reversal permutation ((P·X)(r, ·) = X(n-1-r, ·)), U upper and
// A lower triangular:
//   upper, non-transposed:  U·B = (Uᵀ)ᵀ·B                L = Uᵀ
//   upper, transposed:      P·(Uᵀ·B) = (P·U·P)ᵀ·(P·B)     L = P·U·P
//   lower, non-transposed:  P·(A·B) = (P·Aᵀ·P)ᵀ·(P·B)     L = P·Aᵀ·P
// and each L is lower triangular, so the driver runs Lᵀ·B on it, with B and
// Out row-reversed in the last two cases (lower, transposed needs no map).
// These are memory-bound copies (the TRMM itself is the compute).
#include "hg_internal.h"

#include <type_traits>

namespace hg {
namespace {

constexpr int XT = 64;   // tile edge

// L(r, c) for r >= c tiles only (the driver never reads L's strict upper
// triangle; the diagonal tiles' upper parts get whatever the map yields):
//   MODE 1: A(c, r)            transpose
//   MODE 2: A(n-1-r, n-1-c)    reverse both indices
//   MODE 3: A(n-1-c, n-1-r)    transpose and reverse
//   MODE 4: A(c, r) on the r <= c tiles instead (L upper triangular)
// One workgroup per 64×64 tile of L's lower triangle; the transposing modes
// stage the tile in LDS so that reads and writes both run along columns.
template <int MODE>
__global__ void __launch_bounds__(256) tri_xform_kernel(const _Float16 *__restrict__ A, int64_t lda,
                                                        _Float16 *__restrict__ L, int64_t ldl, int n)
{
    __shared__ _Float16 tile[XT][XT + 2];
    // blockIdx.x → (tile row tr >= tile column tc), row-major over the triangle
    const int b = blockIdx.x;
    int tr = (int)((__builtin_sqrtf(8.0f * (float)b + 1.0f) - 1.0f) * 0.5f);
    while ((tr + 1) * (tr + 2) / 2 <= b)
        ++tr;
    while (tr * (tr + 1) / 2 > b)
        --tr;
    const int tc = b - tr * (tr + 1) / 2;
    const int r0 = (MODE == 4 ? tc : tr) * XT, c0 = (MODE == 4 ? tr : tc) * XT;
    const int t = threadIdx.x;
    const int i = t % XT, g = t / XT;   // i: position along a column, g: column group
    if constexpr (MODE == 2) {
#pragma unroll 4
        for (int q = 0; q < XT / 4; ++q) {
            const int r = r0 + i, c = c0 + g + 4 * q;
            if (r < n && c < n)
                L[r + (int64_t)c * ldl] = A[(n - 1 - r) + (int64_t)(n - 1 - c) * lda];
        }
    } else {
        // Source columns are L's rows: load A's tile column by column.
#pragma unroll 4
        for (int q = 0; q < XT / 4; ++q) {
            const int cl = c0 + i;            // L column ...
            const int rl = r0 + g + 4 * q;    // ... and row of this element
            if (cl < n && rl < n) {
                const int64_t src = MODE == 1 || MODE == 4 ? cl + (int64_t)rl * lda
                                                           : (n - 1 - cl) + (int64_t)(n - 1 - rl) * lda;
                tile[i][g + 4 * q] = A[src];
            }
        }
        __syncthreads();
#pragma unroll 4
        for (int q = 0; q < XT / 4; ++q) {
            const int rl = r0 + i, cl = c0 + g + 4 * q;
            if (rl < n && cl < n)
                L[rl + (int64_t)cl * ldl] = tile[g + 4 * q][i];
        }
    }
}

typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// The same maps with 16-byte accesses, for n a multiple of 64, A and L
// 16-byte aligned and lda, ldl multiples of 8: each wave moves one 64×64
// tile of the triangle (the tile set of tri_xform_kernel).  Lane (rb, cb) =
// (lane / 8, lane % 8):
//   MODE 2 copies columns 8rb..8rb+7 of the L tile, rows 8cb..8cb+7 of each:
//          one 16-byte chunk of A's mirrored column, its 8 elements reversed;
//   MODES 1, 3, 4 load the 8×8 block of L rows 8rb.., columns 8cb.. as 8
//          chunks (L row y, columns x..x+7: A column y, rows x..x+7 for the
//          plain transposes; A column n-1-y, rows n-8-x..n-1-x reversed for
//          MODE 3), transpose it in registers and store 8 L column chunks.
// The 8 lanes of one rb (loads) or one cb (stores) cover a whole 128-byte
// line of one column.
template <int MODE>
__global__ void __launch_bounds__(256) tri_xform64_kernel(const _Float16 *__restrict__ A, int64_t lda,
                                                          _Float16 *__restrict__ L, int64_t ldl, int n,
                                                          int ntiles)
{
    const int b = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (b >= ntiles)
        return;
    int tr = (int)((__builtin_sqrtf(8.0f * (float)b + 1.0f) - 1.0f) * 0.5f);
    while ((tr + 1) * (tr + 2) / 2 <= b)
        ++tr;
    while (tr * (tr + 1) / 2 > b)
        --tr;
    const int tc = b - tr * (tr + 1) / 2;
    const int64_t R0 = (int64_t)(MODE == 4 ? tc : tr) * XT, C0 = (int64_t)(MODE == 4 ? tr : tc) * XT;
    const int lane = threadIdx.x & 63, rb = lane >> 3, cb = lane & 7;
    if constexpr (MODE == 2) {
        const int64_t r = R0 + 8 * cb;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int64_t c = C0 + 8 * rb + k;
            const half8v v = *reinterpret_cast<const half8v *>(A + (n - 1 - c) * lda + (n - 8 - r));
            *reinterpret_cast<half8v *>(L + c * ldl + r) = __builtin_shufflevector(v, v, 7, 6, 5, 4, 3, 2, 1, 0);
        }
    } else {
        const int64_t y0 = R0 + 8 * rb, x = C0 + 8 * cb;
        u32x4v in[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int64_t y = y0 + k;
            if constexpr (MODE == 3) {
                const half8v v = *reinterpret_cast<const half8v *>(A + (n - 1 - y) * lda + (n - 8 - x));
                in[k] = __builtin_bit_cast(u32x4v, __builtin_shufflevector(v, v, 7, 6, 5, 4, 3, 2, 1, 0));
            } else {
                in[k] = *reinterpret_cast<const u32x4v *>(A + y * lda + x);
            }
        }
        // in[e] half k2 = L(y0 + e, x + k2); L column x + k2, rows y0..y0+7:
        // dword d packs rows 2d (low half) and 2d + 1.
#pragma unroll
        for (int k2 = 0; k2 < 8; ++k2) {
            u32x4v o;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t lo = in[2 * d][k2 >> 1], hi = in[2 * d + 1][k2 >> 1];
                o[d] = (k2 & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
            }
            *reinterpret_cast<u32x4v *>(L + (x + k2) * ldl + y0) = o;
        }
    }
}

// D = Sᵀ for row-major fp16 matrices: S is rows×cols (S[r·lds + c]), D is
// cols×rows (D[c·ldd + r]).  64×64 tiles through LDS so that both the reads
// (along S's rows) and the writes (along D's rows) are contiguous.  With
// `vec` (16-byte aligned S and D, lds and ldd multiples of 8) full tiles move
// 16 bytes per lane each way; edge tiles and the other cases go element by
// element.
__global__ void __launch_bounds__(256) transpose_kernel(const _Float16 *__restrict__ S, int64_t lds,
                                                        _Float16 *__restrict__ D, int64_t ldd, int rows,
                                                        int cols, int tiles_c, int vec)
{
    __shared__ __attribute__((aligned(16))) _Float16 tile[XT][XT + 8];
    const int tr = blockIdx.x / tiles_c, tc = blockIdx.x - (blockIdx.x / tiles_c) * tiles_c;
    const int r0 = tr * XT, c0 = tc * XT;
    const int t = threadIdx.x;
    if (vec && r0 + XT <= rows && c0 + XT <= cols) {
        // Thread t: 16-byte chunk t mod 8 of tile rows t/8 and t/8 + 32.
        const int ch = t % 8, rr = t / 8;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int row = rr + 32 * u;
            *reinterpret_cast<half8v *>(&tile[row][8 * ch]) =
                *reinterpret_cast<const half8v *>(S + (int64_t)(r0 + row) * lds + c0 + 8 * ch);
        }
        __syncthreads();
        // D row c0 + cc holds S's column: chunk ch gathers tile rows 8ch..8ch+7.
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int cc = rr + 32 * u;
            half8v v;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e] = tile[8 * ch + e][cc];
            *reinterpret_cast<half8v *>(D + (int64_t)(c0 + cc) * ldd + r0 + 8 * ch) = v;
        }
        return;
    }
    const int i = t % XT, g = t / XT;
#pragma unroll 4
    for (int q = 0; q < XT / 4; ++q) {
        const int r = r0 + g + 4 * q, c = c0 + i;       // read along a row of S
        if (r < rows && c < cols)
            tile[g + 4 * q][i] = S[(int64_t)r * lds + c];
    }
    __syncthreads();
#pragma unroll 4
    for (int q = 0; q < XT / 4; ++q) {
        const int c = c0 + g + 4 * q, r = r0 + i;       // write along a row of D
        if (r < rows && c < cols)
            D[(int64_t)c * ldd + r] = tile[i][g + 4 * q];
    }
}

// Bp(r, j) = B(n-1-r, j), column-major, fp16.  With `vec` (n, ldb, ldp
// multiples of 8, 16-byte aligned B and Bp) each thread moves 8 rows: one
// 16-byte load, the halves reversed in registers, one 16-byte store.
__global__ void __launch_bounds__(256) row_reverse_copy_kernel(const _Float16 *__restrict__ B, int64_t ldb,
                                                               _Float16 *__restrict__ Bp, int64_t ldp,
                                                               int64_t n, int64_t m, int vec)
{
    if (vec) {
        const int64_t n8 = n / 8;
        const int64_t total = n8 * m;
        for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
             idx += (int64_t)gridDim.x * blockDim.x) {
            const int64_t j = idx / n8, q = idx - j * n8;
            const half8v v = *reinterpret_cast<const half8v *>(B + j * ldb + (n - 8 - 8 * q));
            *reinterpret_cast<half8v *>(Bp + j * ldp + 8 * q) =
                __builtin_shufflevector(v, v, 7, 6, 5, 4, 3, 2, 1, 0);
        }
        return;
    }
    const int64_t total = n * m;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t j = idx / n, r = idx - j * n;
        Bp[r + j * ldp] = B[(n - 1 - r) + j * ldb];
    }
}

// Out(r, j) <-> Out(n-1-r, j) for r < n/2, in place, fp32.
__global__ void __launch_bounds__(256) row_reverse_inplace_kernel(float *__restrict__ Out, int64_t ldo,
                                                                  int64_t n, int64_t m)
{
    const int64_t h = n / 2;
    const int64_t total = h * m;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t j = idx / h, r = idx - j * h;
        float *col = Out + j * ldo;
        const float a = col[r], b = col[n - 1 - r];
        col[r] = b;
        col[n - 1 - r] = a;
    }
}

// B(r, j) = fp16(X(r, j)) (round to nearest even), column-major n×m.
// Each thread converts 8 consecutive rows of one column per step; blockIdx.y
// strides over the columns.  VEC: X and B columns start 16-byte aligned, so
// whole groups of 8 move as two float4 loads and one 16-byte store.
template <bool VEC>
__global__ void __launch_bounds__(256) f32_to_f16_kernel(const float *__restrict__ X, int64_t ldx,
                                                         _Float16 *__restrict__ B, int64_t ldb, int64_t n,
                                                         int64_t m)
{
    const int64_t r0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (r0 >= n)
        return;
    for (int64_t j = blockIdx.y; j < m; j += gridDim.y) {
        const float *x = X + j * ldx + r0;
        _Float16 *b = B + j * ldb + r0;
        if (VEC && r0 + 8 <= n) {
            const float4 lo = reinterpret_cast<const float4 *>(x)[0];
            const float4 hi = reinterpret_cast<const float4 *>(x)[1];
            typedef _Float16 h8 __attribute__((ext_vector_type(8)));
            h8 h = {(_Float16)lo.x, (_Float16)lo.y, (_Float16)lo.z, (_Float16)lo.w,
                    (_Float16)hi.x, (_Float16)hi.y, (_Float16)hi.z, (_Float16)hi.w};
            *reinterpret_cast<h8 *>(b) = h;
        } else {
            for (int i = 0; i < 8 && r0 + i < n; ++i)
                b[i] = (_Float16)x[i];
        }
    }
}

// C = alpha·Σ_s P_s + beta·C over S fp32 partial products P_s (row-major
// M×N, ld N, slice elements apart), summed in slice order; the epilogue is the
// GEMM kernels' (fma(alpha, sum, beta·c), or alpha·sum without beta), with
// BETA a compile-time choice as there, so that the same instructions round
// the result (a 16-bit C with beta: one v_fma_mixlo_f16, a single rounding).
// VEC: 4 columns per thread (N % 4 == 0, 16-byte aligned P, C aligned to its
// 4-element vector, ldc % 4 == 0).  blockIdx.y strides over the rows.
template <bool OUT_F16, bool VEC, bool BETA>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float *__restrict__ P, int64_t slice, int S,
                                                            int64_t M, int64_t N, float alpha, float beta,
                                                            void *__restrict__ C, int64_t ldc)
{
    typedef typename std::conditional<OUT_F16, _Float16, float>::type celt;
    const int64_t ncg = VEC ? N / 4 : N;
    const int64_t cg = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (cg >= ncg)
        return;
    constexpr int W = VEC ? 4 : 1;
    for (int64_t i = blockIdx.y; i < M; i += gridDim.y) {
        const int64_t j = cg * W;
        float acc[W];
#pragma unroll
        for (int e = 0; e < W; ++e)
            acc[e] = P[i * N + j + e];
        for (int s = 1; s < S; ++s) {
            if constexpr (VEC) {
                const float4 v = *reinterpret_cast<const float4 *>(P + s * slice + i * N + j);
                acc[0] += v.x;
                acc[1] += v.y;
                acc[2] += v.z;
                acc[3] += v.w;
            } else {
                acc[0] += P[s * slice + i * N + j];
            }
        }
        celt *cp = static_cast<celt *>(C) + i * ldc + j;
        celt out[W];
#pragma unroll
        for (int e = 0; e < W; ++e) {
            const float t = BETA ? __builtin_fmaf(alpha, acc[e], beta * (float)cp[e]) : alpha * acc[e];
            out[e] = (celt)t;
        }
#pragma unroll
        for (int e = 0; e < W; ++e)
            cp[e] = out[e];
    }
}

unsigned grid_for(int64_t total)
{
    int64_t blocks = (total + 255) / 256;
    return (unsigned)(blocks > 65536 ? 65536 : (blocks < 1 ? 1 : blocks));
}

}  // namespace

hipError_t launch_tri_xform(int mode, const _Float16 *A, int64_t lda, _Float16 *L, int64_t ldl,
                            int64_t n, hipStream_t stream)
{
    if (n <= 0)
        return hipSuccess;
    const int64_t nt = (n + XT - 1) / XT;
    const int64_t tiles = nt * (nt + 1) / 2;
    if (tiles > 0x7fffffff || n > 0x7fffffff)
        return hipErrorInvalidValue;
    const bool vec = n % XT == 0 && lda % 8 == 0 && ldl % 8 == 0 && reinterpret_cast<uintptr_t>(A) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(L) % 16 == 0;
    if (vec) {
        const dim3 grid((unsigned)((tiles + 3) / 4));
        switch (mode) {
        case 1:
            hipLaunchKernelGGL(tri_xform64_kernel<1>, grid, dim3(256), 0, stream, A, lda, L, ldl, (int)n, (int)tiles);
            break;
        case 2:
            hipLaunchKernelGGL(tri_xform64_kernel<2>, grid, dim3(256), 0, stream, A, lda, L, ldl, (int)n, (int)tiles);
            break;
        case 3:
            hipLaunchKernelGGL(tri_xform64_kernel<3>, grid, dim3(256), 0, stream, A, lda, L, ldl, (int)n, (int)tiles);
            break;
        case 4:
            hipLaunchKernelGGL(tri_xform64_kernel<4>, grid, dim3(256), 0, stream, A, lda, L, ldl, (int)n, (int)tiles);
            break;
        default:
            return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    switch (mode) {
    case 1:
        hipLaunchKernelGGL(tri_xform_kernel<1>, dim3((unsigned)tiles), dim3(256), 0, stream, A, lda, L, ldl, (int)n);
        break;
    case 2:
        hipLaunchKernelGGL(tri_xform_kernel<2>, dim3((unsigned)tiles), dim3(256), 0, stream, A, lda, L, ldl, (int)n);
        break;
    case 3:
        hipLaunchKernelGGL(tri_xform_kernel<3>, dim3((unsigned)tiles), dim3(256), 0, stream, A, lda, L, ldl, (int)n);
        break;
    case 4:
        hipLaunchKernelGGL(tri_xform_kernel<4>, dim3((unsigned)tiles), dim3(256), 0, stream, A, lda, L, ldl, (int)n);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// D = Sᵀ when rows and cols are multiples of 64 and rows are 16-byte
// aligned, without LDS: each wave moves one 64×64 tile.  Lane (rb, cb) =
// (lane / 8, lane % 8) loads the 8×8 block at S rows 8rb.., columns 8cb..
// (eight 16-byte loads; the 8 lanes of one rb read one whole 128-byte line
// of each row), transposes it in registers and stores 8 rows of D (the 8
// lanes of one cb write one whole 128-byte line of each).
__global__ void __launch_bounds__(256) transpose64_kernel(const _Float16 *__restrict__ S, int64_t lds,
                                                          _Float16 *__restrict__ D, int64_t ldd, int tiles_c,
                                                          int ntiles)
{
    const int tile = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (tile >= ntiles)
        return;
    const int lane = threadIdx.x & 63, rb = lane >> 3, cb = lane & 7;
    const int64_t r0 = (int64_t)(tile / tiles_c) * 64 + 8 * rb;
    const int64_t c0 = (int64_t)(tile % tiles_c) * 64 + 8 * cb;
    u32x4v in[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
        in[k] = *reinterpret_cast<const u32x4v *>(S + (r0 + k) * lds + c0);
    // Output row k2 is S column c0 + k2: element e = S(r0 + e, c0 + k2),
    // i.e. half k2 of in[e]; dword d packs elements 2d (low) and 2d + 1.
#pragma unroll
    for (int k2 = 0; k2 < 8; ++k2) {
        u32x4v o;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t a = in[2 * d][k2 >> 1], b = in[2 * d + 1][k2 >> 1];
            o[d] = (k2 & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
        }
        *reinterpret_cast<u32x4v *>(D + (c0 + k2) * ldd + r0) = o;
    }
}

hipError_t launch_transpose(const _Float16 *S, int64_t lds, _Float16 *D, int64_t ldd, int64_t rows,
                            int64_t cols, hipStream_t stream)
{
    if (rows <= 0 || cols <= 0)
        return hipSuccess;
    const int64_t tr = (rows + XT - 1) / XT, tc = (cols + XT - 1) / XT;
    if (tr * tc > 0x7fffffff || rows > 0x7fffffff || cols > 0x7fffffff)
        return hipErrorInvalidValue;
    const int vec = reinterpret_cast<uintptr_t>(S) % 16 == 0 && reinterpret_cast<uintptr_t>(D) % 16 == 0 &&
                    lds % 8 == 0 && ldd % 8 == 0;
    if (vec && rows % 64 == 0 && cols % 64 == 0) {
        const int64_t nt = (rows / 64) * (cols / 64);
        hipLaunchKernelGGL(transpose64_kernel, dim3((unsigned)((nt + 3) / 4)), dim3(256), 0, stream, S, lds, D,
                           ldd, (int)(cols / 64), (int)nt);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)(tr * tc)), dim3(256), 0, stream, S, lds, D, ldd,
                       (int)rows, (int)cols, (int)tc, vec);
    return hipGetLastError();
}

hipError_t launch_row_reverse_copy(const _Float16 *B, int64_t ldb, _Float16 *Bp, int64_t ldp, int64_t n,
                                   int64_t m, hipStream_t stream)
{
    if (n <= 0 || m <= 0)
        return hipSuccess;
    const int vec = n % 8 == 0 && ldb % 8 == 0 && ldp % 8 == 0 && reinterpret_cast<uintptr_t>(B) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(Bp) % 16 == 0;
    hipLaunchKernelGGL(row_reverse_copy_kernel, dim3(grid_for(vec ? (n / 8) * m : n * m)), dim3(256), 0,
                       stream, B, ldb, Bp, ldp, n, m, vec);
    return hipGetLastError();
}

hipError_t launch_f32_to_f16(const float *X, int64_t ldx, _Float16 *B, int64_t ldb, int64_t n, int64_t m,
                             hipStream_t stream)
{
    if (n <= 0 || m <= 0)
        return hipSuccess;
    const dim3 grid((unsigned)((n + 2047) / 2048), (unsigned)(m < 65535 ? m : 65535));
    const bool vec = (reinterpret_cast<uintptr_t>(X) & 15) == 0 && (reinterpret_cast<uintptr_t>(B) & 15) == 0 &&
                     ldx % 4 == 0 && ldb % 8 == 0;
    if (vec)
        hipLaunchKernelGGL(f32_to_f16_kernel<true>, grid, dim3(256), 0, stream, X, ldx, B, ldb, n, m);
    else
        hipLaunchKernelGGL(f32_to_f16_kernel<false>, grid, dim3(256), 0, stream, X, ldx, B, ldb, n, m);
    return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float *P, int64_t slice, int S, int64_t M, int64_t N, float alpha,
                                float beta, void *C, int64_t ldc, bool out_f16, hipStream_t stream)
{
    if (M <= 0 || N <= 0 || S <= 0)
        return hipSuccess;
    const uintptr_t calign = out_f16 ? 8 : 16;
    const bool vec = N % 4 == 0 && reinterpret_cast<uintptr_t>(P) % 16 == 0 && slice % 4 == 0 &&
                     reinterpret_cast<uintptr_t>(C) % calign == 0 && ldc % 4 == 0;
    const int64_t ncg = vec ? N / 4 : N;
    const dim3 grid((unsigned)((ncg + 255) / 256), (unsigned)(M < 65535 ? M : 65535));
    const int sel = (out_f16 ? 4 : 0) | (vec ? 2 : 0) | (beta != 0.0f ? 1 : 0);
#define HG_REDUCE(F, V, B)                                                                                     \
    hipLaunchKernelGGL((splitk_reduce_kernel<F, V, B>), grid, dim3(256), 0, stream, P, slice, S, M, N, alpha, \
                       beta, C, ldc)
    switch (sel) {
    case 0: HG_REDUCE(false, false, false); break;
    case 1: HG_REDUCE(false, false, true); break;
    case 2: HG_REDUCE(false, true, false); break;
    case 3: HG_REDUCE(false, true, true); break;
    case 4: HG_REDUCE(true, false, false); break;
    case 5: HG_REDUCE(true, false, true); break;
    case 6: HG_REDUCE(true, true, false); break;
    default: HG_REDUCE(true, true, true); break;
    }
#undef HG_REDUCE
    return hipGetLastError();
}

hipError_t launch_row_reverse_inplace(float *Out, int64_t ldo, int64_t n, int64_t m, hipStream_t stream)
{
    if (n <= 1 || m <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(row_reverse_inplace_kernel, dim3(grid_for((n / 2) * m)), dim3(256), 0, stream, Out,
                       ldo, n, m);
    return hipGetLastError();
}

}  // namespace hg
