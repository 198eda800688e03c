/*
 * hgemm.h — C ABI of the MI355X (gfx950) half-precision GEMM library.
 *
 * Two operations:
 *
 *   hgemm             C = alpha·A·B + beta·C, fp16 A and B, fp32 accumulation,
 *                     fp16 or fp32 C.  Problem statement and layouts from
 *                     "Nvidia Tensor Core-MMA PTX编程入门" §4 (A M×K row-major,
 *                     B K×N column-major, C M×N row-major); ragged edges are
 *                     masked as in the tiled matmul of "GPU架构与CUDA"
 *                     (section 共享内存与分块); fp16 inputs with fp32
 *                     accumulation as in its section 混合精度核函数.
 *
 *   trmm_lower_trans  Out = alpha·Aᵀ·B with A lower triangular, computed by
 *                     the recursive 2×2 blocking of
 *                     "异构计算中高性能TRMM与TRSM的递归算法实现" §2.1–§2.2:
 *                     split at n/2 until a block is at most `leaf`, leaf blocks
 *                     by the triangle-masked GEMM kernel, and the A21ᵀ·B2
 *                     updates by hgemm's GEMM kernel.  By default (aligned
 *                     operands, recursion boundaries on 256-column tile edges)
 *                     the whole recursion is one launch: each output tile
 *                     walks its leaf and its updates (in recursion order, or
 *                     the reverse one for the shorter tile of each pair of
 *                     tiles a workgroup takes) and adds the updates in its
 *                     fp32 accumulators.
 *                     hg_trmm_lower_trans_by_level runs the page's schedule
 *                     literally: one launch for the leaves, then one GEMM
 *                     launch with beta = 1 per recursion level.
 *
 *   trsm_lower_trans  X = alpha·A⁻ᵀ·B with A lower triangular: the triangular
 *                     solve of the same page, §2.3, by the same recursion
 *                     (§2.1): the lower half is solved first, the upper
 *                     half's right-hand side is updated by the GEMM kernel
 *                     (alpha = -1), leaves are multiplied by the inverse of
 *                     their diagonal block on the matrix cores.
 *
 * All matrix pointers are DEVICE pointers on the current HIP device.  Calls
 * are asynchronous on `stream` (a hipStream_t; NULL = the default stream);
 * results are valid once the stream has been synchronised.  The library
 * allocates no memory, never copies between host and device and keeps no
 * host state beyond per-device caches (the compute-unit count and the
 * address of hgemm_splitk_noalloc's static device array; atomics), so calls
 * from several host threads are safe (hgemm_splitk_noalloc's calls that
 * overlap on one GPU share that array: see there);
 * hg_trmm_lower_trans_streams creates and destroys HIP events within each
 * call.  The caller owns every buffer, including the device workspaces some
 * entry points take.
 *
 * Return value: 0 on success.  A negative value -i means argument i (1-based,
 * in the order of the prototype) is invalid, following the BLAS xerbla
 * convention; nothing is launched in that case.  A value 1000 + e means the
 * HIP runtime reported hipError_t e at launch.  hg_strerror() names a status.
 */
#ifndef HGEMM_H
#define HGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of C (hgemm, hgemm_bf16) and Out (trmm_lower_trans). */
#define HG_F16 0
#define HG_F32 1
#define HG_BF16 2

/* Triangle and transposition of hg_trmm. */
#define HG_LOWER 0
#define HG_UPPER 1
#define HG_NOTRANS 0
#define HG_TRANS 1

/* Storage order of hgemm_layout's operands. */
#define HG_ROW_MAJOR 0
#define HG_COL_MAJOR 1

/* Activation of hgemm_bias_act. */
#define HG_ACT_NONE 0
#define HG_ACT_RELU 1

#define HG_OK 0
#define HG_ERR_HIP_BASE 1000

/*
 * hgemm — C = alpha·A·B + beta·C.
 *
 *  1 M, 2 N, 3 K : problem sizes, each >= 0.
 *  4 alpha       : scale of the product (fp32).
 *  5 A, 6 lda    : fp16, M×K row-major, element (i,k) at A[i*lda + k];
 *                  lda >= max(1, K).
 *  7 B, 8 ldb    : fp16, K×N column-major, element (k,j) at B[j*ldb + k]
 *                  (equivalently Bᵀ stored N×K row-major); ldb >= max(1, K).
 *  9 beta        : scale of the incoming C (fp32).  When beta == 0, C is
 *                  write-only (NaN or garbage in C does not propagate).
 * 10 C, 11 ldc   : M×N row-major, element (i,j) at C[i*ldc + j], of type
 *                  out_dtype for both the read (beta != 0) and the write;
 *                  ldc >= max(1, N).  Elements outside the M×N window
 *                  (the ldc padding) are never read or written.
 * 12 out_dtype   : HG_F16 (rounded to nearest even) or HG_F32.
 * 13 stream      : hipStream_t to launch on.
 *
 * Arithmetic: each product fp16×fp16 is exact in fp32 and is summed in fp32
 * in an unspecified order; the result is alpha·acc + beta·C_in in fp32, then
 * converted to out_dtype.
 * Quick returns: M == 0 or N == 0 touches nothing.  alpha == 0 or K == 0
 * does not read A or B and sets C = beta·C (C = 0 when beta == 0).
 * A and B may be NULL only when they are not read.  C must not overlap A or B
 * (checked on the host; error -10).  Fast path: A and B 16-byte aligned with
 * lda and ldb multiples of 8; anything else takes a slower, element-wise
 * load path with identical results.
 */
int hgemm(int64_t M, int64_t N, int64_t K, float alpha,
          const void *A, int64_t lda,
          const void *B, int64_t ldb,
          float beta, void *C, int64_t ldc,
          int out_dtype, void *stream);

/*
 * hgemm_bias_act — C = act(alpha·A·B + beta·C + bias), the matmul, bias
 * addition and activation fused into one launch as in "GPU架构与CUDA",
 * section 核函数融合: the sum and the biased value never leave the chip; the
 * only memory traffic beyond hgemm's is the bias vector.
 *
 *  1–12, 15      : as hgemm (13 → 15: stream).
 * 13 bias        : DEVICE pointer to N fp32 values, bias[j] added to every
 *                  element of column j; NULL adds nothing.  Must not overlap
 *                  C (error -13).
 * 14 act         : HG_ACT_NONE, or HG_ACT_RELU: t < 0 becomes +0, NaN passes
 *                  through; anything else is rejected (-14).
 *
 * Per element, in fp32: t = alpha·acc + beta·C_in (as hgemm), t = t + bias[j],
 * t = act(t), then the conversion to out_dtype.  alpha == 0 or K == 0 reads
 * neither A nor B: C = act(beta·C + bias).  With bias NULL and HG_ACT_NONE the
 * result is hgemm's, bit for bit.
 */
int hgemm_bias_act(int64_t M, int64_t N, int64_t K, float alpha,
                   const void *A, int64_t lda,
                   const void *B, int64_t ldb,
                   float beta, void *C, int64_t ldc,
                   int out_dtype, const float *bias, int act, void *stream);

/*
 * hgemm_layout — hgemm with A and B in either storage order (C stays M×N
 * row-major): A M×K row-major (A[i*lda + k], hgemm's) or column-major
 * (A[i + k*lda]); B K×N column-major (B[k + j*ldb], hgemm's) or row-major
 * (B[k*ldb + j], the layout of the matmul in "GPU架构与CUDA").
 *
 *  1 a_layout, 2 b_layout : HG_ROW_MAJOR or HG_COL_MAJOR.
 *  3 M, 4 N, 5 K, 6 alpha, 7 A, 8 lda, 9 B, 10 ldb, 11 beta, 12 C, 13 ldc,
 * 14 out_dtype   : as hgemm; lda >= K (row-major A) or >= M (column-major),
 *                  ldb >= K (column-major B) or >= N (row-major).
 * 15 work        : device workspace, 16-byte aligned, of at least
 * 16 work_bytes    hg_hgemm_layout_workspace_size(...) bytes (0 for hgemm's
 *                  own layouts, which ignore it); must not overlap A, B or C
 *                  (-15; too small: -16).
 * 17 stream      : hipStream_t.
 *
 * An operand that is not K-contiguous is first transposed into the
 * workspace by a tiled copy kernel; the product then runs on hgemm's kernels
 * with the same arithmetic (bit-identical to hgemm on the transposed data).
 */
int hgemm_layout(int a_layout, int b_layout, int64_t M, int64_t N, int64_t K, float alpha,
                 const void *A, int64_t lda, const void *B, int64_t ldb,
                 float beta, void *C, int64_t ldc, int out_dtype,
                 void *work, int64_t work_bytes, void *stream);

/* hg_hgemm_layout_workspace_size — bytes hgemm_layout needs (host only);
 * -1/-2 for a bad layout, -3 for a negative size. */
int64_t hg_hgemm_layout_workspace_size(int a_layout, int b_layout, int64_t M, int64_t N, int64_t K);

/*
 * hgemm_bf16 — hgemm with bf16 A and B ("GPU架构与CUDA", section 混合精度核函数:
 * a lower-precision type for the products, fp32 for the accumulation; bf16
 * keeps fp32's exponent range with an 8-bit significand).
 *
 * Arguments, layouts, quick returns and status codes as hgemm, except:
 *  5 A, 7 B      : bf16 (the upper 16 bits of an IEEE binary32).
 * 12 out_dtype   : HG_BF16 (rounded to nearest even) or HG_F32; HG_F16 is
 *                  rejected (-12).
 * Each bf16×bf16 product is exact in fp32 and summed in fp32, as in hgemm.
 */
int hgemm_bf16(int64_t M, int64_t N, int64_t K, float alpha,
               const void *A, int64_t lda,
               const void *B, int64_t ldb,
               float beta, void *C, int64_t ldc,
               int out_dtype, void *stream);

/*
 * hgemm_bf16_bias_act — hgemm_bias_act with bf16 A and B: C = act(alpha·A·B
 * + beta·C + bias) in one launch, the products as in hgemm_bf16 and the bias
 * and activation as in hgemm_bias_act ("GPU架构与CUDA", sections 混合精度核函数
 * and 核函数融合).  Arguments, layouts and status codes as hgemm_bias_act,
 * except A and B are bf16 and out_dtype is HG_BF16 or HG_F32 (-12).
 */
int hgemm_bf16_bias_act(int64_t M, int64_t N, int64_t K, float alpha,
                        const void *A, int64_t lda, const void *B, int64_t ldb,
                        float beta, void *C, int64_t ldc, int out_dtype,
                        const float *bias, int act, void *stream);

/*
 * trmm_lower_trans — Out = alpha·Aᵀ·B, A lower triangular.
 *
 *  1 n, 2 m      : A is n×n, B and Out are n×m; each >= 0.
 *  3 alpha       : scale (fp32), applied once to every output.
 *  4 A, 5 lda    : fp16, n×n column-major, element (r,c) at A[r + c*lda];
 *                  lda >= max(1, n).  Only the lower triangle (r >= c) is
 *                  read; the strictly upper triangle is never referenced.
 *  6 B, 7 ldb    : fp16, n×m column-major input; ldb >= max(1, n).
 *  8 Out, 9 ldo  : n×m column-major output, element (r,c) at Out[r + c*ldo];
 *                  ldo >= max(1, n); write-only (its previous contents are
 *                  ignored).  Must not overlap A or B (error -8).
 * 10 out_dtype   : HG_F32 (the updates accumulate into Out in fp32; HG_F16
 *                  is rejected with -10).
 * 11 leaf        : recursion cut-off; a diagonal block of size <= leaf is
 *                  handled by the triangle-masked leaf kernel.  leaf <= 0
 *                  selects 256.
 * 12 stream      : hipStream_t to launch on.
 *
 * Order of work: every element of Out receives its leaf term first, then
 * the A21ᵀ·B2 update terms of the recursion nodes above it from the deepest
 * to the outermost -- the order of accumulation of the depth-first
 * recursion.  Each term is a GEMM computed in fp32 and added as
 * Out = alpha·acc (leaf) or Out = fma(alpha, acc, Out) (update, beta = 1).
 * When every recursion boundary falls on a multiple of 256 (n a multiple of
 * 256 split down to leaves of at least 256), the operands are 16-byte
 * aligned with lda, ldb multiples of 8 and there are at least two 256×256
 * output tiles per compute unit, all terms run in one launch in which each
 * output tile walks its own terms and adds each update to the leaf in its
 * fp32 accumulators (alpha applied once, when the tile is written); a
 * workgroup takes output tile columns c and T-1-c of one tile row (T tile
 * columns) in turn, the longer walk in that order, the shorter one in the
 * reverse order, so that concurrent tiles read the same slices of B.  With fewer such tiles, the same one-launch schedule runs on
 * 64×64 output tiles when every boundary falls on a multiple of 64 (leaf
 * >= 64, the same alignment) and n <= 4096, or n <= 8192 with m <= 512, or
 * m·n² <= 2^34.  Otherwise one batched launch runs all leaves and one each
 * update level, rounding Out to fp32 after every update.  The schedules
 * differ only by those fp32 roundings (integer-valued inputs: the same
 * bits; see hg_trmm_lower_trans_by_level).
 */
int trmm_lower_trans(int64_t n, int64_t m, float alpha,
                     const void *A, int64_t lda,
                     const void *B, int64_t ldb,
                     void *Out, int64_t ldo, int out_dtype,
                     int64_t leaf, void *stream);

/*
 * hg_trmm — Out = alpha·op(A)·B for every triangle and transposition
 * ("异构计算中高性能TRMM与TRSM的递归算法实现" §2.1 shows the lower and upper
 * blockings; its §5.1 usage calls the lower, non-transposed product).
 *
 *  1 uplo        : HG_LOWER (A(r,c) read for r >= c) or HG_UPPER (r <= c);
 *                  the other triangle is never referenced.
 *  2 trans       : HG_TRANS (op(A) = Aᵀ) or HG_NOTRANS (op(A) = A).
 *  3 n, 4 m, 5 alpha, 6 A, 7 lda, 8 B, 9 ldb, 10 Out, 11 ldo, 12 out_dtype,
 * 13 leaf        : as trmm_lower_trans (column-major, Out fp32, write-only).
 * 14 work        : device workspace, 16-byte aligned, of at least
 * 15 work_bytes    hg_trmm_workspace_size(uplo, trans, n, m) bytes (0 for
 *                  HG_LOWER/HG_TRANS, which is trmm_lower_trans itself and
 *                  ignores work); must not overlap A, B or Out (-14; too
 *                  small: -15).
 * 16 stream      : hipStream_t to launch on.
 *
 * upper/notrans runs the same recursion on L = Aᵀ, which one copy kernel
 * builds in the workspace.  upper/trans and lower/notrans, when the
 * one-launch schedule applies (see trmm_lower_trans), run it with the
 * triangle on the other side of the GEMM view: each output tile walks K from
 * 0 up to its diagonal block (the recursion's outermost update first, the
 * leaf last; the shorter tile of each pair the other way), on A itself (upper/trans) or on an upper triangular copy of Aᵀ
 * (lower/notrans).  Otherwise they run on a lower triangular L with the row
 * order reversed by P: upper/trans: P·Out = (P·A·P)ᵀ·(P·B); lower/notrans:
 * P·Out = (P·Aᵀ·P)ᵀ·(P·B), B's rows reversed into the workspace and Out's
 * rows reversed in place at the end.
 */
int hg_trmm(int uplo, int trans, int64_t n, int64_t m, float alpha,
            const void *A, int64_t lda,
            const void *B, int64_t ldb,
            void *Out, int64_t ldo, int out_dtype,
            int64_t leaf, void *work, int64_t work_bytes, void *stream);

/*
 * hgemm_splitk — hgemm with K cut into slices that run side by side, for
 * problems whose C has too few tiles to fill the GPU while K is long (the
 * tiled product of "GPU架构与CUDA" 共享内存与分块, its K loop partitioned).
 *
 *  1..12          : as hgemm (fp16 A row-major, B column-major; out_dtype
 *                   HG_F16 or HG_F32).
 * 13 splits       : number of K slices, 1..32 (each at least 64 columns of K,
 *                   fewer if K is short); 0 picks enough slices to give every
 *                   compute unit a 128×128 tile, each slice at least 256
 *                   columns long.  Outside 0..32: -13.
 * 14 work         : device workspace, 16-byte aligned, of at least
 * 15 work_bytes     hg_hgemm_splitk_workspace_size(M, N, K, splits) bytes
 *                   (the fp32 partial products); must not overlap A, B or C
 *                   (-14; too small: -15).
 * 16 stream       : hipStream_t.
 *
 * Each slice's product is accumulated in fp32 as in hgemm and stored in fp32;
 * the slices are then summed in order in fp32 and C = fma(alpha, sum,
 * beta·C) (alpha·sum when beta = 0) is rounded to out_dtype once.  The
 * result depends only on the arguments (no atomics).  With one slice it is
 * hgemm's, bit for bit.
 */
int hgemm_splitk(int64_t M, int64_t N, int64_t K, float alpha,
                 const void *A, int64_t lda, const void *B, int64_t ldb,
                 float beta, void *C, int64_t ldc, int out_dtype, int splits,
                 void *work, int64_t work_bytes, void *stream);

/* hg_hgemm_splitk_workspace_size — bytes hgemm_splitk needs for (M, N, K,
 * splits) on the current device (host only; splits = 0 depends on the
 * device's compute-unit count); -1/-2/-3 for M/N/K out of range, -4 for
 * splits outside 0..32. */
int64_t hg_hgemm_splitk_workspace_size(int64_t M, int64_t N, int64_t K, int splits);

/*
 * hgemm_splitk_noalloc — hgemm_splitk without a workspace argument, for
 * callers that cannot allocate device memory or pass a workspace (code under
 * stream capture, tight serving loops, harnesses that forbid allocation).
 *
 *  1..13          : as hgemm_splitk (splits 0..32; 0 picks the slice count).
 * 14 stream       : hipStream_t.
 *
 * The fp32 partial products go to a static device array of the library,
 * HG_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, which each GPU the library runs
 * on holds until the process ends; the call allocates nothing.  A problem
 * whose partials need more (hg_hgemm_splitk_workspace_size(M, N, K, splits)
 * > HG_NOALLOC_SCRATCH_BYTES) is rejected with HG_ERR_SCRATCH_LIMIT before
 * anything is launched; other arguments are checked as by hgemm_splitk, with
 * its codes.  The result is hgemm_splitk's, bit for bit.  Every call on one
 * GPU uses the same array: calls that overlap in time on one GPU (on
 * different streams, or from different host threads without ordering) race
 * on it and give undefined results; calls on one stream are ordered and safe.
 * The partials are written in full by each call before they are read, so no
 * state carries over from the previous call.
 */
#define HG_NOALLOC_SCRATCH_BYTES (32 << 20)
#define HG_ERR_SCRATCH_LIMIT (-100)
int hgemm_splitk_noalloc(int64_t M, int64_t N, int64_t K, float alpha,
                         const void *A, int64_t lda, const void *B, int64_t ldb,
                         float beta, void *C, int64_t ldc, int out_dtype, int splits,
                         void *stream);

/* hg_trmm_workspace_size — bytes of workspace hg_trmm needs (host only);
 * -1/-2 for a bad uplo/trans, -3/-4 for n/m < 0. */
int64_t hg_trmm_workspace_size(int uplo, int trans, int64_t n, int64_t m);

/*
 * hg_trmm_inplace — B ← alpha·op(A)·B in fp16, the in-place form of
 * "异构计算中高性能TRMM与TRSM的递归算法实现" §2.2 ("B ←").
 *
 *  1 uplo, 2 trans, 3 n, 4 m, 5 alpha, 6 A, 7 lda : as hg_trmm.
 *  8 B, 9 ldb     : fp16 n×m column-major, read as the right-hand side and
 *                   overwritten with the product rounded to nearest even.
 *                   Must not overlap A (-8).
 * 10 leaf        : as hg_trmm.
 * 11 work        : device workspace, 16-byte aligned, of at least
 * 12 work_bytes    hg_trmm_inplace_workspace_size(uplo, trans, n, m) bytes:
 *                  the product (fp32 room) and hg_trmm's own workspace; must
 *                  not overlap A or B (-11; too small: -12).
 * 13 stream      : hipStream_t.
 *
 * B receives hg_trmm's fp32 result rounded to nearest even, bit for bit; no
 * intermediate of the recursion is rounded to fp16.  When hg_trmm would run
 * the one-launch schedule (see trmm_lower_trans), that kernel rounds each
 * finished tile to fp16 into the workspace and one device-to-device copy
 * moves the product into B; otherwise hg_trmm writes the fp32 product into
 * the workspace and one pass rounds it into B.
 */
int hg_trmm_inplace(int uplo, int trans, int64_t n, int64_t m, float alpha,
                    const void *A, int64_t lda, void *B, int64_t ldb,
                    int64_t leaf, void *work, int64_t work_bytes, void *stream);

/* hg_trmm_inplace_workspace_size — bytes hg_trmm_inplace needs (host only);
 * negative values as hg_trmm_workspace_size. */
int64_t hg_trmm_inplace_workspace_size(int uplo, int trans, int64_t n, int64_t m);

/*
 * hg_trmm_lower_trans_by_level — trmm_lower_trans (same arguments, same
 * status codes, the same result up to fp32 rounding) scheduled as in the recursion's
 * description, "异构计算中高性能TRMM与TRSM的递归算法实现" §2.2: one batched
 * launch for all leaves, then one batched GEMM launch (beta = 1) per
 * recursion level, deepest first.  For verification and comparison of the
 * two schedules.
 */
int hg_trmm_lower_trans_by_level(int64_t n, int64_t m, float alpha,
                                 const void *A, int64_t lda,
                                 const void *B, int64_t ldb,
                                 void *Out, int64_t ldo, int out_dtype,
                                 int64_t leaf, void *stream);

/*
 * hg_trmm_lower_trans_streams — hg_trmm_lower_trans_by_level with the
 * independent launches of each phase spread over several streams, as the
 * recursion's usage notes suggest ("异构计算中高性能TRMM与TRSM的递归算法实现"
 * §5.2: several streams for the independent branches): every leaf, then
 * every update of a level, deepest level first, goes to the next stream in
 * turn, and the streams are joined (events) at entry, between phases and at
 * the end.
 *
 *  1..11         : as trmm_lower_trans (no stream argument).
 * 12 streams     : array of nstreams hipStream_t; streams[0] is the caller's:
 *                  the work starts after what is queued on it and, on return,
 *                  everything queued later on it runs after the product.
 *                  NULL: -12.
 * 13 nstreams    : 1..8 (-13 otherwise).
 *
 * Each launch runs the kernel the batched launch of its phase runs, so the
 * result equals hg_trmm_lower_trans_by_level's bit for bit.  The level's
 * batched launch already runs all its branches side by side; this entry
 * point is there to measure the stream form against it.
 */
int hg_trmm_lower_trans_streams(int64_t n, int64_t m, float alpha,
                                const void *A, int64_t lda,
                                const void *B, int64_t ldb,
                                void *Out, int64_t ldo, int out_dtype,
                                int64_t leaf, void *const *streams, int nstreams);

/*
 * trsm_lower_trans — Out = X = alpha·A⁻ᵀ·B, i.e. the X with Aᵀ·X = alpha·B,
 * A lower triangular.
 *
 *  1 n, 2 m      : A is n×n, B and Out are n×m; each >= 0.
 *  3 alpha       : scale of the right-hand side (fp32).
 *  4 A, 5 lda    : fp16, n×n column-major, element (r,c) at A[r + c*lda];
 *                  lda >= max(1, n).  Only the lower triangle (r >= c) is
 *                  read.  The diagonal is not checked: a zero on it gives
 *                  inf/NaN, as the arithmetic does (no singularity test, as
 *                  in BLAS).
 *  6 B, 7 ldb    : fp16, n×m column-major right-hand side; ldb >= max(1, n).
 *  8 Out, 9 ldo  : n×m column-major fp32 solution; ldo >= max(1, n);
 *                  write-only for the caller (the solve keeps running sums
 *                  in it).  Must not overlap A or B (error -8).
 * 10 out_dtype   : HG_F32 (HG_F16 is rejected with -10).
 * 11 leaf        : recursion cut-off, 1..256 (leaf <= 0 selects 256; larger
 *                  values are rejected with -11).  A diagonal block of size
 *                  <= leaf is solved by the leaf step.
 * 12 work        : device workspace, 16-byte aligned, of at least
 * 13 work_bytes    hg_trsm_workspace_size(n, m, leaf) bytes; must not overlap
 *                  A, B or Out (error -12; too small: -13).  Its contents on
 *                  entry are ignored and on return are unspecified.
 * 14 stream      : hipStream_t to launch on.
 *
 * Arithmetic (half precision operands, fp32 accumulation, as in hgemm):
 *   - each leaf's diagonal block is inverted in fp32 and rounded to fp16;
 *   - a leaf's right-hand side alpha·B + (updates so far) is formed in fp32
 *     and rounded to fp16, multiplied by the fp16 inverse with fp32
 *     accumulation, and stored in Out as fp32;
 *   - every update (alpha = -1) takes the solved rows rounded to fp16 as its
 *     GEMM operand and accumulates in fp32 into Out.
 * Each fp16 rounding has relative error <= 2^-11, so X carries an error of
 * order 2^-11 times the condition of the system (ill-conditioned A loses
 * accordingly).  alpha == 0 sets Out = 0 without reading A, B or work.
 * Alignment: A and B 16-byte aligned, lda, ldb multiples of 8 and
 * recursion boundaries (n split down by halving) on multiples of 8 take the
 * vector paths; anything else runs element-wise paths with the same result.
 */
int trsm_lower_trans(int64_t n, int64_t m, float alpha,
                     const void *A, int64_t lda,
                     const void *B, int64_t ldb,
                     void *Out, int64_t ldo, int out_dtype,
                     int64_t leaf, void *work, int64_t work_bytes,
                     void *stream);

/*
 * hg_trsm_workspace_size — bytes of device workspace trsm_lower_trans needs
 * for (n, m, leaf): the fp16 inverses of the leaf blocks plus an fp16 copy
 * of X.  Host only.  Returns 0 when n or m is 0, -1 for n < 0, -2 for
 * m < 0, -3 for leaf > 256 (leaf <= 0 selects 256).
 */
int64_t hg_trsm_workspace_size(int64_t n, int64_t m, int64_t leaf);

/* Human-readable name of a status code (static string, never NULL). */
const char *hg_strerror(int status);

/*
 * hg_trmm_plan — the recursion trmm_lower_trans runs for (n, leaf), for
 * inspection; host only, launches nothing.
 *
 * Writes up to `cap` nodes into `nodes`, 4 int64 per node:
 *   {kind, offset, size, depth}
 *   kind 0 = leaf:   Out[o:o+s] = alpha·tril(A[o:o+s, o:o+s])ᵀ·B[o:o+s]
 *   kind 1 = update: Out[o:o+h] += alpha·A[o+h:o+s, o:o+h]ᵀ·B[o+h:o+s]
 *                    with s = size and h = floor(s/2)
 * in depth-first recursion order, and returns the total node count (which
 * may exceed cap; then only the first cap are written).  Returns -1 for
 * n < 0, -2 when nodes is NULL with cap > 0.
 */
int64_t hg_trmm_plan(int64_t n, int64_t leaf, int64_t *nodes, int64_t cap);

#ifdef __cplusplus
}
#endif

#endif /* HGEMM_H */
