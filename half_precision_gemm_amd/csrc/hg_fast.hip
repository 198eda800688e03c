// hg_fast.hip — the 256×256 fast path of the half-precision GEMM on gfx950.
//
// Same computation and layouts as the general kernel in hg_kernels.hip
// (C = alpha·A·B + beta·C, A M×K row-major, B K×N column-major, fp16 in,
// fp32 accumulate; "Nvidia Tensor Core-MMA PTX编程入门" §4 and the masked
// tiled matmul of "GPU架构与CUDA" 共享内存与分块), for operands whose rows
// are 16-byte aligned and K a multiple of 8; with TRI it is also the
// triangle-masked leaf of the recursive TRMM ("异构计算中高性能TRMM与TRSM的
// 递归算法实现" §2.2), and with TRI and FUSED the whole recursion in one
// launch (see the section on the recursive TRMM below).  Design:
//
//  * One workgroup = 4 waves (one per SIMD) per 256×256 tile, laid out 2×2;
//    each wave owns a 128×128 sub-tile = 8×8 blocks of
//    v_mfma_f32_16x16x32_f16, 256 fp32 accumulators per lane (AGPRs).  The
//    16×16×32 shape draws less power per flop than 32×32×16 on these data,
//    so the chip holds a higher clock.  (HG_FAST_NW=8 builds the 2×4 layout
//    with two waves per SIMD and 128×64 sub-tiles; it was not faster.)
//  * K is walked in BK = 64 stages: one 128-byte cache line per operand row.
//    Operands reach LDS through the gfx950 direct buffer→LDS path
//    (buffer_load_dwordx4 … lds; each wave instruction moves 8 rows × 128
//    bytes): no staging registers, no ds_write.  Lane l fetches the logical
//    16-byte chunk that the XOR swizzle places at position l, so the LDS
//    image is already swizzled for the fragment reads.
//  * The 160 KiB of LDS hold a 3-slot ring of A stages and a 2-slot ring of
//    B stages (32 KiB each); one barrier per stage.
//  * Ragged M/N edges and the K tail are zero-filled by the buffer unit's
//    range check (out-of-range rows and chunks get an offset past the
//    resource size, which loads as zero): no branches in the main loop.
//  * Each stage is four quarters of 16 MFMAs; fragment reads and ring loads
//    are spread evenly over the MFMAs at compile-time positions.
//  * Persistent workgroups (short K): one per CU walks a strided list of
//    tiles; the next tile's first stages are requested before the current
//    tile's epilogue, so loads overlap the stores.
//  * Epilogue: a lane's accumulators are 4 consecutive columns in each of 8
//    column blocks of one row; stored as they are, every store instruction
//    would touch 16 rows with part of a 128-byte line each.  Each 16-row
//    block is instead passed through LDS (the A slot that the next tile's
//    prologue leaves idle) and stored two whole 128-column rows per
//    instruction; the store count is the same.
//
// Workgroup→tile order: tile ids are regrouped per XCD (consecutive
// workgroup ids run on different XCDs, each with its own L2), then each
// XCD's range is walked in bands of 4 tile rows, column by column, so the
// tiles resident on one XCD share A row panels and B column panels.
#include "hg_internal.h"

#include <atomic>
#include <type_traits>
#include <utility>

typedef int32_t hg_int32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint32_t hg_lds_u32;

// The raw buffer→LDS load (LLVM intrinsic; 16 bytes per lane on gfx950).
extern "C" __device__ void hg_raw_buffer_load_lds(hg_int32x4 rsrc, hg_lds_u32 *lds, int size,
                                                  int voffset, int soffset, int offset,
                                                  int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

namespace hg {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// v_mfma_f32_16x16x32 on 16-byte fragments holding fp16 or bf16 values (the
// staging and the fragment reads move bytes and do not depend on the type).
template <bool BF16>
__device__ __forceinline__ floatx4 mfma_16x16x32(const half8 &a, const half8 &b, const floatx4 &c)
{
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

#ifndef HG_FAST_XCD
#define HG_FAST_XCD 1
#endif
#ifndef HG_FAST_PERSIST_MAXK
#define HG_FAST_PERSIST_MAXK 4096
#endif
#ifndef HG_FAST_GROUP
#define HG_FAST_GROUP 4
#endif
#ifndef HG_FAST_EPI_PREFETCH
#define HG_FAST_EPI_PREFETCH 1              // row blocks of C read ahead in the epilogue
#endif
#ifndef HG_FAST_NW
#define HG_FAST_NW 4
#endif
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int NSA = 3, NSB = 2;             // LDS slots of the A and B rings
constexpr int NW = HG_FAST_NW;              // waves per workgroup (4: 2×2, 8: 2×4)
constexpr int WM = 2, WN = NW / 2;
constexpr int THREADS = NW * 64;
constexpr int WTM = BM / WM, WTN = BN / WN; // wave sub-tile (128×128 or 128×64)
constexpr int FB = 16;                      // MFMA output block edge (16×16)
constexpr int KS = 32;                      // k per MFMA
constexpr int TM = WTM / FB, TN = WTN / FB; // 16×16 blocks per wave
constexpr int RB = BK * 2;                  // bytes per LDS row (128: one cache line)
constexpr int KC = BK / 8;                  // 16-byte chunks per row (8)
constexpr int RPL = 256 / RB;               // rows per 256-byte bank line (64 banks)
constexpr int RPI = 1024 / RB;              // rows per buffer→LDS wave instruction (8)
constexpr int RPW = BM / NW;                // tile rows each wave loads, per operand
constexpr int LPS = RPW / RPI;              // load instructions per wave per operand per stage
constexpr int SPS = BK / KS;                // MFMA k-steps per stage (2)
constexpr int NQ = 4;                       // quarters per stage (k-step × half of the A blocks)
constexpr int TMQ = TM / 2;                 // A blocks per quarter
constexpr int PQ = TMQ * TN;                // MFMAs per quarter
constexpr int SLOT = BM * RB;               // bytes of one operand's stage (32 KiB)
constexpr int LDS_B = NSA * SLOT;           // B ring after the A ring
constexpr int LDS_BYTES = (NSA + NSB) * SLOT;
constexpr uint32_t OOB = 0x80000000u;       // offset that the range check rejects
static_assert((NW == 4 || NW == 8) && SPS == 2 && BM == BN && TM == 8, "");
static_assert(LPS * RPI == RPW, "");
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

// Physical 16-byte chunk of logical chunk kc in LDS row r.  The LDS serves a
// 16-byte read for 16 lanes per cycle over 64 four-byte banks (256 bytes);
// a fragment read has 16 consecutive rows at one logical chunk, which this
// XOR spreads over 16 distinct bank groups.
__device__ __forceinline__ int swz(int r, int kc) { return kc ^ ((r / RPL) & (KC - 1)); }

// ---- Schedule of one stage.  Quarter q runs k-step q/2 on A blocks
// (q%2)·TMQ .. +TMQ-1 and all TN B blocks, B block outer (the quarter's A
// blocks are all used by its first TMQ MFMAs, B block j first by MFMA
// TMQ·j; within a B block the A blocks run in snake order).  A fragments are read one quarter ahead (two sets,
// one per quarter parity), B fragments one k-step ahead (two sets, one per
// k-step), half of them in each quarter of the k-step before:
//   q0: A of q1 (stage kt, k-step 0)      + B blocks 0,1 of k-step 1
//   q1: A of q2 (stage kt, k-step 1)      + B blocks 2,3 of k-step 1
//   q2: A of q3 (stage kt, k-step 1) | barrier | B blocks 0,1 of stage kt+1, k-step 0
//   q3: A of q0 (stage kt+1, k-step 0)    + B blocks 2,3 of stage kt+1, k-step 0
// The barrier (in front of MFMA BAR_K of quarter 2) follows every read of
// stage kt and precedes every read of stage kt+1.  Ring loads, LPS/2 per
// quarter: quarters 0 and 1 the A of stage kt+2 (its slot was freed by the
// previous stage's barrier), quarters 2 (after the barrier) and 3 the B of
// stage kt+2 (its slot is the one this barrier frees).
// Op after MFMA k of quarter q: kRA + i reads A block i of the quarter's
// range, kRB + i the quarter's i-th B block, kLD + i ring load i.  Reads and
// loads are spread evenly over the quarter: a wave's LDS traffic stays
// steady instead of arriving in bursts that block its instruction stream
// (with one wave per SIMD, every such stall idles the matrix core).
constexpr int kNone = 0, kRA = 1, kRB = 8, kLD = 16;
constexpr int BAR_K = NW == 8 ? 10 : 13;
__device__ __forceinline__ constexpr int sched8(int q, int k)
{
    if (q == 2) {
        switch (k) {
        case 0: return kRA + 0;
        case 2: return kRA + 1;
        case 4: return kRA + 2;
        case 6: return kRA + 3;
        case 10: return kLD + 0;
        case 11: return kRB + 0;
        case 13: return kRB + 1;
        case 14: return kLD + 1;
        default: return kNone;
        }
    }
    switch (k) {
    case 0: return kRA + 0;
    case 1: return kLD + 0;
    case 2: return kRA + 1;
    case 4: return kRA + 2;
    case 5: return kLD + 1;
    case 6: return kRA + 3;
    case 8: return kRB + 0;
    case 10: return kRB + 1;
    default: return kNone;
    }
}
// Four waves: 32 MFMAs, 4 A + 4 B reads and 4 loads per quarter.
__device__ __forceinline__ constexpr int sched4(int q, int k)
{
    if (q == 2) {
        if (k <= 9 && k % 3 == 0)
            return kRA + k / 3;
        if (k >= 16 && k % 4 == 0)
            return kRB + (k - 16) / 4;
        if (k >= 14 && k <= 26 && k % 4 == 2)
            return kLD + (k - 14) / 4;
        return kNone;
    }
    if (k % 4 == 0)
        return k < 16 ? kRA + k / 4 : kRB + (k - 16) / 4;
    if (k % 8 == 2)
        return kLD + k / 8;
    return kNone;
}
__device__ __forceinline__ constexpr int sched(int q, int k) { return NW == 8 ? sched8(q, k) : sched4(q, k); }

// f(integral_constant<int, i>) for i = 0 .. N-1, so that schedule lookups
// inside f are constant expressions.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}
// Keeps one row block of accumulators in accumulation registers up to this
// point of the epilogue.  Without it the register allocator copies all 256
// accumulators into VGPRs as the K loop exits (about 230 moves), which
// leaves the epilogue too few VGPRs: it spilled a few values and reloaded
// them with a wait for every store issued before.  Pinned block by block,
// each block is read out of its registers where it is consumed.
template <int N>
__device__ __forceinline__ void pin_acc(floatx4 (&blk)[N])
{
#pragma unroll
    for (int j = 0; j < N; ++j)
        __asm__ volatile("" : "+a"(blk[j]));
}

// s_waitcnt on one counter only (the others left at their maxima).
template <int n>
__device__ __forceinline__ void wait_vmcnt()
{
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}
template <int n>
__device__ __forceinline__ void wait_lgkmcnt()
{
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | ((n & 15) << 8));
}

// Raw buffer resource: base address, no stride, `bytes` in range.
__device__ __forceinline__ hg_int32x4 make_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    hg_int32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;
    return r;
}

// Tile id → (batch, tile row, tile column); see the header comment.
__device__ __forceinline__ void map_tile(int id, int total, int tiles_m, int tiles_n, int &batch,
                                         int &tm, int &tn)
{
    const int per = total >> 3, rem = total & 7;
    const int x = id & 7;
    const int q = HG_FAST_XCD ? x * per + min(x, rem) + (id >> 3) : id;
    const int per_batch = tiles_m * tiles_n;
    batch = q / per_batch;
    const int l = q - batch * per_batch;
    constexpr int G = HG_FAST_GROUP;
    const int band = l / (G * tiles_n);
    const int first = band * G;
    const int gsz = min(tiles_m - first, G);
    const int r = l - band * G * tiles_n;
    tm = first + r % gsz;
    tn = r / gsz;
}

// Everything a workgroup needs to know about one tile.
struct TileInfo {
    int batch, m0, n0, N, K, rows_a, rows_b, nk;
    // K stage (BK columns) of loop step kt: kbase + kdir·kt.  The one-launch
    // TRMM's short tiles walk their stages downward (kdir = -1).
    int kbase, kdir;
    hg_int32x4 ra, rb;
};

// First tile with id >= *id (stepping by `stride`) that has work; false if
// none is left.  Entries of a batched launch narrower than the grid leave
// empty tiles, which are skipped here (uniformly for the workgroup).
template <bool TRI>
__device__ __forceinline__ bool find_tile(const GemmParams &p, int &id, int stride, int total,
                                          int tiles_m, int tiles_n, TileInfo &T)
{
    for (; id < total; id += stride) {
        int batch, tm, tn;
        map_tile(id, total, tiles_m, tiles_n, batch, tm, tn);
        const int N = p.e[batch].N;
        const int m0 = tm * BM, n0 = tn * BN;
        if (m0 >= p.M || n0 >= N)
            continue;
        T.batch = batch;
        T.m0 = m0;
        T.n0 = n0;
        T.N = N;
        T.K = p.e[batch].K;
        T.rows_a = min(p.M - m0, BM);
        T.rows_b = min(N - n0, BN);
        // TRI: B element (j, k) counts only for k >= j, so slices wholly
        // left of the tile's first column are skipped.
        T.kbase = TRI ? n0 / BK : 0;
        T.nk = (T.K + BK - 1) / BK - T.kbase;
        T.kdir = 1;
        const _Float16 *Ab = p.A + p.e[batch].a_off + (int64_t)m0 * p.lda;
        const _Float16 *Bb = p.B + p.e[batch].b_off + (int64_t)n0 * p.ldb;
        T.ra = make_rsrc(Ab, (uint32_t)(((int64_t)(T.rows_a - 1) * p.lda + T.K) * 2));
        T.rb = make_rsrc(Bb, (uint32_t)(((int64_t)(T.rows_b - 1) * p.ldb + T.K) * 2));
        return true;
    }
    return false;
}

// ---- Recursive TRMM in one launch ("异构计算中高性能TRMM与TRSM的递归算法实现"
// §2.1–§2.2).  In the GEMM view used here (C = Outᵀ, M = m, N = K = n), the
// recursion splits a diagonal block (o, s) at h = ⌊s/2⌋: the tiles of output
// columns [o, o+h) receive the update over K = [o+h, o+s) (a GEMM with
// β = 1) after everything below that node; a block of at most `leaf`
// columns is a leaf, whose tiles take K from their own first column to the
// leaf's end under the triangle mask.  With every recursion boundary on a
// tile edge, the leaf and the updates that reach one output tile cover
// contiguous K ranges in increasing order -- the leaf's end, then the ends
// of the ancestors whose upper half holds the tile, deepest first, the last
// one n -- which is the order in which the depth-first recursion
// accumulates into that tile.  One workgroup therefore walks K over the
// tile's first column to n (in that order, or -- the short tiles below -- in
// the reverse one), and each update's β = 1
// accumulation into the tile happens in the fp32 accumulators rather than
// through a store and a reload of Out; α, common to the leaf and every
// update, is applied once when the tile is written.  The level-by-level
// launches keep the store between updates.

// Order of the tiles.  Tile column tn (of T = n/256) walks T - tn K blocks
// of 256 (tri_up: tn + 1), so columns c and T-1-c together always walk T + 1:
// a job is the pair of tiles (tm, T-1-c) then (tm, c) of one tile row, and
// every job has the same length.  Jobs are dealt to the persistent
// workgroups one per round, so all workgroups start each round together;
// those of one XCD take a block of HG_TRMM_BAND tile rows × the pair columns
// that the XCD's share of a round covers (ids regrouped per XCD, then bands
// of rows walked pair column by pair column, as for the GEMM's tiles).
// Counting time t in K blocks from the start of a round:
//   lower (not tri_up): the short tile (tm, T-1-c) takes c + 1 blocks,
//   walking down from K block T-1, so it is at K block T-1-t; the long tile
//   (tm, c) then starts at t = c + 1 at K block c and walks up, so it is at K
//   block t - 1 at time t; both whatever c is;
//   tri_up: the long tile (tm, T-1-c) starts at t = 0 at K block 0 and is at
//   K block t; the short tile (tm, c) follows at t = T - c, walking down from
//   its diagonal block c, so it is at K block T - t.
// The tiles of co-resident jobs thus read the same K slabs of the
// right-hand side at the same time and share them in L2, as the tiles of a
// GEMM do.  The long tiles walk K in the recursion's order of accumulation
// (the updates' K ranges after the leaf's; tri_up: the outermost update
// first, the leaf last), the short tiles in the reverse one; the order
// changes only fp32 rounding.  (Walking upward too, the short tiles, a
// quarter of the work at n = 8192, read staggered slabs: 1.5-2 % slower.)
// With T odd, the middle column's tiles pair up by rows (a last odd row is a
// job of one tile) and walk upward.
#ifndef HG_TRMM_BAND
#define HG_TRMM_BAND 4
#endif

// The tile of item `it` (job it/2, its first or second tile) of workgroup
// w, or the next item that has one (it is advanced past missing second
// tiles); false once the workgroup's jobs are done.
__device__ __forceinline__ bool fused_item(const GemmParams &p, int w, int G, int &it, int tiles_m,
                                           int tiles_n, TileInfo &T)
{
    const int P = tiles_n >> 1;                         // pair columns
    const int Jp = tiles_m * P;                         // pair jobs
    const int J = Jp + ((tiles_n & 1) ? (tiles_m + 1) >> 1 : 0);
    constexpr int R = HG_TRMM_BAND;
    for (;; ++it) {
        const int id = w + (it >> 1) * G, second = it & 1;
        if (id >= J)
            return false;
        const int per = J >> 3, rem = J & 7, x = id & 7;
        const int q = x * per + min(x, rem) + (id >> 3);
        int tm, tn;
        if (q < Jp) {
            const int band = q / (R * P);
            const int first = band * R;
            const int gsz = min(tiles_m - first, R);
            const int r = q - band * R * P;
            tm = first + r % gsz;
            const int c = r / gsz;
            tn = second ? c : tiles_n - 1 - c;
        } else {
            tm = 2 * (q - Jp) + second;
            if (tm >= tiles_m)
                continue;                               // a job of one tile
            tn = P;                                     // the middle column
        }
        const int N = p.e[0].N, K = p.e[0].K;
        const int m0 = tm * BM, n0 = tn * BN;
        T.batch = 0;
        T.m0 = m0;
        T.n0 = n0;
        T.N = N;
        T.K = K;
        T.rows_a = min(p.M - m0, BM);
        T.rows_b = min(N - n0, BN);
        const int kt0 = p.tri_up ? 0 : n0 / BK;
        T.nk = p.tri_up ? (n0 + BN) / BK : (K - n0) / BK;
        // The short tile of a pair job walks its stages downward.
        const bool down = q < Jp && second == (p.tri_up ? 1 : 0);
        T.kbase = down ? kt0 + T.nk - 1 : kt0;
        T.kdir = down ? -1 : 1;
        const _Float16 *Ab = p.A + (int64_t)m0 * p.lda;
        const _Float16 *Bb = p.B + (int64_t)n0 * p.ldb;
        T.ra = make_rsrc(Ab, (uint32_t)(((int64_t)(T.rows_a - 1) * p.lda + K) * 2));
        T.rb = make_rsrc(Bb, (uint32_t)(((int64_t)(T.rows_b - 1) * p.ldb + K) * 2));
        return true;
    }
}

template <bool OUT_F16, bool BETA, bool TRI, bool KCHK, bool FUSED, bool EPI, bool IN_BF16>
__global__ void __launch_bounds__(THREADS, 1)
hgemm_fast_kernel(const GemmParams p, int tiles_m, int tiles_n, int total, int cvec)
{
    __shared__ __attribute__((aligned(1024))) unsigned char smem[LDS_BYTES];

    // Lane index, re-materialised at every tile (see the top of the tile loop).
    int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const uint32_t lds_base = (uint32_t)reinterpret_cast<uintptr_t>(smem);
    const int stride = gridDim.x;

    // Load geometry: wave w fills tile rows RPW·w .. RPW·w+RPW-1 of A and of
    // B, RPI rows per instruction; lane l covers row RPI·i + (l div KC) of its
    // group, physical chunk l mod KC, so it fetches the logical chunk lkc[i]
    // that swz() puts there.
    int lkc[LPS];
    // Per-tile byte offsets of this lane's chunks (OOB for rows past the edge).
    uint32_t aoff[LPS], boff[LPS];
    auto set_offsets = [&](const TileInfo &T) {
#pragma unroll
        for (int i = 0; i < LPS; ++i) {
            // swz() XORs the chunk index, so it is its own inverse
            const int row = wave * RPW + i * RPI + lane / KC;
            lkc[i] = swz(row, lane % KC);
        }
        // row r of the wave's share: byte offset r·ld·2, stepping by RPI rows
        const int row0 = wave * RPW + lane / KC;
        const uint32_t a0 = (uint32_t)(row0 * (int)p.lda * 2), sa = (uint32_t)(RPI * (int)p.lda * 2);
        const uint32_t b0 = (uint32_t)(row0 * (int)p.ldb * 2), sb = (uint32_t)(RPI * (int)p.ldb * 2);
#pragma unroll
        for (int i = 0; i < LPS; ++i) {
            const int row = row0 + i * RPI;
            aoff[i] = row < T.rows_a ? a0 + i * sa + lkc[i] * 16 : OOB;
            boff[i] = row < T.rows_b ? b0 + i * sb + lkc[i] * 16 : OOB;
        }
    };
    // Load i of operand `isb` (A or B) of stage kt into that operand's ring
    // slot `slot`.  The stage's K offset is folded into the buffer resource
    // (base advanced, range shortened, both scalar), so the per-lane offset
    // stays the tile's constant and no vector instruction sits in front of
    // the load; a stage past the end of K gets an empty range and is
    // zero-filled, so the ring never needs a branch.  With KCHK (K not a
    // multiple of BK) the last stage is partial: each lane's chunk is checked
    // against K and chunks past it get the out-of-range offset.
    auto issue = [&](const TileInfo &T, bool isb, int kt, int slot, int i) {
        const uint32_t kb = (uint32_t)(T.kbase + T.kdir * kt) * RB;
        const uint32_t sbase = lds_base + (isb ? LDS_B : 0) + slot * SLOT + wave * RPW * RB;
        hg_int32x4 r = isb ? T.rb : T.ra;
        uint32_t off = isb ? boff[i] : aoff[i];
        if constexpr (KCHK) {
            const int kval = T.K - (T.kbase + T.kdir * kt) * BK;  // K % 8 == 0: chunks are all in or all out
            off = lkc[i] * 8 < kval ? off + kb : OOB;
        } else {
            const uint64_t base = ((uint64_t)(uint32_t)r[1] << 32 | (uint32_t)r[0]) + kb;
            r[0] = (int)(uint32_t)base;
            r[1] = (int)(uint32_t)(base >> 32);
            r[2] = kt < T.nk ? (int)((uint32_t)r[2] - kb) : 0;
        }
        hg_raw_buffer_load_lds(r, reinterpret_cast<hg_lds_u32 *>((uintptr_t)(sbase + i * 1024)), 16,
                               (int)off, 0, 0, 0);
    };
    // Every load of the first stages of tile T: A and B of stages 0 and 1
    // (the K loop issues the rest).
    auto prologue = [&](const TileInfo &T) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
            for (int i = 0; i < LPS; ++i)
                issue(T, false, st, st, i);
#pragma unroll
            for (int i = 0; i < LPS; ++i)
                issue(T, true, st, st, i);
        }
    };

    // Fragment of a 16×16×32 MFMA operand: row (lane mod 16) of a 16-row
    // block, logical chunk 4s + (lane div 16) of k-step s (8 consecutive k).
    // The same (lane, element) → k map is used for both operands, so the
    // MFMA contracts matching k.
    auto frag_ptr = [&](bool isb, int slot, int s, int blk) -> const half8 * {
        const int frow = lane & 15;
        const int fhi = lane >> 4;
        const int row = (isb ? wn * WTN : wm * WTM) + blk * FB + frow;
        return reinterpret_cast<const half8 *>(smem + (isb ? LDS_B : 0) + slot * SLOT + row * RB +
                                               swz(frow, KS / 8 * s + fhi) * 16);
    };
    floatx4 acc[TM][TN];
    // A fragments: one set per quarter parity (TMQ blocks each); B
    // fragments: one set per k-step of the stage (all TN blocks).
    half8 fa[2][TMQ], fb[SPS][TN];
    // TRI: the B operand's elements (j, k) with k < j (tri_up: k > j) lie in
    // the other triangle and must count as zero (NaN or Inf stored there
    // must not reach the MFMA).  Only the BN/BK stages of the tile's
    // diagonal block hold such elements.  Once this wave's loads of such a
    // stage have landed, and before the barrier that publishes the stage,
    // each lane zeroes them in its own B row of the stage in LDS (wave w
    // loaded rows RPW·w .. RPW·w + 63): the chunks wholly in the other
    // triangle are overwritten with zeros, the one chunk the diagonal
    // crosses is read, masked and written back.  With jr = (the row's global
    // index) - (the stage's first k), element k of the stage (0..63) is
    // zeroed when k < jr (tri_up: k > jr).
    auto zero_tri = [&](const TileInfo &T, int kt, int slot) {
        const int jr0 = __builtin_amdgcn_readfirstlane(T.n0 + wave * RPW - (T.kbase + T.kdir * kt) * BK);
        const bool up = p.tri_up != 0;
        if (up ? jr0 >= BK - 1 : jr0 + RPW - 1 <= 0)
            return;                                      // nothing to zero in this wave's rows
        const int row = wave * RPW + lane;
        const int jr = jr0 + lane;
        unsigned char *rp = smem + LDS_B + slot * SLOT + row * RB;
        const int kp = jr >> 3;                          // chunk holding k = jr (floor)
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            if (up ? kc > kp : kc < kp)
                *reinterpret_cast<u32x4 *>(rp + swz(row, kc) * 16) = u32x4{0, 0, 0, 0};
        }
        if (kp >= 0 && kp < KC) {
            const int e0 = jr & 7;                       // position of k = jr in its chunk
            u32x4 *cp = reinterpret_cast<u32x4 *>(rp + swz(row, kp) * 16);
            u32x4 w = *cp;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t m = up ? ((2 * d <= e0 ? 0x0000ffffu : 0u) | (2 * d + 1 <= e0 ? 0xffff0000u : 0u))
                                      : ((2 * d >= e0 ? 0x0000ffffu : 0u) | (2 * d + 1 >= e0 ? 0xffff0000u : 0u));
                w[d] &= m;
            }
            *cp = w;
        }
    };
    // Whether loop step kt of tile T is one of its diagonal block's stages:
    // the first BN/BK of its walk, or the last when it walks toward the
    // diagonal (tri_up upward, or lower downward).
    auto tri_stage = [&](const TileInfo &T, int kt) {
        return (p.tri_up != 0) != (T.kdir < 0) ? kt >= T.nk - BN / BK && kt < T.nk
                                               : kt < BN / BK && kt < T.nk;
    };

    int id = FUSED ? 0 : blockIdx.x;  // FUSED: the work item
    TileInfo T;
    if (FUSED ? !fused_item(p, blockIdx.x, stride, id, tiles_m, tiles_n, T)
              : !find_tile<TRI>(p, id, stride, total, tiles_m, tiles_n, T))
        return;
    set_offsets(T);
    prologue(T);

    const float alpha = p.alpha;
    const float beta = p.beta;
    const int64_t ldc = p.ldc;
    // Vector-memory operations an interior epilogue issues after the next
    // tile's prologue (its C_in loads and its stores; all lanes active).
    // The counter retires in issue order, so waiting until at most
    // (loads after stage 0) + EPI_OPS remain means stage 0 has landed while
    // the epilogue's stores are still draining.
    constexpr int EPI_OPS = TM * TN * (BETA ? 2 : 1);
    constexpr int VM_TILE0 = 2 * LPS;       // stage 1's loads, issued after stage 0's
    constexpr int VM_AFTER_EPI = VM_TILE0 + EPI_OPS < 63 ? VM_TILE0 + EPI_OPS : 63;
    int prev = 0;                      // 0: first tile, 1: after an interior epilogue, 2: after an edge one
    for (;;) {
        // Values derived from the lane index are recomputed per tile rather
        // than kept live across the epilogue (where the accumulators need
        // the register file).
        __asm__ volatile("" : "+v"(lane));
        // ---- K loop of tile T.  Stage t's A lives in A slot t mod 3, its B
        // in B slot t mod 2.  First: this wave's loads of stage 0 have
        // landed (an edge epilogue's stores vary per lane, so after one
        // everything is waited for), then everyone else's.
        if (prev == 0)
            wait_vmcnt<VM_TILE0>();
        else if (prev == 1)
            wait_vmcnt<VM_AFTER_EPI>();
        else
            wait_vmcnt<0>();
        if constexpr (TRI) {
            if (tri_stage(T, 0))
                zero_tri(T, 0, 0);
            wait_lgkmcnt<0>();
        }
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // Fragments of quarter 0: A blocks 0..TMQ-1 and every B block of
        // k-step 0.  Drained before the loop, so that the compiler's
        // counter waits inside the loop see only the loop's own reads.
#pragma unroll
        for (int f = 0; f < TMQ; ++f)
            fa[0][f] = *frag_ptr(false, 0, 0, f);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            fb[0][j] = *frag_ptr(true, 0, 0, j);
        wait_lgkmcnt<0>();
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = floatx4{0, 0, 0, 0};
        int as = 0, bs = 0;                       // A and B slots of stage kt
        for (int kt = 0; kt < T.nk; ++kt) {
            const int an = as == NSA - 1 ? 0 : as + 1;   // stage kt+1
            const int a2 = an == NSA - 1 ? 0 : an + 1;   // stage kt+2
            const int bn = bs ^ 1;
            static_for<NQ>([&](auto qc) __attribute__((always_inline)) {
                constexpr int q = decltype(qc)::value;
                constexpr int s = q >> 1, h = q & 1;
                // Ring loads of this quarter: operand, stage, slot, first index.
                constexpr bool lb = q >= 2;
                constexpr int lfirst = (q & 1) * (LPS / 2);
                const int lsl = lb ? bs : a2;
                // Reads of this quarter: A of quarter q+1 (set (q+1)%2, its
                // blocks, its k-step, the next stage's slot for q = 3); B
                // blocks (q%2)·TN/2 .. of the next k-step.
                constexpr int tq = (q + 1) & 3;
                constexpr int ra_set = tq & 1, ra_step = tq >> 1;
                constexpr int rb_step = q < 2 ? 1 : 0;
                const int ra_slot = q == 3 ? an : as;
                const int rb_slot = q < 2 ? bs : bn;
                static_for<PQ>([&](auto kc) __attribute__((always_inline)) {
                    constexpr int k = decltype(kc)::value;
                    if constexpr (q == 2 && k == BAR_K) {
                        // This wave's loads of stage kt+1 have landed (only the
                        // A loads of stage kt+2 may be in flight) and its reads
                        // of stage kt are complete: after the barrier every
                        // wave may read stage kt+1 and refill stage kt's B slot.
                        wait_vmcnt<LPS>();
                        if constexpr (TRI) {
                            if (tri_stage(T, kt + 1))
                                zero_tri(T, kt + 1, bn);
                        }
                        wait_lgkmcnt<0>();
                        __builtin_amdgcn_s_barrier();
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    // B block j outer; A blocks in snake order (reversed for odd
                    // j) so that every two consecutive MFMAs share an operand:
                    // fewer operand bits toggle, which under the board's power
                    // cap holds a slightly higher clock (1.3 % sustained at
                    // 8192³).  The products of one accumulator keep their order.
                    constexpr int j = k / TMQ, a = (j & 1) ? TMQ - 1 - k % TMQ : k % TMQ;
                    acc[h * TMQ + a][j] = mfma_16x16x32<IN_BF16>(fb[s][j], fa[h][a], acc[h * TMQ + a][j]);
                    constexpr int op = sched(q, k);
                    if constexpr (op >= kLD) {
                        issue(T, lb, kt + 2, lsl, lfirst + op - kLD);
                    } else if constexpr (op >= kRB) {
                        constexpr int jb = (q & 1) * (TN / 2) + op - kRB;
                        fb[rb_step][jb] = *frag_ptr(true, rb_slot, rb_step, jb);
                    } else if constexpr (op >= kRA) {
                        constexpr int f = op - kRA;
                        fa[ra_set][f] = *frag_ptr(false, ra_slot, ra_step, ra_set * TMQ + f);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                });
            });
            as = an;
            bs = bn;
        }
        // Ring drained (its last loads are zero fills past the end of K) and
        // every wave done with LDS: the slots are free for the next tile.
        wait_vmcnt<0>();
        wait_lgkmcnt<0>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);

        // EPI: this lane's 4 columns of each column block of an interior
        // tile.  Loaded before the next tile's prologue: the counter retires
        // in issue order, so loads issued after the prologue would also
        // wait for its two stages.
        float bv[EPI ? TN : 1][4];
        if constexpr (EPI) {
            if (T.rows_a == BM && T.rows_b == BN && cvec) {
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        bv[j][e] = p.bias ? p.bias[T.n0 + wn * WTN + j * FB + 4 * (lane >> 4) + e] : -0.0f;
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- Next tile's first stages, in flight during this epilogue.
        int nid = id + stride;
        TileInfo Tn;
        bool more;
        if constexpr (FUSED) {
            nid = id + 1;                 // the next item
            more = fused_item(p, blockIdx.x, stride, nid, tiles_m, tiles_n, Tn);
        } else {
            more = find_tile<TRI>(p, nid, stride, total, tiles_m, tiles_n, Tn);
        }
        if (more) {
            set_offsets(Tn);
            prologue(Tn);
        }
        __builtin_amdgcn_sched_barrier(0);   // those loads precede every epilogue access

        const int frow = lane & 15;
        const int fhi = lane >> 4;
        // ---- Epilogue of tile T.  Block (i, j) of the accumulators is Cᵀ
        // (the B fragment is the MFMA's first operand): lane covers row
        // m0 + wm·WTM + 16i + (lane mod 16) and columns
        // n0 + wn·WTN + 16j + 4·(lane div 16) + 0..3.
        // RD: the epilogue reads C (beta != 0).
        auto epilogue = [&](auto rdc) __attribute__((always_inline)) {
            constexpr bool RD = decltype(rdc)::value;
            // 16-bit C has the input's type (fp16 or bf16).
            typedef typename std::conditional<IN_BF16, __bf16, _Float16>::type e16;
            prev = T.rows_a == BM && T.rows_b == BN && cvec ? 1 : 2;
            if (prev == 1) {
                // Interior tile.  When C is read, its loads run CP row blocks
                // ahead of the stores (the fragment registers are free here),
                // so the epilogue waits on memory about TM/CP times, not TM.
                typedef typename std::conditional<IN_BF16, bf16x4, halfx4>::type vec16;
                typedef typename std::conditional<OUT_F16, vec16, floatx4>::type cvec;
                typedef typename std::conditional<OUT_F16, e16, float>::type celt;
                constexpr int CP = RD ? HG_FAST_EPI_PREFETCH : 1;
                cvec cin[CP][TN];
                auto crow = [&](int i) -> celt * {
                    const int row = T.m0 + wm * WTM + i * FB + frow;
                    return static_cast<celt *>(p.C) + p.e[T.batch].c_off + (int64_t)row * ldc +
                           T.n0 + wn * WTN + 4 * fhi;
                };
                if (RD) {
#pragma unroll
                    for (int i = 0; i < CP; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j)
                            cin[i][j] = *reinterpret_cast<const cvec *>(crow(i) + j * FB);
                }
                // With 128-column wave sub-tiles each 16-row block goes
                // through LDS (A ring slot 2, which the next tile's prologue
                // leaves free; 8 KiB per wave) so that each store instruction
                // writes two whole 128-column rows, i.e. complete 128-byte
                // lines, instead of a half (fp32) or quarter (16-bit) line in
                // each of 16 rows.  The number of stores is unchanged.
                constexpr bool STAGE = TN == 8;
                constexpr int UB = sizeof(cvec);       // one lane's 4 columns
                constexpr int SROW = 32 * UB;          // one staged 128-column row
                constexpr int SSW = OUT_F16 ? 2 : 1;   // bank swizzle: piece ^ (row · SSW)
                unsigned char *stg = smem + 2 * SLOT + wave * (FB * SROW);
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    pin_acc(acc[i]);
                    celt *cr = crow(i);
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        cvec r;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float v = acc[i][j][e];
                            float t = RD ? __builtin_fmaf(alpha, v, beta * (float)cin[i % CP][j][e])
                                         : alpha * v;
                            if constexpr (EPI)
                                t = epi_apply(t, bv[j][e], p.act);
                            if constexpr (OUT_F16 && TRI)
                                t = opaque_f32(t);   // the in-place TRMM: the fp32 result, rounded
                            r[e] = (celt)t;
                        }
                        if constexpr (STAGE)
                            *reinterpret_cast<cvec *>(stg + frow * SROW + ((4 * j + fhi) ^ (frow * SSW)) * UB) = r;
                        else
                            *reinterpret_cast<cvec *>(cr + j * FB) = r;
                    }
                    if constexpr (STAGE) {
                        // A wave's LDS accesses execute in issue order, so the
                        // reads see this block's writes; the fences keep the
                        // compiler from moving LDS accesses across.
                        __atomic_signal_fence(__ATOMIC_SEQ_CST);
                        // All reads of the block first, then the stores, so
                        // that the reads' latencies overlap; the store address
                        // advances by two rows at a time.
                        const int uu = lane & 31;
                        cvec v[TN];
#pragma unroll
                        for (int t = 0; t < TN; ++t) {
                            const int rr = 2 * t + (lane >> 5);
                            v[t] = *reinterpret_cast<const cvec *>(stg + rr * SROW + (uu ^ (rr * SSW)) * UB);
                        }
                        // row (lane div 32), column 4·(lane mod 32) of the block
                        celt *cd = crow(i) + ((lane >> 5) - frow) * ldc + 4 * (uu - fhi);
#pragma unroll
                        for (int t = 0; t < TN; ++t) {
                            *reinterpret_cast<cvec *>(cd) = v[t];
                            cd += 2 * ldc;
                        }
                        __atomic_signal_fence(__ATOMIC_SEQ_CST);
                    }
                    if (RD && i + CP < TM) {
#pragma unroll
                        for (int j = 0; j < TN; ++j)
                            cin[i % CP][j] = *reinterpret_cast<const cvec *>(crow(i + CP) + j * FB);
                    }
                }
            } else {
                // Edge tile: element-wise guarded stores.
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    pin_acc(acc[i]);
                    const int row = T.m0 + wm * WTM + i * FB + frow;
                    if (row >= p.M)
                        continue;
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const int col = T.n0 + wn * WTN + j * FB + 4 * fhi;
                        const int64_t off = p.e[T.batch].c_off + (int64_t)row * ldc + col;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if (col + e >= T.N)
                                continue;
                            const float v = acc[i][j][e];
                            const float b = EPI && p.bias ? p.bias[col + e] : -0.0f;
                            if (OUT_F16) {
                                e16 *cp = static_cast<e16 *>(p.C) + off + e;
                                float t = RD ? __builtin_fmaf(alpha, v, beta * (float)*cp) : alpha * v;
                                if constexpr (EPI)
                                    t = epi_apply(t, b, p.act);
                                if constexpr (TRI)
                                    t = opaque_f32(t);
                                *cp = (e16)t;
                            } else {
                                float *cp = static_cast<float *>(p.C) + off + e;
                                float t = RD ? __builtin_fmaf(alpha, v, beta * *cp) : alpha * v;
                                if constexpr (EPI)
                                    t = epi_apply(t, b, p.act);
                                *cp = t;
                            }
                        }
                    }
                }
            }
        };
        epilogue(std::integral_constant<bool, BETA>{});
        if (!more)
            break;
        T = Tn;
        id = nid;
    }
}

}  // namespace

// Persistent grid size: one workgroup per CU (the 160 KiB ring allows one).
// The count is cached per device; concurrent first calls may both query it
// and store the same value (relaxed atomics: no data race).
int cu_count()
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

namespace {

template <bool OUT_F16, bool BETA, bool TRI, bool EPI, bool IN_BF16 = false>
hipError_t launch(const GemmParams &p, hipStream_t stream)
{
    int maxN = 0;
    for (int b = 0; b < p.nbatch; ++b)
        maxN = p.e[b].N > maxN ? p.e[b].N : maxN;
    const int tiles_m = (p.M + BM - 1) / BM;
    const int tiles_n = (maxN + BN - 1) / BN;
    const int64_t total64 = (int64_t)tiles_m * tiles_n * p.nbatch;
    if (total64 <= 0)
        return hipSuccess;
    if (total64 > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    const uintptr_t align = OUT_F16 ? 8 : 16;
    int cvec = (reinterpret_cast<uintptr_t>(p.C) % align == 0) && (p.ldc % 4 == 0);
    for (int b = 0; b < p.nbatch; ++b)
        cvec = cvec && (p.e[b].c_off % 4 == 0);
    // Persistent grid (one workgroup per CU, a multiple of 8 so that every
    // workgroup's strided tile ids stay on its own XCD) for short K, where
    // the per-tile prologue and epilogue are a large share of a tile; long-K
    // tiles run one workgroup per tile.
    int maxK = 0;
    for (int b = 0; b < p.nbatch; ++b)
        maxK = p.e[b].K > maxK ? p.e[b].K : maxK;
    int64_t grid = total64;
    if (maxK < HG_FAST_PERSIST_MAXK) {
        grid = cu_count();
        grid = grid / 8 * 8 > 0 ? grid / 8 * 8 : grid;
        if (grid > total64)
            grid = total64;
    }
    bool kchk = false;
    for (int b = 0; b < p.nbatch; ++b)
        kchk = kchk || p.e[b].K % BK != 0;
    if (kchk)
        hipLaunchKernelGGL((hgemm_fast_kernel<OUT_F16, BETA, TRI, true, false, EPI, IN_BF16>), dim3((unsigned)grid),
                           dim3(THREADS), 0, stream, p, tiles_m, tiles_n, (int)total64, cvec);
    else
        hipLaunchKernelGGL((hgemm_fast_kernel<OUT_F16, BETA, TRI, false, false, EPI, IN_BF16>), dim3((unsigned)grid),
                           dim3(THREADS), 0, stream, p, tiles_m, tiles_n, (int)total64, cvec);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_trmm_fused(const GemmParams &p, hipStream_t stream, bool out_f16)
{
    const int tiles_m = (p.M + BM - 1) / BM;
    const int tiles_n = p.e[0].N / BN;
    const int64_t total64 = (int64_t)tiles_m * tiles_n;
    if (total64 <= 0)
        return hipSuccess;
    if (total64 > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    const int cvec = reinterpret_cast<uintptr_t>(p.C) % (out_f16 ? 8 : 16) == 0 && p.ldc % 4 == 0;
    // one persistent workgroup per CU, at most one per job (see fused_item)
    const int64_t jobs = (int64_t)tiles_m * (tiles_n / 2) + ((tiles_n & 1) ? (tiles_m + 1) / 2 : 0);
    int64_t grid = cu_count();
    grid = grid / 8 * 8 > 0 ? grid / 8 * 8 : grid;
    if (grid > jobs)
        grid = jobs;
    if (out_f16)
        hipLaunchKernelGGL((hgemm_fast_kernel<true, false, true, false, true, false, false>), dim3((unsigned)grid),
                           dim3(THREADS), 0, stream, p, tiles_m, tiles_n, (int)total64, cvec);
    else
        hipLaunchKernelGGL((hgemm_fast_kernel<false, false, true, false, true, false, false>), dim3((unsigned)grid),
                           dim3(THREADS), 0, stream, p, tiles_m, tiles_n, (int)total64, cvec);
    return hipGetLastError();
}

bool trmm_fused_ok(const GemmParams &p)
{
    if (p.lda > (1 << 21) || p.ldb > (1 << 21) || p.leaf < BN)
        return false;
    // One persistent workgroup per tile at a time: with fewer than two tiles
    // per CU (skinny B: m = 256 gives 16 tiles at n = 4096) the per-level
    // launches, which spread every level over its own grid, are 2–3× faster.
    const int64_t tiles = (int64_t)((p.M + BM - 1) / BM) * (p.e[0].N / BN);
    if (tiles < 2 * (int64_t)cu_count())
        return false;
    if (reinterpret_cast<uintptr_t>(p.A) % 16 != 0 || reinterpret_cast<uintptr_t>(p.B) % 16 != 0 ||
        p.lda % 8 != 0 || p.ldb % 8 != 0)
        return false;
    // Every recursion boundary on a tile edge (and a multiple of BK).
    const int n = p.e[0].N;
    if (n % BN != 0)
        return false;
    struct Frame {
        int o, s;
    };
    Frame st[64];
    int top = 0;
    st[top++] = {0, n};
    while (top > 0) {
        const Frame f = st[--top];
        if (f.o % BN != 0 || f.s % BN != 0)
            return false;
        if (f.s <= p.leaf)
            continue;
        const int h = f.s / 2;
        if (top + 2 > 64)
            return false;
        st[top++] = {f.o, h};
        st[top++] = {f.o + h, f.s - h};
    }
    return true;
}

bool fast_path_ok(const GemmParams &p, const LaunchOpts &o)
{
    if (!o.vec || (o.tri && (o.out_f16 || o.beta_read || o.epi)) || (o.in_bf16 && o.tri))
        return false;
    // 32-bit buffer offsets: every tile's byte range must stay below 2^31.
    if (p.lda > (1 << 21) || p.ldb > (1 << 21))
        return false;
    for (int b = 0; b < p.nbatch; ++b)
        if (p.e[b].K % 8 != 0)
            return false;
    return true;
}

hipError_t launch_gemm_fast(const GemmParams &p, const LaunchOpts &o, hipStream_t stream)
{
    if (o.tri)
        return launch<false, false, true, false>(p, stream);     // TRMM leaves: fp32, written once
    if (o.in_bf16) {
        if (o.epi) {
            if (o.out_f16)
                return o.beta_read ? launch<true, true, false, true, true>(p, stream)
                                   : launch<true, false, false, true, true>(p, stream);
            return o.beta_read ? launch<false, true, false, true, true>(p, stream)
                               : launch<false, false, false, true, true>(p, stream);
        }
        if (o.out_f16)
            return o.beta_read ? launch<true, true, false, false, true>(p, stream)
                               : launch<true, false, false, false, true>(p, stream);
        return o.beta_read ? launch<false, true, false, false, true>(p, stream)
                           : launch<false, false, false, false, true>(p, stream);
    }
    if (o.epi) {
        if (o.out_f16)
            return o.beta_read ? launch<true, true, false, true>(p, stream)
                               : launch<true, false, false, true>(p, stream);
        return o.beta_read ? launch<false, true, false, true>(p, stream)
                           : launch<false, false, false, true>(p, stream);
    }
    if (o.out_f16)
        return o.beta_read ? launch<true, true, false, false>(p, stream)
                           : launch<true, false, false, false>(p, stream);
    return o.beta_read ? launch<false, true, false, false>(p, stream)
                       : launch<false, false, false, false>(p, stream);
}

}  // namespace hg
