// hg_fast.hip — the 256×256 fast path of the half-precision GEMM on gfx950.
//
// Same computation and layouts as the general kernel in hg_kernels.hip
// (C = alpha·A·B + beta·C, A M×K row-major, B K×N column-major, fp16 in,
// fp32 accumulate; "Nvidia Tensor Core-MMA PTX编程入门" §4 and the masked
// tiled matmul of "GPU架构与CUDA" 共享内存与分块), for operands whose rows
// are 16-byte aligned and K a multiple of 8; with TRI it is also the
// triangle-masked leaf of the recursive TRMM ("异构计算中高性能TRMM与TRSM的
// 递归算法实现" §2.2).  Design:
//
//  * One workgroup = 4 waves (2×2) per 256×256 tile; each wave owns a
//    128×128 sub-tile = 4×4 blocks of v_mfma_f32_32x32x16_f16, 256 fp32
//    accumulators per lane (the AGPR file).
//  * K is walked in BK = 64 stages: one 128-byte cache line per operand row,
//    so every L1→L2 request is a whole line (32-wide stages split each line
//    over two requests, which doubled the request rate and the TA stalls).
//    Operands reach LDS through the gfx950 direct buffer→LDS path
//    (buffer_load_dwordx4 … lds; each wave instruction moves 8 rows × 128
//    bytes): no staging registers, no ds_write.  Lane l fetches the logical
//    16-byte chunk that the XOR swizzle places at position l, so the LDS
//    image is already swizzled for the fragment reads.
//  * The 160 KiB of LDS hold a 3-slot ring of A stages and a 2-slot ring of
//    B stages (32 KiB each).  The extra A slot lets A loads run two stages
//    ahead, so each k-step carries the same number of ring loads (4 per
//    wave, evenly spaced) while every load still has at least three k-steps
//    to land; one barrier per stage, in front of its last k-step.
//  * Ragged M/N edges and the K tail are zero-filled by the buffer unit's
//    range check (out-of-range rows and chunks get an offset past the
//    resource size, which loads as zero): no branches in the main loop.
//  * Fragments are double-buffered in registers; within a k-step each MFMA
//    is followed by at most one LDS fragment read (for the next k-step) or
//    one ring load, in a fixed program order.
//  * Persistent workgroups (short K): one per CU walks a strided list of
//    tiles; the next tile's first stages are requested before the current
//    tile's epilogue, so loads overlap the stores.
//
// Workgroup→tile order: tile ids are regrouped per XCD (consecutive
// workgroup ids run on different XCDs, each with its own L2), then each
// XCD's range is walked in bands of 4 tile rows, column by column, so the
// tiles resident on one XCD share A row panels and B column panels.
#include "hg_internal.h"

typedef int32_t hg_int32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint32_t hg_lds_u32;

// The raw buffer→LDS load (LLVM intrinsic; 16 bytes per lane on gfx950).
extern "C" __device__ void hg_raw_buffer_load_lds(hg_int32x4 rsrc, hg_lds_u32 *lds, int size,
                                                  int voffset, int soffset, int offset,
                                                  int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

namespace hg {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Tunables (compile-time).  K is walked in BK = 64 stages (one 128-byte
// cache line per operand row), two LDS stages of 64 KiB; the wave layout is
// WM × WN.
#ifndef HG_FAST_WM
#define HG_FAST_WM 2
#endif
#ifndef HG_FAST_WN
#define HG_FAST_WN 2
#endif
#ifndef HG_FAST_XCD
#define HG_FAST_XCD 1
#endif
#ifndef HG_FAST_PERSIST_MAXK
#define HG_FAST_PERSIST_MAXK 4096
#endif
#ifndef HG_FAST_GROUP
#define HG_FAST_GROUP 4
#endif
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int NSA = 3, NSB = 2;             // LDS slots of the A and B rings
constexpr int WM = HG_FAST_WM, WN = HG_FAST_WN, NW = WM * WN;   // waves per workgroup
constexpr int THREADS = NW * 64;
constexpr int WTM = BM / WM, WTN = BN / WN;                     // wave sub-tile
constexpr int TM = WTM / 32, TN = WTN / 32;                     // 32×32 blocks per wave
constexpr int RB = BK * 2;                  // bytes per LDS row (128: one cache line)
constexpr int KC = BK / 8;                  // 16-byte chunks per row (8)
constexpr int RPL = 256 / RB;               // rows per 256-byte bank line (64 banks)
constexpr int RPI = 1024 / RB;              // rows per buffer→LDS wave instruction (8)
constexpr int RPW = BM / NW;                // tile rows each wave loads, per operand
constexpr int LPS = RPW / RPI;              // load instructions per wave per operand per stage
constexpr int SPS = BK / 16;                // MFMA k-steps per stage (4)
constexpr int SLOT = BM * RB;               // bytes of one operand's stage (32 KiB)
constexpr int LDS_B = NSA * SLOT;           // B ring after the A ring
constexpr int LDS_BYTES = (NSA + NSB) * SLOT;
constexpr uint32_t OOB = 0x80000000u;       // offset that the range check rejects
constexpr int P = TM * TN;                  // MFMAs per k-step
constexpr int R = TM + TN;                  // fragment reads per k-step
constexpr int LH = LPS / 2;                 // loads per k-step
static_assert(SPS == 4 && BM == BN, "");
static_assert(LPS * RPI == RPW && LPS % 2 == 0 && TM >= 2 && TN >= 1, "");
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
static_assert(P >= R + LH, "one fragment read or ring load per MFMA");

// Physical 16-byte chunk of logical chunk kc in LDS row r.  The LDS serves a
// 16-byte read for 16 lanes per cycle over 64 four-byte banks (256 bytes);
// a fragment read has 16 consecutive rows at one logical chunk, which this
// XOR spreads over 16 distinct bank groups.
__device__ __forceinline__ int swz(int r, int kc) { return kc ^ ((r / RPL) & (KC - 1)); }

// Fragment read order within a k-step: A block 0, then every B block, then
// A blocks 1..TM-1 -- the order in which the MFMAs (block row i outer, block
// column j inner) first use them.  f < TM is A block f, else B block f - TM.
__device__ __forceinline__ constexpr int read_order(int o)
{
    return o == 0 ? 0 : (o <= TN ? TM + o - 1 : o - TN);
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
    int batch, m0, n0, N, K, rows_a, rows_b, kt0, nk;
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
        T.kt0 = TRI ? n0 / BK : 0;
        T.nk = (T.K + BK - 1) / BK - T.kt0;
        const _Float16 *Ab = p.A + p.e[batch].a_off + (int64_t)m0 * p.lda;
        const _Float16 *Bb = p.B + p.e[batch].b_off + (int64_t)n0 * p.ldb;
        T.ra = make_rsrc(Ab, (uint32_t)(((int64_t)(T.rows_a - 1) * p.lda + T.K) * 2));
        T.rb = make_rsrc(Bb, (uint32_t)(((int64_t)(T.rows_b - 1) * p.ldb + T.K) * 2));
        return true;
    }
    return false;
}

template <bool OUT_F16, bool BETA, bool TRI>
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
            const int row = wave * RPW + i * RPI + lane / KC;
            int kc = 0;
#pragma unroll
            for (int c = 0; c < KC; ++c)
                kc = swz(row, c) == lane % KC ? c : kc;
            lkc[i] = kc;
        }
#pragma unroll
        for (int i = 0; i < LPS; ++i) {
            const int row = wave * RPW + i * RPI + lane / KC;
            aoff[i] = row < T.rows_a ? (uint32_t)(row * (int)p.lda * 2 + lkc[i] * 16) : OOB;
            boff[i] = row < T.rows_b ? (uint32_t)(row * (int)p.ldb * 2 + lkc[i] * 16) : OOB;
        }
    };
    // Loads q = first .. first+count-1 of operand `isb` (A or B) of stage
    // kt into that operand's ring slot `slot`.  A stage past the end of K
    // has kval <= 0, so every lane gets the out-of-range offset and the slot
    // is zero-filled: the ring never needs a branch.
    auto issue = [&](const TileInfo &T, bool isb, int kt, int slot, int first, int count) {
        const uint32_t kb = (uint32_t)(T.kt0 + kt) * RB;
        const int kval = T.K - (T.kt0 + kt) * BK;  // K % 8 == 0: chunks are all in or all out
        const uint32_t sbase = lds_base + (isb ? LDS_B : 0) + slot * SLOT + wave * RPW * RB;
#pragma unroll
        for (int i = first; i < first + count; ++i) {
            const uint32_t off = lkc[i] * 8 < kval ? (isb ? boff[i] : aoff[i]) + kb : OOB;
            hg_raw_buffer_load_lds(isb ? T.rb : T.ra,
                                   reinterpret_cast<hg_lds_u32 *>((uintptr_t)(sbase + i * 1024)),
                                   16, (int)off, 0, 0, 0);
        }
    };
    // Every load of the first stages of tile T: A and B of stage 0, A of
    // stage 1 and the first half of B of stage 1 (the K loop issues the rest).
    auto prologue = [&](const TileInfo &T) {
        issue(T, false, 0, 0, 0, LPS);
        issue(T, true, 0, 0, 0, LPS);
        issue(T, false, 1, 1, 0, LPS);
        issue(T, true, 1, 1, 0, LH);
    };

    // Fragment reads: row (lane mod 32) of each 32-row block, logical chunk
    // 2s + (lane div 32) of k-step s.  The same (lane, element) → k map is
    // used for both operands, so the MFMA contracts matching k.
    auto frag_addr = [&](int slot, int s, bool isb) -> const unsigned char * {
        const int frow = lane & 31;
        const int fhi = lane >> 5;
        const int row0 = isb ? wn * WTN : wm * WTM;
        return smem + (isb ? LDS_B : 0) + slot * SLOT + (row0 + frow) * RB +
               swz(frow, 2 * s + fhi) * 16;
    };
    floatx16 acc[TM][TN];
    // Fragments are double-buffered: the next k-step's are read into the
    // other set while this k-step's MFMAs run.
    half8 fa[2][TM], fb[2][TN];
    // Fragment f of k-step s: f < TM is A block f, else B block f - TM.
    auto read_frag = [&](int fs, int aslot, int bslot, int s, int f) {
        if (f < TM)
            fa[fs][f] = *reinterpret_cast<const half8 *>(frag_addr(aslot, s, false) + f * 32 * RB);
        else
            fb[fs][f - TM] =
                *reinterpret_cast<const half8 *>(frag_addr(bslot, s, true) + (f - TM) * 32 * RB);
    };
    // TRI: zero the B fragment elements (j, k) with k < j.  Fragment j of
    // k-step s holds row jrow = n0 + wn·WTN + 32j + (lane mod 32) and the 8
    // k from kfirst = (kt0+kt)·BK + 16s + 8·(lane div 32); the first
    // clamp(jrow - kfirst, 0, 8) of them are zeroed by a select (so NaN or
    // Inf stored above the diagonal cannot reach the MFMA).
    auto mask_tri = [&](const TileInfo &T, int fs, int kt, int s) {
        const int frow = lane & 31;
        const int fhi = lane >> 5;
        const int kfirst = (T.kt0 + kt) * BK + 16 * s + 8 * fhi;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int t = T.n0 + wn * WTN + j * 32 + frow - kfirst;   // elements to zero
            u32x4 w = __builtin_bit_cast(u32x4, fb[fs][j]);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t m = (2 * d >= t ? 0x0000ffffu : 0u) | (2 * d + 1 >= t ? 0xffff0000u : 0u);
                w[d] &= m;
            }
            fb[fs][j] = __builtin_bit_cast(half8, w);
        }
    };

    int id = blockIdx.x;
    TileInfo T;
    if (!find_tile<TRI>(p, id, stride, total, tiles_m, tiles_n, T))
        return;
    set_offsets(T);
    prologue(T);

    const float alpha = p.alpha;
    const float beta = p.beta;
    const int64_t ldc = p.ldc;
    // Vector-memory operations an interior epilogue issues after the next
    // tile's first slices (its C_in loads and its stores; all lanes active).
    // The counter retires in issue order, so waiting until at most
    // (first-slice loads) + EPI_OPS remain means slice 0 has landed while
    // the epilogue's stores are still draining.
    constexpr int EPI_OPS = TM * TN * 4 * (BETA ? 2 : 1);
    constexpr int VM_TILE0 = LPS + LH;  // stage 1's loads, issued after stage 0's
    constexpr int VM_AFTER_EPI = VM_TILE0 + EPI_OPS < 63 ? VM_TILE0 + EPI_OPS : 63;
    int prev = 0;                      // 0: first tile, 1: after an interior epilogue, 2: after an edge one
    for (;;) {
        // Values derived from the lane index are recomputed per tile rather
        // than kept live across the epilogue (where the accumulators need
        // the register file).
        __asm__ volatile("" : "+v"(lane));
        // ---- K loop of tile T.  Stage t's A lives in A slot t mod 3, its B
        // in B slot t mod 2.  A slot t mod 3 is free after the barrier in
        // stage t-3 (in front of its last k-step, when every wave has
        // finished reading stage t-3), B slot t mod 2 after the one in stage
        // t-2.  Each k-step of stage kt carries LH ring loads: k-step 3 (after
        // the barrier) the first half of B of stage kt+2, k-step 0 the second
        // half of B of stage kt+1, k-steps 1 and 2 the A of stage kt+2.  The
        // barrier of stage kt publishes stage kt+1 (whose last loads were
        // issued in k-step 0), so every load has at least three k-steps to
        // land.  First: this wave's loads of stage 0 have landed (an edge
        // epilogue's stores vary per lane, so after one everything is waited
        // for), then everyone else's.
        if (prev == 0)
            wait_vmcnt<VM_TILE0>();
        else if (prev == 1)
            wait_vmcnt<VM_AFTER_EPI>();
        else
            wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int f = 0; f < R; ++f)
            read_frag(0, 0, 0, 0, f);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = floatx16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
        int as = 0, bs = 0;                       // A and B slots of stage kt
        for (int kt = 0; kt < T.nk; ++kt) {
            const int an = as == NSA - 1 ? 0 : as + 1;   // stage kt+1
            const int a2 = an == NSA - 1 ? 0 : an + 1;   // stage kt+2
            const int bn = bs ^ 1;
#pragma unroll
            for (int s = 0; s < SPS; ++s) {
                const bool last = s == SPS - 1;
                if (last) {
                    // This wave's loads of stage kt+1 have landed (only the A
                    // loads of stage kt+2 may be in flight) and its reads of
                    // stage kt are complete: after the barrier every wave may
                    // read stage kt+1 and refill stage kt's slots.
                    wait_vmcnt<LPS>();
                    wait_lgkmcnt<0>();
                    __builtin_amdgcn_s_barrier();
                    __builtin_amdgcn_sched_barrier(0);
                }
                const int ra = last ? an : as;     // where the next fragments come from
                const int rb = last ? bn : bs;
                const int rstep = last ? 0 : s + 1;
                const int fs = s & 1;
                if (TRI)
                    mask_tri(T, fs, kt, s);
                // Ring loads of this k-step: operand, stage, slot, first index.
                const bool lb = s == 0 || s == 3;
                const int lkt = s == 0 ? kt + 1 : kt + 2;
                const int lsl = s == 0 ? bn : s == 3 ? bs : a2;
                const int lfirst = s == 0 || s == 2 ? LH : 0;
#pragma unroll
                for (int k = 0; k < P; ++k) {
                    acc[k / TN][k % TN] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        fb[fs][k % TN], fa[fs][k / TN], acc[k / TN][k % TN], 0, 0, 0);
                    // After MFMA k: one ring load every P/LH MFMAs (from the
                    // second on), the next k-step's fragments after the
                    // others, in the order the next k-step consumes them.
                    constexpr int GAP = P / LH;
                    if (k % GAP == GAP / 2 && k / GAP < LH)
                        issue(T, lb, lkt, lsl, lfirst + k / GAP, 1);
                    else {
                        const int o = k - (k >= GAP / 2 ? 1 + (k - GAP / 2) / GAP : 0);
                        if (o < R)
                            read_frag(fs ^ 1, ra, rb, rstep, read_order(o));
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            as = an;
            bs = bn;
        }
        // Ring drained (its last loads are zero fills past the end of K) and
        // every wave done with LDS: the slots are free for the next tile.
        wait_vmcnt<0>();
        wait_lgkmcnt<0>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);

        // ---- Next tile's first slices, in flight during this epilogue.
        int nid = id + stride;
        TileInfo Tn;
        const bool more = find_tile<TRI>(p, nid, stride, total, tiles_m, tiles_n, Tn);
        if (more) {
            set_offsets(Tn);
            prologue(Tn);
        }
        __builtin_amdgcn_sched_barrier(0);   // those loads precede every epilogue access

        const int frow = lane & 31;
        const int fhi = lane >> 5;
        // ---- Epilogue of tile T.  Block (i, j) of the accumulators is Cᵀ
        // (the B fragment is the MFMA's first operand): lane covers row
        // m0 + wm·WTM + 32i + (lane mod 32) and, for register group g,
        // columns n0 + wn·WTN + 32j + 8g + 4·(lane div 32) + 0..3.
        prev = T.rows_a == BM && T.rows_b == BN && cvec ? 1 : 2;
        if (prev == 1) {
            // Interior tile: one row block at a time, all of its C_in loads
            // (beta != 0) issued before any of its stores.
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = T.m0 + wm * WTM + i * 32 + frow;
                const int64_t roff =
                    p.e[T.batch].c_off + (int64_t)row * ldc + T.n0 + wn * WTN + 4 * fhi;
                if (OUT_F16) {
                    _Float16 *cr = static_cast<_Float16 *>(p.C) + roff;
                    halfx4 cin[TN][4];
                    if (BETA) {
#pragma unroll
                        for (int j = 0; j < TN; ++j)
#pragma unroll
                            for (int g = 0; g < 4; ++g)
                                cin[j][g] = *reinterpret_cast<const halfx4 *>(cr + j * 32 + 8 * g);
                    }
#pragma unroll
                    for (int j = 0; j < TN; ++j)
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            halfx4 h;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float v = acc[i][j][4 * g + e];
                                h[e] = (_Float16)(BETA ? __builtin_fmaf(alpha, v, beta * (float)cin[j][g][e])
                                                       : alpha * v);
                            }
                            *reinterpret_cast<halfx4 *>(cr + j * 32 + 8 * g) = h;
                        }
                } else {
                    float *cr = static_cast<float *>(p.C) + roff;
                    floatx4 cin[TN][4];
                    if (BETA) {
#pragma unroll
                        for (int j = 0; j < TN; ++j)
#pragma unroll
                            for (int g = 0; g < 4; ++g)
                                cin[j][g] = *reinterpret_cast<const floatx4 *>(cr + j * 32 + 8 * g);
                    }
#pragma unroll
                    for (int j = 0; j < TN; ++j)
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            floatx4 r;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float v = acc[i][j][4 * g + e];
                                r[e] = BETA ? __builtin_fmaf(alpha, v, beta * cin[j][g][e]) : alpha * v;
                            }
                            *reinterpret_cast<floatx4 *>(cr + j * 32 + 8 * g) = r;
                        }
                }
            }
        } else {
            // Edge tile: element-wise guarded stores.
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = T.m0 + wm * WTM + i * 32 + frow;
                if (row >= p.M)
                    continue;
#pragma unroll
                for (int j = 0; j < TN; ++j) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int col = T.n0 + wn * WTN + j * 32 + 8 * g + 4 * fhi;
                        const int64_t off = p.e[T.batch].c_off + (int64_t)row * ldc + col;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if (col + e >= T.N)
                                continue;
                            const float v = acc[i][j][4 * g + e];
                            if (OUT_F16) {
                                _Float16 *cp = static_cast<_Float16 *>(p.C) + off + e;
                                *cp = (_Float16)(BETA ? __builtin_fmaf(alpha, v, beta * (float)*cp)
                                                      : alpha * v);
                            } else {
                                float *cp = static_cast<float *>(p.C) + off + e;
                                *cp = BETA ? __builtin_fmaf(alpha, v, beta * *cp) : alpha * v;
                            }
                        }
                    }
                }
            }
        }
        if (!more)
            break;
        T = Tn;
        id = nid;
    }
}

// Persistent grid size: one workgroup per CU (the 128 KiB ring allows one).
int cu_count()
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <bool OUT_F16, bool BETA, bool TRI>
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
    hipLaunchKernelGGL((hgemm_fast_kernel<OUT_F16, BETA, TRI>), dim3((unsigned)grid), dim3(THREADS),
                       0, stream, p, tiles_m, tiles_n, (int)total64, cvec);
    return hipGetLastError();
}

}  // namespace

bool fast_path_ok(const GemmParams &p, const LaunchOpts &o)
{
    if (!o.vec || (o.tri && (o.out_f16 || o.beta_read)))
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
        return launch<false, false, true>(p, stream);     // TRMM leaves: fp32, written once
    if (o.out_f16)
        return o.beta_read ? launch<true, true, false>(p, stream)
                           : launch<true, false, false>(p, stream);
    return o.beta_read ? launch<false, true, false>(p, stream)
                       : launch<false, false, false>(p, stream);
}

}  // namespace hg
