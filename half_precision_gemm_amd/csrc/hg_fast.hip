// hg_fast.hip — the 256×256 fast path of the half-precision GEMM on gfx950.
//
// Same computation and layouts as the general kernel in hg_kernels.hip
// (C = alpha·A·B + beta·C, A M×K row-major, B K×N column-major, fp16 in,
// fp32 accumulate; "Nvidia Tensor Core-MMA PTX编程入门" §4 and the masked
// tiled matmul of "GPU架构与CUDA" 共享内存与分块), for operands whose rows
// are 16-byte aligned and K a multiple of 8.  What differs:
//
//  * Global→LDS staging uses the gfx950 direct buffer→LDS path
//    (buffer_load_dwordx4 … lds): no staging registers and no ds_write.
//    Each wave instruction moves 8 rows × 128 bytes; lane l fetches the
//    logical 16-byte chunk (l mod 8) XOR (row mod 8) of its row, so the
//    contiguous LDS image is already XOR-swizzled for the fragment reads.
//  * Ragged M/N edges and the K tail are zero-filled by the buffer unit's
//    range check: out-of-range rows and chunks get an offset past the
//    resource's size, which loads as zero.  No branches in the main loop.
//  * The K loop is software pipelined: the buffer→LDS loads of slice t+1
//    are issued at the top of slice t, MFMA operand fragments of k-step s+1
//    are read from LDS while the 16 MFMAs of k-step s run, and the barrier
//    that hands over the next slice sits in the middle of the last k-step so
//    that its first fragments are already in flight when the slice starts.
//
// One workgroup = 4 waves (2×2) computes a 256×256 tile; each wave owns a
// 128×128 sub-tile = 4×4 blocks of v_mfma_f32_32x32x16_f16, 256 fp32
// accumulators per lane (the AGPR file).  Two LDS stages of 64 KiB each.
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

// Slice depth and ring depth.  BK = 32 with 4 stages keeps three slices in
// flight (about 3000 MFMA cycles of cover for the global latency) in 128 KiB
// of LDS; BK = 64 with 2 stages is the shallow alternative.
#ifndef HG_FAST_BK
#define HG_FAST_BK 32
#endif
#ifndef HG_FAST_NST
#define HG_FAST_NST 4
#endif

#ifndef HG_FAST_WM
#define HG_FAST_WM 2
#endif
#ifndef HG_FAST_WN
#define HG_FAST_WN 2
#endif

constexpr int BM = 256, BN = 256, BK = HG_FAST_BK, NST = HG_FAST_NST;
constexpr int D = NST - 1;                  // prefetch distance in slices
static_assert(D >= 2, "slice kt+1 must be fully issued before iteration kt");
constexpr int WM = HG_FAST_WM, WN = HG_FAST_WN, NW = WM * WN;   // waves per workgroup
constexpr int THREADS = NW * 64;
constexpr int WTM = BM / WM, WTN = BN / WN;                     // wave sub-tile
constexpr int TM = WTM / 32, TN = WTN / 32;                     // 32×32 blocks per wave
constexpr int RB = BK * 2;                  // bytes per LDS row
constexpr int KC = BK / 8;                  // 16-byte chunks per row
#ifndef HG_FAST_RPL
#define HG_FAST_RPL (256 / (HG_FAST_BK * 2))
#endif
constexpr int RPL = HG_FAST_RPL;             // rows per 256-byte bank line (64 banks)
constexpr int RPI = 1024 / RB;              // rows per buffer→LDS wave instruction
constexpr int RPW = BM / NW;                // tile rows each wave loads, per operand
constexpr int LPS = RPW / RPI;              // load instructions per wave per operand
constexpr int SPS = BK / 16;                // MFMA k-steps per slice
constexpr int LDS_A = BM * RB;
constexpr int LDS_STAGE = LDS_A + BN * RB;
constexpr uint32_t OOB = 0x80000000u;       // offset that the range check rejects
static_assert(BK == 32 || BK == 64, "");
static_assert(LPS * RPI == RPW && TM >= 2 && TN >= 1, "");
static_assert(NST >= 2 && NST * LDS_STAGE <= 160 * 1024, "LDS budget");

// Physical 16-byte chunk of logical chunk kc in LDS row r.  The LDS serves a
// 16-byte read for 16 lanes per cycle over 64 four-byte banks (256 bytes);
// a fragment read has 16 consecutive rows at one logical chunk, which this
// XOR spreads over 16 distinct bank groups.
__device__ __forceinline__ int swz(int r, int kc) { return kc ^ ((r / RPL) & (KC - 1)); }

// s_waitcnt vmcnt(n) only (expcnt and lgkmcnt left at their maxima).
template <int n>
__device__ __forceinline__ void wait_vmcnt()
{
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}
// s_waitcnt lgkmcnt(n) only.
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

#ifndef HG_FAST_XCD
#define HG_FAST_XCD 1
#endif
#ifndef HG_FAST_GROUP
#define HG_FAST_GROUP 4
#endif

__device__ __forceinline__ void map_tile(int wg, int total, int tiles_m, int tiles_n, int &batch,
                                         int &tm, int &tn)
{
    const int per = total >> 3, rem = total & 7;
    const int x = wg & 7;
    const int q = HG_FAST_XCD ? x * per + min(x, rem) + (wg >> 3) : wg;
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

template <bool OUT_F16, bool BETA>
__global__ void __launch_bounds__(THREADS, 1)
hgemm_fast_kernel(const GemmParams p, int tiles_m, int tiles_n, int total, int cvec)
{
    __shared__ __attribute__((aligned(1024))) unsigned char smem[NST * LDS_STAGE];

    int batch, tm, tn;
    map_tile(blockIdx.x, total, tiles_m, tiles_n, batch, tm, tn);
    const int M = p.M;
    const int N = p.e[batch].N;
    const int K = p.e[batch].K;
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    if (m0 >= M || n0 >= N)
        return;
    const int64_t lda = p.lda, ldb = p.ldb;
    const int rows_a = min(M - m0, BM);
    const int rows_b = min(N - n0, BN);
    const _Float16 *Ab = p.A + p.e[batch].a_off + (int64_t)m0 * lda;
    const _Float16 *Bb = p.B + p.e[batch].b_off + (int64_t)n0 * ldb;
    const hg_int32x4 ra = make_rsrc(Ab, (uint32_t)(((int64_t)(rows_a - 1) * lda + K) * 2));
    const hg_int32x4 rb = make_rsrc(Bb, (uint32_t)(((int64_t)(rows_b - 1) * ldb + K) * 2));

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;

    // Load geometry: wave w fills tile rows 64w .. 64w+63 of A and of B,
    // RPI rows per instruction; lane l covers row RPI·i + (l div KC) of its
    // group, physical chunk l mod KC, so it fetches the logical chunk that
    // swz() puts there.
    uint32_t aoff[LPS], boff[LPS];
    int lkc[LPS];
#pragma unroll
    for (int i = 0; i < LPS; ++i) {
        const int row = wave * RPW + i * RPI + lane / KC;
        int kc = 0;
#pragma unroll
        for (int c = 0; c < KC; ++c)
            kc = swz(row, c) == lane % KC ? c : kc;
        lkc[i] = kc;
        aoff[i] = row < rows_a ? (uint32_t)(row * (int)lda * 2 + kc * 16) : OOB;
        boff[i] = row < rows_b ? (uint32_t)(row * (int)ldb * 2 + kc * 16) : OOB;
    }
    const uint32_t lds_base = (uint32_t)reinterpret_cast<uintptr_t>(smem);

    // Loads q = first .. first+count-1 of slice kt into ring slot `slot`
    // (q < LPS: A rows, else B rows).  A slice past the end of K has
    // kval <= 0, so every lane gets the out-of-range offset and the slot is
    // zero-filled: the ring never needs a branch.
    auto issue = [&](int kt, int slot, int first, int count) {
        const uint32_t kb = (uint32_t)kt * RB;
        const int kval = K - kt * BK;              // K % 8 == 0: chunks are all in or all out
        const uint32_t sbase = lds_base + slot * LDS_STAGE + wave * RPW * RB;
#pragma unroll
        for (int q = first; q < first + count; ++q) {
            const bool isb = q >= LPS;
            const int i = isb ? q - LPS : q;
            const uint32_t off = lkc[i] * 8 < kval ? (isb ? boff[i] : aoff[i]) + kb : OOB;
            hg_raw_buffer_load_lds(isb ? rb : ra,
                                   reinterpret_cast<hg_lds_u32 *>(
                                       (uintptr_t)(sbase + (isb ? LDS_A : 0) + i * 1024)),
                                   16, (int)off, 0, 0, 0);
        }
    };

    // Fragment reads: row (lane mod 32) of each 32-row block, logical chunk
    // 2s + (lane div 32) of k-step s.
    const int frow = lane & 31;
    const int fhi = lane >> 5;
    auto frag_addr = [&](int slot, int s, bool isb) -> const unsigned char * {
        const int row0 = isb ? wn * WTN : wm * WTM;
        return smem + slot * LDS_STAGE + (isb ? LDS_A : 0) + (row0 + frow) * RB +
               swz(frow, 2 * s + fhi) * 16;
    };

    floatx16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = floatx16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

    half8 fa[2][TM], fb[2][TN];
    // Fragment f of k-step s: f < TM is A block f, else B block f - TM.
    auto read_frag = [&](int fs, int slot, int s, int f) {
        if (f < TM)
            fa[fs][f] = *reinterpret_cast<const half8 *>(frag_addr(slot, s, false) + f * 32 * RB);
        else
            fb[fs][f - TM] =
                *reinterpret_cast<const half8 *>(frag_addr(slot, s, true) + (f - TM) * 32 * RB);
    };
    auto read_frags = [&](int fs, int slot, int s) {
#pragma unroll
        for (int f = 0; f < TM + TN; ++f)
            read_frag(fs, slot, s, f);
    };
    auto mfma = [&](int fs, int i, int j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[fs][j], fa[fs][i], acc[i][j], 0, 0, 0);
    };

    // Ring of NST slices: slice t lives in slot t mod NST.  Slices
    // t+1 .. t+NST-1 are in flight while slice t is multiplied; the slot of
    // slice t-1 is refilled at the top of iteration t, after the barrier of
    // iteration t-1 has seen every wave finish reading it.
    // Ring schedule.  Slice t lives in slot t mod NST and is prefetched
    // D = NST-1 slices ahead: the loads issued while slice kt is multiplied
    // refill the slot of slice kt-1, which every wave finished reading before
    // the barrier of iteration kt-1.
    const int nk = (K + BK - 1) / BK;
    for (int t = 0; t < D; ++t)
        issue(t, t, 0, 2 * LPS);
    wait_vmcnt<2 * LPS * (D - 1)>();             // slice 0 has landed
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(0, 0, 0);
    int slot = 0;                                 // slot of slice kt
    int lslot = D;                                // slot of slice kt + D
    // Each k-step reads the fragments of the next k-step (TM+TN reads) and
    // issues V loads of slice kt+D, spread over its TM·TN MFMAs in a fixed
    // program order (a scheduling fence after every MFMA keeps it).  Before
    // the last k-step the wave waits for slice kt+1 and crosses the barrier,
    // so the last k-step reads slice kt+1's first fragments under its MFMAs.
    // A slice index past the end of K multiplies a zero-filled slot.
    constexpr int P = TM * TN, R = TM + TN, V = 2 * LPS / SPS;
    static_assert(V * SPS == 2 * LPS, "loads must split evenly over the k-steps");
    static_assert(P >= R + 2 * V, "interleave pattern needs enough MFMAs");
    for (int kt = 0; kt < nk; ++kt) {
        const int nxt = slot + 1 == NST ? 0 : slot + 1;
#pragma unroll
        for (int s = 0; s < SPS; ++s) {
            const bool last = s == SPS - 1;
            if (last) {
                // Before the barrier: this wave's loads of slice kt+1 have
                // landed, and its reads of slice kt are complete (after the
                // barrier other waves may start refilling slice kt's slot).
                // Issued after slice kt+1 so far: slices kt+2 .. kt+D-1 and
                // the first SPS-1 k-steps' share of slice kt+D.
                wait_vmcnt<2 * LPS * (D - 2) + V * (SPS - 1)>();
                wait_lgkmcnt<0>();
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
            }
            const int rslot = last ? nxt : slot;   // where the next fragments come from
            const int rstep = last ? 0 : s + 1;
            const int fs = s & 1;
#pragma unroll
            for (int k = 0; k < P; ++k) {
                mfma(fs, k / TN, k % TN);
                if (k < R)                                   // reads early: they gate the next k-step
                    read_frag(fs ^ 1, rslot, rstep, k);
                else if ((k - R) % 2 == 1 && (k - R) / 2 < V)  // loads after them, every other MFMA
                    issue(kt + D, lslot, s * V + (k - R) / 2, 1);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        slot = nxt;
        lslot = lslot + 1 == NST ? 0 : lslot + 1;
    }
    // The ring's last loads (zero fills past the end of K) must land before
    // the workgroup can release its LDS.
    wait_vmcnt<0>();

    // Epilogue: block (i, j) holds Cᵀ; lane covers row m0 + wm·128 + 32i +
    // (lane mod 32) and columns n0 + wn·128 + 32j + 8g + 4·(lane div 32) + 0..3.
    const float alpha = p.alpha;
    const float beta = p.beta;
    const int64_t ldc = p.ldc;
    const bool full = rows_a == BM && rows_b == BN && cvec;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int row = m0 + wm * WTM + i * 32 + frow;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = n0 + wn * WTN + j * 32 + 8 * g + 4 * fhi;
                const floatx4 v = {acc[i][j][4 * g + 0], acc[i][j][4 * g + 1],
                                   acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                const int64_t off = p.e[batch].c_off + (int64_t)row * ldc + col;
                if (full) {
                    if (OUT_F16) {
                        halfx4 *cp = reinterpret_cast<halfx4 *>(static_cast<_Float16 *>(p.C) + off);
                        halfx4 c = {};
                        if (BETA)
                            c = *cp;
                        halfx4 h;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            h[e] = (_Float16)(BETA ? __builtin_fmaf(alpha, v[e], beta * (float)c[e])
                                                   : alpha * v[e]);
                        *cp = h;
                    } else {
                        floatx4 *cp = reinterpret_cast<floatx4 *>(static_cast<float *>(p.C) + off);
                        floatx4 c = {};
                        if (BETA)
                            c = *cp;
                        floatx4 r;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            r[e] = BETA ? __builtin_fmaf(alpha, v[e], beta * c[e]) : alpha * v[e];
                        *cp = r;
                    }
                } else if (row < M) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (col + e < N) {
                            if (OUT_F16) {
                                _Float16 *cp = static_cast<_Float16 *>(p.C) + off + e;
                                const float r = BETA ? __builtin_fmaf(alpha, v[e], beta * (float)*cp)
                                                     : alpha * v[e];
                                *cp = (_Float16)r;
                            } else {
                                float *cp = static_cast<float *>(p.C) + off + e;
                                const float r = BETA ? __builtin_fmaf(alpha, v[e], beta * *cp)
                                                     : alpha * v[e];
                                *cp = r;
                            }
                        }
                    }
                }
            }
        }
    }
}

template <bool OUT_F16, bool BETA>
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
    hipLaunchKernelGGL((hgemm_fast_kernel<OUT_F16, BETA>), dim3((unsigned)total64), dim3(THREADS),
                       0, stream, p, tiles_m, tiles_n, (int)total64, cvec);
    return hipGetLastError();
}

}  // namespace

bool fast_path_ok(const GemmParams &p, const LaunchOpts &o)
{
    if (o.tri || !o.vec)
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
    if (o.out_f16)
        return o.beta_read ? launch<true, true>(p, stream) : launch<true, false>(p, stream);
    return o.beta_read ? launch<false, true>(p, stream) : launch<false, false>(p, stream);
}

}  // namespace hg
