// hg_ring.hip — the small- and mid-tile path of the half-precision GEMM on
// gfx950: C = alpha·A·B + beta·C, A M×K row-major, B K×N column-major, fp16 in,
// fp32 accumulate ("Nvidia Tensor Core-MMA PTX编程入门" §4; masked tiles as in
// the tiled matmul of "GPU架构与CUDA" 共享内存与分块), for operands whose rows
// are 16-byte aligned and K a multiple of 8.
//
// Problems too small to give every CU a 256×256 tile run 64×64 or 128×128
// tiles, where one 64-wide K stage is only 8 or 32 MFMAs per wave: a tile is
// bound by memory latency, not by the matrix cores.  So the K walk is a deep
// ring of LDS stages filled by direct buffer→LDS loads (no staging
// registers): NS stages, NS-1 of them in flight, one barrier per stage.
//
//  * 4 waves (2×2) per tile, 16×16×32 MFMA blocks (B fragment first, so each
//    16×16 result block is Cᵀ and a lane holds 4 consecutive columns of one
//    row); 128-byte LDS rows with the chunk index XOR-swizzled by (row/2) mod
//    8, which the loads realise by having each lane fetch the logical chunk
//    placed at its position; conflict-free 16-byte fragment reads.
//  * Rows past M or N get an offset beyond the buffer range (zero fill); with
//    KCHK (K not a multiple of 64) each lane's chunk is checked against K;
//    stages past the end of K get an empty buffer range.
#include "hg_internal.h"

#include <type_traits>
#include <utility>

typedef int32_t hg_r_int32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint32_t hg_r_lds_u32;

extern "C" __device__ void hg_ring_buffer_load_lds(hg_r_int32x4 rsrc, hg_r_lds_u32 *lds, int size,
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

// v_mfma_f32_16x16x32 on 16-byte fragments of fp16 or bf16 values.
template <bool BF16>
__device__ __forceinline__ floatx4 mfma_16x16x32(const half8 &a, const half8 &b, const floatx4 &c)
{
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

constexpr int BK = 64, RB = 128, KC = 8, THREADS = 256, NWAVES = 4;
constexpr uint32_t OOB = 0x80000000u;

__device__ __forceinline__ int swz(int r, int kc) { return kc ^ ((r >> 1) & (KC - 1)); }

// f(std::integral_constant<int, 0>{}) ... f(std::integral_constant<int, N-1>{}).
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

__device__ __forceinline__ hg_r_int32x4 rsrc_of(const void *base, uint32_t bytes)
{
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    hg_r_int32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;
    return r;
}

// Workgroup id → (batch, tile row, tile column): ids regrouped per XCD, then
// bands of 4 tile rows walked column by column (tiles on one XCD share
// panels in its L2).
__device__ __forceinline__ void ring_map(int wg, int total, int tiles_m, int tiles_n, int &batch,
                                         int &tm, int &tn)
{
    const int per = total >> 3, rem = total & 7;
    const int x = wg & 7;
    const int q = x * per + min(x, rem) + (wg >> 3);
    const int per_batch = tiles_m * tiles_n;
    batch = q / per_batch;
    const int l = q - batch * per_batch;
    const int band = l / (4 * tiles_n);
    const int first = band * 4;
    const int gsz = min(tiles_m - first, 4);
    const int r = l - band * 4 * tiles_n;
    tm = first + r % gsz;
    tn = r / gsz;
}

// TRI: the B operand (N×K) is triangular in the GEMM view: element (j, k)
// counts for k >= j (p.tri_up: k <= j) and the other triangle is never
// used.  A tile walks only the stages that can hold counted elements: from
// its first column's stage on (tri_up: up to the stage of its last column),
// and the elements on the other side of the diagonal in the tile's
// diagonal-block stages are zeroed in LDS once the stage has landed.  With
// one entry of K = N = n this is the whole recursive TRMM in one launch
// (see trmm_ring_fused_ok); with one entry per leaf, the leaves of the
// per-level schedule.
// NSQ: the ring depth, 0 for the default (128 KiB of stages, at most 8);
// NSQ = 5 with 64×64 tiles (80 KiB) lets two workgroups share a CU.
template <int BM, int BN, bool OUT_F16, bool BETA, bool KCHK, bool EPI, bool IN_BF16, bool TRI = false,
          int NSQ = 0>
__global__ void __launch_bounds__(THREADS, 1)
hgemm_ring_kernel(const GemmParams p, int tiles_m, int tiles_n, int total, int cvec)
{
    constexpr int SLOT = (BM + BN) * RB;                   // one stage: A rows then B rows
    constexpr int NS = NSQ > 0 ? NSQ : (128 * 1024) / SLOT < 8 ? (128 * 1024) / SLOT : 8;   // ring depth
    constexpr int WTM = BM / 2, WTN = BN / 2;              // wave sub-tile
    constexpr int TM = WTM / 16, TN = WTN / 16;            // 16×16 blocks per wave
    constexpr int LA = BM / (NWAVES * 8), LB = BN / (NWAVES * 8);   // load instructions per wave
    constexpr int L = LA + LB;                             // ... per stage
    static_assert(NS >= 4 && LA >= 1 && LB >= 1 && (NS - 2) * L <= 63, "");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[NS * SLOT];

    int batch, tm, tn;
    ring_map(blockIdx.x, total, tiles_m, tiles_n, batch, tm, tn);
    const int M = p.M, N = p.e[batch].N, K = p.e[batch].K;
    const int m0 = tm * BM, n0 = tn * BN;
    if (m0 >= M || n0 >= N)
        return;                                            // whole workgroup
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int rows_a = min(M - m0, BM), rows_b = min(N - n0, BN);
    const hg_r_int32x4 ra = rsrc_of(p.A + p.e[batch].a_off + (int64_t)m0 * p.lda,
                                    (uint32_t)(((int64_t)(rows_a - 1) * p.lda + K) * 2));
    const hg_r_int32x4 rb = rsrc_of(p.B + p.e[batch].b_off + (int64_t)n0 * p.ldb,
                                    (uint32_t)(((int64_t)(rows_b - 1) * p.ldb + K) * 2));
    const uint32_t lds_base = (uint32_t)reinterpret_cast<uintptr_t>(smem);
    // Stages kt0 .. kt0 + nk - 1 of K (TRI: only those that can hold counted
    // elements of the tile's columns).
    const int nkk = (K + BK - 1) / BK;
    const int kt0 = TRI && !p.tri_up ? n0 / BK : 0;
    const int nk = TRI ? (p.tri_up ? min(nkk, (n0 + BN + BK - 1) / BK) : nkk - kt0) : nkk;

    // Load i of a wave covers tile rows (wave·(LA or LB) + i)·8 .. +7; lane l
    // takes row +(l div 8) and the logical chunk that swz() puts at l mod 8.
    uint32_t off[L];
    int lkc[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const bool isb = i >= LA;
        const int row = ((isb ? LB : LA) * wave + (isb ? i - LA : i)) * 8 + (lane >> 3);
        const int kc = swz(row, lane & 7);   // swz() XORs the chunk index: its own inverse
        lkc[i] = kc;
        const int rows = isb ? rows_b : rows_a;
        const int64_t ld = isb ? p.ldb : p.lda;
        off[i] = row < rows ? (uint32_t)(row * (int)ld * 2 + kc * 16) : OOB;
    }
    // Load i of stage kt into its ring slot.
    auto issue_one = [&](int kt, int i) __attribute__((always_inline)) {
        const int slot = kt % NS;
        const uint32_t kb = (uint32_t)(kt0 + kt) * RB;
        {
            const bool isb = i >= LA;
            hg_r_int32x4 r = isb ? rb : ra;
            uint32_t o = off[i];
            if constexpr (KCHK) {
                o = lkc[i] * 8 < K - (kt0 + kt) * BK ? o + kb : OOB;
            } else {
                const uint64_t base = ((uint64_t)(uint32_t)r[1] << 32 | (uint32_t)r[0]) + kb;
                r[0] = (int)(uint32_t)base;
                r[1] = (int)(uint32_t)(base >> 32);
                r[2] = kt < nk ? (int)((uint32_t)r[2] - kb) : 0;
            }
            const int row0 = ((isb ? LB : LA) * wave + (isb ? i - LA : i)) * 8;
            const uint32_t dst = lds_base + slot * SLOT + (isb ? BM * RB : 0) + row0 * RB;
            hg_ring_buffer_load_lds(r, reinterpret_cast<hg_r_lds_u32 *>((uintptr_t)dst), 16, (int)o,
                                    0, 0, 0);
        }
    };
    // Every load of stage kt.
    auto issue = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < L; ++i)
            issue_one(kt, i);
    };

    floatx4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = floatx4{0, 0, 0, 0};

#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
        issue(s);
    const int frow = lane & 15, fhi = lane >> 4;
    // Fragments of one stage: both k-steps of the wave's TM A and TN B blocks.
    constexpr int SPS = BK / 32;
    struct Frags {
        half8 a[SPS][TM], b[SPS][TN];
    };
    // Fragment r of stage kt (r < NR: k-step r / (TM + TN), then its TM A
    // blocks and TN B blocks).
    constexpr int NR = SPS * (TM + TN);
    auto read_one = [&](int kt, Frags &f, auto rc) __attribute__((always_inline)) {
        constexpr int r = decltype(rc)::value;
        constexpr int s = r / (TM + TN), q = r % (TM + TN);
        const unsigned char *As = smem + (kt % NS) * SLOT;
        if constexpr (q < TM) {
            const int row = wm * WTM + q * 16 + frow;
            f.a[s][q] = *reinterpret_cast<const half8 *>(As + row * RB + swz(row, 4 * s + fhi) * 16);
        } else {
            const int row = wn * WTN + (q - TM) * 16 + frow;
            f.b[s][q - TM] = *reinterpret_cast<const half8 *>(As + BM * RB + row * RB +
                                                             swz(row, 4 * s + fhi) * 16);
        }
    };
    auto read_stage = [&](int kt, Frags &f) __attribute__((always_inline)) {
        static_for<NR>([&](auto rc) __attribute__((always_inline)) { read_one(kt, f, rc); });
    };
    constexpr int NM = SPS * TN * TM;                      // MFMAs per stage and wave
    constexpr bool SPREAD = BM >= 128;
    // Stage kt's fragments are read one stage ahead, during stage kt-1's
    // MFMAs, so the LDS latency hides behind the matrix core.  In step kt:
    // this wave's loads of stage kt+1 have landed (stages kt+2 .. kt+NS-2 may
    // be in flight); after the barrier everyone's have, and every wave has
    // finished reading stage kt-1 (its MFMAs waited for those reads), whose
    // slot then takes stage kt+NS-1.  Reads past the last stage see the
    // zero-filled slots and are not used.
    // TRI: zero the other triangle's elements of stage kt in its slot, in
    // the B rows this wave loaded (8·LB·wave .. 8·LB·wave + 8·LB - 1), one row
    // per lane: with jr = (the row's column index) - (the stage's first k),
    // element k of the stage (0..63) is zeroed when k < jr (tri_up: k > jr).
    auto zero_tri = [&](int kt) __attribute__((always_inline)) {
        const int jr0 = __builtin_amdgcn_readfirstlane(n0 + 8 * LB * wave - (kt0 + kt) * BK);
        const bool up = p.tri_up != 0;
        if (up ? jr0 >= BK - 1 : jr0 + 8 * LB - 1 <= 0)
            return;
        if (lane < 8 * LB) {
            const int row = 8 * LB * wave + lane;
            const int jr = jr0 + lane;
            unsigned char *rp = smem + (kt % NS) * SLOT + BM * RB + row * RB;
            const int kp = jr >> 3;                         // chunk holding k = jr (floor)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
                if (up ? kc > kp : kc < kp)
                    *reinterpret_cast<u32x4 *>(rp + swz(row, kc) * 16) = u32x4{0, 0, 0, 0};
            if (kp >= 0 && kp < KC) {
                const int e0 = jr & 7;
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
        }
    };
    // Whether stage kt is one of the tile's diagonal-block stages.
    auto tri_stage = [&](int kt) {
        return p.tri_up ? kt >= nk - BN / BK && kt < nk : kt < BN / BK && kt < nk;
    };
    Frags f0, f1;
    wait_vmcnt<(NS - 2) * L>();
    if constexpr (TRI) {
        if (tri_stage(0)) {
            zero_tri(0);
            wait_lgkmcnt<0>();
        }
    }
    __builtin_amdgcn_s_barrier();
    read_stage(0, f0);
    auto step = [&](int kt, const Frags &cur, Frags &nxt) __attribute__((always_inline)) {
        wait_vmcnt<(NS - 3) * L>();
        if constexpr (TRI) {
            if (tri_stage(kt + 1)) {
                zero_tri(kt + 1);
                wait_lgkmcnt<0>();
            }
        }
        __builtin_amdgcn_s_barrier();
        if constexpr (!SPREAD) {
            issue(kt + NS - 1);
            read_stage(kt + 1, nxt);
#pragma unroll
            for (int s = 0; s < SPS; ++s)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int i = 0; i < TM; ++i)
                        acc[i][j] = mfma_16x16x32<IN_BF16>(cur.b[s][j], cur.a[s][i], acc[i][j]);
            return;
        }
        __builtin_amdgcn_sched_barrier(0);
        // 128×128 tiles: the stage's 32 MFMAs per wave with the ring loads of
        // stage kt+NS-1 and the reads of stage kt+1 at fixed positions
        // between them (load l after MFMA l·NM/L, read r after MFMA r·NM/NR).
        // Issued in a burst, the loads wait for the CU's memory path one
        // after another and hold back the wave's MFMAs behind them (2048³:
        // 23.1 -> 20.5 us).  With 64×64 tiles (8 MFMAs per wave) the stage is
        // bound by that path either way and the burst order is kept.
        static_for<NM>([&](auto mc) __attribute__((always_inline)) {
            constexpr int m = decltype(mc)::value;
            constexpr int s = m / (TN * TM), j = m / TM % TN, i = m % TM;
            acc[i][j] = mfma_16x16x32<IN_BF16>(cur.b[s][j], cur.a[s][i], acc[i][j]);
            static_for<L>([&](auto lc) __attribute__((always_inline)) {
                constexpr int l = decltype(lc)::value;
                if constexpr (l * NM / L == m)
                    issue_one(kt + NS - 1, l);
            });
            static_for<NR>([&](auto rc) __attribute__((always_inline)) {
                constexpr int r = decltype(rc)::value;
                if constexpr (r * NM / NR == m)
                    read_one(kt + 1, nxt, rc);
            });
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    for (int kt = 0; kt < nk; kt += 2) {
        step(kt, f0, f1);
        if (kt + 1 < nk)
            step(kt + 1, f1, f0);
    }
    wait_vmcnt<0>();   // the ring's last zero-fill loads (none reach memory) drain before exit

    // Epilogue: lane covers row m0 + wm·WTM + 16i + (lane mod 16) and columns
    // n0 + wn·WTN + 16j + 4·(lane div 16) + 0..3.
    const float alpha = p.alpha, beta = p.beta;
    const int64_t ldc = p.ldc;
    // 16-bit C has the input's type (fp16 or bf16).
    typedef typename std::conditional<IN_BF16, bf16x4, halfx4>::type vec16;
    typedef typename std::conditional<IN_BF16, __bf16, _Float16>::type e16;
    typedef typename std::conditional<OUT_F16, vec16, floatx4>::type cvec_t;
    typedef typename std::conditional<OUT_F16, e16, float>::type celt;
    celt *Cb = static_cast<celt *>(p.C) + p.e[batch].c_off;
    if (rows_a == BM && rows_b == BN && cvec) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = m0 + wm * WTM + i * 16 + frow;
            celt *cr = Cb + (int64_t)row * ldc + n0 + wn * WTN + 4 * fhi;
            cvec_t cin[TN];
            if (BETA) {
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    cin[j] = *reinterpret_cast<const cvec_t *>(cr + j * 16);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                cvec_t r;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v = acc[i][j][e];
                    float t = BETA ? __builtin_fmaf(alpha, v, beta * (float)cin[j][e]) : alpha * v;
                    if constexpr (EPI)
                        t = epi_apply(t, p.bias ? p.bias[n0 + wn * WTN + j * 16 + 4 * fhi + e] : -0.0f,
                                      p.act);
                    if constexpr (OUT_F16 && TRI)
                        t = opaque_f32(t);   // the in-place TRMM: the fp32 result, rounded
                    r[e] = (celt)t;
                }
                *reinterpret_cast<cvec_t *>(cr + j * 16) = r;
            }
        }
    } else {
        // Edge tile: rows past M are skipped; a lane's 4 columns go as one
        // vector access when all are inside N (and C allows it), element by
        // element otherwise.  C is read for the whole row block first.
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = m0 + wm * WTM + i * 16 + frow;
            if (row >= M)
                continue;
            celt *cr = Cb + (int64_t)row * ldc;
            float cin[TN][4];
            if (BETA) {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int col = n0 + wn * WTN + j * 16 + 4 * fhi;
                    if (cvec && col + 3 < N) {
                        const cvec_t c4 = *reinterpret_cast<const cvec_t *>(cr + col);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            cin[j][e] = (float)c4[e];
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            cin[j][e] = col + e < N ? (float)cr[col + e] : 0.0f;
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int col = n0 + wn * WTN + j * 16 + 4 * fhi;
                cvec_t r;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v = acc[i][j][e];
                    float t = BETA ? __builtin_fmaf(alpha, v, beta * cin[j][e]) : alpha * v;
                    if constexpr (EPI)
                        t = epi_apply(t, p.bias && col + e < N ? p.bias[col + e] : -0.0f, p.act);
                    if constexpr (OUT_F16 && TRI)
                        t = opaque_f32(t);
                    r[e] = (celt)t;
                }
                if (cvec && col + 3 < N) {
                    *reinterpret_cast<cvec_t *>(cr + col) = r;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (col + e < N)
                            cr[col + e] = r[e];
                }
            }
        }
    }
}

template <int BM, int BN, bool OUT_F16, bool BETA, bool EPI, bool IN_BF16, bool TRI = false, int NSQ = 0>
hipError_t launch_ring_cfg(const GemmParams &p, hipStream_t stream)
{
    int maxN = 0;
    bool kchk = false;
    for (int b = 0; b < p.nbatch; ++b) {
        maxN = p.e[b].N > maxN ? p.e[b].N : maxN;
        kchk = kchk || p.e[b].K % BK != 0;
    }
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
    if (kchk)
        hipLaunchKernelGGL((hgemm_ring_kernel<BM, BN, OUT_F16, BETA, true, EPI, IN_BF16, TRI, NSQ>), dim3((unsigned)total64),
                           dim3(THREADS), 0, stream, p, tiles_m, tiles_n, (int)total64, cvec);
    else
        hipLaunchKernelGGL((hgemm_ring_kernel<BM, BN, OUT_F16, BETA, false, EPI, IN_BF16, TRI, NSQ>), dim3((unsigned)total64),
                           dim3(THREADS), 0, stream, p, tiles_m, tiles_n, (int)total64, cvec);
    return hipGetLastError();
}

template <int BM, int BN, bool EPI, bool IN_BF16>
hipError_t launch_ring_epi(const GemmParams &p, const LaunchOpts &o, hipStream_t s)
{
    if (o.out_f16)
        return o.beta_read ? launch_ring_cfg<BM, BN, true, true, EPI, IN_BF16>(p, s)
                           : launch_ring_cfg<BM, BN, true, false, EPI, IN_BF16>(p, s);
    return o.beta_read ? launch_ring_cfg<BM, BN, false, true, EPI, IN_BF16>(p, s)
                       : launch_ring_cfg<BM, BN, false, false, EPI, IN_BF16>(p, s);
}

template <int BM, int BN>
hipError_t launch_ring_tile(const GemmParams &p, const LaunchOpts &o, hipStream_t s)
{
    if (o.in_bf16)
        return o.epi ? launch_ring_epi<BM, BN, true, true>(p, o, s) : launch_ring_epi<BM, BN, false, true>(p, o, s);
    return o.epi ? launch_ring_epi<BM, BN, true, false>(p, o, s)
                 : launch_ring_epi<BM, BN, false, false>(p, o, s);
}

}  // namespace

bool ring_path_ok(const GemmParams &p, const LaunchOpts &o)
{
    if (!o.vec || (o.tri && (o.out_f16 || o.beta_read || o.epi || o.in_bf16)))
        return false;
    if (p.lda > (1 << 21) || p.ldb > (1 << 21))
        return false;
    for (int b = 0; b < p.nbatch; ++b)
        if (p.e[b].K % 8 != 0)
            return false;
    return true;
}

bool trmm_ring_fused_ok(const GemmParams &p)
{
    constexpr int T = 64;                                  // tile edge of the Small family
    if (p.lda > (1 << 21) || p.ldb > (1 << 21) || p.leaf < T)
        return false;
    if (reinterpret_cast<uintptr_t>(p.A) % 16 != 0 || reinterpret_cast<uintptr_t>(p.B) % 16 != 0 ||
        p.lda % 8 != 0 || p.ldb % 8 != 0)
        return false;
    // Every recursion boundary on a 64-column tile edge.
    const int n = p.e[0].N;
    if (n % T != 0)
        return false;
    struct Frame {
        int o, s;
    };
    Frame st[64];
    int top = 0;
    st[top++] = {0, n};
    while (top > 0) {
        const Frame f = st[--top];
        if (f.o % T != 0 || f.s % T != 0)
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

hipError_t launch_trmm_fused_ring(const GemmParams &p, hipStream_t stream, bool out_f16)
{
    // With at least two tiles per CU, a 5-stage ring (80 KiB) lets two
    // workgroups share each CU: n = m = 2048 (1024 tiles) 33.0 -> 21.9 us.
    // With fewer tiles one workgroup per CU gets the deeper default ring.
    const int64_t tiles = (int64_t)((p.M + 63) / 64) * ((p.e[0].N + 63) / 64);
    const bool two = tiles >= 2 * (int64_t)cu_count();
    if (out_f16)
        return two ? launch_ring_cfg<64, 64, true, false, false, false, true, 5>(p, stream)
                   : launch_ring_cfg<64, 64, true, false, false, false, true>(p, stream);
    return two ? launch_ring_cfg<64, 64, false, false, false, false, true, 5>(p, stream)
               : launch_ring_cfg<64, 64, false, false, false, false, true>(p, stream);
}

hipError_t launch_gemm_ring(const GemmParams &p, const LaunchOpts &o, hipStream_t stream)
{
    if (o.tri)   // fp32 C written once (TRMM leaves and the one-launch ring TRMM)
        return o.tile == Tile::Mid ? launch_ring_cfg<128, 128, false, false, false, false, true>(p, stream)
                                   : launch_ring_cfg<64, 64, false, false, false, false, true>(p, stream);
    if (o.tile == Tile::Mid)
        return launch_ring_tile<128, 128>(p, o, stream);
    return launch_ring_tile<64, 64>(p, o, stream);
}

}  // namespace hg
