// Expert GEMMs for many rows per expert: LDS-tiled scaled FP4 x FP8 MFMA.
//
// A workgroup computes a tile of BN weight rows x BM dispatched rows of one
// expert.  Its NW wavefronts (four, or eight for the 256-row tiles) form
// a 2 x NW/2 grid: wavefront (wn, wm) owns weight rows [wn BN/2, (wn+1) BN/2)
// of the tile (BN/32 16-row MFMA groups) and BM/(NW/2) dispatched rows from
// wm BM/(NW/2).  The operands of KU K steps of 128 (one stage) are brought
// into LDS with direct global-to-LDS loads, double-buffered: the loads of
// stage u+1 are in flight while stage u is computed.  A four-wavefront
// workgroup fits in half a CU's LDS and registers, so two independent
// workgroups share every CU: while one waits at its barrier or on memory,
// the other's MFMAs run (measured faster than one workgroup of eight
// wavefronts over the same rows, whose halves wait at the same barriers, and
// than three-stage rings at one workgroup per CU).
//
// Tiles: 128-row tiles (MFMA-bound prefill sizes) take 256 weight rows (or
// 128 when 256 would leave fewer than three rounds of items) and one K step
// per stage; 64-row tiles (HBM-bound) take 128 weight rows and two K steps
// per stage, so every weight row is read 128 contiguous bytes at a time.
// Up to 16 expected rows per expert (decode) 32-row tiles keep three such
// stages in LDS at two workgroups per CU, two of them in flight: a stage's
// weight loads go out last, and the wait before a stage leaves the next
// stage's weight loads outstanding.
// Past 512 expected rows per expert both GEMMs take 256 x 256 tiles on
// eight wavefronts, one workgroup per CU: the two 128-row halves share one
// weight stage, so a CU moves 48 KB per K step for 256 MFMAs instead of 64 KB.
//
// GEMM1 tile: BN/2 intermediate columns.  Each wavefront holds BN/4 of them
// as BN/64 gate groups and the matching up groups, so the clamped SwiGLU and
// the MX FP8 requant (32-column blocks) happen in registers.  GEMM2 tile: BN
// output columns, y rounded to bf16 (the combine's input).
//
// Work items are (row tile of one expert, N tile), derived on every
// workgroup from counts as in the skinny kernels, and taken in a grid-stride
// loop.
#include <cstdlib>
#include <mutex>
#include <type_traits>

#include "moe_common.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
// Tile of BN weight rows (256 or 128) x BM dispatched rows (32 to 256); one
// LDS stage holds KU K steps of 128 (1 or 2); 32-row tiles keep three stages.
template <int BM, int BN, int KU>
struct TileLds {
    static_assert(KU == 1 || KU == 2, "one or two K steps per stage");
    static constexpr int kW = BN * 64 * KU;    // FP4 weight tile, one stage
    static constexpr int kX = BM * 128 * KU;   // FP8 activation rows, one stage
    static constexpr int kStage = kW + kX;
    static constexpr int kStages = BM == 32 ? 3 : 2;   // stages resident in LDS
    static constexpr int kWE = BN * 16;        // weight exponents of four K steps
    static constexpr int kXE = BM * 16;        // activation exponents of four K steps
    static constexpr int kExp = kWE + kXE;
    static constexpr int kExpSlots = 2;
    // the stage ring, grown where the bf16 y tile of a 256-row tile needs
    // more (that tile runs one workgroup per CU)
    static constexpr int kPipe = kStages * kStage + kExpSlots * kExp;
    static constexpr int kYTile = BM * (BN * 2 + 16);
    static constexpr int kRing = BM == 256 && kYTile > kPipe ? kYTile : kPipe;
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 lds_read16(const uint8_t *p)
{
    return *reinterpret_cast<const u32x4 *>(p);
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(uint8_t *p)
{
    return (uint32_t)(uintptr_t)(lds_u8 *)p;
}

// global -> LDS without registers: lane l's SIZE bytes from base + voff land
// at LDS address m0 + SIZE * l (m0 is wavefront-uniform).  Issued as inline
// assembly so that the waits are exactly the ones this file writes: the
// loads count in vmcnt like any vector memory load.  An LDS DMA reads m0 one
// wait state after an SALU write of m0 at the earliest, hence the s_nop.
// kStream marks data read once (non-temporal: the L2 evicts it first, so it
// does not push out the activation rows that other tiles read again).
// kL2 reads data that another CU of the same XCD wrote earlier in the same
// launch: sc0 makes the load miss the CU's own L1, which may hold the line
// from before the write, and take it from the XCD's L2, where the write is.
template <int SIZE, bool kStream = false, bool kL2 = false>
__device__ __forceinline__ void g2lds(const uint8_t *base, uint32_t voff, uint32_t m0)
{
    static_assert(SIZE == 16 || SIZE == 4, "dword and dwordx4 LDS DMA only");
    static_assert(!(kStream && kL2), "one cache policy");
    if (SIZE == 16 && kL2)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 sc0" ::"s"(m0),
                     "v"(voff), "s"(base)
                     : "memory", "m0");
    else if (SIZE == 16 && kStream)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(m0),
                     "v"(voff), "s"(base)
                     : "memory", "m0");
    else if (SIZE == 16)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0),
                     "v"(voff), "s"(base)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" ::"s"(m0),
                     "v"(voff), "s"(base)
                     : "memory", "m0");
}

// The workgroup barrier without the memory fence __syncthreads() adds (that
// fence would wait for every outstanding load, prefetches included).
__device__ __forceinline__ void raw_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Operands of one GEMM launch.
struct TiledArgs {
    const uint8_t *act, *act_s;             // FP8 activation rows (x or h) and exponents
    const int32_t *counts, *offsets, *row_route;
    const uint8_t *w, *ws;                  // W13 or W2 codes and exponents
    uint8_t *h_out, *hs_out;                // GEMM1 output
    uint16_t *y_out;                        // GEMM2 output, bf16 rows, or
    uint8_t *y8_out, *y8s_out;              // MX FP8 rows (y_out null)
};

// One work item: N tile nt of row chunk q.  prefix holds the chunk plan,
// arow (BM ints) and lds (the stage ring) are the workgroup's.  kL2: GEMM2
// reads h through the XCD's L2, past the CU's L1 (the persistent layer,
// where GEMM1 items of the same launch and XCD wrote it).  Ends with the
// workgroup's LDS still in use: the caller synchronises before the next item.
template <bool kGemm1, int BM, int BN, int KU, bool kL2, int NW = 4>
__device__ __forceinline__ void tiled_item(const Shape &s, const TiledArgs &g,
                                           const int *prefix, int *arow, uint8_t *lds, int q,
                                           int nt)
{
    const int32_t *__restrict__ counts = g.counts;
    const int32_t *__restrict__ offsets = g.offsets;
    const int32_t *__restrict__ row_route = g.row_route;
    uint8_t *__restrict__ h_out = g.h_out;
    uint8_t *__restrict__ hs_out = g.hs_out;
    uint16_t *__restrict__ y_out = g.y_out;
    using L = TileLds<BM, BN, KU>;
    // 64-row tiles: an expert's weights are read by one row chunk (as a
    // rule), so they stream through the L2 without displacing the
    // activation rows; 128-row tiles reuse each weight tile across row chunks
    constexpr bool kStreamW = BM <= 64;
    constexpr int GW = BN / 32;             // 16-row weight groups per wavefront
    constexpr int NTH = NW * 64;            // threads
    constexpr int NWM = NW / 2;             // wavefronts along the rows
    constexpr int WI = BN * KU / (16 * NW); // weight load instructions per wavefront and stage
    constexpr int TBL = BM / (8 * NW);      // activation load instructions per wavefront and K step
    constexpr int TB = BM / (16 * NWM);     // 16-row activation blocks per wavefront
    constexpr int NS = L::kStages;
    constexpr int WROW = 64 * KU;           // LDS bytes of one weight row in a stage
    constexpr int WSWZ = 4 * KU - 1;        // chunk swizzle mask of the weight rows
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i16 = lane & 15, kq = lane >> 4;
    const int wn = wave & 1, wm = wave >> 1;
    const int H = s.H, I = s.I;
    const int KT = kGemm1 ? H : I;          // contraction length
    const int KS = KT / 128;                // K steps
    const int U = (KS + KU - 1) / KU;       // stages
    {
        const int e = __builtin_amdgcn_readfirstlane(chunk_expert(prefix, s.E_local, q));
        const int c = q - prefix[e];
        const int row0 = __builtin_amdgcn_readfirstlane(offsets[e] + c * BM);
        const int nrows = min(BM, used_rows(s, counts[e]) - c * BM);
        // wavefront-uniform bases: expert e's weight rows and, for GEMM2, the
        // tile's first h row, so every 32-bit lane offset below stays inside
        // one expert's weights or one row tile (GEMM1's gathered x rows are
        // addressed from x itself: T * H < 2^32 is checked on the host)
        const size_t wrows = kGemm1 ? 2 * (size_t)I : (size_t)H;
        const uint8_t *__restrict__ w = g.w + (size_t)e * wrows * (size_t)(KT / 2);
        const uint8_t *__restrict__ ws = g.ws + (size_t)e * wrows * (size_t)(KT / 32);
        const uint8_t *__restrict__ act = kGemm1 ? g.act : g.act + (size_t)row0 * (size_t)KT;
        const uint8_t *__restrict__ act_s =
            kGemm1 ? g.act_s : g.act_s + (size_t)row0 * (size_t)(KT / 32);
        if (tid < BM) {
            const int r = min(tid, nrows - 1);
            arow[tid] = kGemm1 ? row_route[row0 + r] / s.K : r;
        }
        __syncthreads();

        // weight row (within expert e's rows of W) of tile row r
        auto wrow_of = [&](int r) -> uint32_t {
            const int grp = r >> 4, rr = r & 15;
            if (kGemm1) {
                // group grp: wavefront half grp / GW; within it GW/2 gate
                // groups, then the GW/2 matching up groups
                const int half = grp / GW, up = (grp % GW) >= GW / 2, cb = grp % (GW / 2);
                return (uint32_t)((up ? I : 0) + nt * (BN / 2) + (BN / 4) * half + 16 * cb + rr);
            }
            return (uint32_t)(nt * BN + r);
        };
        // LDS layout of a stage: weight tile row r at WROW r (64 bytes of
        // each row per K step, so WROW = 64 or 128), then activation rows:
        // K step kk of the stage at kW + BM 128 kk, tile row R at 128 R of
        // it.  The 16-byte chunk c of a row sits at position c ^ swz(row),
        // swz = (row >> 1) & (WROW/16 - 1) (weights) or (row >> 1) & 7
        // (activations), so the MFMA fragment reads below hit every LDS bank
        // once.  Loads are row-major (WROW/16 or eight consecutive lanes
        // cover one row): the global-to-LDS path moves that several times
        // faster than lanes walking down the rows, and HBM serves whole
        // 128-byte row pieces (two K steps per stage) markedly faster than
        // 64-byte ones.
        //
        // Weight instruction i brings tile rows rpi h .. rpi h + rpi - 1 with
        // rpi = 1024 / WROW and h = wave + NW i: lane l -> row
        // rpi h + l / (WROW/16), chunk (l mod WROW/16) ^ swz.  Activation
        // instruction i of a K step brings tile rows 8h.., h = wave + NW i:
        // lane l -> row R = 8h + (l >> 3), chunk (l & 7) ^ swz.
        constexpr int LPR = WROW / 16;      // lanes per weight row
        uint32_t woff[WI], xoff[TBL];
        bool xrow_used[TBL];   // activation rows past nrows are not loaded
#pragma unroll
        for (int i = 0; i < WI; ++i) {
            const int r = (64 / LPR) * (wave + NW * i) + lane / LPR;
            const int cc = (lane % LPR) ^ ((r >> 1) & WSWZ);
            woff[i] = wrow_of(r) * (uint32_t)(KT / 2) + 16u * (uint32_t)cc;
        }
#pragma unroll
        for (int i = 0; i < TBL; ++i) {
            const int h = wave + NW * i, R = 8 * h + (lane >> 3);
            const int cc = (lane & 7) ^ ((R >> 1) & 7);
            xoff[i] = (uint32_t)arow[R] * (uint32_t)KT + 16u * (uint32_t)cc;
            xrow_used[i] = R < nrows;
        }
        // exponents, four K steps (16 bytes) per row at a time: wavefront
        // v < BN/64 brings weight rows 64 v + l, wavefront v < BM/64
        // activation rows 64 v + l.
        // The last group of a row is read from 16 bytes before the row's
        // end, so no read passes it (KS >= 4).
        const int we_wave = wave % (BN / 64);
        constexpr int XEW = BM >= 64 ? BM / 64 : 1;   // wavefronts loading activation exponents
        const int xe_wave = wave % XEW;
        const uint32_t weoff = wrow_of(64 * we_wave + lane) * (uint32_t)(KT / 32);
        const uint32_t xeoff = (uint32_t)arow[min(64 * xe_wave + lane, BM - 1)] * (uint32_t)(KT / 32);
        const bool xe_used = 64 * xe_wave + lane < nrows;
        auto ebase = [&](int grp) -> int { return min(16 * grp, KT / 32 - 16); };

        const uint32_t lds0 = lds_addr(lds);
        const uint32_t lds_w = __builtin_amdgcn_readfirstlane(lds0 + 1024u * wave);
        const uint32_t lds_x = __builtin_amdgcn_readfirstlane(lds0 + L::kW + 1024u * wave);
        const uint32_t lds_e = lds0 + NS * L::kStage;
        const uint32_t lds_we = __builtin_amdgcn_readfirstlane(lds_e + 1024u * we_wave);
        const uint32_t lds_xe = __builtin_amdgcn_readfirstlane(lds_e + L::kWE + 1024u * xe_wave);
        // stage u: K steps KU u .. (the last stage of an odd KS with KU = 2
        // holds one step; its other half is neither loaded nor read)
        // the weight loads of a stage, then its activation rows and exponents
        auto issue_w = [&](int u) {
            const uint32_t st = (uint32_t)((u % NS) * L::kStage);
            const int ks0 = KU * u;
            const int nk = min(KU, KS - ks0);
            if (nk == KU) {
#pragma unroll
                for (int i = 0; i < WI; ++i)
                    g2lds<16, kStreamW>(w, woff[i] + (uint32_t)ks0 * 64u, lds_w + st + (uint32_t)(NW * 1024) * i);
            } else {
                // one K step of a 128-byte row layout: only chunks 0..3
                // (positions c ^ swz) are read; load them, skip the rest
#pragma unroll
                for (int i = 0; i < WI; ++i)
                    if (((lane % LPR) ^ ((((64 / LPR) * (wave + NW * i) + lane / LPR) >> 1) & WSWZ)) < 4)
                        g2lds<16, kStreamW>(w, woff[i] + (uint32_t)ks0 * 64u, lds_w + st + (uint32_t)(NW * 1024) * i);
            }
        };
        auto issue_x = [&](int u) {
            const uint32_t st = (uint32_t)((u % NS) * L::kStage);
            const int ks0 = KU * u;
            const int nk = min(KU, KS - ks0);
#pragma unroll
            for (int kk = 0; kk < KU; ++kk)
                if (kk < nk) {
#pragma unroll
                    for (int i = 0; i < TBL; ++i)
                        if (xrow_used[i])
                            g2lds<16, false, kL2>(act, xoff[i] + (uint32_t)(ks0 + kk) * 128u,
                                      lds_x + st + (uint32_t)(kk * BM * 128) + (uint32_t)(NW * 1024) * i);
                }
            if ((ks0 & 3) == 0) {
                const int grp = ks0 >> 2;
                const uint32_t es = (uint32_t)((grp % L::kExpSlots) * L::kExp);
                const uint32_t eb = (uint32_t)ebase(grp);
                // one wavefront per 64-row block (no two load the same rows)
                if (wave < BN / 64)
                    g2lds<16>(ws, weoff + eb, lds_we + es);
                if (wave < XEW && xe_used)
                    g2lds<16, false, kL2>(act_s, xeoff + eb, lds_xe + es);
            }
        };
        // three stages: a stage's weight loads go last, so that waiting for
        // all but WI loads leaves the next stage's weight stream in flight
        auto issue = [&](int u) {
            if (NS == 3) {
                issue_x(u);
                issue_w(u);
            } else {
                issue_w(u);
                issue_x(u);
            }
        };

        v4f acc[GW][TB];
#pragma unroll
        for (int i = 0; i < GW; ++i)
#pragma unroll
            for (int j = 0; j < TB; ++j)
                acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

        // per-lane LDS offsets of the fragment reads (see the layout above);
        // K step kk of a stage reads chunks 4 kk + kq of the weight rows
        const int arow0 = wn * GW * 16 * WROW + WROW * i16;
        const int xrow = wm * (BM / NWM) + i16;
        const int bfrag_lo = L::kW + 128 * xrow + 16 * (kq ^ ((i16 >> 1) & 7));
        const int bfrag_hi = L::kW + 128 * xrow + 16 * ((kq + 4) ^ ((i16 >> 1) & 7));
        const int wexp = NS * L::kStage + 16 * (wn * (BN / 2) + i16) + kq;
        const int xexp = NS * L::kStage + L::kWE + 16 * xrow + kq;

        // 16-row activation blocks of this wavefront that hold dispatched
        // rows (the MFMAs of the others would only feed discarded columns)
        // (wavefront-uniform: read into a scalar register, so the guards
        // below are scalar branches, not lane masks around every MFMA)
        const int nlive_lane = min(TB, max(0, (nrows - wm * (BM / NWM) + 15) >> 4));
        const int nlive = __builtin_amdgcn_readfirstlane(nlive_lane);

        // The K loop, instantiated per count NL of this wavefront's live
        // 16-row blocks (NL = TB in all but an expert's last row tile): it
        // reads the fragments and exponents of a K step and issues its
        // GW x NL MFMAs with no branch between them.  Per-block guards
        // inside the loop would split it into one basic block per MFMA and
        // serialise every LDS read with the MFMAs that use it.
        auto k_loop = [&](auto nl_tag) {
            constexpr int NL = decltype(nl_tag)::value;   // live 16-row blocks
        issue(0);
        if (NS == 3 && U > 1)
            issue(1);
        for (int u = 0; u < U; ++u) {
            if (NS == 3) {
                // stage u + 1 (issued last) may keep its WI weight loads in
                // flight when it is a whole stage (vector memory operations
                // count down in issue order, the previous item's stores
                // included); a partial stage u + 1 waits for everything
                if (u + 1 < U && KU * (u + 2) <= KS)
                    wait_vmcnt<WI>();
                else
                    wait_vmcnt<0>();
                // every wavefront's loads of stage u are done and every
                // wavefront is done with stage u - 1, whose buffer u + 2 takes
                raw_barrier();
                if (u + 2 < U)
                    issue(u + 2);
            } else {
                // this wavefront's loads of stage u are the only ones
                // outstanding; after the barrier every wavefront's are done
                // and nobody reads the other stage any more, so the next
                // stage's loads go there
                wait_vmcnt<0>();
                raw_barrier();
                if (u + 1 < U)
                    issue(u + 1);
            }
            const uint8_t *st = lds + (u % NS) * L::kStage;
#pragma unroll
            for (int kk = 0; kk < KU; ++kk) {
                const int ks = KU * u + kk;
                if (ks >= KS)
                    break;
                const uint8_t *ex = lds + ((ks >> 2) % L::kExpSlots) * L::kExp + (4 * ks - ebase(ks >> 2));
                const uint8_t *sx = st + kk * (BM * 128);
                const int afrag = arow0 + 16 * ((4 * kk + kq) ^ ((i16 >> 1) & WSWZ));
                // the activation fragments of the NL live blocks, then per
                // weight group its fragment and NL MFMAs; weight fragments
                // double-buffered, so group i + 1's read is in flight while
                // group i's MFMAs issue
                if constexpr (NL > 0) {
                v8i b[NL];
                int sb[NL];
#pragma unroll
                for (int j = 0; j < NL; ++j) {
                    const u32x4 lo = lds_read16(sx + bfrag_lo + j * 2048);
                    const u32x4 hi = lds_read16(sx + bfrag_hi + j * 2048);
                    b[j] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                    sb[j] = ex[xexp + j * 256];
                }
                u32x4 a_cur = lds_read16(st + afrag);
                int sa_cur = ex[wexp];
#pragma unroll
                for (int i = 0; i < GW; ++i) {
                    u32x4 a_nxt = a_cur;
                    int sa_nxt = sa_cur;
                    if (i + 1 < GW) {
                        a_nxt = lds_read16(st + afrag + (i + 1) * 16 * WROW);
                        sa_nxt = ex[wexp + (i + 1) * 256];
                    }
                    const v8i a = v8i{(int)a_cur[0], (int)a_cur[1], (int)a_cur[2],
                                      (int)a_cur[3], 0, 0, 0, 0};
#pragma unroll
                    for (int j = 0; j < NL; ++j)
                        acc[i][j] = mfma_w4a8(a, b[j], acc[i][j], sa_cur, sb[j]);
                    a_cur = a_nxt;
                    sa_cur = sa_nxt;
                }
                }
            }
        }
        };
        // one instance per count of live blocks (each straight-line; a
        // wavefront whose blocks all lie past the tile's rows still loads
        // its share of the stages and keeps the barriers, without MFMAs)
        if (__builtin_expect(nlive == TB, 1))
            k_loop(std::integral_constant<int, TB>{});
        else if constexpr (TB >= 4) {
            if (nlive == 3)
                k_loop(std::integral_constant<int, (TB >= 4 ? 3 : 0)>{});
            else if (nlive == 2)
                k_loop(std::integral_constant<int, (TB >= 4 ? 2 : 0)>{});
            else if (nlive == 1)
                k_loop(std::integral_constant<int, 1>{});
            else
                k_loop(std::integral_constant<int, 0>{});
        } else if constexpr (TB == 2) {
            if (nlive == 1)
                k_loop(std::integral_constant<int, 1>{});
            else
                k_loop(std::integral_constant<int, 0>{});
        } else {
            k_loop(std::integral_constant<int, 0>{});
        }

        // epilogue: lane holds tile row (wm BM/NWM + 16j + i16), weight rows
        // 4kq..4kq+3 of each of its GW groups.  On the 128- and 256-row
        // tiles its thread indices come from an opaque copy of the thread id,
        // so the compiler recomputes the epilogue's LDS and global addresses
        // here instead of hoisting them out of the item loop and holding them
        // (spilled, 4 to 46 registers) across the K loop.
        int tid_e = tid;
        if constexpr (BM >= 128)
            asm volatile("" : "+v"(tid_e));
        {
        const int tid = tid_e, lane = tid & 63, wave = tid >> 6;
        const int i16 = lane & 15, kq = lane >> 4;
        const int wn = wave & 1, wm = wave >> 1;
        if constexpr (kGemm1) {
            constexpr int CB = GW / 2;   // 16-column blocks of h per wavefront
            // the h codes go through LDS (rows of BN/2 + 16 bytes, so the
            // 4-byte writes of a wavefront hit distinct banks), then out as
            // whole 16-byte pieces of rows
            constexpr int HP = BN / 2 + 16;
            static_assert(BM * HP <= L::kRing,
                          "h tile fits the stage ring");
            __syncthreads();   // every wavefront is done with the stage ring
#pragma unroll
            for (int j = 0; j < TB; ++j) {
                const int m = wm * (BM / NWM) + 16 * j + i16;
                float hv[CB][4];
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        hv[cb][v] = swiglu_clamped(acc[cb][j][v], acc[cb + CB][j][v],
                                                   s.gate_limit, s.up_limit);
#pragma unroll
                for (int blk = 0; blk < CB / 2; ++blk) {
                    float amax = 0.0f;
#pragma unroll
                    for (int cb = 2 * blk; cb < 2 * blk + 2; ++cb)
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            amax = fmaxf(amax, fabsf(hv[cb][v]));
                    amax = fmaxf(amax, __shfl_xor(amax, 16));
                    amax = fmaxf(amax, __shfl_xor(amax, 32));
                    const int E = mx8_block_exponent(amax);
                    const int tcol = (BN / 4) * wn + 32 * blk;   // column in the tile
#pragma unroll
                    for (int cb = 2 * blk; cb < 2 * blk + 2; ++cb)
                        *reinterpret_cast<uint32_t *>(lds + m * HP + tcol + 16 * (cb - 2 * blk) +
                                                      4 * kq) =
                            mx8_pack4(hv[cb][0], hv[cb][1], hv[cb][2], hv[cb][3], E, amax);
                    if (m < nrows && kq == 0)
                        hs_out[(size_t)(row0 + m) * (size_t)(I / 32) + (nt * (BN / 2) + tcol) / 32] =
                            (uint8_t)(E + 127);
                }
            }
            __syncthreads();
            constexpr int PR = BN / 32;                // 16-byte pieces per row
#pragma unroll
            for (int p = 0; p < (BM * PR + NTH - 1) / NTH; ++p) {
                const int piece = p * NTH + tid, r = piece / PR, c = piece % PR;
                if (piece < BM * PR && r < nrows)
                    *reinterpret_cast<u32x4 *>(h_out + (size_t)(row0 + r) * (size_t)I +
                                               (size_t)nt * (BN / 2) + 16 * c) =
                        lds_read16(lds + r * HP + 16 * c);
            }
        } else if (g.y8_out) {
            // MX FP8 rows: one exponent per 32 consecutive output columns
            // (weight groups 2b and 2b + 1 of a wavefront, met across the
            // four lanes kq of a route), by the requant's rule; the codes go
            // through LDS (rows of BN + 16 bytes, so the 4-byte writes of a
            // wavefront hit distinct banks), then out as whole 16-byte pieces
            // of rows
            constexpr int YP = BN + 16;
            static_assert(BM * YP <= L::kRing, "y code tile fits the stage ring");
            static_assert(GW % 2 == 0, "32-column blocks");
            __syncthreads();   // every wavefront is done with the stage ring
#pragma unroll
            for (int j = 0; j < TB; ++j) {
                const int m = wm * (BM / NWM) + 16 * j + i16;
#pragma unroll
                for (int blk = 0; blk < GW / 2; ++blk) {
                    float amax = 0.0f;
#pragma unroll
                    for (int i = 2 * blk; i < 2 * blk + 2; ++i)
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            amax = fmaxf(amax, fabsf(acc[i][j][v]));
                    amax = fmaxf(amax, __shfl_xor(amax, 16));
                    amax = fmaxf(amax, __shfl_xor(amax, 32));
                    const int E = mx8_block_exponent(amax);
                    const int tcol = (BN / 2) * wn + 32 * blk;   // column in the tile
#pragma unroll
                    for (int i = 2 * blk; i < 2 * blk + 2; ++i)
                        *reinterpret_cast<uint32_t *>(lds + m * YP + tcol + 16 * (i - 2 * blk) +
                                                      4 * kq) =
                            mx8_pack4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3], E,
                                      amax);
                    if (m < nrows && kq == 0)
                        g.y8s_out[(size_t)(row0 + m) * (size_t)(H / 32) + (nt * BN + tcol) / 32] =
                            (uint8_t)(E + 127);
                }
            }
            __syncthreads();
            constexpr int PR = BN / 16;                // 16-byte pieces per row
#pragma unroll
            for (int p = 0; p < (BM * PR + NTH - 1) / NTH; ++p) {
                const int piece = p * NTH + tid, r = piece / PR, c = piece % PR;
                if (piece < BM * PR && r < nrows)
                    *reinterpret_cast<u32x4 *>(g.y8_out + (size_t)(row0 + r) * (size_t)H +
                                               (size_t)nt * BN + 16 * c) =
                        lds_read16(lds + r * YP + 16 * c);
            }
        } else {
            // the bf16 tile goes through LDS (rows of BN*2 + 16 bytes: the
            // fragment writes of a half-wavefront hit distinct banks), then
            // out as whole 16-byte pieces of rows, 32 lanes to a 512-byte row
            constexpr int PITCH = BN * 2 + 16;
            static_assert(BM * PITCH <= L::kRing,
                          "y tile fits the stage ring");
            __syncthreads();   // every wavefront is done with the stage ring
#pragma unroll
            for (int j = 0; j < TB; ++j) {
                const int m = wm * (BM / NWM) + 16 * j + i16;
#pragma unroll
                for (int i = 0; i < GW; ++i)
                    *reinterpret_cast<uint2 *>(lds + m * PITCH + 2 * ((BN / 2) * wn + 16 * i + 4 * kq)) =
                        uint2{f32_to_bf16(acc[i][j][0]) | (f32_to_bf16(acc[i][j][1]) << 16),
                              f32_to_bf16(acc[i][j][2]) | (f32_to_bf16(acc[i][j][3]) << 16)};
            }
            __syncthreads();
            constexpr int PR = BN / 8;                 // 16-byte pieces per row
#pragma unroll
            for (int p = 0; p < BM * PR / NTH; ++p) {
                const int piece = p * NTH + tid, r = piece / PR, c = piece % PR;
                if (r < nrows)
                    *reinterpret_cast<u32x4 *>(y_out + (size_t)(row0 + r) * (size_t)H +
                                               (size_t)nt * BN + 8 * c) = lds_read16(lds + r * PITCH + 16 * c);
            }
        }
        }
    }
}

// LDS of a workgroup running BM-row tiles with the given stage ring.
template <int BM, int BN, int KU>
struct TileShared {
    using L = TileLds<BM, BN, KU>;
    __align__(16) uint8_t ring[L::kRing];
    int prefix[kMaxLocalExperts + 1];
    int arow[BM];
};

// ---------------------------------------------------------------------------
// The persistent layer for 128-row tiles: GEMM1 + SwiGLU + requant and GEMM2
// in one launch, one work queue per XCD.  Row chunk q belongs to queue
// q mod nq; a workgroup serves the queue of the XCD it runs on (hardware
// XCC id mod nq, nq = the device's XCD count), so the h rows of a chunk are
// written and read through one L2.  A queue hands out tickets for first
// every GEMM1 item of its chunks, then every GEMM2 item; a GEMM2 item of
// chunk q waits until ready[q] counts all NT1 GEMM1 items of q, so GEMM2
// starts on the first chunks while GEMM1 finishes the last ones.  A
// workgroup takes its next ticket when it starts an item (the atomic's
// round trip hides behind the item); tickets go out in dependency order
// and a workgroup's tickets rise, so every wait is on items that running
// workgroups hold and reach first.  A GEMM1 item counts in ready[q] once
// its h stores are in the L2; GEMM2 reads h past the CU's L1.
// sync[32 x] is queue x's ticket counter (one 128-byte line each),
// sync[256 + q] = ready[q], all zero at launch.  Every wait is bounded by
// max_polls: past the bound the workgroup counts the timeout in status[2]
// and goes on (its GEMM2 item may then read h before it is written), so
// the caller sees a failed layer instead of a GPU that never finishes.
template <int BM, int BN1, int BN2, int KU>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
layer_persistent_kernel(Shape s, TiledArgs g1, TiledArgs g2, int32_t *sync, int32_t *status,
                        int nq, int max_polls)
{
    // one stage ring, sized for the wider of the two weight tiles
    __shared__ TileShared<BM, (BN1 > BN2 ? BN1 : BN2), KU> sh;
    __shared__ int ticket_sh;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int NT1 = s.I / (BN1 / 2), NT2 = s.H / BN2;
    const int nchunks = plan_chunks(s, g1.counts, BM, sh.prefix);
    unsigned xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    const int x = (int)(xcc & 7u) % nq;
    const int mine = nchunks > x ? (nchunks - x + nq - 1) / nq : 0;
    const int n1 = mine * NT1, n2 = mine * NT2;
    int32_t *ticket = sync + 32 * x, *ready = sync + 256;
    // wavefront 0 takes tickets (whole-wavefront atomic, value 1 in lane 0:
    // control flow stays uniform) and hands them to the others through LDS
    if (wave == 0) {
        const int t0 = atomicAdd(ticket, lane == 0 ? 1 : 0);
        ticket_sh = __builtin_amdgcn_readfirstlane(t0);
    }
    __syncthreads();
    for (;;) {
        const int t = ticket_sh;
        __syncthreads();
        if (t >= n1 + n2)
            break;
        int next = 0;
        if (wave == 0)
            next = atomicAdd(ticket, lane == 0 ? 1 : 0);
        if (t < n1) {
            const int q = x + nq * (t / NT1), nt = t % NT1;
            tiled_item<true, BM, BN1, KU, false>(s, g1, sh.prefix, sh.arow, sh.ring, q, nt);
            wait_vmcnt<0>();   // this thread's h stores are in the L2
            __syncthreads();   // ... and every thread's
            if (wave == 0)
                atomicAdd(&ready[q], lane == 0 ? 1 : 0);
        } else {
            const int q = x + nq * ((t - n1) / NT2), nt = (t - n1) % NT2;
            if (wave == 0) {
                bool done = false;
                for (int it = 0; it < max_polls; ++it) {
                    const int v = __builtin_amdgcn_readfirstlane(
                        __hip_atomic_load(&ready[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
                    if (v >= NT1) {
                        done = true;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
                if (!done)
                    atomicAdd(&status[2], lane == 0 ? 1 : 0);
            }
            __syncthreads();
            tiled_item<false, BM, BN2, KU, true>(s, g2, sh.prefix, sh.arow, sh.ring, q, nt);
        }
        if (wave == 0)
            ticket_sh = __builtin_amdgcn_readfirstlane(next);
        __syncthreads();
    }
}

__global__ void __launch_bounds__(256) fill_zero_kernel(int32_t *p, int n)
{
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256)
        p[i] = 0;
}

// Row chunk q and N tile nt of grid-stride item `item` (workgroup blockIdx.x
// of a launch whose workgroup b runs on XCD b mod 8).  With bq = 0 items go
// chunk-major (item = q * NT + nt).  With bq > 0 the (chunk, N tile) grid is
// cut into blocks of bq chunks x bnt N tiles (clipped at the edges), blocks
// row-major, items row-major inside a block; in every full round of the
// grid-stride loop the G / 8 workgroups of one XCD take consecutive items
// of that order, so the workgroups that share an XCD's L2 work on one block
// at a time: each activation tile is read by bnt of them, each weight tile
// by bq (chunk-major, an XCD's workgroups hold ~G / 8 / 3 chunks x 3 N
// tiles of each round).  The last, partial round keeps the plain order.
// A bijection of [0, items) onto the grid, every q < nchunks and nt < NT.
__device__ __forceinline__ void tile_of_item(long item, long items, int nchunks, int NT, int bq,
                                             int bnt, int &q, int &nt)
{
    long e = item;
    const long G = gridDim.x;
    const long base = item - blockIdx.x;
    if (bq > 0 && (G & 7) == 0 && base + G <= items)
        e = base + (long)(blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    if (bq <= 0) {
        q = (int)(e / NT);
        nt = (int)(e - (long)q * NT);
        return;
    }
    const long per_row = (long)bq * NT;
    const int qb = (int)(e / per_row);
    long rem = e - (long)qb * per_row;
    const int rows_q = min(bq, nchunks - qb * bq);
    const int nb = (int)(rem / (rows_q * bnt));
    rem -= (long)nb * rows_q * bnt;
    const int w = min(bnt, NT - nb * bnt);
    q = qb * bq + (int)(rem / w);
    nt = nb * bnt + (int)(rem % w);
}

template <bool kGemm1, int BM, int BN, int KU, int NW>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
gemm_tiled_kernel(Shape s, TiledArgs g, int bq, int bnt)
{
    __shared__ TileShared<BM, BN, KU> sh;
    const int NT = kGemm1 ? s.I / (BN / 2) : s.H / BN;
    const int nchunks = plan_chunks<NW * 64>(s, g.counts, BM, sh.prefix);
    const long items = (long)nchunks * NT;
    for (long item = blockIdx.x; item < items; item += gridDim.x) {
        int q, nt;
        tile_of_item(item, items, nchunks, NT, bq, bnt, q, nt);
        tiled_item<kGemm1, BM, BN, KU, false, NW>(s, g, sh.prefix, sh.arow, sh.ring, q, nt);
        __syncthreads();
    }
}

template <typename KernelT>
int tiled_grid(KernelT kernel, long upper_items, int threads = kThreads)
{
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) !=
            hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    long g = (long)device_cu_count() * per_cu;
    if (upper_items < g)
        g = upper_items;
    return (int)(g < 1 ? 1 : g);
}

long tile_upper_bound(const moe_shape &s, int bm)
{
    const long rows = s.dispatch_mode == MOE_DISPATCH_FIXED_SLOT
                          ? (long)s.E_local * s.capacity
                          : (long)s.T * s.K;
    return rows / bm + s.E_local;
}

} // namespace

// Rows per expert the host expects: every slot routed, experts equally likely.
static double per_expert_rows(const moe_shape &s)
{
    return (double)s.T * s.K / (double)(s.E_total > 0 ? s.E_total : 1);
}

// Row tiles by the expected rows per expert:
// - 32-row tiles up to 16 (decode: GEMM1 and GEMM2 -5%; 1,024 tokens -3 to
//   -7%; at 2,048 tokens and on the Flash shape, where experts pass 32 rows
//   and stream their weights twice, +30 to +60%);
// - 64-row tiles up to 96.  An expert past 64 rows streams its weights twice
//   (64-row tiles read them non-temporally), yet on the Flash shape with a
//   tenth of the slots -1 (57 rows per expert on average) the 64-row tiles
//   still win, 334 against 360 us for GEMM1; with no -1 slots (64 rows) the
//   128-row tiles win, 354 against 434 us;
// - 128-row tiles above, and 256-row tiles from 512 (eight wavefronts, one
//   workgroup per CU; at 65,536 tokens, GEMM alone: GEMM1 1,999 against
//   2,151 us for 128 x 256 tiles, GEMM2 1,115 against 1,186).
// The host sees neither the -1 slots nor the skew, so shapes near the bounds
// are left to the tuned table.  tiled_bm gives the class (64 or 128),
// tiled_config the tile.
int tiled_bm(const moe_shape &s)
{
    const double per_expert = per_expert_rows(s);
    return per_expert <= 96.0 ? 64 : 128;
}

namespace {

// Weight rows per tile: 256, or 128 when the expected number of items with
// 256 would leave fewer than three rounds for the resident workgroups (two
// per CU), so the last, partly filled round costs little.
int tiled_bn(const moe_shape &s, bool gemm1)
{
    const double per_expert = per_expert_rows(s);
    const int bm = tiled_bm(s);
    const double tiles = (double)s.E_local * (double)(long)((per_expert + bm - 1) / bm);
    const double nt256 = gemm1 ? s.I / 128 : s.H / 256;
    const bool fits256 = gemm1 ? s.I % 128 == 0 : s.H % 256 == 0;
    if (!fits256)
        return 128;
    return tiles * nt256 < 3.0 * 2 * device_cu_count() ? 128 : 256;
}

// Tile shape and K steps per LDS stage.  Two steps per stage (128 bytes of
// every weight row per load) stream HBM faster; they double the stage, so
// they are used where two workgroups per CU still fit: 64-row tiles, which
// are HBM-bound, take 128 weight rows and two steps.
struct TiledConfig {
    int bm, bn, ku;
};

// The tile shapes compiled for both GEMMs (a tuned table may name only these).
constexpr TiledConfig kTiledShapes[] = {{32, 128, 2},  {64, 128, 2},  {64, 256, 1},
                                        {128, 128, 1}, {128, 256, 1}, {256, 256, 1}};

// A tuned table ("[FlyDSL] Add full-expert DeepSeek V4.1 Flash MegaMoE tuning
// for gfx950", tuning: one config per shape and token bucket, a count between
// two buckets taking the larger one): entries set through
// moe_set_tile_table, read by every launch under a lock.
constexpr int kMaxTileEntries = 256;
std::mutex g_table_mu;
moe_tile_entry g_table[kMaxTileEntries];
int g_table_n = 0;

bool table_lookup(const moe_shape &s, bool gemm1, TiledConfig *out)
{
    std::lock_guard<std::mutex> lock(g_table_mu);
    int best = -1;
    for (int i = 0; i < g_table_n; ++i) {
        const moe_tile_entry &e = g_table[i];
        if (e.gemm != (gemm1 ? 1 : 2) || e.H != s.H || e.I != s.I || e.K != s.K ||
            e.E_total != s.E_total || e.E_local != s.E_local || e.max_tokens < s.T)
            continue;
        // N tiles must cover the output columns exactly
        if (gemm1 ? s.I % (e.bn / 2) != 0 : s.H % e.bn != 0)
            continue;
        if (best < 0 || e.max_tokens < g_table[best].max_tokens)
            best = i;
    }
    if (best < 0)
        return false;
    *out = TiledConfig{g_table[best].bm, g_table[best].bn, g_table[best].ku};
    return true;
}

TiledConfig tiled_config(const moe_shape &s, bool gemm1)
{
    TiledConfig c;
    if (table_lookup(s, gemm1, &c))
        return c;
    const int bm = tiled_bm(s), bn = tiled_bn(s, gemm1);
    const double per_expert = per_expert_rows(s);
    if (bm == 64)
        return per_expert <= 16.0 ? TiledConfig{32, 128, 2} : TiledConfig{64, 128, 2};
    if (bn == 256 && per_expert >= 512.0)
        return {256, 256, 1};
    return {bm, bn, 1};
}

template <bool kGemm1, int BM, int BN, int KU>
hipError_t launch_tiled(const moe_shape &sh, const uint8_t *act, const uint8_t *act_s,
                        const int32_t *counts, const int32_t *offsets, const int32_t *row_route,
                        const uint8_t *w, const uint8_t *ws, uint8_t *h, uint8_t *hs, const YRows &y,
                        hipStream_t st)
{
    // eight wavefronts for the 256-row tile, four otherwise
    constexpr int NW = BM == 256 ? 8 : 4;
    auto k = gemm_tiled_kernel<kGemm1, BM, BN, KU, NW>;
    const long nt = kGemm1 ? sh.I / (BN / 2) : sh.H / BN;
    const int grid = tiled_grid(k, tile_upper_bound(sh, BM) * nt, NW * 64);
    // MFMA-bound tiles (weight tiles reused by several row chunks) take the
    // blocked item order: an XCD's grid / 8 workgroups of a round share
    // 8 N tiles (or all, when fewer) and grid / 64 row chunks
    int bq = 0, bnt = 0;
    if (BM >= 128 && grid % 8 == 0) {
        bnt = nt < 8 ? (int)nt : 8;
        bq = grid / 8 / bnt > 1 ? grid / 8 / bnt : 1;
    }
    k<<<grid, NW * 64, 0, st>>>(to_dev(sh),
                                 TiledArgs{act, act_s, counts, offsets, row_route, w, ws, h, hs,
                                           y.bf16, y.codes, y.scales},
                                 bq, bnt);
    return hipGetLastError();
}

template <bool kGemm1>
hipError_t launch_tiled_any(const moe_shape &sh, const uint8_t *act, const uint8_t *act_s,
                            const int32_t *counts, const int32_t *offsets,
                            const int32_t *row_route, const uint8_t *w, const uint8_t *ws,
                            uint8_t *h, uint8_t *hs, const YRows &y, hipStream_t st)
{
    const TiledConfig c = tiled_config(sh, kGemm1);
#define MOE_TILED_CASE(BM, BN, KU)                                                                \
    if (c.bm == BM && c.bn == BN && c.ku == KU)                                                   \
        return launch_tiled<kGemm1, BM, BN, KU>(sh, act, act_s, counts, offsets, row_route, w, ws, \
                                                h, hs, y, st);
    MOE_TILED_CASE(32, 128, 2)
    MOE_TILED_CASE(64, 128, 2)
    MOE_TILED_CASE(64, 256, 1)
    MOE_TILED_CASE(128, 128, 1)
    MOE_TILED_CASE(256, 256, 1)
#undef MOE_TILED_CASE
    return launch_tiled<kGemm1, 128, 256, 1>(sh, act, act_s, counts, offsets, row_route, w, ws, h,
                                             hs, y, st);
}

} // namespace

hipError_t launch_gemm1_tiled(const moe_shape &sh, const uint8_t *x, const uint8_t *xs,
                              const int32_t *counts, const int32_t *offsets,
                              const int32_t *row_route, const uint8_t *w13, const uint8_t *w13s,
                              uint8_t *h, uint8_t *hs, hipStream_t st)
{
    return launch_tiled_any<true>(sh, x, xs, counts, offsets, row_route, w13, w13s, h, hs,
                                  YRows{nullptr, nullptr, nullptr}, st);
}

// XCDs of the device: the MI355X has 32 CUs per XCD, and its partition modes
// give a device 1, 2, 4 or 8 of them (0 for any other CU count).
static int xcd_count()
{
    const int cus = device_cu_count();
    return cus == 32 || cus == 64 || cus == 128 || cus == 256 ? cus / 32 : 0;
}

int set_tile_table(const moe_tile_entry *entries, int n)
{
    if (n < 0 || n > kMaxTileEntries || (n > 0 && !entries))
        return MOE_EINVAL;
    for (int i = 0; i < n; ++i) {
        const moe_tile_entry &e = entries[i];
        bool known = false;
        for (const TiledConfig &c : kTiledShapes)
            known |= c.bm == e.bm && c.bn == e.bn && c.ku == e.ku;
        if (!known || (e.gemm != 1 && e.gemm != 2) || e.max_tokens < 0)
            return MOE_EINVAL;
    }
    std::lock_guard<std::mutex> lock(g_table_mu);
    for (int i = 0; i < n; ++i)
        g_table[i] = entries[i];
    g_table_n = n;
    return MOE_OK;
}

bool tile_config_of(const moe_shape &s, bool gemm1, int *bm, int *bn, int *ku)
{
    if (!(gemm1 ? use_tiled_gemm1(s) : use_tiled_gemm2(s)))
        return false;
    const TiledConfig c = tiled_config(s, gemm1);
    *bm = c.bm;
    *bn = c.bn;
    *ku = c.ku;
    return true;
}

// The tile config of the persistent layer: that of the launches, with
// 256-row tiles run as 128 rows (the persistent kernels are built for four
// wavefronts and two workgroups per CU).
static TiledConfig persistent_config(const moe_shape &sh, bool gemm1)
{
    TiledConfig c = tiled_config(sh, gemm1);
    if (c.bm == 256)
        c.bm = 128;
    return c;
}

// The persistent layer takes the tiled GEMMs when both use the same row
// tile: 128 rows with one K step per stage (any weight tile widths) or 32 or
// 64 rows with two K steps and 128 weight rows; on a device whose XCDs it
// can tell apart.
bool persistent_supported(const moe_shape &sh)
{
    if (sh.H < 512 || sh.I < 512 || xcd_count() == 0)
        return false;
    const TiledConfig a = persistent_config(sh, true), b = persistent_config(sh, false);
    if (a.bm == 128 && b.bm == 128 && a.ku == 1 && b.ku == 1)
        return true;
    return (a.bm == 32 || a.bm == 64) && b.bm == a.bm && a.ku == 2 && b.ku == 2 && a.bn == 128 &&
           b.bn == 128;
}

int persistent_sync_words(const moe_shape &sh) { return 256 + (int)tile_upper_bound(sh, 32); }

// Polls of a persistent wait before it gives up (2^22 polls of s_sleep 2,
// about a second); MOE_PERSISTENT_MAX_POLLS in the environment, read at
// every launch, lowers it (0: no poll, every wait gives up at once), so a
// test can make the waits give up while every kernel still exits normally.
static int persistent_max_polls()
{
    constexpr int kDefault = 1 << 22;
    const char *v = getenv("MOE_PERSISTENT_MAX_POLLS");
    if (!v || !*v)
        return kDefault;
    char *end = nullptr;
    const long n = strtol(v, &end, 10);
    return *end == 0 && n >= 0 && n < kDefault ? (int)n : kDefault;
}

hipError_t launch_layer_persistent(const moe_shape &sh, const uint8_t *x, const uint8_t *xs,
                                   const int32_t *counts, const int32_t *offsets,
                                   const int32_t *row_route, const uint8_t *w13,
                                   const uint8_t *w13s, const uint8_t *w2, const uint8_t *w2s,
                                   uint8_t *h, uint8_t *hs, const YRows &y, int32_t *sync,
                                   int32_t *status, hipStream_t st)
{
    const int nsync = persistent_sync_words(sh);
    fill_zero_kernel<<<(nsync + 255) / 256, 256, 0, st>>>(sync, nsync);
    const TiledArgs g1{x, xs, counts, offsets, row_route, w13, w13s, h, hs, nullptr, nullptr,
                       nullptr};
    const TiledArgs g2{h, hs, counts, offsets, nullptr, w2, w2s, nullptr, nullptr, y.bf16,
                       y.codes, y.scales};
    const TiledConfig c1 = persistent_config(sh, true);
    const int bn1 = c1.bn, bn2 = persistent_config(sh, false).bn;
    const int nq = xcd_count();
    // workgroup b runs on XCD b mod nq: a grid of nq or more workgroups puts
    // at least one on every XCD, so every queue is served
    auto go = [&](auto k, int bm, int b1, int b2) {
        const long items = tile_upper_bound(sh, bm) * (long)(sh.I / (b1 / 2) + sh.H / b2);
        const int grid = tiled_grid(k, items);
        k<<<grid > nq ? grid : nq, kThreads, 0, st>>>(to_dev(sh), g1, g2, sync, status, nq,
                                                        persistent_max_polls());
    };
    if (c1.bm == 32)
        go(layer_persistent_kernel<32, 128, 128, 2>, 32, 128, 128);
    else if (c1.bm == 64)
        go(layer_persistent_kernel<64, 128, 128, 2>, 64, 128, 128);
    else if (bn1 == 256 && bn2 == 256)
        go(layer_persistent_kernel<128, 256, 256, 1>, 128, 256, 256);
    else if (bn1 == 256)
        go(layer_persistent_kernel<128, 256, 128, 1>, 128, 256, 128);
    else if (bn2 == 256)
        go(layer_persistent_kernel<128, 128, 256, 1>, 128, 128, 256);
    else
        go(layer_persistent_kernel<128, 128, 128, 1>, 128, 128, 128);
    return hipGetLastError();
}

hipError_t launch_gemm2_tiled(const moe_shape &sh, const uint8_t *h, const uint8_t *hs,
                              const int32_t *counts, const int32_t *offsets, const uint8_t *w2,
                              const uint8_t *w2s, const YRows &y, hipStream_t st)
{
    return launch_tiled_any<false>(sh, h, hs, counts, offsets, nullptr, w2, w2s, nullptr,
                                   nullptr, y, st);
}

} // namespace moe
