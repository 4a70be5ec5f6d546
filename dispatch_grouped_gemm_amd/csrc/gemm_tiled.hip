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

#include "dispatch_dev.hpp"

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
        const uint8_t *__restrict__ w = uniform_ptr(g.w + (size_t)e * wrows * (size_t)(KT / 2));
        const uint8_t *__restrict__ ws = uniform_ptr(g.ws + (size_t)e * wrows * (size_t)(KT / 32));
        const uint8_t *__restrict__ act =
            uniform_ptr(kGemm1 ? g.act : g.act + (size_t)row0 * (size_t)KT);
        const uint8_t *__restrict__ act_s =
            uniform_ptr(kGemm1 ? g.act_s : g.act_s + (size_t)row0 * (size_t)(KT / 32));
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
                    __builtin_nontemporal_store(
                        lds_read16(lds + r * YP + 16 * c),
                        reinterpret_cast<u32x4 *>(g.y8_out + (size_t)(row0 + r) * (size_t)H +
                                                  (size_t)nt * BN + 16 * c));
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
            // non-temporal: y is read once, by the combine (the stores drain
            // sooner, and the next item's first wait, which counts them,
            // ends sooner: -1% GEMM2 at 65,536 tokens, -6% at 2,048)
            constexpr int PR = BN / 8;                 // 16-byte pieces per row
#pragma unroll
            for (int p = 0; p < BM * PR / NTH; ++p) {
                const int piece = p * NTH + tid, r = piece / PR, c = piece % PR;
                if (r < nrows)
                    __builtin_nontemporal_store(
                        lds_read16(lds + r * PITCH + 16 * c),
                        reinterpret_cast<u32x4 *>(y_out + (size_t)(row0 + r) * (size_t)H +
                                                  (size_t)nt * BN + 8 * c));
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
// The persistent layer: dispatch, GEMM1 + SwiGLU + requant, GEMM2 and the
// combine in one launch ("MegaMoEV2: fuse Dispatch, GEMM1, GEMM2 and Combine
// into one kernel", Technical Details, large input: one persistent kernel
// overlaps the stages).  Every workgroup of the grid (all resident: the grid
// is the device's CUs times the kernel's occupancy) runs the phases in turn:
//
//  1. Dispatch.  Slice b of the route slots (b below min(grid, kMaxSlices)):
//     compact: per-wavefront histograms, the slice's totals into row b of a
//     table; after a grid barrier every workgroup sums the table (segment
//     sizes, and for its own slice the rows before it), scans the experts
//     and scatters its slots stably; a second barrier publishes row_route
//     and route_row.  Fixed-slot: wave-aggregated claims on per-expert
//     counters in the header, then one barrier.
//  2. GEMM1 and GEMM2 from one work queue per XCD (chunk q on queue q mod
//     nq, served by the workgroups running on that XCD, so h is written and
//     read through one L2): all GEMM1 tickets of a queue before its GEMM2
//     tickets; a GEMM2 item of chunk q waits until ready[q] counts all NT1
//     GEMM1 items of q.  Tickets map to (chunk, N tile) in blocks of bq
//     chunks x bnt N tiles, so each round of an XCD's workgroups shares
//     weight tiles and activation rows in its L2 (the pages' n-major claims
//     when an expert is large: a weight tile serves bq row chunks in turn).
//  3. After a grid barrier (every workgroup done with its tickets, y made
//     visible device-wide), the combine of every token.
//
// Barriers: each workgroup makes its stores visible at device scope (a
// release fence, once per barrier and workgroup), adds itself to a counter
// and polls it (relaxed), then takes an acquire fence.  Every wait is
// bounded by max_polls: a barrier that gives up is counted and sends its
// workgroup straight to the end, so no phase ever reads data that was not
// written (a GEMM2 wait that gives up goes on with h that may be stale but
// is in bounds); the caller sees the count in status[2].
//
// The header (the first kHdrWords words of the workspace) must be zero at
// launch; the last workgroup to finish copies the status words out and
// zeroes it again, so a workspace stays ready for the next call.
constexpr int kHdrTicket = 0;      // + 32 x: ticket counter of XCD queue x < 8
constexpr int kHdrBarrier = 256;   // barrier arrivals, cumulative
constexpr int kHdrDepart = 288;    // workgroups finished
constexpr int kHdrInvalid = 320;   // ids outside [-1, E_total)
constexpr int kHdrDropped = 352;   // fixed-slot routes past capacity
constexpr int kHdrTimeouts = 384;  // waits that gave up
constexpr int kHdrClaims = 512;    // fixed-slot claim counter of each local expert
constexpr int kMaxSlices = 256;    // compact histogram table rows
constexpr int kSliceSlots = 2048;  // fewest route slots per dispatch slice
static_assert(kHdrClaims + kMaxLocalExperts <= kPersistentHeaderWords, "header size");

struct FusedArgs {
    const int32_t *ids, *valid;
    const float *tw;
    const uint8_t *x, *xs, *w13, *w13s, *w2, *w2s;
    int32_t *counts, *offsets, *row_route, *route_row, *status;
    int32_t *hdr;      // kPersistentHeaderWords, zero at launch and at exit
    int32_t *table;    // [kMaxSlices][E_local + 1] slice histograms (compact)
    int32_t *ready;    // nready words: finished GEMM1 items per row chunk
    int nready;
    uint8_t *h, *hs;
    uint16_t *y;       // bf16 rows, or
    uint8_t *y8, *y8s; // MX FP8 rows
    uint16_t *out;
};

// Wavefront 0 polls *p (relaxed, device scope) until it reaches target, at
// most max_polls times; returns whether it did (in every lane).
__device__ __forceinline__ bool poll_at_least(const int32_t *p, int target, int max_polls)
{
    for (int it = 0; it < max_polls; ++it) {
        const int v = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        if (v >= target)
            return true;
        __builtin_amdgcn_s_sleep(2);
    }
    return false;
}

// Grid barrier number n (1, 2, ...): true when every workgroup of the grid
// arrived.  ok_sh is the workgroup's LDS word for the result.
__device__ __forceinline__ bool grid_barrier(int32_t *hdr, int n, int max_polls, int *ok_sh)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    wait_vmcnt<0>();   // this thread's stores are done
    __syncthreads();   // ... and every thread's
    if (wave == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        atomicAdd(&hdr[kHdrBarrier], lane == 0 ? 1 : 0);
        const bool ok = poll_at_least(&hdr[kHdrBarrier], n * (int)gridDim.x, max_polls);
        if (!ok)
            atomicAdd(&hdr[kHdrTimeouts], lane == 0 ? 1 : 0);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        if (lane == 0)
            *ok_sh = ok;
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(*ok_sh) != 0;
}

// Ticket t of a queue with `mine` row chunks and NT N tiles -> (local chunk
// index, N tile): blocks of bq chunks x bnt N tiles, clipped at the edges,
// chunk blocks outer, N blocks inner, chunk-major inside a block.
__device__ __forceinline__ void queue_item(int t, int mine, int NT, int bq, int bnt, int &qi,
                                           int &nt)
{
    const int full = bq * NT;
    const int qb = t / full, r = t - qb * full;
    const int cb = min(bq, mine - qb * bq);
    const int nb = r / (cb * bnt), r2 = r - nb * cb * bnt;
    const int nbw = min(bnt, NT - nb * bnt);
    qi = qb * bq + r2 / nbw;
    nt = nb * bnt + r2 % nbw;
}

// The combine of token t over chunks c0 .. c0 + nc - 1 of 64 pieces of its
// row (lane l takes piece 64 c + l of each): the kept routes in ascending k,
// each route's pieces loaded together, the same float32 arithmetic as
// combine_cols / combine8_cols (so the same bits).  kFP8: pieces of 16
// columns of MX FP8 rows, else 8 columns of bf16 rows.
template <bool kFP8, int U>
__device__ __forceinline__ void combine_row_part(const Shape &s, const FusedArgs &a, int t, int c0,
                                                 int nc)
{
#pragma clang fp contract(off)
    constexpr int V = kFP8 ? 16 : 8;
    const int lane = threadIdx.x & 63;
    float acc[U][V];
#pragma unroll
    for (int j = 0; j < U; ++j)
#pragma unroll
        for (int v = 0; v < V; ++v)
            acc[j][v] = 0.0f;
    for (int k = 0; k < s.K; ++k) {
        const int row = __builtin_amdgcn_readfirstlane(a.route_row[(size_t)t * s.K + k]);
        if (row < 0)
            continue;
        const float w = a.tw[(size_t)t * s.K + k];
        uint4 q[U];
        int e[U];
#pragma unroll
        for (int j = 0; j < U; ++j)
            if (j < nc) {
                const int col = ((c0 + j) * 64 + lane) * V;
                if (kFP8) {
                    q[j] = *reinterpret_cast<const uint4 *>(a.y8 + (size_t)row * s.H + col);
                    e[j] = (int)a.y8s[(size_t)row * (s.H / 32) + col / 32] - 127;
                } else {
                    q[j] = *reinterpret_cast<const uint4 *>(a.y + (size_t)row * s.H + col);
                }
            }
#pragma unroll
        for (int j = 0; j < U; ++j) {
            if (j >= nc)
                break;
            const uint32_t wd[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                if (kFP8) {
                    const float v[4] = {__builtin_amdgcn_cvt_f32_fp8((int)wd[d], 0),
                                        __builtin_amdgcn_cvt_f32_fp8((int)wd[d], 1),
                                        __builtin_amdgcn_cvt_f32_fp8((int)wd[d], 2),
                                        __builtin_amdgcn_cvt_f32_fp8((int)wd[d], 3)};
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const float p = w * ldexpf(v[b], e[j]);
                        acc[j][4 * d + b] = acc[j][4 * d + b] + p;
                    }
                } else {
                    const float p0 = w * __uint_as_float(wd[d] << 16);
                    const float p1 = w * __uint_as_float(wd[d] & 0xffff0000u);
                    acc[j][2 * d] = acc[j][2 * d] + p0;
                    acc[j][2 * d + 1] = acc[j][2 * d + 1] + p1;
                }
            }
        }
    }
    typedef unsigned int u4v __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int j = 0; j < U; ++j) {
        if (j >= nc)
            break;
        const int col = ((c0 + j) * 64 + lane) * V;
        u4v *dst = reinterpret_cast<u4v *>(a.out + (size_t)t * s.H + col);
#pragma unroll
        for (int g = 0; g < V / 8; ++g) {
            uint32_t o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                o[i] = f32_to_bf16(acc[j][8 * g + 2 * i]) |
                       (f32_to_bf16(acc[j][8 * g + 2 * i + 1]) << 16);
            __builtin_nontemporal_store(u4v{o[0], o[1], o[2], o[3]}, dst + g);
        }
    }
}

// The combine phase: wavefront tasks of up to U 64-piece chunks of one
// token's row where a row is a whole number of such chunks (H a multiple of
// 512 for bf16 rows, 1024 for FP8 rows), else one piece per thread.
template <bool kFP8>
__device__ __forceinline__ void combine_phase(const Shape &s, const FusedArgs &a)
{
    constexpr int U = kFP8 ? 4 : 8;   // 64 float32 sums per lane either way
    const int V = kFP8 ? kCombine8Vec : kCombineVec;
    const int NTH = blockDim.x, NW = NTH / 64;
    const int pieces = s.H / V;
    if (pieces % 64 == 0) {
        const int C = pieces / 64, TPR = (C + U - 1) / U;
        const long tasks = (long)s.T * TPR;
        for (long task = (long)blockIdx.x * NW + (threadIdx.x >> 6); task < tasks;
             task += (long)gridDim.x * NW) {
            const int t = __builtin_amdgcn_readfirstlane((int)(task / TPR));
            const int c0 = __builtin_amdgcn_readfirstlane((int)(task - (long)t * TPR) * U);
            combine_row_part<kFP8, U>(s, a, t, c0, min(U, C - c0));
        }
        return;
    }
    const long n = (long)s.T * pieces;
    for (long i = (long)blockIdx.x * NTH + threadIdx.x; i < n; i += (long)gridDim.x * NTH) {
        const int t = (int)(i / pieces);
        const int col = (int)(i - (long)t * pieces) * V;
        if (kFP8)
            combine8_cols(s, a.tw, a.route_row, a.y8, a.y8s, a.out, t, col);
        else
            combine_cols(s, a.tw, a.route_row, a.y, a.out, t, col);
    }
}

template <int BM, int BN1, int BN2, int KU, int NW>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
layer_persistent_kernel(Shape s, FusedArgs a, int nq, int max_polls)
{
    constexpr int NTH = NW * 64;
    constexpr int BN = BN1 > BN2 ? BN1 : BN2;
    // (within 80 KB for the 128-row tiles: two workgroups per CU)
    __shared__ TileShared<BM, BN, KU> sh;
    __shared__ int ticket_sh, ok_sh;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = gridDim.x, blk = blockIdx.x;
    const int E = s.E_local, E1 = E + 1;
    const bool fixed = s.mode == MOE_DISPATCH_FIXED_SLOT;
    int32_t *hdr = a.hdr;
    int barriers = 0;
    bool ok = true;

    // ---- 1. dispatch -------------------------------------------------------
    // LDS (the stage ring, free until the GEMMs): per-wavefront histograms
    // [NW][E], partial table sums [2 NW][E + 1], segment sizes [E] and
    // offsets [E + 1]
    int *wh = reinterpret_cast<int *>(sh.ring);
    int *part = wh + NW * E;
    int *cnt = part + 2 * NW * E1;
    int *offs = cnt + E;
    static_assert(sizeof(sh.ring) >= sizeof(int) * (NW * kMaxLocalExperts +
                                                    2 * NW * (kMaxLocalExperts + 1) +
                                                    2 * kMaxLocalExperts + 1),
                  "dispatch tables fit the stage ring");
    const long n = (long)s.T * s.K;
    const long nv = valid_slots(s, a.valid);
    // slices of at least kSliceSlots slots (the table every workgroup sums
    // then has few rows), at most one per workgroup and kMaxSlices
    const long want = (n + kSliceSlots - 1) / kSliceSlots;
    const int nsl = (int)min((long)min(G, kMaxSlices), want > 0 ? want : 1L);
    const long per = (n + nsl - 1) / nsl;
    const long sb = blk < nsl ? min(n, per * blk) : n, se = blk < nsl ? min(n, sb + per) : n;
    const long pw = (se - sb + NW - 1) / NW;
    const long wb = min(se, sb + pw * wave), we = min(se, wb + pw);
    for (int i = blk * NTH + tid; i < a.nready; i += G * NTH)
        a.ready[i] = 0;
    if (fixed) {
        int inv = 0, drop = 0;
        if (blk < nsl)
            claim_slots<kBatch, false>(s, a.ids, wb, we, nv, hdr + kHdrClaims, a.row_route,
                                       a.route_row, inv, drop);
        inv = wave_sum(inv);
        drop = wave_sum(drop);
        if (inv)
            atomicAdd(&hdr[kHdrInvalid], lane == 0 ? inv : 0);
        if (drop)
            atomicAdd(&hdr[kHdrDropped], lane == 0 ? drop : 0);
        ok = grid_barrier(hdr, ++barriers, max_polls, &ok_sh);
        if (ok && blk == 0) {
            for (int e = tid; e < E; e += NTH) {
                a.counts[e] = __hip_atomic_load(&hdr[kHdrClaims + e], __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
                a.offsets[e] = e * s.capacity;
            }
            if (tid == 0)
                a.offsets[E] = E * s.capacity;
        }
    } else {
        if (blk < nsl) {
            for (int i = tid; i < NW * E; i += NTH)
                wh[i] = 0;
            __syncthreads();
            const int inv = wave_histogram<kBatch>(s, a.ids, wb, we, nv, wh + wave * E);
            if (inv)
                atomicAdd(&hdr[kHdrInvalid], lane == 0 ? inv : 0);
            __syncthreads();
            for (int e = tid; e < E; e += NTH) {
                int c = 0;
                for (int w = 0; w < NW; ++w)
                    c += wh[w * E + e];
                a.table[(size_t)blk * E1 + e] = c;
            }
        }
        ok = grid_barrier(hdr, ++barriers, max_polls, &ok_sh);
        if (ok && (blk < nsl || blk == 0)) {
            // wavefront w sums table rows w, w + NW, ...: over all slices
            // (segment sizes) and over the slices before this one
            for (int c = lane; c < E; c += 64) {
                int before = 0, all = 0;
#pragma unroll 8
                for (int b = wave; b < nsl; b += NW) {
                    const int v = a.table[(size_t)b * E1 + c];
                    all += v;
                    before += b < blk ? v : 0;
                }
                part[wave * E1 + c] = all;
                part[(NW + wave) * E1 + c] = before;
            }
            __syncthreads();
            for (int e = tid; e < E; e += NTH) {
                int all = 0;
                for (int w = 0; w < NW; ++w)
                    all += part[w * E1 + e];
                cnt[e] = all;
            }
            __syncthreads();
            scan_experts<NTH>(E, [&](int e) { return cnt[e]; }, offs);
            if (blk == 0) {
                for (int e = tid; e < E; e += NTH) {
                    a.counts[e] = cnt[e];
                    a.offsets[e] = offs[e];
                }
                if (tid == 0)
                    a.offsets[E] = offs[E];
            }
            if (blk < nsl) {
                // this slice's first row in each segment, then per wavefront
                for (int e = tid; e < E; e += NTH) {
                    int run = offs[e];
                    for (int w = 0; w < NW; ++w)
                        run += part[(NW + w) * E1 + e];
                    for (int w = 0; w < NW; ++w) {
                        const int c = wh[w * E + e];
                        wh[w * E + e] = run;
                        run += c;
                    }
                }
                __syncthreads();
                for (long base = wb; base < we; base += 64 * kBatch) {
                    int ex[kBatch];
                    load_keys<kBatch>(s, a.ids, base, we, nv, ex);
                    scatter_keys<kBatch>(ex, base, we, wh + wave * E, a.row_route, a.route_row);
                }
            }
        }
    }
    // counts, offsets, row_route and route_row published to every workgroup
    if (ok)
        ok = grid_barrier(hdr, ++barriers, max_polls, &ok_sh);

    // ---- 2. GEMM1 and GEMM2 from the XCD's queue -------------------------------
    if (ok) {
        const int NT1 = s.I / (BN1 / 2), NT2 = s.H / BN2;
        const int nchunks =
            __builtin_amdgcn_readfirstlane(plan_chunks<NTH>(s, a.counts, BM, sh.prefix));
        unsigned xcc;
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
        const int x = (int)(xcc & 7u) % nq;
        const int mine = nchunks > x ? (nchunks - x + nq - 1) / nq : 0;
        const int n1 = mine * NT1, n2 = mine * NT2;
        // blocks of bq chunks x bnt N tiles per round of the XCD's workgroups
        const int per_xcd = G / nq > 0 ? G / nq : 1;
        const int bnt1 = min(NT1, 8), bnt2 = min(NT2, 8);
        const int bq1 = max(1, per_xcd / bnt1), bq2 = max(1, per_xcd / bnt2);
        const TiledArgs g1{a.x, a.xs, a.counts, a.offsets, a.row_route, a.w13, a.w13s, a.h, a.hs,
                           nullptr, nullptr, nullptr};
        const TiledArgs g2{a.h, a.hs, a.counts, a.offsets, nullptr, a.w2, a.w2s, nullptr, nullptr,
                           a.y, a.y8, a.y8s};
        int32_t *ticket = hdr + kHdrTicket + 32 * x;
        if (wave == 0) {
            const int t0 = atomicAdd(ticket, lane == 0 ? 1 : 0);
            ticket_sh = __builtin_amdgcn_readfirstlane(t0);
        }
        __syncthreads();
        for (;;) {
            const int t = __builtin_amdgcn_readfirstlane(ticket_sh);
            __syncthreads();
            if (t >= n1 + n2)
                break;
            int next = 0;
            if (wave == 0)
                next = atomicAdd(ticket, lane == 0 ? 1 : 0);
            int qi, nt;
            if (t < n1) {
                queue_item(t, mine, NT1, bq1, bnt1, qi, nt);
                const int q = x + nq * qi;
                tiled_item<true, BM, BN1, KU, false, NW>(s, g1, sh.prefix, sh.arow, sh.ring, q,
                                                         nt);
                wait_vmcnt<0>();   // this thread's h stores are in the L2
                __syncthreads();   // ... and every thread's
                if (wave == 0)
                    atomicAdd(&a.ready[q], lane == 0 ? 1 : 0);
            } else {
                queue_item(t - n1, mine, NT2, bq2, bnt2, qi, nt);
                const int q = x + nq * qi;
                if (wave == 0) {
                    const bool done = poll_at_least(&a.ready[q], NT1, max_polls);
                    if (!done)
                        atomicAdd(&hdr[kHdrTimeouts], lane == 0 ? 1 : 0);
                    if (lane == 0)
                        ok_sh = done;
                }
                __syncthreads();
                // a wait that gave up: this workgroup takes no more tickets
                // (the layer is reported failed), so a lost GEMM1 item costs
                // one bounded wait per workgroup, not one per GEMM2 item
                if (!__builtin_amdgcn_readfirstlane(ok_sh)) {
                    ok = false;
                    break;
                }
                tiled_item<false, BM, BN2, KU, true, NW>(s, g2, sh.prefix, sh.arow, sh.ring, q,
                                                         nt);
            }
            if (wave == 0)
                ticket_sh = __builtin_amdgcn_readfirstlane(next);
            __syncthreads();
        }
        // every workgroup that reached the GEMMs meets here (also one whose
        // wait gave up, so the others are not held up by it)
        const bool met = grid_barrier(hdr, ++barriers, max_polls, &ok_sh);
        ok = ok && met;
    }

    // ---- 3. combine ---------------------------------------------------------------
    if (ok) {
        if (a.y8)
            combine_phase<true>(s, a);
        else
            combine_phase<false>(s, a);
    }

    // ---- the end: the last workgroup reports and clears the header -------------
    __syncthreads();
    if (wave == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const int old = __builtin_amdgcn_readfirstlane(atomicAdd(&hdr[kHdrDepart], lane == 0 ? 1 : 0));
        if (old == G - 1) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            if (lane == 0) {
                a.status[0] = __hip_atomic_load(&hdr[kHdrInvalid], __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
                a.status[1] = __hip_atomic_load(&hdr[kHdrDropped], __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
                a.status[2] = __hip_atomic_load(&hdr[kHdrTimeouts], __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
                a.status[3] = 0;
            }
            for (int i = lane; i < kPersistentHeaderWords; i += 64)
                __hip_atomic_store(&hdr[i], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
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

// The tile config of the persistent layer: that of the launches.  The
// 256-row tile (eight wavefronts, one workgroup per CU) runs when both GEMMs
// take it; a 256-row tile next to another row tile runs as 128 rows.
static TiledConfig persistent_config(const moe_shape &sh, bool gemm1)
{
    const TiledConfig a = tiled_config(sh, true), b = tiled_config(sh, false);
    TiledConfig c = gemm1 ? a : b;
    if (c.bm == 256 && !(a.bm == 256 && b.bm == 256))
        c = TiledConfig{128, 256, 1};
    return c;
}

// The persistent layer takes the tiled GEMMs when both use the same row
// tile: 256 rows (256 weight rows, one K step), 128 rows with one K step per
// stage (any weight tile widths), or 32 or 64 rows with two K steps and 128
// weight rows; on a device whose XCDs it can tell apart.
bool persistent_supported(const moe_shape &sh)
{
    if (sh.H < 512 || sh.I < 512 || xcd_count() == 0 || sh.E_local > kMaxLocalExperts)
        return false;
    const TiledConfig a = persistent_config(sh, true), b = persistent_config(sh, false);
    if (a.bm == 256 && b.bm == 256)
        return a.bn == 256 && b.bn == 256 && a.ku == 1 && b.ku == 1;
    if (a.bm == 128 && b.bm == 128 && a.ku == 1 && b.ku == 1)
        return true;
    return (a.bm == 32 || a.bm == 64) && b.bm == a.bm && a.ku == 2 && b.ku == 2 && a.bn == 128 &&
           b.bn == 128;
}

int persistent_ready_words(const moe_shape &sh) { return (int)tile_upper_bound(sh, 32); }

size_t persistent_table_bytes(const moe_shape &sh)
{
    return sizeof(int32_t) * (size_t)kMaxSlices * (size_t)(sh.E_local + 1);
}

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

hipError_t launch_layer_persistent(const moe_shape &sh, const int32_t *ids, const int32_t *valid,
                                   const float *tw, const uint8_t *x, const uint8_t *xs,
                                   const uint8_t *w13, const uint8_t *w13s, const uint8_t *w2,
                                   const uint8_t *w2s, const PersistentBufs &b, const YRows &y,
                                   uint16_t *out, hipStream_t st)
{
    const FusedArgs a{ids,       valid,      tw,      x,         xs,       w13,
                      w13s,      w2,         w2s,     b.counts,  b.offsets, b.row_route,
                      b.route_row, b.status, b.hdr,   b.table,   b.ready,  persistent_ready_words(sh),
                      b.h,       b.hs,       y.bf16,  y.codes,   y.scales, out};
    const TiledConfig c1 = persistent_config(sh, true), c2 = persistent_config(sh, false);
    const int nq = xcd_count();
    // every workgroup resident at once (the grid barriers wait for all of
    // them): the device's CUs times the kernel's occupancy
    auto go = [&](auto k, int nw) {
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, nw * 64, 0) != hipSuccess ||
            per_cu < 1)
            per_cu = 1;
        const int grid = device_cu_count() * per_cu;
        k<<<grid, nw * 64, 0, st>>>(to_dev(sh), a, nq, persistent_max_polls());
    };
    if (c1.bm == 256)
        go(layer_persistent_kernel<256, 256, 256, 1, 8>, 8);
    else if (c1.bm == 32)
        go(layer_persistent_kernel<32, 128, 128, 2, 4>, 4);
    else if (c1.bm == 64)
        go(layer_persistent_kernel<64, 128, 128, 2, 4>, 4);
    else if (c1.bn == 256 && c2.bn == 256)
        go(layer_persistent_kernel<128, 256, 256, 1, 4>, 4);
    else if (c1.bn == 256)
        go(layer_persistent_kernel<128, 256, 128, 1, 4>, 4);
    else if (c2.bn == 256)
        go(layer_persistent_kernel<128, 128, 256, 1, 4>, 4);
    else
        go(layer_persistent_kernel<128, 128, 128, 1, 4>, 4);
    return hipGetLastError();
}

namespace {
__global__ void __launch_bounds__(256) zero_words_kernel(int32_t *p, int n)
{
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256)
        p[i] = 0;
}
} // namespace

hipError_t launch_zero_words(int32_t *p, int words, hipStream_t st)
{
    zero_words_kernel<<<(words + 255) / 256, 256, 0, st>>>(p, words);
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
