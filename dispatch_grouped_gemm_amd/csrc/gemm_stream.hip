// Packed-weight expert GEMMs, for the row tiles whose GEMMs are bound by the
// weight stream (the 32- and 64-row tile classes: decode and the mid
// sizes).  ("full-expert DeepSeek V4.1 Flash MegaMoE tuning",
// Changes and tuning: weight pipelining and the B cache policy are among the
// searched knobs; the packed order is an internal layout, written once by
// moe_pack_weights.)
//
// Packed layout of a weight matrix W [E, N, K/2] (FP4 codes) with exponents
// Ws [E, N, K/32], N rows in groups of 16, K in steps of 128:
//   codes  P[e][ks][g][lane][16 bytes] = W[e][16 g + (lane & 15)]
//                                          [64 ks + 16 (lane >> 4) .. + 16]
//   scales S[e][ks4][g][lane][j]       = Ws[e][16 g + (lane & 15)]
//                                          [4 (4 ks4 + j) + (lane >> 4)]
//          (j < 4; K steps past the last are zero bytes)
// so one K step of a 16-row group is 1 KiB in the scaled MFMA's FP4 lane
// order (lane l: row l mod 16, 32 K values 32 (l div 16) ..) and one dword
// per lane holds its exponents of four K steps.  K-step major: the
// wavefronts of a launch, which advance through K at about the same pace,
// read one contiguous span of the weights at a time.
//
// A workgroup of four or eight wavefronts takes an item (row chunk, one
// slice of the weight rows per wavefront); a wavefront's slice is GEMM1 32
// intermediate columns (their gate and up groups, 64 W13 rows, so the
// requant's 32-column block stays in the wavefront) or GEMM2 64 output
// columns.  Each wavefront
// streams its four weight groups into registers four K steps ahead with
// 1 KiB buffer loads (no LDS for weights).  The activation fragments (the
// gathered x rows, or h rows) go through a two-stage LDS ring by LDS DMA,
// two K steps per stage, each K step fetched once per workgroup, one
// barrier per stage; their exponents go through LDS too, four K steps at a
// time.  Read by every wavefront into its own registers instead, the
// activations quadruple the L1 traffic and the L1, not HBM, becomes the
// bound.  Every output element is the same sequence of scaled MFMAs over
// ascending K steps as in the LDS-tiled kernels, and the epilogues are
// theirs, so the bits are the same.
#include <type_traits>

#include "moe_common.hpp"

namespace moe {

namespace {

constexpr int kStreamBigRows = 96;
// wavefronts per workgroup of the 96-row kernels (one workgroup per CU at
// two wavefronts per SIMD with eight): GEMM2 shares each activation stage
// among eight (half the activation fetches per weight byte: Flash 135 ->
// 133 us, V4 at 2,048 tokens 110 -> 106 us); GEMM1 keeps two workgroups of
// four per CU, whose items (two to three per workgroup) then overlap one
// another's start (eight: V4 at 2,048 tokens 183 -> 203 us)
template <bool kGemm1>
constexpr int kStreamBigWaves = kGemm1 ? 4 : 8;

typedef unsigned int u32x4s __attribute__((ext_vector_type(4)));

struct StreamArgs {
    const uint8_t *act, *act_s;          // x (GEMM1, gathered) or h (GEMM2) rows
    const int32_t *counts, *offsets, *row_route;
    const uint8_t *wp, *wps;             // packed W13 or W2 codes and exponents
    uint8_t *h_out, *hs_out;             // GEMM1 output
    uint16_t *y_out;                     // GEMM2 output, bf16 rows, or
    uint8_t *y8_out, *y8s_out;           // MX FP8 rows
};

// Buffer loads: a wavefront-uniform resource (base and byte range, in
// SGPRs), a 32-bit lane offset and a uniform offset (an SGPR), so a lane
// keeps one VGPR per address stream.  Bytes past the range read as zero.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRawBufferFlags = 0x00020000;   // raw bytes, 32-bit data format
constexpr int kNonTemporal = 2;               // cache policy bit nt

__device__ __forceinline__ Rsrc make_rsrc(const uint8_t *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(uniform_ptr(base)), (short)0,
                                             (int)bytes, kRawBufferFlags);
}

template <int kAux = 0>
__device__ __forceinline__ u32x4s load16(Rsrc r, uint32_t voff, int soff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, soff, kAux);
}

__device__ __forceinline__ uint32_t load4(Rsrc r, uint32_t voff, int soff)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, soff, 0);
}

// Scaled MFMA with the weight exponent taken from byte SEL of a dword that
// holds four K steps' exponents (the instruction's scale byte select).
template <int SEL>
__device__ __forceinline__ v4f mfma_w4a8_sel(const v8i &a_fp4, const v8i &b_fp8, v4f c,
                                             uint32_t sa4, int sb)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a_fp4, b_fp8, c, 4, 0, SEL, (int)sa4,
                                                            0, sb);
}

__device__ __forceinline__ u32x4s lds_read16(const uint8_t *p)
{
    return *reinterpret_cast<const u32x4s *>(p);
}

// LDS bytes of one activation stage: two K steps of NL 16-row blocks, each
// block step 2 KiB (16 rows of 128 bytes, their 16-byte columns swizzled).
template <int NL>
constexpr int kStageBytes = 2 * NL * 2 * 1024;

// One work item of a workgroup: NL (1 .. TB) live 16-row blocks of the chunk
// at rows row0 .. row0 + nrows - 1 of expert e; wavefront w takes slice
// kW sg + w (four weight groups).  Each K step's activation fragments are
// fetched once per workgroup and shared through the LDS ring; every
// wavefront streams its own weights into registers.
template <bool kGemm1, int TB, int NL, int kW>
__device__ __forceinline__ void stream_item(const Shape &s, const StreamArgs &g, int e, int row0,
                                            int nrows, int sg, uint8_t *lds)
{
    const int lane = threadIdx.x & 63, i16 = lane & 15, kq = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int H = s.H, I = s.I;
    const int KT = kGemm1 ? H : I;
    const int KS = KT / 128, KS4 = (KS + 3) / 4;
    const int N = kGemm1 ? 2 * I : H;
    const int G = N / 16;
    const int S = kGemm1 ? I / 32 : H / 64;
    const int slice = kW * sg + wave;
    const bool live = slice < S;
    const Rsrc null_r = make_rsrc(g.wp, 0);
    // the wavefront's four 16-row weight groups: GEMM1 the gate groups of
    // intermediate columns 32 slice .. + 31, then their up groups; GEMM2
    // output columns 64 slice .. + 63.  Offsets within expert e's packed
    // codes (K-step major: 1 KiB per group and K step, a K step's groups
    // adjacent) and exponents (256 bytes per group and four K steps).  A
    // slice past the last (the workgroup's last wavefronts where S is not a
    // multiple of kW) reads zeros and stores nothing.
    const Rsrc wr_r =
        live ? make_rsrc(g.wp + (size_t)e * G * KS * 1024, (uint32_t)(G * KS * 1024)) : null_r;
    const Rsrc ws_r =
        live ? make_rsrc(g.wps + (size_t)e * G * KS4 * 256, (uint32_t)(G * KS4 * 256)) : null_r;
    int wgo[4], sgo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int grp = kGemm1 ? (i < 2 ? 2 * slice + i : (I / 16) + 2 * slice + (i - 2))
                               : 4 * slice + i;
        wgo[i] = grp * 1024;
        sgo[i] = grp * 256;
    }
    const uint32_t wl = 16 * lane, sl = 4 * lane;
    // activation rows (rows past nrows repeat the last): GEMM1 gathered x
    // rows (T H < 2^32), GEMM2 the chunk's h rows
    auto arow_of = [&](int r) -> uint32_t {
        r = min(r, nrows - 1);
        return kGemm1 ? (uint32_t)(g.row_route[row0 + r] / s.K) : (uint32_t)r;
    };
    // A K step of a 16-row block sits in LDS as 16 rows of 128 bytes, row r's
    // 16-byte column c at slot c ^ swz(r), swz(r) = (r >> 1) & 7 (the eight
    // lanes of a fragment read that share a column hit distinct banks).  This
    // wavefront fetches row octet (wave >> 1) & 1 of its blocks (every block
    // with four wavefronts; with eight, the blocks j = wave >> 2 mod 2): lane
    // l the column stored at slot l & 7 of row 8 ((wave >> 1) & 1) + (l >> 3),
    // so an instruction reads eight whole 128-byte lines.
    constexpr int kBP = kW / 4;                   // block phases
    constexpr int kOwn = (NL + kBP - 1) / kBP;    // blocks per wavefront, at most
    const int bp = wave >> 2;
    const int rl = 8 * ((wave >> 1) & 1) + (lane >> 3);
    const uint32_t col = 16 * ((lane & 7) ^ ((rl >> 1) & 7));
    uint32_t ao[kOwn];
#pragma unroll
    for (int m = 0; m < kOwn; ++m)
        ao[m] = arow_of(16 * min(kBP * m + bp, NL - 1) + rl) * (uint32_t)KT + col;
    // the MFMA lane (i16, kq) reads columns kq and kq + 4 of row i16
    const uint32_t frag_lo = 128 * i16 + 16 * (kq ^ ((i16 >> 1) & 7));
    const uint32_t frag_hi = frag_lo ^ 64;
    // activation exponents, shared through LDS like the fragments: four K
    // steps at a time, per block 64 dwords, lane (i16, kq)'s dword the four
    // block exponents of K step 4 q + kq of its row; a step reads byte kq of
    // lane i16 + 16 (ks mod 4)'s dword.  This wavefront loads blocks
    // wave + kW n (n < kAxLoads, clamped to the last block: a repeated block
    // is the same bytes written twice).
    constexpr int kAxLoads = (NL + kW - 1) / kW;
    uint32_t axrow[kAxLoads];
    int axblk[kAxLoads];
#pragma unroll
    for (int n = 0; n < kAxLoads; ++n) {
        axblk[n] = min(wave + kW * n, NL - 1);
        axrow[n] = arow_of(16 * axblk[n] + i16) * (uint32_t)(KT / 32);   // the row's first exponent byte
    }

    v4f acc[4][NL];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NL; ++j)
            acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // weight fragments of K steps ks .. ks + 3 (slot ks mod 4) and their
    // exponents, four K steps to a dword, double-buffered
    u32x4s wr[4][4];
    uint32_t we[2][4];
    // this wavefront's share of stage p (K steps 2 p, 2 p + 1): step
    // 2 p + (wave & 1), row octet (wave >> 1) & 1, of its blocks, straight
    // into the ring (LDS DMA: lane l's 16 bytes land at 16 l of a 1 KiB
    // block).  A step past the last reloads the last (never read).  These
    // loads are inline assembly, out of the compiler's wait accounting: the
    // waits for them are the explicit ones below, and the compiler's own
    // waits for its loads, which do not count them, only wait longer than
    // needed.
    const uint8_t *act = kGemm1 ? g.act : g.act + (size_t)row0 * KT;
    const uint32_t ring = lds_addr(lds) + (wave & 1) * (NL * 2048) + ((wave >> 1) & 1) * 1024 +
                          bp * 2048;
    auto stage_load = [&](int p) {
        const uint8_t *base = act + (size_t)min(2 * p + (wave & 1), KS - 1) * 128;
        const uint32_t m0 = ring + (p & 1) * kStageBytes<NL>;
#pragma unroll
        for (int m = 0; m < kOwn; ++m)
            if (kBP * m + bp < NL)
                g2lds<16>(base, ao[m], m0 + m * (kBP * 2048));
    };
    // exponents of K steps 4 q .. 4 q + 3 into buffer q mod 2 (a step past
    // the last reloads the last)
    const uint8_t *act_s = kGemm1 ? g.act_s : g.act_s + (size_t)row0 * (KT / 32);
    const uint8_t *ax_lds = lds + 2 * kStageBytes<TB>;
    auto ax_load = [&](int q) {
        const uint32_t voff = 4 * min(4 * q + kq, KS - 1);
        const uint32_t m0 = lds_addr(const_cast<uint8_t *>(ax_lds)) + (q & 1) * (NL * 256);
#pragma unroll
        for (int n = 0; n < kAxLoads; ++n)
            g2lds<4>(act_s, axrow[n] + voff, m0 + axblk[n] * 256);
    };
    const int np = (KS + 1) / 2, nq = (KS + 3) / 4;
    // every wavefront is done with the previous item's ring: its reads are
    // consumed, and its loads into the ring (the last group's exponent loads
    // among them, which no wait of that item covers) are done before the
    // barrier, so none lands in this item's ring
    asm volatile("" ::: "memory");
    wait_vmcnt<0>();
    raw_barrier();
    stage_load(0);
    ax_load(0);
    // the first four K steps of weights, after the ring loads so that the
    // first stage waits for those alone (kPrologue operations follow them)
    constexpr int kPrologue = 16 + 4;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            wr[d][i] = load16<kNonTemporal>(d < KS ? wr_r : null_r, wl, wgo[i] + d * G * 1024);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        we[0][i] = load4(ws_r, sl, sgo[i]);

    // Stage p is in the ring once this wavefront's loads of it are done
    // (issued at the start of stage p - 1, or in the prologue) and, after
    // the barrier, every wavefront's; every wavefront is then also done
    // reading stage p - 1, whose buffer takes p + 1.  kAfter: the vector
    // memory operations issued after the stage loads by then -- the
    // exponents of the next four K steps (kAxLoads activation DMA dwords, 4
    // weight dwords) where stage p - 1 began a group of four K steps, and
    // two K steps of weight fragments (8).  The empty asm keeps every memory
    // operation on its side of the count.  The activation exponents of a
    // group, loaded at the start of the group before, are done by the wait
    // of the group's first stage (loaded before that stage's fragments).
    auto stage_begin = [&](int p, auto after) {
        asm volatile("" ::: "memory");
        if (p == 0)
            wait_vmcnt<kPrologue>();
        else
            wait_vmcnt<decltype(after)::value>();
        raw_barrier();
        if (p + 1 < np)
            stage_load(p + 1);
    };

    // K step ks = 4 q + D: its weight exponents are byte D of we[0].
    // Prefetches past the last K step go to a null resource (no memory
    // access, zeros), so every step issues the same loads and the buffers
    // rotate without copies; steps past the last skip the MFMAs.
    auto step = [&](int q, auto dc) {
        constexpr int D = decltype(dc)::value;
        const int ks = 4 * q + D;
        if (ks < KS) {
            const uint8_t *b =
                lds + ((2 * q + D / 2) & 1) * kStageBytes<NL> + (D & 1) * (NL * 2048);
#pragma unroll
            for (int j = 0; j < NL; ++j) {
                const u32x4s lo = lds_read16(b + j * 2048 + frag_lo),
                             hi = lds_read16(b + j * 2048 + frag_hi);
                const v8i bj = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                const int sb = ax_lds[(q & 1) * (NL * 256) + j * 256 + 4 * (i16 + 16 * D) + kq];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const v8i a = v8i{(int)wr[D][i][0], (int)wr[D][i][1], (int)wr[D][i][2],
                                      (int)wr[D][i][3], 0, 0, 0, 0};
                    acc[i][j] = mfma_w4a8_sel<D>(a, bj, acc[i][j], we[0][i], sb);
                }
            }
        }
        // the scheduler would hoist the next loads into this slot above the
        // MFMAs that read it (two live copies, then register moves that wait
        // on the loads) or sink them to the end of the unrolled body (the
        // next step waits on them at once): keep every step's loads in place
        __builtin_amdgcn_sched_barrier(0);
        // this slot's next weight fragments: K step ks + 4
        {
            const Rsrc r = ks + 4 < KS ? wr_r : null_r;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                wr[D][i] = load16<kNonTemporal>(r, wl, wgo[i] + (ks + 4) * G * 1024);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    for (int q = 0; q < nq; ++q) {
        stage_begin(2 * q, std::integral_constant<int, 8>{});
        // the next four K steps' activation and weight exponents (past the
        // last group too: the wait counts assume these loads in every group)
        ax_load(q + 1);
        {
            const Rsrc r = 4 * q + 4 < KS ? ws_r : null_r;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                we[1][i] = load4(r, sl, sgo[i] + (q + 1) * G * 256);
        }
        step(q, std::integral_constant<int, 0>{});
        step(q, std::integral_constant<int, 1>{});
        stage_begin(2 * q + 1, std::integral_constant<int, kAxLoads + 4 + 8>{});
        step(q, std::integral_constant<int, 2>{});
        step(q, std::integral_constant<int, 3>{});
#pragma unroll
        for (int i = 0; i < 4; ++i)
            we[0][i] = we[1][i];
    }
    if (!live)
        return;

    // epilogue: lane holds rows 16 j + i16, columns 4 kq .. 4 kq + 3 of each
    // of its four groups
    if (kGemm1) {
        const int c0 = 32 * slice;
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            float hv[2][4];
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    hv[cb][v] = swiglu_clamped(acc[cb][j][v], acc[cb + 2][j][v], s.gate_limit,
                                               s.up_limit);
            float amax = 0.0f;
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    amax = fmaxf(amax, fabsf(hv[cb][v]));
            amax = fmaxf(amax, __shfl_xor(amax, 16));
            amax = fmaxf(amax, __shfl_xor(amax, 32));
            const int E = mx8_block_exponent(amax);
            const int m = 16 * j + i16;
            if (m < nrows) {
                uint8_t *hr = g.h_out + (size_t)(row0 + m) * I + c0 + 4 * kq;
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
                    *reinterpret_cast<uint32_t *>(hr + 16 * cb) =
                        mx8_pack4(hv[cb][0], hv[cb][1], hv[cb][2], hv[cb][3], E, amax);
                if (kq == 0)
                    g.hs_out[(size_t)(row0 + m) * (I / 32) + c0 / 32] = (uint8_t)(E + 127);
            }
        }
    } else if (g.y8_out) {
        const int n0 = 64 * slice;
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int m = 16 * j + i16;
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                float amax = 0.0f;
#pragma unroll
                for (int i = 2 * blk; i < 2 * blk + 2; ++i)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        amax = fmaxf(amax, fabsf(acc[i][j][v]));
                amax = fmaxf(amax, __shfl_xor(amax, 16));
                amax = fmaxf(amax, __shfl_xor(amax, 32));
                const int E = mx8_block_exponent(amax);
                if (m < nrows) {
                    uint8_t *yr = g.y8_out + (size_t)(row0 + m) * H + n0 + 32 * blk + 4 * kq;
#pragma unroll
                    for (int i = 2 * blk; i < 2 * blk + 2; ++i)
                        *reinterpret_cast<uint32_t *>(yr + 16 * (i - 2 * blk)) =
                            mx8_pack4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3],
                                      E, amax);
                    if (kq == 0)
                        g.y8s_out[(size_t)(row0 + m) * (H / 32) + (n0 + 32 * blk) / 32] =
                            (uint8_t)(E + 127);
                }
            }
        }
    } else {
        const int n0 = 64 * slice;
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int m = 16 * j + i16;
            if (m >= nrows)
                continue;
            uint16_t *yr = g.y_out + (size_t)(row0 + m) * H + n0 + 4 * kq;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<uint2 *>(yr + 16 * i) =
                    uint2{f32_to_bf16(acc[i][j][0]) | (f32_to_bf16(acc[i][j][1]) << 16),
                          f32_to_bf16(acc[i][j][2]) | (f32_to_bf16(acc[i][j][3]) << 16)};
        }
    }
}

// The item code for NL live blocks, NL = nl (1 .. TB), each count its own
// straight-line instance.
template <bool kGemm1, int TB, int kW, int NL = 1>
__device__ __forceinline__ void dispatch_nl(int nl, const Shape &s, const StreamArgs &g, int e,
                                            int row0, int nrows, int sg, uint8_t *lds)
{
    if (nl == NL)
        stream_item<kGemm1, TB, NL, kW>(s, g, e, row0, nrows, sg, lds);
    else if constexpr (NL < TB)
        dispatch_nl<kGemm1, TB, kW, NL + 1>(nl, s, g, e, row0, nrows, sg, lds);
}

// Workgroup items: (row chunk q of BM rows, group of kW slices)
// chunk-major.  Workgroup b runs on XCD b mod X (X XCDs, the grid a
// multiple of X); XCD x takes the contiguous block x of the item list, so
// the items of a chunk, which read the same activation rows, mostly share
// one XCD's L2.
template <bool kGemm1, int BM, int kW>
__global__ void __launch_bounds__(64 * kW) __attribute__((amdgpu_waves_per_eu(2)))
gemm_stream_kernel(Shape s, StreamArgs g, int X)
{
    constexpr int TB = BM / 16;
    __shared__ int prefix[kMaxLocalExperts + 1];
    // the fragment ring, then the activation exponents (two buffers)
    __shared__ __attribute__((aligned(16))) uint8_t ring[2 * kStageBytes<TB> + 2 * TB * 256];
    const int nchunks = plan_chunks<64 * kW>(s, g.counts, BM, prefix);
    const int S = kGemm1 ? s.I / 32 : s.H / 64;
    const int SG = (S + kW - 1) / kW;
    const long items = (long)nchunks * SG;
    const long per = (items + X - 1) / X;
    const int xcd = blockIdx.x % X, nb = gridDim.x / X;
    for (long t = blockIdx.x / X; t < per; t += nb) {
        const long item = xcd * per + t;
        if (item >= items)
            break;
        const int q = __builtin_amdgcn_readfirstlane((int)(item / SG));
        const int sg = __builtin_amdgcn_readfirstlane((int)(item - (long)q * SG));
        const int e = __builtin_amdgcn_readfirstlane(chunk_expert(prefix, s.E_local, q));
        const int c = q - prefix[e];
        const int row0 = __builtin_amdgcn_readfirstlane(g.offsets[e] + c * BM);
        const int nrows =
            __builtin_amdgcn_readfirstlane(min(BM, used_rows(s, g.counts[e]) - c * BM));
        const int nl = min((nrows + 15) >> 4, TB);
        dispatch_nl<kGemm1, TB, kW>(nl, s, g, e, row0, nrows, sg, ring);
    }
}

// Packing, one thread per (expert, group, K step, lane): 16 code bytes; and
// per (expert, group, four K steps, lane): 4 exponent bytes.
__global__ void __launch_bounds__(256)
pack_codes_kernel(const uint8_t *__restrict__ w, uint8_t *__restrict__ p, int E, int N, int K)
{
    const int KS = K / 128, G = N / 16;
    const long n = (long)E * KS * G * 64;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
        const int lane = (int)(i & 63);
        const long blk = i >> 6;   // (e * KS + ks) * G + g
        const int gi = (int)(blk % G);
        const long eks = blk / G;
        const int ks = (int)(eks % KS);
        const long e = eks / KS;
        const long row = e * N + 16 * gi + (lane & 15);
        *reinterpret_cast<uint4 *>(p + i * 16) = *reinterpret_cast<const uint4 *>(
            w + row * (K / 2) + 64 * ks + 16 * (lane >> 4));
    }
}

__global__ void __launch_bounds__(256)
pack_scales_kernel(const uint8_t *__restrict__ ws, uint8_t *__restrict__ ps, int E, int N, int K)
{
    const int KS = K / 128, KS4 = (KS + 3) / 4, G = N / 16;
    const long n = (long)E * KS4 * G * 64;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
        const int lane = (int)(i & 63);
        const long blk = i >> 6;   // (e * KS4 + ks4) * G + g
        const int gi = (int)(blk % G);
        const long eks = blk / G;
        const int ks4 = (int)(eks % KS4);
        const long e = eks / KS4;
        const long row = e * N + 16 * gi + (lane & 15);
        uint32_t v = 0;
        for (int j = 0; j < 4; ++j) {
            const int ks = 4 * ks4 + j;
            if (ks < KS)
                v |= (uint32_t)ws[row * (K / 32) + 4 * ks + (lane >> 4)] << (8 * j);
        }
        *reinterpret_cast<uint32_t *>(ps + i * 4) = v;
    }
}

// The inverse of the two packing passes (moe_unpack_weights).
__global__ void __launch_bounds__(256)
unpack_codes_kernel(const uint8_t *__restrict__ p, uint8_t *__restrict__ w, int E, int N, int K)
{
    const int KS = K / 128, G = N / 16;
    const long n = (long)E * KS * G * 64;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
        const int lane = (int)(i & 63);
        const long blk = i >> 6;   // (e * KS + ks) * G + g
        const int gi = (int)(blk % G);
        const long eks = blk / G;
        const int ks = (int)(eks % KS);
        const long e = eks / KS;
        const long row = e * N + 16 * gi + (lane & 15);
        *reinterpret_cast<uint4 *>(w + row * (K / 2) + 64 * ks + 16 * (lane >> 4)) =
            *reinterpret_cast<const uint4 *>(p + i * 16);
    }
}

__global__ void __launch_bounds__(256)
unpack_scales_kernel(const uint8_t *__restrict__ ps, uint8_t *__restrict__ ws, int E, int N,
                     int K)
{
    const int KS = K / 128, KS4 = (KS + 3) / 4, G = N / 16;
    const long n = (long)E * KS4 * G * 64;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
        const int lane = (int)(i & 63);
        const long blk = i >> 6;   // (e * KS4 + ks4) * G + g
        const int gi = (int)(blk % G);
        const long eks = blk / G;
        const int ks4 = (int)(eks % KS4);
        const long e = eks / KS4;
        const long row = e * N + 16 * gi + (lane & 15);
        const uint32_t v = *reinterpret_cast<const uint32_t *>(ps + i * 4);
        for (int j = 0; j < 4; ++j) {
            const int ks = 4 * ks4 + j;
            if (ks < KS)
                ws[row * (K / 32) + 4 * ks + (lane >> 4)] = (uint8_t)(v >> (8 * j));
        }
    }
}

int stream_grid(const void *kernel, int threads)
{
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) !=
            hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    return device_cu_count() * per_cu;
}

// XCDs the grid spreads over round-robin: the MI355X has 32 CUs per XCD
// (1 where the CU count says otherwise, or the grid is not a multiple).
int stream_xcds(int grid)
{
    const int cus = device_cu_count();
    const int x = cus % 32 == 0 ? cus / 32 : 1;
    return x > 0 && grid % x == 0 ? x : 1;
}

template <bool kGemm1>
hipError_t launch_stream(const moe_shape &sh, const StreamArgs &g, int bm, hipStream_t st)
{
    if (bm == 32) {
        auto k = gemm_stream_kernel<kGemm1, 32, 4>;
        const int grid = stream_grid(reinterpret_cast<const void *>(k), 256);
        k<<<grid, 256, 0, st>>>(to_dev(sh), g, stream_xcds(grid));
    } else {
        constexpr int kW = kStreamBigWaves<kGemm1>;
        auto k = gemm_stream_kernel<kGemm1, kStreamBigRows, kW>;
        const int grid = stream_grid(reinterpret_cast<const void *>(k), 64 * kW);
        k<<<grid, 64 * kW, 0, st>>>(to_dev(sh), g, stream_xcds(grid));
    }
    return hipGetLastError();
}

// Chunk rows of the packed kernels: 32 where the tile rule takes 32-row
// tiles, else kStreamBigRows.  A chunk costs MFMAs for its live 16-row
// blocks only, so the taller chunk loses nothing where experts hold fewer
// rows, and where they hold more than 64 (Flash: 64 expected) it keeps an
// expert in one chunk, its weights read once.
int stream_bm(const moe_shape &s, bool gemm1)
{
    int bm = 0, bn = 0, ku = 0;
    tile_config_of(s, gemm1, &bm, &bn, &ku);
    return bm == 32 ? 32 : kStreamBigRows;
}

} // namespace

size_t packed_codes_bytes(int E, int N, int K) { return (size_t)E * N * (size_t)(K / 2); }

size_t packed_scales_bytes(int E, int N, int K)
{
    const int KS4 = (K / 128 + 3) / 4;
    return (size_t)E * (size_t)(N / 16) * KS4 * 256;
}

hipError_t launch_pack(const uint8_t *w, const uint8_t *ws, uint8_t *p, uint8_t *ps, int E,
                       int N, int K, hipStream_t st)
{
    const long nc = (long)E * (N / 16) * (K / 128) * 64;
    const long nsc = (long)E * (N / 16) * ((K / 128 + 3) / 4) * 64;
    auto grid = [](long n) { return (unsigned)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536); };
    pack_codes_kernel<<<grid(nc), 256, 0, st>>>(w, p, E, N, K);
    pack_scales_kernel<<<grid(nsc), 256, 0, st>>>(ws, ps, E, N, K);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t *p, const uint8_t *ps, uint8_t *w, uint8_t *ws, int E,
                         int N, int K, hipStream_t st)
{
    const long nc = (long)E * (N / 16) * (K / 128) * 64;
    const long nsc = (long)E * (N / 16) * ((K / 128 + 3) / 4) * 64;
    auto grid = [](long n) { return (unsigned)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536); };
    unpack_codes_kernel<<<grid(nc), 256, 0, st>>>(p, w, E, N, K);
    unpack_scales_kernel<<<grid(nsc), 256, 0, st>>>(ps, ws, E, N, K);
    return hipGetLastError();
}

bool use_stream_gemm(const moe_shape &s, bool gemm1)
{
    int bm = 0, bn = 0, ku = 0;
    return tile_config_of(s, gemm1, &bm, &bn, &ku) && bm <= 64;
}

hipError_t launch_gemm1_stream(const moe_shape &sh, const uint8_t *x, const uint8_t *xs,
                               const int32_t *counts, const int32_t *offsets,
                               const int32_t *row_route, const uint8_t *w13p,
                               const uint8_t *w13ps, uint8_t *h, uint8_t *hs, hipStream_t st)
{
    const StreamArgs g{x, xs, counts, offsets, row_route, w13p, w13ps, h, hs, nullptr, nullptr,
                       nullptr};
    return launch_stream<true>(sh, g, stream_bm(sh, true), st);
}

hipError_t launch_gemm2_stream(const moe_shape &sh, const uint8_t *h, const uint8_t *hs,
                               const int32_t *counts, const int32_t *offsets,
                               const uint8_t *w2p, const uint8_t *w2ps, const YRows &y,
                               hipStream_t st)
{
    const StreamArgs g{h, hs, counts, offsets, nullptr, w2p, w2ps, nullptr, nullptr, y.bf16,
                       y.codes, y.scales};
    return launch_stream<false>(sh, g, stream_bm(sh, false), st);
}

} // namespace moe
