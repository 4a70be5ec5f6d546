// Expert GEMMs for many rows per expert: LDS-tiled scaled FP4 x FP8 MFMA.
//
// A workgroup computes a tile of 256 weight rows x BM dispatched rows of one
// expert.  Its four wavefronts form a 2 x 2 grid: wavefront (wn, wm) owns
// weight rows [128 wn, 128 wn + 128) of the tile (eight 16-row MFMA groups)
// and dispatched rows [wm BM/2, (wm+1) BM/2).  Every K step of 128 is
// brought into LDS with direct global-to-LDS loads, double-buffered: the
// loads of step k+1 are in flight while step k is computed.  Each workgroup
// fits in half a CU's LDS and registers, so two independent workgroups share
// every CU: while one waits at its barrier or on LDS, the other's MFMAs run
// (measured faster than one workgroup of eight wavefronts, whose halves wait
// at the same barriers, and than three-stage rings at one workgroup per CU).
//
// GEMM1 tile: 128 intermediate columns j0..j0+127.  Wavefront wn holds the
// 64 columns j0+64wn.. as four gate groups and the four matching up groups,
// so the clamped SwiGLU and the MX FP8 requant (two 32-column blocks) happen
// in registers.  GEMM2 tile: 256 output columns, y kept in float32.
//
// Work items are (row tile of one expert, N tile), derived on every
// workgroup from counts as in the skinny kernels, and taken in a grid-stride
// loop.
#include "moe_common.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
// Tile of BN weight rows (256 or 128) x BM dispatched rows (64 or 128).
template <int BM, int BN>
struct TileLds {
    static constexpr int kW = BN * 64;    // FP4 weight tile, one K step
    static constexpr int kX = BM * 128;   // FP8 activation rows, one K step
    static constexpr int kStage = kW + kX;
    static constexpr int kStages = 2;     // K steps resident in LDS (2 to 4)
    static constexpr int kWE = BN * 16;   // weight exponents of four K steps
    static constexpr int kXE = BM * 16;   // activation exponents of four K steps
    static constexpr int kExp = kWE + kXE;
    static constexpr int kExpSlots = 2;
    // loads one wavefront issues per K step (BN/64 weight instructions, BM/32
    // activation instructions) and per four K steps (one weight-exponent and
    // one activation-exponent instruction)
    static constexpr int kDataLoads = BN / 64 + BM / 32;
    static constexpr int kExpLoads = 2;
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
template <int SIZE>
__device__ __forceinline__ void g2lds(const uint8_t *base, uint32_t voff, uint32_t m0)
{
    static_assert(SIZE == 16 || SIZE == 4, "dword and dwordx4 LDS DMA only");
    if (SIZE == 16)
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

// Wait until at most `steps` K steps' loads (of which `exps` start an
// exponent group) are outstanding; steps <= 2, exps <= 1.
template <typename L>
__device__ __forceinline__ void wait_loads(int steps, int exps)
{
    constexpr int D = L::kDataLoads, E = L::kExpLoads;
    switch (steps * 2 + exps) {
    case 2: wait_vmcnt<D>(); break;
    case 3: wait_vmcnt<D + E>(); break;
    case 4: wait_vmcnt<2 * D>(); break;
    case 5: wait_vmcnt<2 * D + E>(); break;
    default: wait_vmcnt<0>(); break;
    }
}

template <bool kGemm1, int BM, int BN>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
gemm_tiled_kernel(Shape s, const uint8_t *__restrict__ act, const uint8_t *__restrict__ act_s,
                  const int32_t *__restrict__ counts, const int32_t *__restrict__ offsets,
                  const int32_t *__restrict__ row_route, const uint8_t *__restrict__ w,
                  const uint8_t *__restrict__ ws, uint8_t *__restrict__ h_out,
                  uint8_t *__restrict__ hs_out, float *__restrict__ y_out)
{
    using L = TileLds<BM, BN>;
    constexpr int GW = BN / 32;             // 16-row weight groups per wavefront
    constexpr int WI = BN / 64;             // weight load instructions per wavefront
    constexpr int TB = BM / 32;             // 16-row activation blocks per wavefront
    constexpr int NS = L::kStages;
    __shared__ __align__(16) uint8_t lds[NS * L::kStage + L::kExpSlots * L::kExp];
    __shared__ int prefix[kMaxLocalExperts + 1];
    __shared__ int arow[BM];                // activation row of each tile row

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i16 = lane & 15, kq = lane >> 4;
    const int wn = wave & 1, wm = wave >> 1;
    const int H = s.H, I = s.I;
    const int KT = kGemm1 ? H : I;          // contraction length
    const int KS = KT / 128;
    const int NT = kGemm1 ? I / (BN / 2) : H / BN;
    const int nchunks = plan_chunks(s, counts, BM, prefix);
    const long items = (long)nchunks * NT;

    for (long item = blockIdx.x; item < items; item += gridDim.x) {
        const int q = (int)(item / NT), nt = (int)(item - (long)q * NT);
        const int e = chunk_expert(prefix, s.E_local, q);
        const int c = q - prefix[e];
        const int row0 = offsets[e] + c * BM;
        const int nrows = min(BM, used_rows(s, counts[e]) - c * BM);
        if (tid < BM) {
            const int r = min(tid, nrows - 1);
            arow[tid] = kGemm1 ? row_route[row0 + r] / s.K : row0 + r;
        }
        __syncthreads();

        // weight row (within the expert's rows of W) of tile row r
        auto wrow_of = [&](int r) -> uint32_t {
            const int grp = r >> 4, rr = r & 15;
            if (kGemm1) {
                // group grp: wavefront half grp / GW; within it GW/2 gate
                // groups, then the GW/2 matching up groups
                const int half = grp / GW, up = (grp % GW) >= GW / 2, cb = grp % (GW / 2);
                return (uint32_t)(e * 2 * I + (up ? I : 0) + nt * (BN / 2) + (BN / 4) * half +
                                  16 * cb + rr);
            }
            return (uint32_t)(e * H + nt * BN + r);
        };
        // LDS layout of a stage: weight group g (tile rows 16g..16g+15) at
        // 1024 g as 64-byte rows, activation tile row R at kW + 128 R; the
        // 16-byte chunk c of a row sits at position c ^ swz(row) with
        // swz = (row >> 1) & 3 (weights) or (row >> 1) & 7 (activations), so
        // the MFMA fragment reads below hit every LDS bank once.  Loads are
        // row-major (four or eight consecutive lanes cover one row), which
        // the global-to-LDS path moves several times faster than lanes
        // walking down the rows.
        //
        // Weight instruction i (< BN/64) brings group g = wave + 4i: lane l -> row
        // 16g + (l >> 2), chunk (l & 3) ^ swz.  Activation instruction i
        // brings tile rows 8h.. with h = wave + 4i: lane l -> row
        // R = 8h + (l >> 3), chunk (l & 7) ^ swz.
        uint32_t woff[WI], xoff[TB];
#pragma unroll
        for (int i = 0; i < WI; ++i) {
            const int g = wave + 4 * i, rr = lane >> 2;
            const int c = (lane & 3) ^ ((rr >> 1) & 3);
            woff[i] = wrow_of(16 * g + rr) * (uint32_t)(KT / 2) + 16u * (uint32_t)c;
        }
#pragma unroll
        for (int i = 0; i < TB; ++i) {
            const int h = wave + 4 * i, R = 8 * h + (lane >> 3);
            const int c = (lane & 7) ^ ((R >> 1) & 7);
            xoff[i] = (uint32_t)arow[R] * (uint32_t)KT + 16u * (uint32_t)c;
        }
        // exponents, four K steps (16 bytes) per row at a time: wavefront v
        // brings weight rows 64 (v mod BN/64) + l and activation rows
        // 64 (v mod BM/64) + l (where there are fewer than four such row
        // blocks, two wavefronts write the same bytes to the same place).
        // The last group of a row is read from 16 bytes before the row's
        // end, so no read passes it (KS >= 4).
        const int we_wave = wave % (BN / 64);
        const int xe_wave = wave % (BM / 64);
        const uint32_t weoff = wrow_of(64 * we_wave + lane) * (uint32_t)(KT / 32);
        const uint32_t xeoff = (uint32_t)arow[64 * xe_wave + lane] * (uint32_t)(KT / 32);
        auto ebase = [&](int grp) -> int { return min(16 * grp, KT / 32 - 16); };

        const uint32_t lds0 = lds_addr(lds);
        const uint32_t lds_w = __builtin_amdgcn_readfirstlane(lds0 + 1024u * wave);
        const uint32_t lds_x = __builtin_amdgcn_readfirstlane(lds0 + L::kW + 1024u * wave);
        const uint32_t lds_e = lds0 + NS * L::kStage;
        const uint32_t lds_we = __builtin_amdgcn_readfirstlane(lds_e + 1024u * we_wave);
        const uint32_t lds_xe = __builtin_amdgcn_readfirstlane(lds_e + L::kWE + 1024u * xe_wave);
        auto issue = [&](int ks) {
            const uint32_t st = (uint32_t)((ks % NS) * L::kStage);
#pragma unroll
            for (int i = 0; i < WI; ++i)
                g2lds<16>(w, woff[i] + (uint32_t)ks * 64u, lds_w + st + 4096u * i);
#pragma unroll
            for (int i = 0; i < TB; ++i)
                g2lds<16>(act, xoff[i] + (uint32_t)ks * 128u, lds_x + st + 4096u * i);
            if ((ks & 3) == 0) {
                const int grp = ks >> 2;
                const uint32_t es = (uint32_t)((grp % L::kExpSlots) * L::kExp);
                const uint32_t eb = (uint32_t)ebase(grp);
                g2lds<16>(ws, weoff + eb, lds_we + es);
                g2lds<16>(act_s, xeoff + eb, lds_xe + es);
            }
        };

        v4f acc[GW][TB];
#pragma unroll
        for (int i = 0; i < GW; ++i)
#pragma unroll
            for (int j = 0; j < TB; ++j)
                acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

        // per-lane LDS offsets of the fragment reads (see the layout above)
        const int afrag = wn * GW * 1024 + 64 * i16 + 16 * (kq ^ ((i16 >> 1) & 3));
        const int xrow = wm * (BM / 2) + i16;
        const int bfrag_lo = L::kW + 128 * xrow + 16 * (kq ^ ((i16 >> 1) & 7));
        const int bfrag_hi = L::kW + 128 * xrow + 16 * ((kq + 4) ^ ((i16 >> 1) & 7));
        const int wexp = NS * L::kStage + 16 * (wn * (BN / 2) + i16) + kq;
        const int xexp = NS * L::kStage + L::kWE + 16 * xrow + kq;

#pragma unroll
        for (int p = 0; p < NS - 1; ++p)
            if (p < KS)
                issue(p);
        for (int ks = 0; ks < KS; ++ks) {
            // this wavefront's loads of step ks are done once at most the
            // loads of the later steps already issued (up to NS-2 of them)
            // are outstanding; then all wavefronts' are
            {
                const int later = min(NS - 2, KS - 1 - ks);
                int exps = 0;
                for (int t = ks + 1; t <= ks + later; ++t)
                    exps += (t & 3) == 0;
                wait_loads<L>(later, exps);
            }
            raw_barrier();
            if (ks + NS - 1 < KS)
                issue(ks + NS - 1);
            const uint8_t *st = lds + (ks % NS) * L::kStage;
            const uint8_t *ex = lds + ((ks >> 2) % L::kExpSlots) * L::kExp + (4 * ks - ebase(ks >> 2));
            v8i b[TB];
            int sb[TB];
#pragma unroll
            for (int j = 0; j < TB; ++j) {
                const u32x4 lo = lds_read16(st + bfrag_lo + j * 2048);
                const u32x4 hi = lds_read16(st + bfrag_hi + j * 2048);
                b[j] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                           (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                sb[j] = ex[xexp + j * 256];
            }
#pragma unroll
            for (int i = 0; i < GW; ++i) {
                const u32x4 a4 = lds_read16(st + afrag + i * 1024);
                const v8i a = v8i{(int)a4[0], (int)a4[1], (int)a4[2], (int)a4[3], 0, 0, 0, 0};
                const int sa = ex[wexp + i * 256];
#pragma unroll
                for (int j = 0; j < TB; ++j)
                    acc[i][j] = mfma_w4a8(a, b[j], acc[i][j], sa, sb[j]);
            }
        }

        // epilogue: lane holds tile row (wm*BM/2 + 16j + i16), weight rows
        // 4kq..4kq+3 of each of its GW groups
        if (kGemm1) {
            constexpr int CB = GW / 2;   // 16-column blocks of h per wavefront
#pragma unroll
            for (int j = 0; j < TB; ++j) {
                const int m = wm * (BM / 2) + 16 * j + i16;
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
                    if (m < nrows) {
                        const size_t row = (size_t)(row0 + m);
                        const int col0 = nt * (BN / 2) + (BN / 4) * wn + 32 * blk;
#pragma unroll
                        for (int cb = 2 * blk; cb < 2 * blk + 2; ++cb) {
                            uint32_t pk = 0;
#pragma unroll
                            for (int v = 0; v < 4; ++v)
                                pk |= f32_to_e4m3(ldexpf(hv[cb][v], -E)) << (8 * v);
                            *reinterpret_cast<uint32_t *>(h_out + row * (size_t)I + col0 +
                                                          16 * (cb - 2 * blk) + 4 * kq) = pk;
                        }
                        if (kq == 0)
                            hs_out[row * (size_t)(I / 32) + col0 / 32] = (uint8_t)(E + 127);
                    }
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < TB; ++j) {
                const int m = wm * (BM / 2) + 16 * j + i16;
                if (m < nrows) {
                    float *yr = y_out + (size_t)(row0 + m) * (size_t)H + (size_t)nt * BN +
                                (BN / 2) * wn + 4 * kq;
#pragma unroll
                    for (int i = 0; i < GW; ++i)
                        *reinterpret_cast<float4 *>(yr + 16 * i) =
                            float4{acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
                }
            }
        }
        __syncthreads();
    }
}

template <typename KernelT>
int tiled_grid(KernelT kernel, long upper_items)
{
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) !=
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

int tiled_bm(const moe_shape &s)
{
    const double per_expert = (double)s.T * s.K / (double)(s.E_total > 0 ? s.E_total : 1);
    return per_expert <= 96.0 ? 64 : 128;
}

namespace {

// Weight rows per tile: 256, or 128 when the expected number of items with
// 256 would leave fewer than three rounds for the resident workgroups (two
// per CU), so the last, partly filled round costs little.
int tiled_bn(const moe_shape &s, bool gemm1)
{
    const double per_expert = (double)s.T * s.K / (double)(s.E_total > 0 ? s.E_total : 1);
    const int bm = tiled_bm(s);
    const double tiles = (double)s.E_local * (double)(long)((per_expert + bm - 1) / bm);
    const double nt256 = gemm1 ? s.I / 128 : s.H / 256;
    const bool fits256 = gemm1 ? s.I % 128 == 0 : s.H % 256 == 0;
    if (!fits256)
        return 128;
    return tiles * nt256 < 3.0 * 2 * device_cu_count() ? 128 : 256;
}

template <bool kGemm1, int BM, int BN>
hipError_t launch_tiled(const moe_shape &sh, const uint8_t *act, const uint8_t *act_s,
                        const int32_t *counts, const int32_t *offsets, const int32_t *row_route,
                        const uint8_t *w, const uint8_t *ws, uint8_t *h, uint8_t *hs, float *y,
                        hipStream_t st)
{
    auto k = gemm_tiled_kernel<kGemm1, BM, BN>;
    const long nt = kGemm1 ? sh.I / (BN / 2) : sh.H / BN;
    const int grid = tiled_grid(k, tile_upper_bound(sh, BM) * nt);
    k<<<grid, kThreads, 0, st>>>(to_dev(sh), act, act_s, counts, offsets, row_route, w, ws, h, hs,
                                 y);
    return hipGetLastError();
}

template <bool kGemm1>
hipError_t launch_tiled_any(const moe_shape &sh, const uint8_t *act, const uint8_t *act_s,
                            const int32_t *counts, const int32_t *offsets,
                            const int32_t *row_route, const uint8_t *w, const uint8_t *ws,
                            uint8_t *h, uint8_t *hs, float *y, hipStream_t st)
{
    const int bm = tiled_bm(sh), bn = tiled_bn(sh, kGemm1);
    if (bm == 64 && bn == 128)
        return launch_tiled<kGemm1, 64, 128>(sh, act, act_s, counts, offsets, row_route, w, ws, h,
                                             hs, y, st);
    if (bm == 64)
        return launch_tiled<kGemm1, 64, 256>(sh, act, act_s, counts, offsets, row_route, w, ws, h,
                                             hs, y, st);
    if (bn == 128)
        return launch_tiled<kGemm1, 128, 128>(sh, act, act_s, counts, offsets, row_route, w, ws,
                                              h, hs, y, st);
    return launch_tiled<kGemm1, 128, 256>(sh, act, act_s, counts, offsets, row_route, w, ws, h,
                                          hs, y, st);
}

} // namespace

hipError_t launch_gemm1_tiled(const moe_shape &sh, const uint8_t *x, const uint8_t *xs,
                              const int32_t *counts, const int32_t *offsets,
                              const int32_t *row_route, const uint8_t *w13, const uint8_t *w13s,
                              uint8_t *h, uint8_t *hs, hipStream_t st)
{
    return launch_tiled_any<true>(sh, x, xs, counts, offsets, row_route, w13, w13s, h, hs,
                                  nullptr, st);
}

hipError_t launch_gemm2_tiled(const moe_shape &sh, const uint8_t *h, const uint8_t *hs,
                              const int32_t *counts, const int32_t *offsets, const uint8_t *w2,
                              const uint8_t *w2s, float *y, hipStream_t st)
{
    return launch_tiled_any<false>(sh, h, hs, counts, offsets, nullptr, w2, w2s, nullptr,
                                   nullptr, y, st);
}

} // namespace moe
