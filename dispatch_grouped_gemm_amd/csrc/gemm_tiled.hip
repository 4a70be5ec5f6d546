// Expert GEMMs for many rows per expert: LDS-tiled scaled FP4 x FP8 MFMA.
//
// A workgroup computes a tile of 256 weight rows x BM dispatched rows of one
// expert.  Its four wavefronts form a 2 x 2 grid: wavefront (wn, wm) owns
// weight rows [128 wn, 128 wn + 128) of the tile (eight 16-row MFMA groups)
// and dispatched rows [wm BM/2, (wm+1) BM/2).  Every K step of 128 is staged
// in LDS, double-buffered: the global loads of step k+1 are in flight while
// the MFMAs of step k run.  LDS holds the operands in MFMA fragment order
// (one 16-byte slot per lane), so every fragment read is one linear
// ds_read_b128 without bank conflicts.
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
constexpr int kBN = 256;          // weight rows per tile
constexpr int kGroups = kBN / 16; // 16-row MFMA groups per tile

template <int BM>
struct TileLds {
    static constexpr int kW = kBN * 64;   // FP4 weight tile, one K step
    static constexpr int kX = BM * 128;   // FP8 activation tile
    static constexpr int kWE = kBN * 4;   // weight exponents (4 blocks per row)
    static constexpr int kXE = BM * 4;    // activation exponents
    static constexpr int kStage = kW + kX + kWE + kXE;
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 lds_read16(const uint8_t *p)
{
    return *reinterpret_cast<const u32x4 *>(p);
}

// Global loads of one K step of the tile into registers.
template <int WPT, int XPT>
__device__ __forceinline__ void tile_gload(u32x4 (&wreg)[WPT], u32x4 (&xreg)[XPT], uint32_t &wereg,
                                           uint32_t &xereg, const uint8_t *w,
                                           const uint32_t (&woff)[WPT], const uint8_t *x,
                                           const uint32_t (&xoff)[XPT], const uint8_t *we,
                                           uint32_t weoff, const uint8_t *xe, uint32_t xeoff,
                                           int ks, bool has_xe)
{
#pragma unroll
    for (int i = 0; i < WPT; ++i)
        wreg[i] = *reinterpret_cast<const u32x4 *>(w + (woff[i] + (uint32_t)ks * 64u));
#pragma unroll
    for (int i = 0; i < XPT; ++i)
        xreg[i] = *reinterpret_cast<const u32x4 *>(x + (xoff[i] + (uint32_t)ks * 128u));
    wereg = *reinterpret_cast<const uint32_t *>(we + (weoff + (uint32_t)ks * 4u));
    if (has_xe)
        xereg = *reinterpret_cast<const uint32_t *>(xe + (xeoff + (uint32_t)ks * 4u));
}

// The registers of one K step into an LDS stage (fragment order).
// LDS slot of weight piece p = tid + 256 i (tile row p/4, chunk p%4) and of
// activation piece p (tile row p/8, chunk p%8), in MFMA fragment order.
__device__ __forceinline__ int wpiece_slot(int p)
{
    const int r = p >> 2, ch = p & 3;
    return ((r >> 4) * 64 + (r & 15) + 16 * ch) * 16;
}

__device__ __forceinline__ int xpiece_slot(int p)
{
    const int r = p >> 3, ch = p & 7;
    return (((r >> 4) * 2 + (ch >> 2)) * 64 + (r & 15) + 16 * (ch & 3)) * 16;
}

template <int WPT, int XPT>
__device__ __forceinline__ void tile_lstore(uint8_t *st, const u32x4 (&wreg)[WPT],
                                            const u32x4 (&xreg)[XPT], uint32_t wereg,
                                            uint32_t xereg, int x_off, int we_off, int xe_off,
                                            int tid, bool has_xe)
{
#pragma unroll
    for (int i = 0; i < WPT; ++i)
        *reinterpret_cast<u32x4 *>(st + wpiece_slot(tid + 256 * i)) = wreg[i];
#pragma unroll
    for (int i = 0; i < XPT; ++i)
        *reinterpret_cast<u32x4 *>(st + x_off + xpiece_slot(tid + 256 * i)) = xreg[i];
    *reinterpret_cast<uint32_t *>(st + we_off + 4 * tid) = wereg;
    if (has_xe)
        *reinterpret_cast<uint32_t *>(st + xe_off + 4 * tid) = xereg;
}

// One K step from LDS stage BUF: the next step's global loads are issued
// first, the MFMAs run, then the next step goes to the other stage.
template <int BUF, int TB, int WPT, int XPT, int STAGE>
__device__ __forceinline__ void
tile_step(v4f (&acc)[8][TB], uint8_t *lds, int ks, int KS, int afrag, int bfrag, int wexp,
          int xexp, u32x4 (&wreg)[WPT], u32x4 (&xreg)[XPT], uint32_t &wereg, uint32_t &xereg,
          const uint8_t *w, const uint32_t (&woff)[WPT], const uint8_t *x,
          const uint32_t (&xoff)[XPT], const uint8_t *we, uint32_t weoff, const uint8_t *xe,
          uint32_t xeoff, int x_off, int we_off, int xe_off, int tid, bool has_xe)
{
    const bool more = ks + 1 < KS;
    if (more)
        tile_gload<WPT, XPT>(wreg, xreg, wereg, xereg, w, woff, x, xoff, we, weoff, xe, xeoff,
                             ks + 1, has_xe);
    const uint8_t *st = lds + BUF * STAGE;
    v8i b[TB];
    int sb[TB];
#pragma unroll
    for (int j = 0; j < TB; ++j) {
        const u32x4 lo = lds_read16(st + bfrag + j * 2048);
        const u32x4 hi = lds_read16(st + bfrag + j * 2048 + 1024);
        b[j] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        sb[j] = st[xexp + j * 64];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const u32x4 a4 = lds_read16(st + afrag + i * 1024);
        const v8i a = v8i{(int)a4[0], (int)a4[1], (int)a4[2], (int)a4[3], 0, 0, 0, 0};
        const int sa = st[wexp + i * 64];
#pragma unroll
        for (int j = 0; j < TB; ++j)
            acc[i][j] = mfma_w4a8(a, b[j], acc[i][j], sa, sb[j]);
    }
    if (more)
        tile_lstore<WPT, XPT>(lds + (BUF ^ 1) * STAGE, wreg, xreg, wereg, xereg, x_off, we_off,
                              xe_off, tid, has_xe);
    __syncthreads();
}

template <bool kGemm1, int BM>
__global__ void __launch_bounds__(kThreads)
gemm_tiled_kernel(Shape s, const uint8_t *__restrict__ act, const uint8_t *__restrict__ act_s,
                  const int32_t *__restrict__ counts, const int32_t *__restrict__ offsets,
                  const int32_t *__restrict__ row_route, const uint8_t *__restrict__ w,
                  const uint8_t *__restrict__ ws, uint8_t *__restrict__ h_out,
                  uint8_t *__restrict__ hs_out, float *__restrict__ y_out)
{
    using L = TileLds<BM>;
    constexpr int TB = BM / 32;             // 16-row activation blocks per wavefront
    constexpr int WPT = kBN * 4 / kThreads; // 16-byte weight pieces per thread and K step
    constexpr int XPT = BM * 8 / kThreads;  // 16-byte activation pieces per thread
    __shared__ __align__(16) uint8_t lds[2 * L::kStage];
    __shared__ int prefix[kMaxLocalExperts + 1];
    __shared__ int arow[BM];                // activation row of each tile row

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i16 = lane & 15, kq = lane >> 4;
    const int wn = wave & 1, wm = wave >> 1;
    const int H = s.H, I = s.I;
    const int KT = kGemm1 ? H : I;          // contraction length
    const int KS = KT / 128;
    const int NT = kGemm1 ? I / 128 : H / kBN;
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

        // byte offsets of this thread's pieces (all buffers are below 4 GiB)
        auto wrow_of = [&](int r) -> uint32_t {
            const int grp = r >> 4, rr = r & 15;
            if (kGemm1) {
                // group grp: wavefront half grp/8, up if (grp/4)&1, column block grp%4
                const int half = grp >> 3, up = (grp >> 2) & 1, cb = grp & 3;
                return (uint32_t)(e * 2 * I + (up ? I : 0) + nt * 128 + 64 * half + 16 * cb + rr);
            }
            return (uint32_t)(e * H + nt * kBN + r);
        };
        uint32_t woff[WPT], xoff[XPT];
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int p = tid + kThreads * i;
            woff[i] = wrow_of(p >> 2) * (uint32_t)(KT / 2) + (uint32_t)(p & 3) * 16u;
        }
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int p = tid + kThreads * i;
            xoff[i] = (uint32_t)arow[p >> 3] * (uint32_t)KT + (uint32_t)(p & 7) * 16u;
        }
        const uint32_t weoff = wrow_of(tid) * (uint32_t)(KT / 32);
        const uint32_t xeoff = (uint32_t)arow[tid < BM ? tid : 0] * (uint32_t)(KT / 32);

        u32x4 wreg[WPT], xreg[XPT];
        uint32_t wereg = 0, xereg = 0;
        v4f acc[8][TB];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < TB; ++j)
                acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

        // per-lane LDS bases: fragment slot of this lane, its exponent bytes
        const int frag = lane * 16;
        const int wexp = L::kW + L::kX + i16 * 4 + kq + wn * 8 * 64;
        const int xexp = L::kW + L::kX + L::kWE + i16 * 4 + kq + wm * TB * 64;
        const int afrag = frag + wn * 8 * 1024;
        const int bfrag = L::kW + frag + wm * TB * 2048;

        tile_gload<WPT, XPT>(wreg, xreg, wereg, xereg, w, woff, act, xoff, ws, weoff, act_s, xeoff,
                             0, tid < BM);
        tile_lstore<WPT, XPT>(lds, wreg, xreg, wereg, xereg, L::kW, L::kX + L::kW,
                              L::kW + L::kX + L::kWE, tid, tid < BM);
        __syncthreads();
        for (int ks = 0; ks < KS; ks += 2) {
            tile_step<0, TB, WPT, XPT, L::kStage>(acc, lds, ks, KS, afrag, bfrag, wexp, xexp, wreg,
                                                  xreg, wereg, xereg, w, woff, act, xoff, ws,
                                                  weoff, act_s, xeoff, L::kW, L::kW + L::kX,
                                                  L::kW + L::kX + L::kWE, tid, tid < BM);
            if (ks + 1 < KS)
                tile_step<1, TB, WPT, XPT, L::kStage>(acc, lds, ks + 1, KS, afrag, bfrag, wexp,
                                                      xexp, wreg, xreg, wereg, xereg, w, woff, act,
                                                      xoff, ws, weoff, act_s, xeoff, L::kW,
                                                      L::kW + L::kX, L::kW + L::kX + L::kWE,
                                                      tid, tid < BM);
        }

        // epilogue: lane holds tile row (wm*BM/2 + 16j + i16), weight rows
        // 4kq..4kq+3 of each of its eight groups
        if (kGemm1) {
#pragma unroll
            for (int j = 0; j < TB; ++j) {
                const int m = wm * (BM / 2) + 16 * j + i16;
                float hv[4][4];
#pragma unroll
                for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        hv[cb][v] = swiglu_clamped(acc[cb][j][v], acc[cb + 4][j][v], s.gate_limit,
                                                   s.up_limit);
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) {
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
                        const int col0 = nt * 128 + 64 * wn + 32 * blk;
#pragma unroll
                        for (int cb = 2 * blk; cb < 2 * blk + 2; ++cb) {
                            uint32_t pk = 0;
#pragma unroll
                            for (int v = 0; v < 4; ++v)
                                pk |= f32_to_e4m3(ldexpf(hv[cb][v], -E)) << (8 * v);
                            *reinterpret_cast<uint32_t *>(h_out + row * (size_t)I + nt * 128 +
                                                          64 * wn + 16 * cb + 4 * kq) = pk;
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
                    float *yr = y_out + (size_t)(row0 + m) * (size_t)H + (size_t)nt * kBN +
                                128 * wn + 4 * kq;
#pragma unroll
                    for (int i = 0; i < 8; ++i)
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

hipError_t launch_gemm1_tiled(const moe_shape &sh, const uint8_t *x, const uint8_t *xs,
                              const int32_t *counts, const int32_t *offsets,
                              const int32_t *row_route, const uint8_t *w13, const uint8_t *w13s,
                              uint8_t *h, uint8_t *hs, hipStream_t st)
{
    const Shape s = to_dev(sh);
    const long nt = sh.I / 128;
    if (tiled_bm(sh) == 64) {
        auto k = gemm_tiled_kernel<true, 64>;
        const int grid = tiled_grid(k, tile_upper_bound(sh, 64) * nt);
        k<<<grid, kThreads, 0, st>>>(s, x, xs, counts, offsets, row_route, w13, w13s, h, hs,
                                     nullptr);
    } else {
        auto k = gemm_tiled_kernel<true, 128>;
        const int grid = tiled_grid(k, tile_upper_bound(sh, 128) * nt);
        k<<<grid, kThreads, 0, st>>>(s, x, xs, counts, offsets, row_route, w13, w13s, h, hs,
                                     nullptr);
    }
    return hipGetLastError();
}

hipError_t launch_gemm2_tiled(const moe_shape &sh, const uint8_t *h, const uint8_t *hs,
                              const int32_t *counts, const int32_t *offsets, const uint8_t *w2,
                              const uint8_t *w2s, float *y, hipStream_t st)
{
    const Shape s = to_dev(sh);
    const long nt = sh.H / kBN;
    if (tiled_bm(sh) == 64) {
        auto k = gemm_tiled_kernel<false, 64>;
        const int grid = tiled_grid(k, tile_upper_bound(sh, 64) * nt);
        k<<<grid, kThreads, 0, st>>>(s, h, hs, counts, offsets, nullptr, w2, w2s, nullptr,
                                     nullptr, y);
    } else {
        auto k = gemm_tiled_kernel<false, 128>;
        const int grid = tiled_grid(k, tile_upper_bound(sh, 128) * nt);
        k<<<grid, kThreads, 0, st>>>(s, h, hs, counts, offsets, nullptr, w2, w2s, nullptr,
                                     nullptr, y);
    }
    return hipGetLastError();
}

} // namespace moe
