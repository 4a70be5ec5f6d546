// Expert GEMMs for few rows per expert (decode-sized batches): the weights
// are streamed once from HBM straight into scaled FP4 x FP8 MFMAs and every
// weight fragment is applied to all rows of a chunk (up to 16*NMB rows)
// while it is in registers.
//
// The E8M0 exponents of an item's weight and activation rows are copied to
// LDS once per item (coalesced dword loads); the K loop reads them there.
//
// Work items are (row chunk of one expert, N tile); a workgroup of four
// wavefronts takes items in a grid-stride loop.  The four wavefronts split
// the K steps of an item (wavefront w takes K steps w, w+4, ...), so their
// loads of each weight row together cover 256 contiguous bytes, and their
// partial sums meet in LDS before the epilogue.
//
// GEMM1 tile: 32 intermediate columns j0..j0+31, i.e. W13 rows
// j0..j0+31 (gate) and I+j0..I+j0+31 (up), four 16-row MFMA groups.  The
// epilogue applies the clamped SwiGLU to matching gate/up accumulators and
// requantises the 32 columns as one MX FP8 block.
// GEMM2 tile: 64 output columns, four 16-row MFMA groups of W2; y rows are
// kept in float32 for the combine.
#include "moe_common.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ v8i load_fp4_frag(const uint8_t *p)
{
    const uint4 q = *reinterpret_cast<const uint4 *>(p);
    return v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
}

// FP8 operand of one K step: lane group g takes bytes [16g, 16g+16) and
// [64+16g, 64+16g+16) of the 128-byte K step (p points at the first).
__device__ __forceinline__ v8i load_fp8_frag(const uint8_t *p)
{
    const uint4 lo = *reinterpret_cast<const uint4 *>(p);
    const uint4 hi = *reinterpret_cast<const uint4 *>(p + 64);
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
               (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// Copy the E8M0 exponent rows of one item into LDS (row stride `stride`
// bytes, `nbytes` used bytes per row, a multiple of 4): rows [0, nrows)
// come from src_rows(r); the workgroup shares the copy.
template <typename RowFn>
__device__ __forceinline__ void stage_exponents(uint8_t *dst, int stride, int nbytes, int nrows,
                                                RowFn src_row)
{
    const int words = nbytes >> 2;
    for (int i = threadIdx.x; i < nrows * words; i += kThreads) {
        const int r = i / words, c = i - r * words;
        const uint32_t v = reinterpret_cast<const uint32_t *>(src_row(r))[c];
        *reinterpret_cast<uint32_t *>(dst + r * stride + 4 * c) = v;
    }
}

// Sum the four wavefronts' accumulators in LDS: red[(mb*4 + g)*4 + v][lane].
template <int NMB>
__device__ __forceinline__ void reduce_waves(v4f (&acc)[NMB][4], float *red, int nmb_act)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int w = 0; w < 4; ++w) {
        if (wave == w) {
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) {
                if (mb < nmb_act) {
#pragma unroll
                    for (int g = 0; g < 4; ++g)
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            float *p = red + ((mb * 4 + g) * 4 + v) * 64 + lane;
                            *p = (w == 0 ? 0.0f : *p) + acc[mb][g][v];
                        }
                }
            }
        }
        __syncthreads();
    }
}

template <int NMB>
__global__ void __launch_bounds__(kThreads)
gemm1_skinny_kernel(Shape s, const uint8_t *__restrict__ x, const uint8_t *__restrict__ xs,
                    const int32_t *__restrict__ counts, const int32_t *__restrict__ offsets,
                    const int32_t *__restrict__ row_route, const uint8_t *__restrict__ w13,
                    const uint8_t *__restrict__ w13s, uint8_t *__restrict__ h,
                    uint8_t *__restrict__ hs)
{
    constexpr int CH = 16 * NMB;
    __shared__ int prefix[kMaxLocalExperts + 1];
    __shared__ int tok[CH];
    __shared__ float red[NMB * 4 * 4 * 64];
    extern __shared__ uint8_t exps[]; // [64 weight rows + CH x rows][H/32 + 4]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i16 = lane & 15, kq = lane >> 4;
    const int H = s.H, I = s.I, KS = H / 128;
    const int es = H / 32 + 4;
    uint8_t *wexp = exps, *xexp = exps + 64 * es;
    const int nchunks = plan_chunks(s, counts, CH, prefix);
    const int NT = I / 32;
    const long items = (long)nchunks * NT;

    for (long item = blockIdx.x; item < items; item += gridDim.x) {
        const int q = (int)(item / NT), nt = (int)(item - (long)q * NT);
        const int e = chunk_expert(prefix, s.E_local, q);
        const int c = q - prefix[e];
        const int rows_e = used_rows(s, counts[e]);
        const int row0 = offsets[e] + c * CH;
        const int nrows = min(CH, rows_e - c * CH);
        const int nmb_act = (nrows + 15) >> 4;
        const int j0 = nt * 32;
        if (tid < CH)
            tok[tid] = tid < nrows ? row_route[row0 + tid] / s.K : 0;
        // W13 rows of the tile: r in [0, 64) is gate/up group r/16, row r%16
        stage_exponents(wexp, es, H / 32, 64, [&](int r) {
            const int g = r >> 4;
            const size_t wrow = (size_t)e * 2 * I + (g >= 2 ? I : 0) + j0 + 16 * (g & 1) + (r & 15);
            return w13s + wrow * (size_t)(H / 32);
        });
        stage_exponents(xexp, es, H / 32, nrows, [&](int r) {
            return xs + (size_t)(row_route[row0 + r] / s.K) * (size_t)(H / 32);
        });
        __syncthreads();

        const uint8_t *wp[4];
        const uint8_t *wsp[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const size_t wrow = (size_t)e * 2 * I + (g >= 2 ? I : 0) + j0 + 16 * (g & 1) + i16;
            wp[g] = w13 + wrow * (size_t)(H / 2) + kq * 16;
            wsp[g] = wexp + (g * 16 + i16) * es + kq;
        }
        const uint8_t *xp[NMB];
        const uint8_t *xsp[NMB];
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
            const int rloc = min(mb * 16 + i16, nrows - 1);
            const size_t t = (size_t)tok[rloc];
            xp[mb] = x + t * (size_t)H + kq * 16;
            xsp[mb] = xexp + rloc * es + kq;
        }

        v4f acc[NMB][4];
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                acc[mb][g] = v4f{0.f, 0.f, 0.f, 0.f};

        for (int ks = wave; ks < KS; ks += 4) {
            v8i a[4];
            int sa[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                a[g] = load_fp4_frag(wp[g] + ks * 64);
                sa[g] = wsp[g][ks * 4];
            }
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) {
                if (mb < nmb_act) {
                    const v8i b = load_fp8_frag(xp[mb] + ks * 128);
                    const int sb = xsp[mb][ks * 4];
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        acc[mb][g] = mfma_w4a8(a[g], b, acc[mb][g], sa[g], sb);
                }
            }
        }
        reduce_waves<NMB>(acc, red, nmb_act);

        // epilogue: wavefront w finishes row block w
        if (wave < nmb_act) {
            const int mb = wave;
            const int rloc = mb * 16 + i16;
            float hv[8];
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float gt = red[((mb * 4 + half) * 4 + v) * 64 + lane];
                    const float up = red[((mb * 4 + 2 + half) * 4 + v) * 64 + lane];
                    hv[half * 4 + v] = swiglu_clamped(gt, up, s.gate_limit, s.up_limit);
                }
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                amax = fmaxf(amax, fabsf(hv[i]));
            amax = fmaxf(amax, __shfl_xor(amax, 16));
            amax = fmaxf(amax, __shfl_xor(amax, 32));
            const int E = mx8_block_exponent(amax);
            uint32_t pk[2] = {0u, 0u};
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    pk[half] |= f32_to_e4m3(ldexpf(hv[half * 4 + v], -E)) << (8 * v);
            if (rloc < nrows) {
                const size_t row = (size_t)(row0 + rloc);
                uint8_t *hr = h + row * (size_t)I + j0 + 4 * kq;
                *reinterpret_cast<uint32_t *>(hr) = pk[0];
                *reinterpret_cast<uint32_t *>(hr + 16) = pk[1];
                if (kq == 0)
                    hs[row * (size_t)(I / 32) + nt] = (uint8_t)(E + 127);
            }
        }
        __syncthreads();
    }
}

template <int NMB>
__global__ void __launch_bounds__(kThreads)
gemm2_skinny_kernel(Shape s, const uint8_t *__restrict__ h, const uint8_t *__restrict__ hs,
                    const int32_t *__restrict__ counts, const int32_t *__restrict__ offsets,
                    const uint8_t *__restrict__ w2, const uint8_t *__restrict__ w2s,
                    float *__restrict__ y)
{
    constexpr int CH = 16 * NMB;
    __shared__ int prefix[kMaxLocalExperts + 1];
    __shared__ float red[NMB * 4 * 4 * 64];
    extern __shared__ uint8_t exps[]; // [64 weight rows + CH h rows][I/32 + 4]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i16 = lane & 15, kq = lane >> 4;
    const int H = s.H, I = s.I, KS = I / 128;
    const int es = I / 32 + 4;
    uint8_t *wexp = exps, *hexp = exps + 64 * es;
    const int nchunks = plan_chunks(s, counts, CH, prefix);
    const int NT = H / 64;
    const long items = (long)nchunks * NT;

    for (long item = blockIdx.x; item < items; item += gridDim.x) {
        const int q = (int)(item / NT), nt = (int)(item - (long)q * NT);
        const int e = chunk_expert(prefix, s.E_local, q);
        const int c = q - prefix[e];
        const int rows_e = used_rows(s, counts[e]);
        const int row0 = offsets[e] + c * CH;
        const int nrows = min(CH, rows_e - c * CH);
        const int nmb_act = (nrows + 15) >> 4;
        const int n0 = nt * 64;
        stage_exponents(wexp, es, I / 32, 64, [&](int r) {
            return w2s + ((size_t)e * H + n0 + r) * (size_t)(I / 32);
        });
        stage_exponents(hexp, es, I / 32, nrows, [&](int r) {
            return hs + (size_t)(row0 + r) * (size_t)(I / 32);
        });
        __syncthreads();

        const uint8_t *wp[4];
        const uint8_t *wsp[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const size_t wrow = (size_t)e * H + n0 + 16 * g + i16;
            wp[g] = w2 + wrow * (size_t)(I / 2) + kq * 16;
            wsp[g] = wexp + (16 * g + i16) * es + kq;
        }
        const uint8_t *hp[NMB];
        const uint8_t *hsp[NMB];
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
            const int rloc = min(mb * 16 + i16, nrows - 1);
            const size_t row = (size_t)(row0 + rloc);
            hp[mb] = h + row * (size_t)I + kq * 16;
            hsp[mb] = hexp + rloc * es + kq;
        }

        v4f acc[NMB][4];
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                acc[mb][g] = v4f{0.f, 0.f, 0.f, 0.f};

        for (int ks = wave; ks < KS; ks += 4) {
            v8i a[4];
            int sa[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                a[g] = load_fp4_frag(wp[g] + ks * 64);
                sa[g] = wsp[g][ks * 4];
            }
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) {
                if (mb < nmb_act) {
                    const v8i b = load_fp8_frag(hp[mb] + ks * 128);
                    const int sb = hsp[mb][ks * 4];
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        acc[mb][g] = mfma_w4a8(a[g], b, acc[mb][g], sa[g], sb);
                }
            }
        }
        reduce_waves<NMB>(acc, red, nmb_act);

        if (wave < nmb_act) {
            const int mb = wave;
            const int rloc = mb * 16 + i16;
            if (rloc < nrows) {
                float *yr = y + (size_t)(row0 + rloc) * (size_t)H + n0 + 4 * kq;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float *r = red + (mb * 4 + g) * 4 * 64 + lane;
                    *reinterpret_cast<float4 *>(yr + 16 * g) =
                        float4{r[0], r[64], r[128], r[192]};
                }
            }
        }
        __syncthreads();
    }
}

int g_cu_count = 0;

template <typename KernelT>
int grid_for(KernelT kernel, long upper_items, size_t dyn_lds)
{
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, dyn_lds) !=
            hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    long g = (long)device_cu_count() * per_cu;
    if (upper_items < g)
        g = upper_items;
    return (int)(g < 1 ? 1 : g);
}

// Upper bound of the row chunks any dispatch result can produce.
long chunk_upper_bound(const moe_shape &s, int ch)
{
    const long rows = s.dispatch_mode == MOE_DISPATCH_FIXED_SLOT
                          ? (long)s.E_local * s.capacity
                          : (long)s.T * s.K;
    return rows / ch + s.E_local;
}

// Expected rows per local expert under uniform routing; the kernel family is
// chosen from this host-known figure only, never from device data.
double rows_per_expert(const moe_shape &s)
{
    return (double)s.T * s.K / (double)(s.E_total > 0 ? s.E_total : 1);
}

bool use_tiled_gemm1(const moe_shape &s) { return rows_per_expert(s) > 24.0; }

bool use_tiled_gemm2(const moe_shape &s) { return rows_per_expert(s) > 24.0 && s.H % 256 == 0; }

// Rows per chunk: enough for the expected rows of an expert, at most 64.
int pick_nmb(const moe_shape &s)
{
    const double per_expert = (double)s.T * s.K / (double)(s.E_total > 0 ? s.E_total : 1);
    if (per_expert <= 16.0)
        return 1;
    if (per_expert <= 32.0)
        return 2;
    return 4;
}

} // namespace

int device_cu_count()
{
    if (g_cu_count == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            n > 0)
            g_cu_count = n;
        else
            g_cu_count = 256;
    }
    return g_cu_count;
}

hipError_t launch_gemm1(const moe_shape &sh, const uint8_t *x, const uint8_t *xs,
                        const int32_t *counts, const int32_t *offsets, const int32_t *row_route,
                        const uint8_t *w13, const uint8_t *w13s, uint8_t *h, uint8_t *hs,
                        hipStream_t st)
{
    if (use_tiled_gemm1(sh))
        return launch_gemm1_tiled(sh, x, xs, counts, offsets, row_route, w13, w13s, h, hs, st);
    const Shape s = to_dev(sh);
    const int nmb = pick_nmb(sh);
    const long nt = sh.I / 32;
#define MOE_LAUNCH_G1(N)                                                                          \
    do {                                                                                          \
        auto k = gemm1_skinny_kernel<N>;                                                          \
        const size_t lds = (size_t)(64 + 16 * N) * (sh.H / 32 + 4);                               \
        const int grid = grid_for(k, chunk_upper_bound(sh, 16 * N) * nt, lds);                    \
        k<<<grid, kThreads, lds, st>>>(s, x, xs, counts, offsets, row_route, w13, w13s, h, hs);   \
    } while (0)
    if (nmb == 1)
        MOE_LAUNCH_G1(1);
    else if (nmb == 2)
        MOE_LAUNCH_G1(2);
    else
        MOE_LAUNCH_G1(4);
#undef MOE_LAUNCH_G1
    return hipGetLastError();
}

hipError_t launch_gemm2(const moe_shape &sh, const uint8_t *h, const uint8_t *hs,
                        const int32_t *counts, const int32_t *offsets, const uint8_t *w2,
                        const uint8_t *w2s, float *y, hipStream_t st)
{
    if (use_tiled_gemm2(sh))
        return launch_gemm2_tiled(sh, h, hs, counts, offsets, w2, w2s, y, st);
    const Shape s = to_dev(sh);
    const int nmb = pick_nmb(sh);
    const long nt = sh.H / 64;
#define MOE_LAUNCH_G2(N)                                                                          \
    do {                                                                                          \
        auto k = gemm2_skinny_kernel<N>;                                                          \
        const size_t lds = (size_t)(64 + 16 * N) * (sh.I / 32 + 4);                               \
        const int grid = grid_for(k, chunk_upper_bound(sh, 16 * N) * nt, lds);                    \
        k<<<grid, kThreads, lds, st>>>(s, h, hs, counts, offsets, w2, w2s, y);                    \
    } while (0)
    if (nmb == 1)
        MOE_LAUNCH_G2(1);
    else if (nmb == 2)
        MOE_LAUNCH_G2(2);
    else
        MOE_LAUNCH_G2(4);
#undef MOE_LAUNCH_G2
    return hipGetLastError();
}

} // namespace moe
