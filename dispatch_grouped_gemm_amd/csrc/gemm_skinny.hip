// Expert GEMMs without LDS tiles, for contractions shorter than four K steps
// of 128 (the LDS-tiled kernels take all others): the weights are streamed
// from HBM straight into scaled FP4 x FP8 MFMAs and every weight fragment is
// applied to all rows of a chunk (up to 16*NMB rows) while it is in
// registers.
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
// rounded to bf16 for the combine.
#include <cmath>

#include "moe_common.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
// Resident wavefronts per SIMD the skinny GEMM1 is compiled for (register
// budget 512 / kGemm1Waves per lane): three wavefronts with two K steps in
// flight each stream W13 faster than four with one (measured on the
// 7168 x 3072 decode shape: 183 against 199 us; one row block per chunk).
// GEMM2, whose items are a
// third as long, is faster with the plain loop at four wavefronts.
constexpr int kGemm1Waves = 3;

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

// LDS row stride of staged exponent rows of a contraction of length k:
// 16-byte aligned when the row (k/32 bytes) is a whole number of 16-byte
// chunks, with 16 bytes of padding so the K loop's byte reads of sixteen
// consecutive rows fall in different LDS banks; 4 bytes of padding else.
__host__ __device__ constexpr int exp_stride(int k)
{
    return (k / 32) % 16 == 0 ? k / 32 + 16 : k / 32 + 4;
}

// Copy the E8M0 exponent rows of one item into LDS (row stride `stride`
// bytes, `nbytes` used bytes per row, a multiple of 4): rows [0, nrows)
// come from src_row(r); the workgroup shares the copy, in 16-byte pieces
// when the rows allow (a quarter of the load instructions), else in dwords.
template <typename RowFn>
__device__ __forceinline__ void stage_exponents(uint8_t *dst, int stride, int nbytes, int nrows,
                                                RowFn src_row)
{
    if (nbytes % 16 == 0) {
        const int pieces = nbytes >> 4;
        for (int i = threadIdx.x; i < nrows * pieces; i += kThreads) {
            const int r = i / pieces, c = i - r * pieces;
            const uint4 v = reinterpret_cast<const uint4 *>(src_row(r))[c];
            *reinterpret_cast<uint4 *>(dst + r * stride + 16 * c) = v;
        }
        return;
    }
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

// Operands of one K step (128 K values) of an item: four 16-row FP4 weight
// fragments and one 16-row FP8 activation fragment per row block, with their
// exponents.
template <int NMB>
struct KStep {
    v8i a[4];
    int sa[4];
    v8i b[NMB];
    int sb[NMB];
};

// Where this lane's operands of an item are at K step 0: weight codes at
// wbase + woff[g] and activation codes at xbase + xoff[mb] (workgroup-uniform
// bases, 32-bit lane offsets), exponents in LDS at wsp[g] / xsp[mb].
template <int NMB>
struct KPtrs {
    const uint8_t *wbase, *xbase;
    uint32_t woff[4], xoff[NMB];
    const uint8_t *wsp[4], *xsp[NMB];
};

template <int NMB>
__device__ __forceinline__ void fetch_step(KStep<NMB> &f, const KPtrs<NMB> &p, int ks)
{
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        f.a[g] = load_fp4_frag(p.wbase + (p.woff[g] + (uint32_t)ks * 64u));
        f.sa[g] = p.wsp[g][ks * 4];
    }
    // every row block is loaded (offsets of missing rows repeat the last
    // row), so the loads of a step are unconditional
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
        f.b[mb] = load_fp8_frag(p.xbase + (p.xoff[mb] + (uint32_t)ks * 128u));
        f.sb[mb] = p.xsp[mb][ks * 4];
    }
}

template <int NMB>
__device__ __forceinline__ void mma_step(v4f (&acc)[NMB][4], const KStep<NMB> &f, int nmb_act)
{
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
        if (mb < nmb_act) {
#pragma unroll
            for (int g = 0; g < 4; ++g)
                acc[mb][g] = mfma_w4a8(f.a[g], f.b[mb], acc[mb][g], f.sa[g], f.sb[mb]);
        }
    }
}

// This wavefront's K steps ks = wave, wave + 4, ... < KS.  With kPrefetch
// the loads of the next step are in flight while the current step's MFMAs
// run (twice the bytes in flight per wavefront, at the price of the
// registers of a second step).
template <bool kPrefetch, int NMB>
__device__ __forceinline__ void k_loop(v4f (&acc)[NMB][4], const KPtrs<NMB> &p, int KS, int wave,
                                       int nmb_act)
{
    if (!kPrefetch) {
        for (int ks = wave; ks < KS; ks += 4) {
            KStep<NMB> f;
            fetch_step(f, p, ks);
            mma_step(acc, f, nmb_act);
        }
        return;
    }
    const int n = wave < KS ? (KS - wave + 3) / 4 : 0;
    if (n == 0)
        return;
    KStep<NMB> f0, f1;
    fetch_step(f0, p, wave);
    int j = 0;
    for (; j + 2 < n; j += 2) {
        fetch_step(f1, p, wave + 4 * (j + 1));
        mma_step(acc, f0, nmb_act);
        fetch_step(f0, p, wave + 4 * (j + 2));
        mma_step(acc, f1, nmb_act);
    }
    if (j + 1 < n) {
        fetch_step(f1, p, wave + 4 * (j + 1));
        mma_step(acc, f0, nmb_act);
        mma_step(acc, f1, nmb_act);
    } else {
        mma_step(acc, f0, nmb_act);
    }
}

// Pointers of one layer call, shared by the item bodies below.
struct LayerPtrs {
    const uint8_t *x, *xs;
    const int32_t *counts, *offsets, *row_route;
    const uint8_t *w13, *w13s, *w2, *w2s;
    uint8_t *h, *hs;
    uint16_t *y;           // bf16 rows, or
    uint8_t *y8, *y8s;     // MX FP8 rows (y null)
};

// Where an item's rows are: expert e, rows [row0, row0 + nrows).
struct Chunk {
    int e, row0, nrows;
};

__device__ __forceinline__ Chunk chunk_of(const Shape &s, const int *prefix,
                                          const int32_t *__restrict__ counts,
                                          const int32_t *__restrict__ offsets, int ch, int q)
{
    Chunk c;
    c.e = chunk_expert(prefix, s.E_local, q);
    const int k = q - prefix[c.e];
    c.row0 = offsets[c.e] + k * ch;
    c.nrows = min(ch, used_rows(s, counts[c.e]) - k * ch);
    return c;
}

// GEMM1 + SwiGLU + requant of 32 intermediate columns j0 = 32 nt .. of one
// row chunk.  LDS: tok[16 NMB], red[NMB*4*4*64], exps[(64 + 16 NMB) * es].
template <int NMB>
__device__ __forceinline__ void gemm1_item(const Shape &s, const LayerPtrs &p, const Chunk &c,
                                           int nt, int *tok, float *red, uint8_t *exps)
{
    constexpr int CH = 16 * NMB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i16 = lane & 15, kq = lane >> 4;
    const int H = s.H, I = s.I, KS = H / 128;
    const int es = exp_stride(H);
    uint8_t *wexp = exps, *xexp = exps + 64 * es;
    const int e = c.e, row0 = c.row0, nrows = c.nrows;
    const int nmb_act = (nrows + 15) >> 4;
    const int j0 = nt * 32;
    if (tid < CH)
        tok[tid] = tid < nrows ? p.row_route[row0 + tid] / s.K : 0;
    // W13 rows of the tile: r in [0, 64) is gate/up group r/16, row r%16
    stage_exponents(wexp, es, H / 32, 64, [&](int r) {
        const int g = r >> 4;
        const size_t wrow = (size_t)e * 2 * I + (g >= 2 ? I : 0) + j0 + 16 * (g & 1) + (r & 15);
        return p.w13s + wrow * (size_t)(H / 32);
    });
    stage_exponents(xexp, es, H / 32, nrows, [&](int r) {
        return p.xs + (size_t)(p.row_route[row0 + r] / s.K) * (size_t)(H / 32);
    });
    __syncthreads();

    KPtrs<NMB> kp;
    kp.wbase = p.w13 + ((size_t)e * 2 * I + j0) * (size_t)(H / 2);
    kp.xbase = p.x;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const uint32_t r = (g >= 2 ? I : 0) + 16 * (g & 1) + i16;
        kp.woff[g] = r * (uint32_t)(H / 2) + kq * 16;
        kp.wsp[g] = wexp + (g * 16 + i16) * es + kq;
    }
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
        const int rloc = min(mb * 16 + i16, nrows - 1);
        kp.xoff[mb] = (uint32_t)tok[rloc] * (uint32_t)H + kq * 16;
        kp.xsp[mb] = xexp + rloc * es + kq;
    }

    v4f acc[NMB][4];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            acc[mb][g] = v4f{0.f, 0.f, 0.f, 0.f};
    k_loop<NMB == 1, NMB>(acc, kp, KS, wave, nmb_act);
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
        const uint32_t pk[2] = {mx8_pack4(hv[0], hv[1], hv[2], hv[3], E, amax),
                                mx8_pack4(hv[4], hv[5], hv[6], hv[7], E, amax)};
        if (rloc < nrows) {
            const size_t row = (size_t)(row0 + rloc);
            uint8_t *hr = p.h + row * (size_t)I + j0 + 4 * kq;
            *reinterpret_cast<uint32_t *>(hr) = pk[0];
            *reinterpret_cast<uint32_t *>(hr + 16) = pk[1];
            if (kq == 0)
                p.hs[row * (size_t)(I / 32) + nt] = (uint8_t)(E + 127);
        }
    }
    __syncthreads();
}

// GEMM2 of 64 output columns n0 = 64 nt .. of one row chunk (y in bf16).
// LDS: red[NMB*4*4*64], exps[(64 + 16 NMB) * exp_stride(I)].
template <int NMB>
__device__ __forceinline__ void gemm2_item(const Shape &s, const LayerPtrs &p, const Chunk &c,
                                           int nt, float *red, uint8_t *exps)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i16 = lane & 15, kq = lane >> 4;
    const int H = s.H, I = s.I, KS = I / 128;
    const int es = exp_stride(I);
    uint8_t *wexp = exps, *hexp = exps + 64 * es;
    const int e = c.e, row0 = c.row0, nrows = c.nrows;
    const int nmb_act = (nrows + 15) >> 4;
    const int n0 = nt * 64;
    stage_exponents(wexp, es, I / 32, 64, [&](int r) {
        return p.w2s + ((size_t)e * H + n0 + r) * (size_t)(I / 32);
    });
    stage_exponents(hexp, es, I / 32, nrows, [&](int r) {
        return p.hs + (size_t)(row0 + r) * (size_t)(I / 32);
    });
    __syncthreads();

    KPtrs<NMB> kp;
    kp.wbase = p.w2 + ((size_t)e * H + n0) * (size_t)(I / 2);
    kp.xbase = p.h + (size_t)row0 * (size_t)I;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        kp.woff[g] = (uint32_t)(16 * g + i16) * (uint32_t)(I / 2) + kq * 16;
        kp.wsp[g] = wexp + (16 * g + i16) * es + kq;
    }
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
        const int rloc = min(mb * 16 + i16, nrows - 1);
        kp.xoff[mb] = (uint32_t)rloc * (uint32_t)I + kq * 16;
        kp.xsp[mb] = hexp + rloc * es + kq;
    }

    v4f acc[NMB][4];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            acc[mb][g] = v4f{0.f, 0.f, 0.f, 0.f};
    k_loop<false, NMB>(acc, kp, KS, wave, nmb_act);
    reduce_waves<NMB>(acc, red, nmb_act);

    if (wave < nmb_act && p.y8) {
        // MX FP8 rows: lane (i16, kq) holds columns n0 + 16 g + 4 kq + v;
        // the 32-column block b is groups 2b and 2b + 1 of the four lanes kq
        // of a route (every lane takes part in the exchanges; rows past
        // nrows repeat the last row and are not stored)
        const int mb = wave;
        const int rloc = mb * 16 + i16;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            float v[2][4];
            float amax = 0.0f;
#pragma unroll
            for (int g = 0; g < 2; ++g)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    v[g][q] = red[(mb * 4 + 2 * blk + g) * 4 * 64 + lane + 64 * q];
                    amax = fmaxf(amax, fabsf(v[g][q]));
                }
            amax = fmaxf(amax, __shfl_xor(amax, 16));
            amax = fmaxf(amax, __shfl_xor(amax, 32));
            const int E = mx8_block_exponent(amax);
            if (rloc < nrows) {
                uint8_t *yr = p.y8 + (size_t)(row0 + rloc) * (size_t)H + n0 + 32 * blk + 4 * kq;
#pragma unroll
                for (int g = 0; g < 2; ++g)
                    *reinterpret_cast<uint32_t *>(yr + 16 * g) =
                        mx8_pack4(v[g][0], v[g][1], v[g][2], v[g][3], E, amax);
                if (kq == 0)
                    p.y8s[(size_t)(row0 + rloc) * (size_t)(H / 32) + (n0 + 32 * blk) / 32] =
                        (uint8_t)(E + 127);
            }
        }
    } else if (wave < nmb_act) {
        const int mb = wave;
        const int rloc = mb * 16 + i16;
        if (rloc < nrows) {
            uint16_t *yr = p.y + (size_t)(row0 + rloc) * (size_t)H + n0 + 4 * kq;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float *r = red + (mb * 4 + g) * 4 * 64 + lane;
                *reinterpret_cast<uint2 *>(yr + 16 * g) =
                    uint2{f32_to_bf16(r[0]) | (f32_to_bf16(r[64]) << 16),
                          f32_to_bf16(r[128]) | (f32_to_bf16(r[192]) << 16)};
            }
        }
    }
    __syncthreads();
}

template <int NMB>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(NMB == 4 ? 2 : kGemm1Waves)))
gemm1_skinny_kernel(Shape s, LayerPtrs p)
{
    constexpr int CH = 16 * NMB;
    __shared__ int prefix[kMaxLocalExperts + 1];
    __shared__ int tok[CH];
    __shared__ float red[NMB * 4 * 4 * 64];
    extern __shared__ __align__(16) uint8_t exps[];
    const int nchunks = plan_chunks(s, p.counts, CH, prefix);
    const int NT = s.I / 32;
    const long items = (long)nchunks * NT;
    for (long item = blockIdx.x; item < items; item += gridDim.x) {
        const int q = (int)(item / NT), nt = (int)(item - (long)q * NT);
        gemm1_item<NMB>(s, p, chunk_of(s, prefix, p.counts, p.offsets, CH, q), nt, tok, red, exps);
    }
}

template <int NMB>
__global__ void __launch_bounds__(kThreads)
gemm2_skinny_kernel(Shape s, LayerPtrs p)
{
    constexpr int CH = 16 * NMB;
    __shared__ int prefix[kMaxLocalExperts + 1];
    __shared__ float red[NMB * 4 * 4 * 64];
    extern __shared__ __align__(16) uint8_t exps[];
    const int nchunks = plan_chunks(s, p.counts, CH, prefix);
    const int NT = s.H / 64;
    const long items = (long)nchunks * NT;
    for (long item = blockIdx.x; item < items; item += gridDim.x) {
        const int q = (int)(item / NT), nt = (int)(item - (long)q * NT);
        gemm2_item<NMB>(s, p, chunk_of(s, prefix, p.counts, p.offsets, CH, q), nt, red, exps);
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

// Rows per chunk: enough for nearly every expert's rows in one pass over its
// weights (mean + 3 standard deviations of the binomial route count, + 1),
// at most 64; a second chunk of an expert streams its weights again.
int pick_nmb(const moe_shape &s)
{
    const double mu = rows_per_expert(s);
    const double need = mu + 3.0 * std::sqrt(mu) + 1.0;
    if (need <= 16.0)
        return 1;
    if (need <= 32.0)
        return 2;
    return 4;
}

} // namespace

// The tiled kernels need a contraction of at least four K steps (512); where
// they have it they are faster at every row count (measured on the V4 and
// Flash shapes from 2.7 to 1000 rows per expert: their 64-row tiles read
// each weight row 128 contiguous bytes at a time, which HBM serves faster
// than the 64-byte fragments these kernels stream), so the kernels here
// serve the shorter contractions.
bool use_tiled_gemm1(const moe_shape &s) { return s.H >= 512; }

bool use_tiled_gemm2(const moe_shape &s) { return s.I >= 512; }

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
    LayerPtrs p{};
    p.x = x;
    p.xs = xs;
    p.counts = counts;
    p.offsets = offsets;
    p.row_route = row_route;
    p.w13 = w13;
    p.w13s = w13s;
    p.h = h;
    p.hs = hs;
    const int nmb = pick_nmb(sh);
    const long nt = sh.I / 32;
#define MOE_LAUNCH_G1(N)                                                                          \
    do {                                                                                          \
        auto k = gemm1_skinny_kernel<N>;                                                          \
        const size_t lds = (size_t)(64 + 16 * N) * exp_stride(sh.H);                              \
        const int grid = grid_for(k, chunk_upper_bound(sh, 16 * N) * nt, lds);                    \
        k<<<grid, kThreads, lds, st>>>(s, p);                                                     \
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
                        const uint8_t *w2s, const YRows &y, hipStream_t st)
{
    if (use_tiled_gemm2(sh))
        return launch_gemm2_tiled(sh, h, hs, counts, offsets, w2, w2s, y, st);
    const Shape s = to_dev(sh);
    LayerPtrs p{};
    p.h = const_cast<uint8_t *>(h);
    p.hs = const_cast<uint8_t *>(hs);
    p.counts = counts;
    p.offsets = offsets;
    p.w2 = w2;
    p.w2s = w2s;
    p.y = y.bf16;
    p.y8 = y.codes;
    p.y8s = y.scales;
    const int nmb = pick_nmb(sh);
    const long nt = sh.H / 64;
#define MOE_LAUNCH_G2(N)                                                                          \
    do {                                                                                          \
        auto k = gemm2_skinny_kernel<N>;                                                          \
        const size_t lds = (size_t)(64 + 16 * N) * exp_stride(sh.I);                              \
        const int grid = grid_for(k, chunk_upper_bound(sh, 16 * N) * nt, lds);                    \
        k<<<grid, kThreads, lds, st>>>(s, p);                                                     \
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
