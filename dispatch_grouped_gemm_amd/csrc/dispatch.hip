// Route dispatch for gfx950: compact (histogram -> exclusive scan -> stable
// scatter) and fixed-slot (atomic claim of a slot in a per-expert segment of
// fixed capacity, no prepare pass).
//
// Both modes group the same routes: a slot (t, k) is kept when its id names
// one of this GPU's experts.  Compact packs the kept routes of each expert
// contiguously in ascending route order r = t*K + k; fixed-slot gives each
// route the next free slot of its expert, in whatever order the claims land.
//
// Stable ranks inside a wavefront come from ballots: the lanes that hold the
// same expert form a 64-bit mask, a lane's rank is the popcount of the mask
// below it, and one leader per expert does the bookkeeping for the group.
#include "dispatch_dev.hpp"

namespace moe {

namespace {

constexpr int kThreads = 1024; // 16 wavefronts
constexpr int kWaves = kThreads / 64;
constexpr int kSlotsPerWaveLarge = 128;
constexpr int kLargeBatch = kSlotsPerWaveLarge / 64;
constexpr int kSlotsPerBlockLarge = kWaves * kSlotsPerWaveLarge;
// Dispatches of at most this many slots run in one workgroup (measured, back
// to back: compact 6144 slots 10.3 us in one workgroup, 7.7 us over three in
// two launches; fixed-slot 24,576 slots 8.6 us in one workgroup, 10.9 us as
// reset + claim).  Past one workgroup's 2048 slots the compact passes run
// workgroups in parallel; a fixed-slot claim is one LDS atomic per route.
constexpr long kCompactOneWgSlots = kSlotsPerBlockLarge;
constexpr long kFixedOneWgSlots = 32768;

// Stable scatter of the slots [b, e), keys loaded P batches at a time.
template <int P>
__device__ void wave_scatter(const Shape &s, const int32_t *__restrict__ ids, long b, long e,
                             long nv, int *base_row, int32_t *__restrict__ row_route,
                             int32_t *__restrict__ route_row)
{
    for (long base = b; base < e; base += 64 * P) {
        int ex[P];
        load_keys<P>(s, ids, base, e, nv, ex);
        scatter_keys<P>(ex, base, e, base_row, row_route, route_row);
    }
}

// Exclusive scan of v over the 1024 threads; returns the exclusive prefix
// and writes the total to *total (every thread).
__device__ int block_exclusive_scan(int v, int *total)
{
    __shared__ int wsum[kWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int inc = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(inc, d);
        if (lane >= d)
            inc += o;
    }
    if (lane == 63)
        wsum[wave] = inc;
    __syncthreads();
    int base = 0, all = 0;
    for (int w = 0; w < kWaves; ++w) {
        const int x = wsum[w];
        if (w < wave)
            base += x;
        all += x;
    }
    __syncthreads();
    *total = all;
    return base + inc - v;
}

// ---- compact, one workgroup ------------------------------------------------

__global__ void __launch_bounds__(kThreads)
compact_small_kernel(Shape s, const int32_t *__restrict__ ids, int32_t *__restrict__ counts,
                     int32_t *__restrict__ offsets, int32_t *__restrict__ row_route,
                     int32_t *__restrict__ route_row, int32_t *__restrict__ status,
                     int32_t *__restrict__ zero, int nzero, QuantJob quant,
                     const int32_t *__restrict__ valid)
{
    // workgroups past the first quantise the activation rows
    if (blockIdx.x > 0) {
        quant_mx8_part(quant, (long)(blockIdx.x - 1) * kThreads + threadIdx.x,
                       (long)(gridDim.x - 1) * kThreads);
        return;
    }
    for (int i = threadIdx.x; i < nzero; i += kThreads)
        zero[i] = 0;
    const long nv = valid_slots(s, valid);
    extern __shared__ int hist[]; // [kWaves][E_local]
    __shared__ int invalid_total;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int E = s.E_local;
    const long n = (long)s.T * s.K;
    const long per_wave = (n + kWaves - 1) / kWaves;
    const long b = min(n, per_wave * wave), e = min(n, b + per_wave);

    for (int i = tid; i < kWaves * E; i += kThreads)
        hist[i] = 0;
    if (tid == 0)
        invalid_total = 0;
    __syncthreads();
    const int inv = wave_histogram<kBatch>(s, ids, b, e, nv, hist + wave * E);
    if (lane == 0 && inv)
        atomicAdd(&invalid_total, inv);
    __syncthreads();

    // totals per expert, exclusive scan over experts
    int cnt = 0;
    if (tid < E)
        for (int w = 0; w < kWaves; ++w)
            cnt += hist[w * E + tid];
    int total;
    const int off = block_exclusive_scan(tid < E ? cnt : 0, &total);
    if (tid < E) {
        counts[tid] = cnt;
        offsets[tid] = off;
        int run = off; // per-wavefront bases, wavefronts in slot order
        for (int w = 0; w < kWaves; ++w) {
            const int c = hist[w * E + tid];
            hist[w * E + tid] = run;
            run += c;
        }
    }
    if (tid == 0) {
        offsets[E] = total;
        status[0] = invalid_total;
        status[1] = status[2] = status[3] = 0;
    }
    __syncthreads();
    wave_scatter<kBatch>(s, ids, b, e, nv, hist + wave * E, row_route, route_row);
}

// ---- compact, many workgroups ------------------------------------------------

// Pass 1: per-workgroup histograms; scratch[blk][E] holds the invalid count.
__global__ void __launch_bounds__(kThreads)
compact_hist_kernel(Shape s, const int32_t *__restrict__ ids, int32_t *__restrict__ scratch,
                    const int32_t *__restrict__ valid)
{
    const long nv = valid_slots(s, valid);
    extern __shared__ int hist[]; // [E_local]
    __shared__ int invalid_total;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int E = s.E_local;
    const long n = (long)s.T * s.K;
    for (int i = tid; i < E; i += kThreads)
        hist[i] = 0;
    if (tid == 0)
        invalid_total = 0;
    __syncthreads();
    const long b = min(n, (long)blockIdx.x * kSlotsPerBlockLarge + (long)wave * kSlotsPerWaveLarge);
    const long e = min(n, b + kSlotsPerWaveLarge);
    // wavefronts share the workgroup histogram: add with LDS atomics
    int inv = 0;
    for (long base = b; base < e; base += 64 * kLargeBatch) {
        int ex[kLargeBatch];
        load_keys<kLargeBatch>(s, ids, base, e, nv, ex);
#pragma unroll
        for (int p = 0; p < kLargeBatch; ++p) {
            if (ex[p] >= 0)
                atomicAdd(&hist[ex[p]], 1);
            inv += ex[p] == -2;
        }
    }
    inv = wave_sum(inv);
    if (lane == 0 && inv)
        atomicAdd(&invalid_total, inv);
    __syncthreads();
    int32_t *row = scratch + (size_t)blockIdx.x * (E + 1);
    for (int i = tid; i < E; i += kThreads)
        row[i] = hist[i];
    if (tid == 0)
        row[E] = invalid_total;
}

// Pass 2: the stable scatter of each workgroup's slots.  A workgroup sums the
// pass-1 table itself: over the workgroups before it (its first row within
// each expert's segment) and over all of them (the segment sizes, scanned
// over the experts into the offsets); the first workgroup also writes the
// counts, offsets and status.  Each wavefront loads its keys once.
__global__ void __launch_bounds__(kThreads)
compact_scatter_kernel(Shape s, int nblk, const int32_t *__restrict__ ids,
                       const int32_t *__restrict__ scratch, int32_t *__restrict__ counts,
                       int32_t *__restrict__ offsets, int32_t *__restrict__ status,
                       int32_t *__restrict__ row_route, int32_t *__restrict__ route_row,
                       const int32_t *__restrict__ valid)
{
    const long nv = valid_slots(s, valid);
    // [kWaves][E] histograms, then [kWaves][E+1] partial sums before / all
    extern __shared__ int lds[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int E = s.E_local, E1 = E + 1;
    int *hist = lds;
    int *part_before = hist + kWaves * E;
    int *part_all = part_before + kWaves * E1;
    const long n = (long)s.T * s.K;
    const long b = min(n, (long)blockIdx.x * kSlotsPerBlockLarge + (long)wave * kSlotsPerWaveLarge);
    const long e = min(n, b + kSlotsPerWaveLarge);
    int ex[kLargeBatch];
    load_keys<kLargeBatch>(s, ids, b, e, nv, ex);
    // wavefront w sums the rows of workgroups w, w + 16, ... of the table
    for (int c = lane; c < E1; c += 64) {
        int before = 0, all = 0;
#pragma unroll 4
        for (int w = wave; w < nblk; w += kWaves) {
            const int v = scratch[(size_t)w * E1 + c];
            all += v;
            before += w < (int)blockIdx.x ? v : 0;
        }
        part_before[wave * E1 + c] = before;
        part_all[wave * E1 + c] = all;
    }
    for (int i = tid; i < kWaves * E; i += kThreads)
        hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int p = 0; p < kLargeBatch; ++p)
        if (ex[p] >= 0)
            atomicAdd(&hist[wave * E + ex[p]], 1);
    int before = 0, all = 0;
    if (tid < E1)
        for (int w = 0; w < kWaves; ++w) {
            before += part_before[w * E1 + tid];
            all += part_all[w * E1 + tid];
        }
    int total;
    const int off = block_exclusive_scan(tid < E ? all : 0, &total);
    // block_exclusive_scan ends with a barrier: the histograms are complete
    if (tid < E) {
        int run = off + before; // per-wavefront bases, wavefronts in slot order
        for (int w = 0; w < kWaves; ++w) {
            const int c = hist[w * E + tid];
            hist[w * E + tid] = run;
            run += c;
        }
    }
    if (blockIdx.x == 0) {
        if (tid < E) {
            counts[tid] = all;
            offsets[tid] = off;
        }
        if (tid == E) {
            offsets[E] = total;
            status[0] = all; // column E holds the invalid ids
            status[1] = status[2] = status[3] = 0;
        }
    }
    __syncthreads();
    scatter_keys<kLargeBatch>(ex, b, e, hist + wave * E, row_route, route_row);
}

// ---- fixed-slot ----------------------------------------------------------------

__global__ void __launch_bounds__(kThreads)
fixed_small_kernel(Shape s, const int32_t *__restrict__ ids, int32_t *__restrict__ counts,
                   int32_t *__restrict__ offsets, int32_t *__restrict__ row_route,
                   int32_t *__restrict__ route_row, int32_t *__restrict__ status,
                   int32_t *__restrict__ zero, int nzero, QuantJob quant,
                   const int32_t *__restrict__ valid)
{
    // workgroups past the first quantise the activation rows
    if (blockIdx.x > 0) {
        quant_mx8_part(quant, (long)(blockIdx.x - 1) * kThreads + threadIdx.x,
                       (long)(gridDim.x - 1) * kThreads);
        return;
    }
    for (int i = threadIdx.x; i < nzero; i += kThreads)
        zero[i] = 0;
    extern __shared__ int cnt[]; // [E_local]
    __shared__ int inv_total, drop_total;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int E = s.E_local;
    const long n = (long)s.T * s.K;
    for (int i = tid; i < E; i += kThreads)
        cnt[i] = 0;
    if (tid == 0)
        inv_total = drop_total = 0;
    __syncthreads();
    const long per_wave = (n + kWaves - 1) / kWaves;
    const long b = min(n, per_wave * wave), e = min(n, b + per_wave);
    int invalid = 0, dropped = 0;
    claim_slots<kBatch, true>(s, ids, b, e, valid_slots(s, valid), cnt, row_route, route_row,
                              invalid, dropped);
    invalid = wave_sum(invalid);
    dropped = wave_sum(dropped);
    if (lane == 0) {
        if (invalid)
            atomicAdd(&inv_total, invalid);
        if (dropped)
            atomicAdd(&drop_total, dropped);
    }
    __syncthreads();
    for (int i = tid; i <= E; i += kThreads) {
        if (i < E)
            counts[i] = cnt[i];
        offsets[i] = i * s.capacity;
    }
    if (tid == 0) {
        status[0] = inv_total;
        status[1] = drop_total;
        status[2] = status[3] = 0;
    }
}

__global__ void __launch_bounds__(256)
fixed_reset_kernel(Shape s, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                   int32_t *__restrict__ status)
{
    for (int i = blockIdx.x * 256 + threadIdx.x; i <= s.E_local; i += gridDim.x * 256) {
        if (i < s.E_local)
            counts[i] = 0;
        offsets[i] = i * s.capacity;
    }
    if (blockIdx.x == 0 && threadIdx.x < 4)
        status[threadIdx.x] = 0;
}

__global__ void __launch_bounds__(kThreads)
fixed_claim_kernel(Shape s, const int32_t *__restrict__ ids, int32_t *__restrict__ counts,
                   int32_t *__restrict__ row_route, int32_t *__restrict__ route_row,
                   int32_t *__restrict__ status, const int32_t *__restrict__ valid)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long n = (long)s.T * s.K;
    const long b = min(n, (long)blockIdx.x * kSlotsPerBlockLarge + (long)wave * kSlotsPerWaveLarge);
    const long e = min(n, b + kSlotsPerWaveLarge);
    int invalid = 0, dropped = 0;
    claim_slots<kLargeBatch, false>(s, ids, b, e, valid_slots(s, valid), counts, row_route,
                                    route_row, invalid, dropped);
    invalid = wave_sum(invalid);
    dropped = wave_sum(dropped);
    if (lane == 0) {
        if (invalid)
            atomicAdd(&status[0], invalid);
        if (dropped)
            atomicAdd(&status[1], dropped);
    }
}

long num_slots(const moe_shape &s) { return (long)s.T * s.K; }

int large_blocks(const moe_shape &s)
{
    return (int)((num_slots(s) + kSlotsPerBlockLarge - 1) / kSlotsPerBlockLarge);
}

} // namespace

bool dispatch_is_single_block(const moe_shape &s)
{
    return num_slots(s) <= (s.dispatch_mode == MOE_DISPATCH_COMPACT ? kCompactOneWgSlots
                                                                    : kFixedOneWgSlots);
}

size_t dispatch_scratch_bytes(const moe_shape &s)
{
    if (s.dispatch_mode != MOE_DISPATCH_COMPACT || dispatch_is_single_block(s))
        return 0;
    return (size_t)large_blocks(s) * (size_t)(s.E_local + 1) * sizeof(int32_t);
}

hipError_t launch_dispatch(const moe_shape &sh, const int32_t *ids, int32_t *counts,
                           int32_t *offsets, int32_t *row_route, int32_t *route_row,
                           int32_t *status, void *scratch, hipStream_t st, int32_t *zero,
                           int nzero, const QuantJob *quant, const int32_t *valid)
{
    const bool one = dispatch_is_single_block(sh);
    if (nzero > 0 && !one)
        return hipErrorInvalidValue;
    const Shape s = to_dev(sh);
    const size_t E = (size_t)sh.E_local;
    // one-workgroup paths: the quant rides in extra workgroups of the launch
    const QuantJob qj = quant ? *quant : QuantJob{nullptr, nullptr, nullptr, 0};
    const int grid = 1 + (qj.blocks > 0 ? quant_blocks(qj, kThreads) : 0);
    if (!one && qj.blocks > 0) {
        const hipError_t e = launch_quant_mxfp8(qj, st);
        if (e != hipSuccess)
            return e;
    }
    if (sh.dispatch_mode == MOE_DISPATCH_COMPACT) {
        if (one) {
            compact_small_kernel<<<grid, kThreads, kWaves * E * sizeof(int), st>>>(
                s, ids, counts, offsets, row_route, route_row, status, zero, nzero, qj, valid);
            return hipGetLastError();
        }
        const int nblk = large_blocks(sh);
        int32_t *blk = static_cast<int32_t *>(scratch);
        compact_hist_kernel<<<nblk, kThreads, E * sizeof(int), st>>>(s, ids, blk, valid);
        const size_t lds = (kWaves * E + 2 * kWaves * (E + 1)) * sizeof(int);
        compact_scatter_kernel<<<nblk, kThreads, lds, st>>>(s, nblk, ids, blk, counts, offsets,
                                                           status, row_route, route_row, valid);
        return hipGetLastError();
    }
    if (one) {
        fixed_small_kernel<<<grid, kThreads, E * sizeof(int), st>>>(
            s, ids, counts, offsets, row_route, route_row, status, zero, nzero, qj, valid);
        return hipGetLastError();
    }
    fixed_reset_kernel<<<(int)((E + 256) / 256), 256, 0, st>>>(s, counts, offsets, status);
    fixed_claim_kernel<<<large_blocks(sh), kThreads, 0, st>>>(s, ids, counts, row_route, route_row,
                                                              status, valid);
    return hipGetLastError();
}

} // namespace moe
