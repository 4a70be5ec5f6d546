// Wavefront helpers of the route dispatch, shared by the dispatch kernels
// and the persistent layer: grouping of lanes by key with ballots (stable
// ranks), the valid-row count, batched key loads, per-wavefront histograms,
// the stable scatter of one batch and the fixed-slot claims.
#pragma once

#include "moe_common.hpp"

namespace moe {

struct Match {
    int rank;                 // lanes below with the same key
    int count;                // lanes with the same key
    unsigned long long mask;  // those lanes
};

// Group the active lanes of the wavefront by key.
__device__ __forceinline__ Match wave_match(int key, bool active)
{
    Match m{0, 0, 0ull};
    const unsigned long long lt = __lanemask_lt();
    unsigned long long rem = __ballot(active);
    while (rem) {
        const int leader = __ffsll((long long)rem) - 1;
        const int k = __builtin_amdgcn_readlane(key, leader);
        const bool mine = active && key == k;
        const unsigned long long mk = __ballot(mine);
        if (mine) {
            m.rank = __popcll(mk & lt);
            m.count = __popcll(mk);
            m.mask = mk;
        }
        rem &= ~mk;
    }
    return m;
}

__device__ __forceinline__ int wave_sum(int v)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1)
        v += __shfl_xor(v, d);
    return v;
}

// Slots a wavefront reads per batch: the id loads of a batch are all in
// flight together, so a wavefront waits for memory once per 64 * P slots
// rather than once per 64.
constexpr int kBatch = 8;

// Slots of the tokens the call counts: rows t >= *valid are padding (their
// slots read as -1, no expert), the count clamped to [0, T]; all T rows when
// valid is null.  Read on the device, so a replayed graph follows the count
// the caller wrote for that replay ("feat(moe): route before the rows move;
// per-pass real row counts", Per-pass real row counts).
__device__ __forceinline__ long valid_slots(const Shape &s, const int32_t *valid)
{
    if (!valid)
        return (long)s.T * s.K;
    const int v = *valid;
    return (long)(v < 0 ? 0 : (v > s.T ? s.T : v)) * s.K;
}

// Local expert (route_local) of the slots base + 64 p + lane, p < P; -1 past
// e and past the valid slots nv.
template <int P>
__device__ __forceinline__ void load_keys(const Shape &s, const int32_t *__restrict__ ids,
                                          long base, long e, long nv, int (&ex)[P])
{
    const int lane = threadIdx.x & 63;
    const long lim = e < nv ? e : nv;
    int raw[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const long r = base + 64 * p + lane;
        raw[p] = r < lim ? ids[r] : -1;
    }
#pragma unroll
    for (int p = 0; p < P; ++p)
        ex[p] = route_local(s, raw[p]);
}

// Per-wavefront histogram of the slots [b, e) into hist_row (LDS); returns
// the wavefront's count of invalid ids (in every lane).
template <int P>
__device__ int wave_histogram(const Shape &s, const int32_t *__restrict__ ids, long b, long e,
                              long nv, int *hist_row)
{
    int invalid = 0;
    for (long base = b; base < e; base += 64 * P) {
        int ex[P];
        load_keys<P>(s, ids, base, e, nv, ex);
#pragma unroll
        for (int p = 0; p < P; ++p) {
            if (base + 64 * p >= e)
                break;
            if (ex[p] >= 0)
                atomicAdd(&hist_row[ex[p]], 1);
            invalid += ex[p] == -2;
        }
    }
    return wave_sum(invalid);
}

// Stable scatter of the slots base + 64 p + lane below e, whose keys ex[]
// were loaded by load_keys: base_row[ex] (LDS, this wavefront's own row) is
// the next row of expert ex for this wavefront.
template <int P>
__device__ __forceinline__ void scatter_keys(const int (&ex)[P], long base, long e, int *base_row,
                                             int32_t *__restrict__ row_route,
                                             int32_t *__restrict__ route_row)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        if (base + 64 * p >= e)
            break;
        const long r = base + 64 * p + lane;
        const Match m = wave_match(ex[p], ex[p] >= 0);
        int row = -1;
        if (ex[p] >= 0)
            row = base_row[ex[p]] + m.rank;
        // every lane has read its base before a leader moves it on
        __builtin_amdgcn_wave_barrier();
        if (ex[p] >= 0 && m.rank == 0)
            base_row[ex[p]] += m.count;
        __builtin_amdgcn_wave_barrier();
        if (r < e) {
            route_row[r] = row;
            if (row >= 0)
                row_route[row] = (int32_t)r;
        }
    }
}

// Claim one slot per kept route.  kPerLane (counters in LDS): every lane
// takes its own slot with an LDS atomic (the order of a segment is free in
// fixed-slot mode).  Otherwise (counters in global memory) the leader of each
// expert group adds the group's size to the expert's counter and hands out
// consecutive slots, one global atomic per expert and wavefront.
template <int P, bool kPerLane>
__device__ void claim_slots(const Shape &s, const int32_t *__restrict__ ids, long b, long e,
                            long nv, int32_t *cnt, int32_t *__restrict__ row_route,
                            int32_t *__restrict__ route_row, int &invalid, int &dropped)
{
    const int lane = threadIdx.x & 63;
    for (long base = b; base < e; base += 64 * P) {
        int exs[P];
        load_keys<P>(s, ids, base, e, nv, exs);
#pragma unroll
        for (int p = 0; p < P; ++p) {
            if (base + 64 * p >= e)
                break;
            const long r = base + 64 * p + lane;
            const int ex = exs[p];
            if (kPerLane) {
                int row = -1;
                if (ex >= 0) {
                    const int slot = atomicAdd(&cnt[ex], 1);
                    if (slot < s.capacity)
                        row = ex * s.capacity + slot;
                    else
                        ++dropped;
                }
                invalid += ex == -2;
                if (r < e) {
                    route_row[r] = row;
                    if (row >= 0)
                        row_route[row] = (int32_t)r;
                }
                continue;
            }
            const Match m = wave_match(ex, ex >= 0);
            int first = 0;
            if (ex >= 0 && m.rank == 0)
                first = atomicAdd(&cnt[ex], m.count);
            const int leader = ex >= 0 ? __ffsll((long long)m.mask) - 1 : lane;
            first = __shfl(first, leader);
            int row = -1;
            if (ex >= 0) {
                const int slot = first + m.rank;
                if (slot < s.capacity)
                    row = ex * s.capacity + slot;
                else
                    ++dropped;
            }
            invalid += ex == -2;
            if (r < e) {
                route_row[r] = row;
                if (row >= 0)
                    row_route[row] = (int32_t)r;
            }
        }
    }
}

} // namespace moe
