// Combine: each token's kept routes (bf16 or MX FP8 y rows), weighted by their routing
// weights and summed in float32 in ascending k, rounded to bf16 once.  Slots whose
// route_row is -1 (pad, foreign, invalid or dropped) contribute nothing, so
// the result does not depend on their weights.  No atomics: a thread owns 8
// output columns of one token, which makes the sum order fixed; it loads the
// token's slots, then all its kept routes' y pieces at once.
#include "moe_common.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;

// A row of a multiple of 64 * kPair pieces (H a multiple of 1024): lane l of
// a wavefront takes pieces p + l and p + l + 64 of one token (each load
// instruction still reads 1 KiB of contiguous y), so each lane keeps two
// pieces of every kept route in flight; the sums are combine_cols' (the
// same bits).
constexpr int kPair = 2;

__global__ void __launch_bounds__(kThreads)
combine_pair_kernel(Shape s, const float *__restrict__ tw, const int32_t *__restrict__ route_row,
                    const uint16_t *__restrict__ y, uint16_t *__restrict__ out)
{
#pragma clang fp contract(off)
    const int pieces = s.H / kCombineVec;
    const long wid = ((long)blockIdx.x * kThreads + threadIdx.x) >> 6;   // wavefront
    const int lane = threadIdx.x & 63;
    const long groups = (long)s.T * (pieces / (64 * kPair));
    if (wid >= groups)
        return;
    const int per_row = pieces / (64 * kPair);
    const int t = __builtin_amdgcn_readfirstlane((int)(wid / per_row));
    const int p0 = (int)(wid - (long)t * per_row) * 64 * kPair + lane;
    constexpr int kMaxK = 8;
    const size_t slot0 = (size_t)t * s.K;
    int rows[kMaxK];
    float w[kMaxK];
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
        rows[k] = k < s.K ? route_row[slot0 + k] : -1;
        w[k] = k < s.K ? tw[slot0 + k] : 0.0f;
    }
    uint4 q[kMaxK][kPair];
#pragma unroll
    for (int k = 0; k < kMaxK; ++k)
        if (rows[k] >= 0)
#pragma unroll
            for (int j = 0; j < kPair; ++j)
                q[k][j] = *reinterpret_cast<const uint4 *>(y + (size_t)rows[k] * s.H +
                                                           (size_t)(p0 + 64 * j) * kCombineVec);
    float acc[kPair][kCombineVec];
#pragma unroll
    for (int j = 0; j < kPair; ++j)
#pragma unroll
        for (int i = 0; i < kCombineVec; ++i)
            acc[j][i] = 0.0f;
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
        if (rows[k] < 0)
            continue;
#pragma unroll
        for (int j = 0; j < kPair; ++j) {
            const uint32_t wd[4] = {q[k][j].x, q[k][j].y, q[k][j].z, q[k][j].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float lo = __uint_as_float(wd[i] << 16);
                const float hi = __uint_as_float(wd[i] & 0xffff0000u);
                const float pl = w[k] * lo, ph = w[k] * hi;
                acc[j][2 * i] = acc[j][2 * i] + pl;
                acc[j][2 * i + 1] = acc[j][2 * i + 1] + ph;
            }
        }
    }
    typedef unsigned int u4v __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int j = 0; j < kPair; ++j) {
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = f32_to_bf16(acc[j][2 * i]) | (f32_to_bf16(acc[j][2 * i + 1]) << 16);
        __builtin_nontemporal_store(
            u4v{o[0], o[1], o[2], o[3]},
            reinterpret_cast<u4v *>(out + (size_t)t * s.H + (size_t)(p0 + 64 * j) * kCombineVec));
    }
}

__global__ void __launch_bounds__(kThreads)
combine_kernel(Shape s, const float *__restrict__ tw, const int32_t *__restrict__ route_row,
               const uint16_t *__restrict__ y, uint16_t *__restrict__ out)
{
    // one flat index over (token, 8-column piece): no idle threads at the
    // end of a row
    const int pieces = s.H / kCombineVec;
    const long i = (long)blockIdx.x * kThreads + threadIdx.x;
    if (i >= (long)s.T * pieces)
        return;
    const int t = (int)(i / pieces);
    const int col = (int)(i - (long)t * pieces) * kCombineVec;
    // a row of a multiple of 64 pieces puts every wavefront inside one token:
    // its slots and weights are then read once per wavefront (scalar loads)
    if ((pieces & 63) == 0)
        combine_cols(s, tw, route_row, y, out, __builtin_amdgcn_readfirstlane(t), col);
    else
        combine_cols(s, tw, route_row, y, out, t, col);
}

// MX FP8 rows where a row is a multiple of 128 pieces of 8 columns (H a
// multiple of 1024): lane l of a wavefront takes columns 8 (p + l) and
// 8 (p + l + 64) of one token, 8 codes and their block's exponent byte
// each, so each lane keeps two loads of every kept route in flight (each
// instruction reads 512 contiguous bytes of codes); the arithmetic is
// combine8_cols' (the same bits).
__global__ void __launch_bounds__(kThreads)
combine_fp8_pair_kernel(Shape s, const float *__restrict__ tw,
                        const int32_t *__restrict__ route_row, const uint8_t *__restrict__ yc,
                        const uint8_t *__restrict__ ys, uint16_t *__restrict__ out)
{
#pragma clang fp contract(off)
    constexpr int V = 8;
    const int pieces = s.H / V;
    const long wid = ((long)blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int lane = threadIdx.x & 63;
    const int per_row = pieces / (64 * kPair);
    if (wid >= (long)s.T * per_row)
        return;
    const int t = __builtin_amdgcn_readfirstlane((int)(wid / per_row));
    const int p0 = (int)(wid - (long)t * per_row) * 64 * kPair + lane;
    constexpr int kMaxK = 8;
    const size_t slot0 = (size_t)t * s.K;
    int rows[kMaxK];
    float w[kMaxK];
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
        rows[k] = k < s.K ? route_row[slot0 + k] : -1;
        w[k] = k < s.K ? tw[slot0 + k] : 0.0f;
    }
    uint2 q[kMaxK][kPair];
    int e[kMaxK][kPair];
#pragma unroll
    for (int k = 0; k < kMaxK; ++k)
        if (rows[k] >= 0)
#pragma unroll
            for (int j = 0; j < kPair; ++j) {
                const int col = (p0 + 64 * j) * V;
                q[k][j] = *reinterpret_cast<const uint2 *>(yc + (size_t)rows[k] * s.H + col);
                e[k][j] = (int)ys[(size_t)rows[k] * (s.H / 32) + col / 32] - 127;
            }
    float acc[kPair][V];
#pragma unroll
    for (int j = 0; j < kPair; ++j)
#pragma unroll
        for (int i = 0; i < V; ++i)
            acc[j][i] = 0.0f;
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
        if (rows[k] < 0)
            continue;
#pragma unroll
        for (int j = 0; j < kPair; ++j) {
            const int wd[2] = {(int)q[k][j].x, (int)q[k][j].y};
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                const float v[4] = {__builtin_amdgcn_cvt_f32_fp8(wd[d], 0),
                                    __builtin_amdgcn_cvt_f32_fp8(wd[d], 1),
                                    __builtin_amdgcn_cvt_f32_fp8(wd[d], 2),
                                    __builtin_amdgcn_cvt_f32_fp8(wd[d], 3)};
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const float p = w[k] * ldexpf(v[b], e[k][j]);
                    acc[j][4 * d + b] = acc[j][4 * d + b] + p;
                }
            }
        }
    }
    typedef unsigned int u4v __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int j = 0; j < kPair; ++j) {
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = f32_to_bf16(acc[j][2 * i]) | (f32_to_bf16(acc[j][2 * i + 1]) << 16);
        __builtin_nontemporal_store(
            u4v{o[0], o[1], o[2], o[3]},
            reinterpret_cast<u4v *>(out + (size_t)t * s.H + (size_t)(p0 + 64 * j) * V));
    }
}

__global__ void __launch_bounds__(kThreads)
combine_fp8_kernel(Shape s, const float *__restrict__ tw, const int32_t *__restrict__ route_row,
                   const uint8_t *__restrict__ yc, const uint8_t *__restrict__ ys,
                   uint16_t *__restrict__ out)
{
    const int pieces = s.H / kCombine8Vec;
    const long i = (long)blockIdx.x * kThreads + threadIdx.x;
    if (i >= (long)s.T * pieces)
        return;
    const int t = (int)(i / pieces);
    const int col = (int)(i - (long)t * pieces) * kCombine8Vec;
    combine8_cols(s, tw, route_row, yc, ys, out, t, col);
}

} // namespace

hipError_t launch_combine_fp8(const moe_shape &sh, const float *tw, const int32_t *route_row,
                              const uint8_t *y_codes, const uint8_t *y_scales, uint16_t *out,
                              hipStream_t st)
{
    const Shape s = to_dev(sh);
    if ((sh.H / 8) % (64 * kPair) == 0) {
        const long threads = (long)sh.T * (sh.H / 8 / kPair);
        const long grid = (threads + kThreads - 1) / kThreads;
        combine_fp8_pair_kernel<<<(unsigned)grid, kThreads, 0, st>>>(s, tw, route_row, y_codes,
                                                                     y_scales, out);
        return hipGetLastError();
    }
    const long threads = (long)sh.T * (sh.H / kCombine8Vec);
    const long grid = (threads + kThreads - 1) / kThreads;
    combine_fp8_kernel<<<(unsigned)grid, kThreads, 0, st>>>(s, tw, route_row, y_codes, y_scales,
                                                            out);
    return hipGetLastError();
}

hipError_t launch_combine(const moe_shape &sh, const float *tw, const int32_t *route_row,
                          const uint16_t *y, uint16_t *out, hipStream_t st)
{
    const Shape s = to_dev(sh);
    const int pieces = sh.H / kCombineVec;
    if (pieces % (64 * kPair) == 0) {
        const long threads = (long)sh.T * (pieces / kPair);
        const long grid = (threads + kThreads - 1) / kThreads;
        combine_pair_kernel<<<(unsigned)grid, kThreads, 0, st>>>(s, tw, route_row, y, out);
        return hipGetLastError();
    }
    const long threads = (long)sh.T * pieces;
    const long grid = (threads + kThreads - 1) / kThreads;
    combine_kernel<<<(unsigned)grid, kThreads, 0, st>>>(s, tw, route_row, y, out);
    return hipGetLastError();
}

} // namespace moe
