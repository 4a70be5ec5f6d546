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

// The combine of MX FP8 rows (e4m3 codes [R, H], E8M0 bytes [R, H/32]): a
// thread owns 16 columns of one token (one 16-byte piece of each kept row
// and its block's exponent byte); every value is decoded exactly (the
// hardware e4m3 conversion, then ldexp by byte - 127), then summed as in
// combine_cols: float32, k ascending, a product then an add per term, one
// bf16 rounding.
constexpr int kCombine8Vec = 16;

__global__ void __launch_bounds__(kThreads)
combine_fp8_kernel(Shape s, const float *__restrict__ tw, const int32_t *__restrict__ route_row,
                   const uint8_t *__restrict__ yc, const uint8_t *__restrict__ ys,
                   uint16_t *__restrict__ out)
{
#pragma clang fp contract(off)
    const int pieces = s.H / kCombine8Vec;
    const long i = (long)blockIdx.x * kThreads + threadIdx.x;
    if (i >= (long)s.T * pieces)
        return;
    const int t = (int)(i / pieces);
    const int col = (int)(i - (long)t * pieces) * kCombine8Vec;
    constexpr int kMaxK = 8;
    const size_t slot0 = (size_t)t * s.K;
    int rows[kMaxK];
    float w[kMaxK];
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
        rows[k] = k < s.K ? route_row[slot0 + k] : -1;
        w[k] = k < s.K ? tw[slot0 + k] : 0.0f;
    }
    uint4 q[kMaxK];
    int e[kMaxK];
#pragma unroll
    for (int k = 0; k < kMaxK; ++k)
        if (rows[k] >= 0) {
            q[k] = *reinterpret_cast<const uint4 *>(yc + (size_t)rows[k] * s.H + col);
            e[k] = (int)ys[(size_t)rows[k] * (s.H / 32) + col / 32] - 127;
        }
    float acc[kCombine8Vec];
#pragma unroll
    for (int j = 0; j < kCombine8Vec; ++j)
        acc[j] = 0.0f;
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
        if (rows[k] < 0)
            continue;
        const int wd[4] = {(int)q[k].x, (int)q[k].y, (int)q[k].z, (int)q[k].w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const float v[4] = {__builtin_amdgcn_cvt_f32_fp8(wd[d], 0),
                                __builtin_amdgcn_cvt_f32_fp8(wd[d], 1),
                                __builtin_amdgcn_cvt_f32_fp8(wd[d], 2),
                                __builtin_amdgcn_cvt_f32_fp8(wd[d], 3)};
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float p = w[k] * ldexpf(v[b], e[k]);
                acc[4 * d + b] = acc[4 * d + b] + p;
            }
        }
    }
    uint32_t o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        o[j] = f32_to_bf16(acc[2 * j]) | (f32_to_bf16(acc[2 * j + 1]) << 16);
    typedef unsigned int u4v __attribute__((ext_vector_type(4)));
    u4v *dst = reinterpret_cast<u4v *>(out + (size_t)t * s.H + col);
    __builtin_nontemporal_store(u4v{o[0], o[1], o[2], o[3]}, dst);
    __builtin_nontemporal_store(u4v{o[4], o[5], o[6], o[7]}, dst + 1);
}

} // namespace

hipError_t launch_combine_fp8(const moe_shape &sh, const float *tw, const int32_t *route_row,
                              const uint8_t *y_codes, const uint8_t *y_scales, uint16_t *out,
                              hipStream_t st)
{
    const Shape s = to_dev(sh);
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
    const long threads = (long)sh.T * (sh.H / kCombineVec);
    const long grid = (threads + kThreads - 1) / kThreads;
    combine_kernel<<<(unsigned)grid, kThreads, 0, st>>>(s, tw, route_row, y, out);
    return hipGetLastError();
}

} // namespace moe
