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
