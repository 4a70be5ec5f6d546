// Combine: each token's kept routes (bf16 y rows), weighted by their routing
// weights and summed in float32 in ascending k, rounded to bf16 once.  Slots whose
// route_row is -1 (pad, foreign, invalid or dropped) contribute nothing, so
// the result does not depend on their weights.  No atomics: a thread owns 8
// output columns of one token, which makes the sum order fixed.
#include "moe_common.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads)
combine_kernel(Shape s, const float *__restrict__ tw, const int32_t *__restrict__ route_row,
               const uint16_t *__restrict__ y, uint16_t *__restrict__ out)
{
    const int per_token = (s.H + kThreads * kCombineVec - 1) / (kThreads * kCombineVec);
    const int t = blockIdx.x / per_token;
    const int col = ((blockIdx.x - t * per_token) * kThreads + threadIdx.x) * kCombineVec;
    combine_cols(s, tw, route_row, y, out, t, col);
}

} // namespace

hipError_t launch_combine(const moe_shape &sh, const float *tw, const int32_t *route_row,
                          const uint16_t *y, uint16_t *out, hipStream_t st)
{
    const Shape s = to_dev(sh);
    const int per_block = kThreads * kCombineVec;
    const long grid = (long)((sh.H + per_block - 1) / per_block) * sh.T;
    combine_kernel<<<(unsigned)grid, kThreads, 0, st>>>(s, tw, route_row, y, out);
    return hipGetLastError();
}

} // namespace moe
