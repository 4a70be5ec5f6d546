// Combine: each token's kept routes, weighted by their routing weights and
// summed in float32 in ascending k, rounded to bf16 once.  Slots whose
// route_row is -1 (pad, foreign, invalid or dropped) contribute nothing, so
// the result does not depend on their weights.  No atomics: a thread owns 8
// output columns of one token, which makes the sum order fixed.
#include "moe_common.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kCols = 8; // output columns per thread

__global__ void __launch_bounds__(kThreads)
combine_kernel(Shape s, const float *__restrict__ tw, const int32_t *__restrict__ route_row,
               const float *__restrict__ y, uint16_t *__restrict__ out)
{
    // a rounded product, then a rounded add: no fused multiply-add
#pragma clang fp contract(off)
    const int per_token = (s.H + kThreads * kCols - 1) / (kThreads * kCols);
    const int t = blockIdx.x / per_token;
    const int col = ((blockIdx.x - t * per_token) * kThreads + threadIdx.x) * kCols;
    if (col >= s.H)
        return;
    float acc[kCols];
#pragma unroll
    for (int i = 0; i < kCols; ++i)
        acc[i] = 0.0f;
    const size_t slot0 = (size_t)t * s.K;
    for (int k = 0; k < s.K; ++k) {
        const int row = route_row[slot0 + k];
        if (row < 0)
            continue;
        const float w = tw[slot0 + k];
        const float4 *yr = reinterpret_cast<const float4 *>(y + (size_t)row * s.H + col);
        const float4 a = yr[0], b = yr[1];
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < kCols; ++i) {
            const float p = w * v[i];
            acc[i] = acc[i] + p;
        }
    }
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o[i] = f32_to_bf16(acc[2 * i]) | (f32_to_bf16(acc[2 * i + 1]) << 16);
    *reinterpret_cast<uint4 *>(out + (size_t)t * s.H + col) = uint4{o[0], o[1], o[2], o[3]};
}

} // namespace

hipError_t launch_combine(const moe_shape &sh, const float *tw, const int32_t *route_row,
                          const float *y, uint16_t *out, hipStream_t st)
{
    const Shape s = to_dev(sh);
    const int per_block = kThreads * kCols;
    const long grid = (long)((sh.H + per_block - 1) / per_block) * sh.T;
    combine_kernel<<<(unsigned)grid, kThreads, 0, st>>>(s, tw, route_row, y, out);
    return hipGetLastError();
}

} // namespace moe
