// BF16 activation rows to MX FP8 1x32 (e4m3 codes + E8M0 exponents) as a
// kernel of its own, on the caller's stream: the large-input form of the
// quant in front of the layer ("MegaMoEV2: fuse dispatch, GEMM1, GEMM2 and
// combine into one kernel", Summary).  The one-workgroup dispatch paths run
// the same device code in extra workgroups of their launch instead
// (dispatch.hip).  HBM-bound: 2 bytes read and 33/32 bytes written per value.
#include "moe_common.hpp"

namespace moe {

namespace {

constexpr int kQuantThreads = 256;

__global__ void __launch_bounds__(kQuantThreads) quant_mxfp8_kernel(QuantJob q)
{
    quant_mx8_part(q, (long)blockIdx.x * kQuantThreads + threadIdx.x,
                   (long)gridDim.x * kQuantThreads);
}

} // namespace

// Enough workgroups for one pass over the blocks, at most eight per CU (the
// grid-stride loop covers the rest).
int quant_blocks(const QuantJob &q, int threads)
{
    const long want = (4 * q.blocks + threads - 1) / threads;
    const long cap = 8L * device_cu_count() * (kQuantThreads / 64) / (threads / 64);
    const long n = want < cap ? want : cap;
    return (int)(n < 1 ? 1 : n);
}

hipError_t launch_quant_mxfp8(const QuantJob &q, hipStream_t st)
{
    if (q.blocks <= 0)
        return hipSuccess;
    quant_mxfp8_kernel<<<quant_blocks(q, kQuantThreads), kQuantThreads, 0, st>>>(q);
    return hipGetLastError();
}

} // namespace moe
