// Internal declarations shared by the gfx950 kernels of the a8w4 MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_a8w4.h"

namespace moe {

constexpr int kMaxLocalExperts = 512;
// int32 words at the start of the moe_forward workspace that the persistent
// layer keeps its counters in (zero before its first call, zero after each)
constexpr int kPersistentHeaderWords = 1024;

// Kernel-side copy of moe_shape, passed by value.
struct Shape {
    int T, H, I, K;
    int E_total, expert_begin, E_local;
    int mode, capacity;
    float gate_limit, up_limit;
};

inline Shape to_dev(const moe_shape &s)
{
    return Shape{s.T, s.H, s.I, s.K, s.E_total, s.expert_begin, s.E_local,
                 s.dispatch_mode, s.capacity, s.gate_limit, s.up_limit};
}

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// A pointer every lane holds the same value of, in scalar registers (the
// LDS DMA loads and the saddr form of the global loads take their base from
// an SGPR pair).
__device__ __forceinline__ const uint8_t *uniform_ptr(const uint8_t *p)
{
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const uint8_t *>(((uint64_t)hi << 32) | lo);
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(uint8_t *p)
{
    return (uint32_t)(uintptr_t)(lds_u8 *)p;
}

// global -> LDS without registers: lane l's SIZE bytes from base + voff land
// at LDS address m0 + SIZE * l (m0 is wavefront-uniform).  Issued as inline
// assembly so that the waits are exactly the ones this file writes: the
// loads count in vmcnt like any vector memory load.  An LDS DMA reads m0 one
// wait state after an SALU write of m0 at the earliest, hence the s_nop.
// kStream marks data read once (non-temporal: the L2 evicts it first, so it
// does not push out the activation rows that other tiles read again).
// kL2 reads data that another CU of the same XCD wrote earlier in the same
// launch: sc0 makes the load miss the CU's own L1, which may hold the line
// from before the write, and take it from the XCD's L2, where the write is.
template <int SIZE, bool kStream = false, bool kL2 = false>
__device__ __forceinline__ void g2lds(const uint8_t *base, uint32_t voff, uint32_t m0)
{
    static_assert(SIZE == 16 || SIZE == 4, "dword and dwordx4 LDS DMA only");
    static_assert(!(kStream && kL2), "one cache policy");
    // both are wavefront-uniform by construction; readfirstlane tells the
    // compiler so where its analysis cannot see it (it costs nothing when
    // the values already sit in scalar registers)
    m0 = __builtin_amdgcn_readfirstlane(m0);
    base = uniform_ptr(base);
    if (SIZE == 16 && kL2)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 sc0" ::"s"(m0),
                     "v"(voff), "s"(base)
                     : "memory", "m0");
    else if (SIZE == 16 && kStream)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(m0),
                     "v"(voff), "s"(base)
                     : "memory", "m0");
    else if (SIZE == 16)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0),
                     "v"(voff), "s"(base)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" ::"s"(m0),
                     "v"(voff), "s"(base)
                     : "memory", "m0");
}

// The workgroup barrier without the memory fence __syncthreads() adds (that
// fence would wait for every outstanding load, prefetches included).
__device__ __forceinline__ void raw_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// ---------------------------------------------------------------------------
// Route filter: local expert of an id, -1 (pad slot or another GPU's expert)
// or -2 (id outside [-1, E_total)).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int route_local(const Shape &s, int id)
{
    if (id == -1)
        return -1;
    if ((unsigned)id >= (unsigned)s.E_total)
        return -2;
    const int e = id - s.expert_begin;
    return (unsigned)e < (unsigned)s.E_local ? e : -1;
}

// Rows of expert e actually held by its segment.
__device__ __forceinline__ int used_rows(const Shape &s, int count)
{
    return s.mode == MOE_DISPATCH_FIXED_SLOT ? min(count, s.capacity) : count;
}

// ---------------------------------------------------------------------------
// Scaled MFMA: D(16x16) += A(16x128) * B(128x16) with one E8M0 exponent per
// 32 K values of every A row and every B column.  Lane l serves row / column
// (l & 15); with g = l >> 4:
//   A, MXFP4 (weights): 16 bytes in the low four dwords, K = 32g .. 32g+31,
//     two values per byte, low nibble first;
//   B, MXFP8 (activations): bytes 0..15 hold K = 16g .. 16g+15 and bytes
//     16..31 hold K = 64+16g .. 64+16g+15;
//   the exponent byte (bits 0..7) of lane l scales K block g (K = 32g ..
//     32g+31) of its row / column, whichever lanes hold that block's data;
//   D: lane l holds column (l & 15), rows 4g .. 4g+3.
// ---------------------------------------------------------------------------
__device__ __forceinline__ v4f mfma_w4a8(const v8i &a_fp4, const v8i &b_fp8, v4f c, int sa,
                                         int sb)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a_fp4, b_fp8, c, 4, 0, 0, sa, 0,
                                                            sb);
}

// float -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint32_t f32_to_bf16(float v)
{
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return 0x7FC0u;
    const uint32_t lsb = (u >> 16) & 1u;
    return (u + 0x7FFFu + lsb) >> 16;
}

// Exponent of the 1x32 block: floor(log2(amax)) - 8 clamped to [-127, 127].
__device__ __forceinline__ int mx8_block_exponent(float amax)
{
    if (!(amax > 0.0f))
        return 0;
    int ex;
    (void)frexpf(amax, &ex);                    // amax in [2^(ex-1), 2^ex)
    int E = ex - 1 - 8;
    return E < -127 ? -127 : (E > 127 ? 127 : E);
}

// Four values of a 1x32 block with exponent E as e4m3 codes, the first in
// the low byte, by the hardware conversion (v_cvt_pk_fp8_f32, OCP e4m3 on
// gfx950, round to nearest even): each value is first scaled by 2^-E (exact)
// and clamped to +-448, so the conversion never overflows.  A block whose
// largest magnitude is zero is all +0 codes (-0 inputs included), as its
// exponent byte is 127.  Checked against the oracle on every bf16 value
// below 2^9 at a block exponent of 0 (the scaling is exact, so that covers
// every exponent), and on float32 values through GEMM1's requant codes.
__device__ __forceinline__ uint32_t mx8_pack4(float a, float b, float c, float d, int E,
                                              float amax)
{
    if (!(amax > 0.0f))
        return 0u;
    auto sc = [E](float v) { return __builtin_amdgcn_fmed3f(ldexpf(v, -E), -448.0f, 448.0f); };
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(sc(a), sc(b), 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(sc(c), sc(d), r, true);
    return (uint32_t)r;
}

// ---------------------------------------------------------------------------
// BF16 activation rows to MX FP8 (the 1x32 rule of the requant above): the
// step in front of the layer ("MegaMoEV2: fuse dispatch, GEMM1, GEMM2 and
// combine into one kernel", Summary: the small-input path fuses the quant,
// the large-input path runs it as its own kernel on the caller's stream).
// Four consecutive threads take one 32-value block, thread j the values
// 8j .. 8j+7 (one 16-byte load, one 8-byte store); the block's amax meets
// over two lane exchanges.  Thread tid of nthreads (nthreads a multiple of
// four) walks the blocks with a stride of nthreads / 4, four at a time.
// ---------------------------------------------------------------------------
struct QuantJob {
    const uint16_t *x;   // [rows, H] bf16
    uint8_t *codes;      // [rows, H] e4m3
    uint8_t *scales;     // [rows, H / 32] E8M0
    long blocks;         // rows * H / 32
};

__device__ __forceinline__ void quant_mx8_part(const QuantJob &q, long tid, long nthreads)
{
    // four blocks per pass, their loads issued together (the stream needs
    // several loads in flight per thread to cover the memory latency)
    constexpr int kU = 4;
    const int j = (int)(tid & 3);
    const long step = nthreads >> 2;
    for (long g0 = tid >> 2; g0 < q.blocks; g0 += kU * step) {
        uint4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const long g = g0 + u * step;
            if (g < q.blocks)
                v[u] = *reinterpret_cast<const uint4 *>(q.x + 32 * g + 8 * j);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const long g = g0 + u * step;
            if (g >= q.blocks)
                break;
            const float f[8] = {
                __uint_as_float(v[u].x << 16), __uint_as_float(v[u].x & 0xFFFF0000u),
                __uint_as_float(v[u].y << 16), __uint_as_float(v[u].y & 0xFFFF0000u),
                __uint_as_float(v[u].z << 16), __uint_as_float(v[u].z & 0xFFFF0000u),
                __uint_as_float(v[u].w << 16), __uint_as_float(v[u].w & 0xFFFF0000u)};
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                amax = fmaxf(amax, fabsf(f[i]));
            amax = fmaxf(amax, __shfl_xor(amax, 1));
            amax = fmaxf(amax, __shfl_xor(amax, 2));
            const int E = mx8_block_exponent(amax);
            *reinterpret_cast<uint2 *>(q.codes + 32 * g + 8 * j) =
                uint2{mx8_pack4(f[0], f[1], f[2], f[3], E, amax),
                      mx8_pack4(f[4], f[5], f[6], f[7], E, amax)};
            if (j == 0)
                q.scales[g] = (uint8_t)(E + 127);
        }
    }
}

// Clamped SwiGLU: min(g, gl) * sigmoid(min(g, gl)) * clamp(u, -ul, ul), the
// logistic from the hardware exp and reciprocal (v_exp_f32, v_rcp_f32: a
// few float32 ulps; the value is requantised to 3 mantissa bits next).
__device__ __forceinline__ float swiglu_clamped(float g, float u, float gl, float ul)
{
    const float gc = fminf(g, gl);
    const float uc = fminf(fmaxf(u, -ul), ul);
    return gc * __builtin_amdgcn_rcpf(1.0f + __expf(-gc)) * uc;
}

// ---------------------------------------------------------------------------
// Exclusive prefix over the local experts of f(e) >= 0, shared by the
// workgroup: out[e] = sum of f over experts < e, out[E] = total (returned).
// NT = threads of the workgroup (a multiple of 64, at most 1024); each
// thread sums up to 4 experts, which covers E_local <= 512 for NT >= 128.
// ---------------------------------------------------------------------------
template <int NT, typename F>
__device__ __forceinline__ int scan_experts(int E, F f, int *out)
{
    static_assert(NT % 64 == 0 && NT >= 128 && NT <= 1024, "scan_experts: workgroup size");
    const int tid = threadIdx.x;
    int local[4];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = tid * 4 + i;
        const int n = e < E ? f(e) : 0;
        local[i] = n;
        sum += n;
    }
    // inclusive scan of sum over the NT threads
    const int lane = tid & 63, wave = tid >> 6;
    int inc = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(inc, d);
        if (lane >= d)
            inc += o;
    }
    __shared__ int wtot[NT / 64];
    if (lane == 63)
        wtot[wave] = inc;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w)
        base += wtot[w];
    int run = base + inc - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = tid * 4 + i;
        if (e < E)
            out[e] = run;
        run += local[i];
    }
    if (tid == NT - 1)
        out[E] = base + inc;
    __syncthreads();
    return out[E];
}

// Row chunks of the expert segments: every workgroup derives the same plan
// from counts.  prefix[e] = first chunk of expert e, prefix[E] = total.
template <int NT = 256>
__device__ __forceinline__ int plan_chunks(const Shape &s, const int *__restrict__ counts, int ch,
                                           int *prefix)
{
    return scan_experts<NT>(
        s.E_local, [&](int e) { return (used_rows(s, counts[e]) + ch - 1) / ch; }, prefix);
}

// Expert owning chunk q: the last e with prefix[e] <= q.
__device__ __forceinline__ int chunk_expert(const int *prefix, int E, int q)
{
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (prefix[mid] <= q)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// ---------------------------------------------------------------------------
// Combine of output columns [col, col + 8) of token t: the kept routes in
// ascending k, each a rounded product then a rounded add (no fused
// multiply-add) on the bf16 y values widened to float32, one bf16 rounding
// at the end.
// ---------------------------------------------------------------------------
constexpr int kCombineVec = 8;

__device__ __forceinline__ void combine_cols(const Shape &s, const float *__restrict__ tw,
                                             const int32_t *__restrict__ route_row,
                                             const uint16_t *__restrict__ y,
                                             uint16_t *__restrict__ out, int t, int col)
{
#pragma clang fp contract(off)
    if (col >= s.H)
        return;
    // the token's slots first, then every kept route's 16 bytes of y, all in
    // flight together; the sum itself runs in ascending k
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
#pragma unroll
    for (int k = 0; k < kMaxK; ++k)
        if (rows[k] >= 0)
            q[k] = *reinterpret_cast<const uint4 *>(y + (size_t)rows[k] * s.H + col);
    float acc[kCombineVec];
#pragma unroll
    for (int i = 0; i < kCombineVec; ++i)
        acc[i] = 0.0f;
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
        if (rows[k] < 0)
            continue;
        const uint32_t wd[4] = {q[k].x, q[k].y, q[k].z, q[k].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = __uint_as_float(wd[i] << 16);
            const float hi = __uint_as_float(wd[i] & 0xffff0000u);
            const float p0 = w[k] * lo, p1 = w[k] * hi;
            acc[2 * i] = acc[2 * i] + p0;
            acc[2 * i + 1] = acc[2 * i + 1] + p1;
        }
    }
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o[i] = f32_to_bf16(acc[2 * i]) | (f32_to_bf16(acc[2 * i + 1]) << 16);
    // the layer never reads its output again: a non-temporal store keeps the
    // y rows other threads still read in the L2 (-9% at 65,536 tokens)
    typedef unsigned int u4v __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(u4v{o[0], o[1], o[2], o[3]},
                                reinterpret_cast<u4v *>(out + (size_t)t * s.H + col));
}

// The combine of MX FP8 rows (e4m3 codes [R, H], E8M0 bytes [R, H/32]) for
// output columns [col, col + 16) of token t: one 16-byte piece of each kept
// row and its block's exponent byte; every value is decoded exactly (the
// hardware e4m3 conversion, then ldexp by byte - 127), then summed as in
// combine_cols: float32, k ascending, a product then an add per term, one
// bf16 rounding.
constexpr int kCombine8Vec = 16;

__device__ __forceinline__ void combine8_cols(const Shape &s, const float *__restrict__ tw,
                                              const int32_t *__restrict__ route_row,
                                              const uint8_t *__restrict__ yc,
                                              const uint8_t *__restrict__ ys,
                                              uint16_t *__restrict__ out, int t, int col)
{
#pragma clang fp contract(off)
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

// ---------------------------------------------------------------------------
// Host-side launchers (defined in the kernel sources).
// ---------------------------------------------------------------------------
size_t dispatch_scratch_bytes(const moe_shape &s);
bool dispatch_is_single_block(const moe_shape &s);
// zero[0 .. nzero) is cleared by the dispatch launch (one workgroup paths
// only).  With a quant job the activation quant runs first: in the same
// launch as a one-workgroup dispatch (extra workgroups), else as its own
// launch before the dispatch.  valid (device int32, may be null) is the
// count of real tokens: rows past it are padding, routed nowhere.
hipError_t launch_dispatch(const moe_shape &s, const int32_t *ids, int32_t *counts,
                           int32_t *offsets, int32_t *row_route, int32_t *route_row,
                           int32_t *status, void *scratch, hipStream_t st,
                           int32_t *zero = nullptr, int nzero = 0,
                           const QuantJob *quant = nullptr, const int32_t *valid = nullptr);
// workgroups of `threads` threads that the quant job wants (at least one)
int quant_blocks(const QuantJob &q, int threads);
hipError_t launch_quant_mxfp8(const QuantJob &q, hipStream_t st);
hipError_t launch_gemm1(const moe_shape &s, const uint8_t *x, const uint8_t *xs,
                        const int32_t *counts, const int32_t *offsets, const int32_t *row_route,
                        const uint8_t *w13, const uint8_t *w13s, uint8_t *h, uint8_t *hs,
                        hipStream_t st);
// GEMM2 output rows: bf16 [R, H] (codes and scales null), or MX FP8 rows,
// e4m3 codes [R, H] and E8M0 bytes [R, H/32] by the requant's 1x32 rule
// (bf16 null).
struct YRows {
    uint16_t *bf16;
    uint8_t *codes, *scales;
};
hipError_t launch_gemm2(const moe_shape &s, const uint8_t *h, const uint8_t *hs,
                        const int32_t *counts, const int32_t *offsets, const uint8_t *w2,
                        const uint8_t *w2s, const YRows &y, hipStream_t st);
int tiled_bm(const moe_shape &s);
bool use_tiled_gemm1(const moe_shape &s);
bool use_tiled_gemm2(const moe_shape &s);
// tuned tile table (copied in; MOE_OK or MOE_EINVAL) and the tile shape a
// launch of the tiled GEMM would take (false where the register-streaming
// kernels serve the shape)
int set_tile_table(const moe_tile_entry *entries, int n);
bool tile_config_of(const moe_shape &s, bool gemm1, int *bm, int *bn, int *ku);
hipError_t launch_gemm1_tiled(const moe_shape &s, const uint8_t *x, const uint8_t *xs,
                              const int32_t *counts, const int32_t *offsets,
                              const int32_t *row_route, const uint8_t *w13, const uint8_t *w13s,
                              uint8_t *h, uint8_t *hs, hipStream_t st);
hipError_t launch_gemm2_tiled(const moe_shape &s, const uint8_t *h, const uint8_t *hs,
                              const int32_t *counts, const int32_t *offsets, const uint8_t *w2,
                              const uint8_t *w2s, const YRows &y, hipStream_t st);
bool persistent_supported(const moe_shape &s);
// words of the persistent layer's per-chunk ready counters
int persistent_ready_words(const moe_shape &s);
// bytes of its dispatch table
size_t persistent_table_bytes(const moe_shape &s);
// The whole layer in one persistent launch: dispatch, GEMM1 + SwiGLU +
// requant, GEMM2 and the combine.  hdr (kPersistentHeaderWords) must be zero
// at launch and is zero again when the kernel ends; a wait that gives up
// counts in status[2].
struct PersistentBufs {
    int32_t *counts, *offsets, *row_route, *route_row, *status;
    int32_t *hdr, *table, *ready;
    uint8_t *h, *hs;
};
hipError_t launch_layer_persistent(const moe_shape &s, const int32_t *ids, const int32_t *valid,
                                   const float *tw, const uint8_t *x, const uint8_t *xs,
                                   const uint8_t *w13, const uint8_t *w13s, const uint8_t *w2,
                                   const uint8_t *w2s, const PersistentBufs &b, const YRows &y,
                                   uint16_t *out, hipStream_t st);
// zero the first `words` words of p (the persistent header of a workspace)
hipError_t launch_zero_words(int32_t *p, int words, hipStream_t st);
hipError_t launch_combine(const moe_shape &s, const float *tw, const int32_t *route_row,
                          const uint16_t *y, uint16_t *out, hipStream_t st);
hipError_t launch_combine_fp8(const moe_shape &s, const float *tw, const int32_t *route_row,
                              const uint8_t *y_codes, const uint8_t *y_scales, uint16_t *out,
                              hipStream_t st);

// Packed weights of the register-streaming GEMMs (E experts, N rows of K
// values each): byte sizes, the packing launch, whether a GEMM of this shape
// takes them (its tile has 32 or 64 rows), and the two GEMM launches.
size_t packed_codes_bytes(int E, int N, int K);
size_t packed_scales_bytes(int E, int N, int K);
hipError_t launch_pack(const uint8_t *w, const uint8_t *ws, uint8_t *p, uint8_t *ps, int E,
                       int N, int K, hipStream_t st);
hipError_t launch_unpack(const uint8_t *p, const uint8_t *ps, uint8_t *w, uint8_t *ws, int E,
                         int N, int K, hipStream_t st);
bool use_stream_gemm(const moe_shape &s, bool gemm1);
hipError_t launch_gemm1_stream(const moe_shape &s, const uint8_t *x, const uint8_t *xs,
                               const int32_t *counts, const int32_t *offsets,
                               const int32_t *row_route, const uint8_t *w13p,
                               const uint8_t *w13ps, uint8_t *h, uint8_t *hs, hipStream_t st);
hipError_t launch_gemm2_stream(const moe_shape &s, const uint8_t *h, const uint8_t *hs,
                               const int32_t *counts, const int32_t *offsets,
                               const uint8_t *w2p, const uint8_t *w2ps, const YRows &y,
                               hipStream_t st);

int device_cu_count();

} // namespace moe
