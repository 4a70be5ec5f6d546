// C ABI of the a8w4 MoE layer: argument checks (all before the first
// launch), workspace layout and the launch sequence.
#include <math.h>

#include <mutex>

#include "moe_common.hpp"

namespace {

using moe::kMaxLocalExperts;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// The kernels move codes, exponents and rows in 16-byte pieces.
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

template <typename... P>
bool all_aligned16(const P *...p)
{
    return (aligned16(p) && ...);
}

// Byte layout of the moe_forward workspace.
struct Layout {
    size_t hdr, counts, offsets, row_route, route_row, status, sync, scratch, h, hs, y, ys, xq,
        xqs, total;
};

Layout layout_of(const moe_shape &s)
{
    const size_t R = (size_t)moe_row_capacity(&s);
    const size_t TK = (size_t)s.T * (size_t)s.K;
    Layout L{};
    size_t p = 0;
    // the persistent layer's counters: first, at a fixed place, so they stay
    // where they were when a workspace serves other shapes
    L.hdr = p;
    p = align_up(p + sizeof(int32_t) * (size_t)moe::kPersistentHeaderWords);
    L.counts = p;
    p = align_up(p + sizeof(int32_t) * (size_t)s.E_local);
    L.offsets = p;
    p = align_up(p + sizeof(int32_t) * ((size_t)s.E_local + 1));
    L.row_route = p;
    p = align_up(p + sizeof(int32_t) * R);
    L.route_row = p;
    p = align_up(p + sizeof(int32_t) * TK);
    L.status = p;
    p = align_up(p + sizeof(int32_t) * 4);
    L.sync = p;
    p = align_up(p + sizeof(int32_t) * (size_t)moe::persistent_ready_words(s));
    L.scratch = p;
    {
        const size_t a = moe::dispatch_scratch_bytes(s), b = moe::persistent_table_bytes(s);
        p = align_up(p + (a > b ? a : b));
    }
    L.h = p;
    p = align_up(p + R * (size_t)s.I);
    L.hs = p;
    p = align_up(p + R * (size_t)(s.I / 32));
    // y: bf16 rows, or MX FP8 rows (codes, then exponent bytes at ys)
    L.y = p;
    L.ys = align_up(p + R * (size_t)s.H);
    {
        const size_t bf16_end = p + R * (size_t)s.H * sizeof(uint16_t);
        const size_t fp8_end = L.ys + R * (size_t)(s.H / 32);
        p = align_up(bf16_end > fp8_end ? bf16_end : fp8_end);
    }
    // MX FP8 activations of moe_forward_bf16
    L.xq = p;
    p = align_up(p + (size_t)s.T * (size_t)s.H);
    L.xqs = p;
    p = align_up(p + (size_t)s.T * (size_t)(s.H / 32));
    L.total = p;
    return L;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

// ---------------------------------------------------------------------------
// Scratch of moe_forward_static: the moe_forward workspace as a file-scope
// device array, for callers that cannot allocate.  Each device the library
// runs on holds its own copy until the process ends.  On the host the
// array's name stands for no device address: its address on a device comes
// from hipGetSymbolAddress with that device current, once per device, and
// only that pointer is ever handed to a kernel.
// ---------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = size_t(128) << 20;
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device, or nullptr.
void *static_scratch(int *dev_out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    *dev_out = dev;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

hipStream_t as_stream(void *p) { return static_cast<hipStream_t>(p); }

} // namespace

extern "C" {

int moe_check_shape(const moe_shape *s)
{
    if (!s)
        return MOE_EINVAL;
    if (s->T < 0 || s->H <= 0 || s->I <= 0 || s->K < 1 || s->E_total < 1 || s->E_local < 1 ||
        s->expert_begin < 0)
        return MOE_EINVAL;
    if (s->dispatch_mode != MOE_DISPATCH_COMPACT && s->dispatch_mode != MOE_DISPATCH_FIXED_SLOT)
        return MOE_EINVAL;
    if (s->dispatch_mode == MOE_DISPATCH_FIXED_SLOT && s->capacity < 1)
        return MOE_EINVAL;
    if (isnan(s->gate_limit) || isnan(s->up_limit))
        return MOE_EINVAL;
    if ((long long)s->expert_begin + s->E_local > s->E_total)
        return MOE_EINVAL;
    if (s->K > 8 || s->E_local > kMaxLocalExperts)
        return MOE_ENOTSUP;
    if (s->H % 128 != 0 || s->I % 128 != 0)
        return MOE_ENOTSUP;
    if ((long long)s->T * s->K >= (1ll << 31))
        return MOE_ENOTSUP;
    // the kernels address a gathered activation row (token t of x) and a row
    // of one expert's weights with 32-bit byte offsets from a wavefront-
    // uniform base: x itself, and the expert's first weight row
    if ((long long)s->T * s->H >= (1ll << 32) || (long long)s->I * s->H >= (1ll << 32))
        return MOE_ENOTSUP;
    if (s->dispatch_mode == MOE_DISPATCH_FIXED_SLOT &&
        (long long)s->E_local * s->capacity >= (1ll << 31))
        return MOE_ENOTSUP;
    return MOE_OK;
}

int64_t moe_row_capacity(const moe_shape *s)
{
    if (moe_check_shape(s) != MOE_OK)
        return -1;
    if (s->dispatch_mode == MOE_DISPATCH_FIXED_SLOT)
        return (int64_t)s->E_local * s->capacity;
    return (int64_t)s->T * s->K;
}

size_t moe_dispatch_workspace_size(const moe_shape *s)
{
    if (moe_check_shape(s) != MOE_OK)
        return 0;
    return moe::dispatch_scratch_bytes(*s);
}

size_t moe_workspace_size(const moe_shape *s)
{
    if (moe_check_shape(s) != MOE_OK)
        return 0;
    return layout_of(*s).total;
}

int moe_workspace_init(void *ws, size_t ws_bytes, void *stream)
{
    const size_t need = sizeof(int32_t) * (size_t)moe::kPersistentHeaderWords;
    if (!ws || ws_bytes < need || ((uintptr_t)ws % kAlign) != 0)
        return MOE_EWORKSPACE;
    return hip_status(moe::launch_zero_words(static_cast<int32_t *>(ws),
                                             moe::kPersistentHeaderWords, as_stream(stream)));
}

int64_t moe_workspace_status_offset(const moe_shape *s)
{
    if (moe_check_shape(s) != MOE_OK)
        return -1;
    return (int64_t)layout_of(*s).status;
}

static int dispatch_impl(const moe_shape *s, const int32_t *ids, const int32_t *valid,
                         int32_t *counts, int32_t *offsets, int32_t *row_route,
                         int32_t *route_row, int32_t *status, void *ws, size_t ws_bytes,
                         void *stream)
{
    int rc = moe_check_shape(s);
    if (rc != MOE_OK)
        return rc;
    if (!counts || !offsets || !status)
        return MOE_EINVAL;
    if (s->T > 0 && (!ids || !row_route || !route_row))
        return MOE_EINVAL;
    const size_t need = moe::dispatch_scratch_bytes(*s);
    if (need && (!ws || ws_bytes < need))
        return MOE_EWORKSPACE;
    return hip_status(moe::launch_dispatch(*s, ids, counts, offsets, row_route, route_row, status,
                                           ws, as_stream(stream), nullptr, 0, nullptr, valid));
}

int moe_dispatch(const moe_shape *s, const int32_t *ids, int32_t *counts, int32_t *offsets,
                 int32_t *row_route, int32_t *route_row, int32_t *status, void *ws,
                 size_t ws_bytes, void *stream)
{
    return dispatch_impl(s, ids, nullptr, counts, offsets, row_route, route_row, status, ws,
                         ws_bytes, stream);
}

int moe_dispatch_valid(const moe_shape *s, const int32_t *ids, const int32_t *num_valid_tokens,
                       int32_t *counts, int32_t *offsets, int32_t *row_route, int32_t *route_row,
                       int32_t *status, void *ws, size_t ws_bytes, void *stream)
{
    if (s && s->T > 0 && !num_valid_tokens)
        return moe_check_shape(s) != MOE_OK ? moe_check_shape(s) : MOE_EINVAL;
    return dispatch_impl(s, ids, num_valid_tokens, counts, offsets, row_route, route_row, status,
                         ws, ws_bytes, stream);
}

int moe_gemm1_swiglu(const moe_shape *s, const uint8_t *x, const uint8_t *xs,
                     const int32_t *counts, const int32_t *offsets, const int32_t *row_route,
                     const uint8_t *w13, const uint8_t *w13s, uint8_t *h, uint8_t *hs,
                     void *stream)
{
    int rc = moe_check_shape(s);
    if (rc != MOE_OK)
        return rc;
    if (s->T == 0)
        return MOE_OK;
    if (!x || !xs || !counts || !offsets || !row_route || !w13 || !w13s || !h || !hs)
        return MOE_EINVAL;
    if (!all_aligned16(x, xs, w13, w13s, h, hs))
        return MOE_EINVAL;
    return hip_status(moe::launch_gemm1(*s, x, xs, counts, offsets, row_route, w13, w13s, h, hs,
                                        as_stream(stream)));
}

int moe_gemm2(const moe_shape *s, const uint8_t *h, const uint8_t *hs, const int32_t *counts,
              const int32_t *offsets, const uint8_t *w2, const uint8_t *w2s, uint16_t *y,
              void *stream)
{
    int rc = moe_check_shape(s);
    if (rc != MOE_OK)
        return rc;
    if (s->T == 0)
        return MOE_OK;
    if (!h || !hs || !counts || !offsets || !w2 || !w2s || !y)
        return MOE_EINVAL;
    if (!all_aligned16(h, hs, w2, w2s, y))
        return MOE_EINVAL;
    return hip_status(moe::launch_gemm2(*s, h, hs, counts, offsets, w2, w2s,
                                        moe::YRows{y, nullptr, nullptr}, as_stream(stream)));
}

int moe_gemm2_fp8(const moe_shape *s, const uint8_t *h, const uint8_t *hs, const int32_t *counts,
                  const int32_t *offsets, const uint8_t *w2, const uint8_t *w2s, uint8_t *y_fp8,
                  uint8_t *y_scale, void *stream)
{
    int rc = moe_check_shape(s);
    if (rc != MOE_OK)
        return rc;
    if (s->T == 0)
        return MOE_OK;
    if (!h || !hs || !counts || !offsets || !w2 || !w2s || !y_fp8 || !y_scale)
        return MOE_EINVAL;
    if (!all_aligned16(h, hs, w2, w2s, y_fp8))
        return MOE_EINVAL;
    return hip_status(moe::launch_gemm2(*s, h, hs, counts, offsets, w2, w2s,
                                        moe::YRows{nullptr, y_fp8, y_scale}, as_stream(stream)));
}

int moe_gemm1_swiglu_packed(const moe_shape *s, const uint8_t *x, const uint8_t *xs,
                            const int32_t *counts, const int32_t *offsets,
                            const int32_t *row_route, const uint8_t *w13p, const uint8_t *w13ps,
                            uint8_t *h, uint8_t *hs, void *stream)
{
    int rc = moe_check_shape(s);
    if (rc != MOE_OK)
        return rc;
    if (!moe::use_stream_gemm(*s, true))
        return MOE_ENOTSUP;
    if (s->T == 0)
        return MOE_OK;
    if (!x || !xs || !counts || !offsets || !row_route || !w13p || !w13ps || !h || !hs)
        return MOE_EINVAL;
    if (!all_aligned16(x, xs, w13p, w13ps, h, hs))
        return MOE_EINVAL;
    return hip_status(moe::launch_gemm1_stream(*s, x, xs, counts, offsets, row_route, w13p,
                                               w13ps, h, hs, as_stream(stream)));
}

int moe_gemm2_packed(const moe_shape *s, const uint8_t *h, const uint8_t *hs,
                     const int32_t *counts, const int32_t *offsets, const uint8_t *w2p,
                     const uint8_t *w2ps, uint16_t *y_bf16, uint8_t *y_fp8, uint8_t *y_scale,
                     void *stream)
{
    int rc = moe_check_shape(s);
    if (rc != MOE_OK)
        return rc;
    if (!moe::use_stream_gemm(*s, false))
        return MOE_ENOTSUP;
    if (s->T == 0)
        return MOE_OK;
    // exactly one output form: bf16 rows, or MX FP8 codes with exponents
    const bool fp8 = y_fp8 || y_scale;
    if (!h || !hs || !counts || !offsets || !w2p || !w2ps || fp8 == (y_bf16 != nullptr) ||
        (fp8 && (!y_fp8 || !y_scale)))
        return MOE_EINVAL;
    if (!all_aligned16(h, hs, w2p, w2ps, y_bf16, y_fp8))
        return MOE_EINVAL;
    return hip_status(moe::launch_gemm2_stream(*s, h, hs, counts, offsets, w2p, w2ps,
                                               moe::YRows{y_bf16, y_fp8, y_scale},
                                               as_stream(stream)));
}

int moe_quant_mxfp8(const moe_shape *s, const uint16_t *x, uint8_t *xq, uint8_t *xqs,
                    void *stream)
{
    int rc = moe_check_shape(s);
    if (rc != MOE_OK)
        return rc;
    if (s->T == 0)
        return MOE_OK;
    if (!x || !xq || !xqs)
        return MOE_EINVAL;
    if (!all_aligned16(x, xq))
        return MOE_EINVAL;
    const moe::QuantJob q{x, xq, xqs, (long)s->T * (s->H / 32)};
    return hip_status(moe::launch_quant_mxfp8(q, as_stream(stream)));
}

int moe_combine(const moe_shape *s, const float *tw, const int32_t *route_row, const uint16_t *y,
                uint16_t *out, void *stream)
{
    int rc = moe_check_shape(s);
    if (rc != MOE_OK)
        return rc;
    if (s->T == 0)
        return MOE_OK;
    if (!tw || !route_row || !y || !out)
        return MOE_EINVAL;
    if (!all_aligned16(y, out))
        return MOE_EINVAL;
    return hip_status(moe::launch_combine(*s, tw, route_row, y, out, as_stream(stream)));
}

int moe_combine_fp8(const moe_shape *s, const float *tw, const int32_t *route_row,
                    const uint8_t *y_fp8, const uint8_t *y_scale, uint16_t *out, void *stream)
{
    int rc = moe_check_shape(s);
    if (rc != MOE_OK)
        return rc;
    if (s->T == 0)
        return MOE_OK;
    if (!tw || !route_row || !y_fp8 || !y_scale || !out)
        return MOE_EINVAL;
    if (!all_aligned16(y_fp8, out))
        return MOE_EINVAL;
    return hip_status(
        moe::launch_combine_fp8(*s, tw, route_row, y_fp8, y_scale, out, as_stream(stream)));
}

int moe_resolve_y_format(const moe_shape *s, int32_t y_format)
{
    int rc = moe_check_shape(s);
    if (rc != MOE_OK)
        return rc;
    if (y_format == MOE_Y_BF16 || y_format == MOE_Y_FP8)
        return y_format;
    if (y_format != MOE_Y_AUTO)
        return MOE_EINVAL;
    // many rows per expert: where the tile rule reads weights through the
    // cache (tiles of 128 rows or more, from 96 expected rows per local
    // expert under uniform routing), from host-known sizes only
    return (double)s->T * s->K / (double)s->E_total > 96.0 ? MOE_Y_FP8 : MOE_Y_BF16;
}

} // extern "C"

namespace {

// The layer; `persistent` runs it as one persistent launch (dispatch, both
// GEMMs and the combine).
// With x_bf16 the activations arrive as bf16 rows and are quantised into the
// workspace first (x and xs are then ignored).
// Packed weights of the register-streaming GEMMs (either pair may be null).
struct Packed {
    const uint8_t *w13, *w13s, *w2, *w2s;
};

int forward_impl(const moe_shape *s, const uint8_t *x, const uint8_t *xs, const int32_t *ids,
                 const float *tw, const uint8_t *w13, const uint8_t *w13s, const uint8_t *w2,
                 const uint8_t *w2s, uint16_t *out, void *ws, size_t ws_bytes, void *stream,
                 bool persistent, const uint16_t *x_bf16 = nullptr,
                 const int32_t *valid = nullptr, size_t need_bytes = 0,
                 int32_t y_format = MOE_Y_BF16, const Packed &pk = Packed{})
{
    int rc = moe_check_shape(s);
    if (rc != MOE_OK)
        return rc;
    const int yf = moe_resolve_y_format(s, y_format);
    if (yf < 0)
        return yf;
    if (persistent && !moe::persistent_supported(*s))
        return MOE_ENOTSUP;
    if (s->T == 0)
        return MOE_OK;
    const Layout L = layout_of(*s);
    uint8_t *base = static_cast<uint8_t *>(ws);
    moe::QuantJob quant{nullptr, nullptr, nullptr, 0};
    if (x_bf16) {
        if (!all_aligned16(x_bf16))
            return MOE_EINVAL;
        if (base) {
            x = base + L.xq;
            xs = base + L.xqs;
            quant = moe::QuantJob{x_bf16, base + L.xq, base + L.xqs, (long)s->T * (s->H / 32)};
        }
    }
    if (!ids || !tw || !w13 || !w13s || !w2 || !w2s || !out || (!x_bf16 && (!x || !xs)))
        return MOE_EINVAL;
    if (!ws || ws_bytes < (need_bytes ? need_bytes : L.total) || ((uintptr_t)ws % kAlign) != 0)
        return MOE_EWORKSPACE;
    if (!all_aligned16(x, xs, w13, w13s, w2, w2s, out))
        return MOE_EINVAL;
    if ((!pk.w13 != !pk.w13s) || (!pk.w2 != !pk.w2s) ||
        !all_aligned16(pk.w13, pk.w13s, pk.w2, pk.w2s))
        return MOE_EINVAL;
    const moe::QuantJob *qj = x_bf16 ? &quant : nullptr;
    int32_t *counts = reinterpret_cast<int32_t *>(base + L.counts);
    int32_t *offsets = reinterpret_cast<int32_t *>(base + L.offsets);
    int32_t *row_route = reinterpret_cast<int32_t *>(base + L.row_route);
    int32_t *route_row = reinterpret_cast<int32_t *>(base + L.route_row);
    int32_t *status = reinterpret_cast<int32_t *>(base + L.status);
    void *scratch = base + L.scratch;
    uint8_t *h = base + L.h;
    uint8_t *hs = base + L.hs;
    const moe::YRows y = yf == MOE_Y_FP8
                             ? moe::YRows{nullptr, base + L.y, base + L.ys}
                             : moe::YRows{reinterpret_cast<uint16_t *>(base + L.y), nullptr,
                                          nullptr};
    hipStream_t st = as_stream(stream);
    if (persistent) {
        // one launch (after the activation quant, when the rows come as bf16)
        hipError_t e = qj ? moe::launch_quant_mxfp8(*qj, st) : hipSuccess;
        const moe::PersistentBufs pb{counts,
                                     offsets,
                                     row_route,
                                     route_row,
                                     status,
                                     reinterpret_cast<int32_t *>(base + L.hdr),
                                     reinterpret_cast<int32_t *>(scratch),
                                     reinterpret_cast<int32_t *>(base + L.sync),
                                     h,
                                     hs};
        if (e == hipSuccess)
            e = moe::launch_layer_persistent(*s, ids, valid, tw, x, xs, w13, w13s, w2, w2s, pb,
                                             y, out, st);
        return hip_status(e);
    }
    hipError_t e = moe::launch_dispatch(*s, ids, counts, offsets, row_route, route_row, status,
                                        scratch, st, nullptr, 0, qj, valid);
    if (e == hipSuccess)
        e = pk.w13 && moe::use_stream_gemm(*s, true)
                ? moe::launch_gemm1_stream(*s, x, xs, counts, offsets, row_route, pk.w13,
                                           pk.w13s, h, hs, st)
                : moe::launch_gemm1(*s, x, xs, counts, offsets, row_route, w13, w13s, h, hs, st);
    if (e == hipSuccess)
        e = pk.w2 && moe::use_stream_gemm(*s, false)
                ? moe::launch_gemm2_stream(*s, h, hs, counts, offsets, pk.w2, pk.w2s, y, st)
                : moe::launch_gemm2(*s, h, hs, counts, offsets, w2, w2s, y, st);
    if (e == hipSuccess)
        e = y.bf16 ? moe::launch_combine(*s, tw, route_row, y.bf16, out, st)
                   : moe::launch_combine_fp8(*s, tw, route_row, y.codes, y.scales, out, st);
    return hip_status(e);
}

} // namespace

extern "C" {

int moe_forward(const moe_shape *s, const uint8_t *x, const uint8_t *xs, const int32_t *ids,
                const float *tw, const uint8_t *w13, const uint8_t *w13s, const uint8_t *w2,
                const uint8_t *w2s, uint16_t *out, void *ws, size_t ws_bytes, void *stream)
{
    return forward_impl(s, x, xs, ids, tw, w13, w13s, w2, w2s, out, ws, ws_bytes, stream, false);
}

size_t moe_static_scratch_bytes(void) { return kStaticScratchBytes; }

size_t moe_forward_static_need(const moe_shape *s)
{
    if (moe_check_shape(s) != MOE_OK)
        return 0;
    // the MX FP8 path uses the workspace up to the bf16-input area
    return layout_of(*s).xq;
}

int moe_forward_static(const moe_shape *s, const uint8_t *x, const uint8_t *xs,
                       const int32_t *ids, const float *tw, const uint8_t *w13,
                       const uint8_t *w13s, const uint8_t *w2, const uint8_t *w2s, uint16_t *out,
                       void *stream)
{
    int rc = moe_check_shape(s);
    if (rc != MOE_OK)
        return rc;
    if (s->T == 0)
        return MOE_OK;
    if (layout_of(*s).xq > kStaticScratchBytes)
        return MOE_ESCRATCH;
    int dev = -1;
    void *ws = static_scratch(&dev);
    if (!ws)
        return MOE_EHIP;
    return forward_impl(s, x, xs, ids, tw, w13, w13s, w2, w2s, out, ws, kStaticScratchBytes,
                        stream, false, nullptr, nullptr, layout_of(*s).xq);
}

int moe_forward_persistent(const moe_shape *s, const uint8_t *x, const uint8_t *xs,
                           const int32_t *ids, const float *tw, const uint8_t *w13,
                           const uint8_t *w13s, const uint8_t *w2, const uint8_t *w2s,
                           uint16_t *out, void *ws, size_t ws_bytes, void *stream)
{
    return forward_impl(s, x, xs, ids, tw, w13, w13s, w2, w2s, out, ws, ws_bytes, stream, true);
}

int moe_forward_bf16(const moe_shape *s, const uint16_t *x_bf16, const int32_t *ids,
                     const float *tw, const uint8_t *w13, const uint8_t *w13s, const uint8_t *w2,
                     const uint8_t *w2s, uint16_t *out, void *ws, size_t ws_bytes, void *stream)
{
    if (s && s->T > 0 && !x_bf16)
        return moe_check_shape(s) != MOE_OK ? moe_check_shape(s) : MOE_EINVAL;
    return forward_impl(s, nullptr, nullptr, ids, tw, w13, w13s, w2, w2s, out, ws, ws_bytes,
                        stream, false, x_bf16);
}

int moe_forward_ex(const moe_shape *s, const moe_forward_args *a, void *ws, size_t ws_bytes,
                   void *stream)
{
    int rc = moe_check_shape(s);
    if (rc != MOE_OK)
        return rc;
    if (!a)
        return MOE_EINVAL;
    // exactly one activation form
    const bool fp8 = a->x_fp8 || a->x_scale, bf16 = a->x_bf16 != nullptr;
    if (fp8 == bf16)
        return s->T == 0 ? MOE_OK : MOE_EINVAL;
    return forward_impl(s, a->x_fp8, a->x_scale, a->topk_ids, a->topk_w, a->w13, a->w13_scale,
                        a->w2, a->w2_scale, a->out_bf16, ws, ws_bytes, stream, a->persistent != 0,
                        a->x_bf16, a->num_valid_tokens, 0, a->y_format,
                        Packed{a->w13_packed, a->w13_packed_scale, a->w2_packed,
                               a->w2_packed_scale});
}

static bool pack_dims_ok(int32_t E, int32_t N, int32_t K)
{
    return E >= 1 && N >= 64 && K >= 128 && N % 64 == 0 && K % 128 == 0 &&
           (long double)E * N * (K / 2) < (long double)(1ll << 40);
}

size_t moe_packed_codes_bytes(int32_t E, int32_t N, int32_t K)
{
    return pack_dims_ok(E, N, K) ? moe::packed_codes_bytes(E, N, K) : 0;
}

size_t moe_packed_scales_bytes(int32_t E, int32_t N, int32_t K)
{
    return pack_dims_ok(E, N, K) ? moe::packed_scales_bytes(E, N, K) : 0;
}

int moe_pack_weights(const uint8_t *w, const uint8_t *w_scale, int32_t E, int32_t N, int32_t K,
                     uint8_t *packed, uint8_t *packed_scale, void *stream)
{
    if (!pack_dims_ok(E, N, K) || !w || !w_scale || !packed || !packed_scale ||
        !all_aligned16(w, w_scale, packed, packed_scale))
        return MOE_EINVAL;
    return hip_status(moe::launch_pack(w, w_scale, packed, packed_scale, E, N, K,
                                       as_stream(stream)));
}

int moe_unpack_weights(const uint8_t *packed, const uint8_t *packed_scale, int32_t E, int32_t N,
                       int32_t K, uint8_t *w, uint8_t *w_scale, void *stream)
{
    if (!pack_dims_ok(E, N, K) || !w || !w_scale || !packed || !packed_scale ||
        !all_aligned16(w, w_scale, packed, packed_scale))
        return MOE_EINVAL;
    return hip_status(moe::launch_unpack(packed, packed_scale, w, w_scale, E, N, K,
                                         as_stream(stream)));
}

int moe_set_tile_table(const moe_tile_entry *entries, int32_t n)
{
    return moe::set_tile_table(entries, n);
}

int moe_get_tile_config(const moe_shape *s, int32_t gemm, moe_tile_entry *out)
{
    int rc = moe_check_shape(s);
    if (rc != MOE_OK)
        return rc;
    if (!out || (gemm != 1 && gemm != 2))
        return MOE_EINVAL;
    int bm = 0, bn = 0, ku = 0;
    if (!moe::tile_config_of(*s, gemm == 1, &bm, &bn, &ku))
        return MOE_ENOTSUP;
    *out = moe_tile_entry{gemm, s->H, s->I, s->K, s->E_total, s->E_local, s->T, bm, bn, ku};
    return MOE_OK;
}

const char *moe_strerror(int code)
{
    switch (code) {
    case MOE_OK:
        return "ok";
    case MOE_EINVAL:
        return "invalid argument";
    case MOE_ENOTSUP:
        return "shape not supported (H and I multiples of 128, K <= 8, E_local <= 512, "
               "T*H and I*H below 2^32)";
    case MOE_EWORKSPACE:
        return "workspace missing, too small or not 256-byte aligned";
    case MOE_EHIP:
        return "HIP launch failed";
    case MOE_ESCRATCH:
        return "shape needs more than the static scratch of moe_forward_static "
               "(moe_forward_static_need > moe_static_scratch_bytes)";
    default:
        return "unknown error";
    }
}

} // extern "C"
