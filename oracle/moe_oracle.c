/*
 * moe_oracle.c -- plain, slow CPU oracle of one GPU's share of the a8w4 MoE
 * expert layer.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg call it; the GPU library never does, and the
 * two share no code, header, table or constant.
 *
 * What it computes (the layer as the pages describe it):
 *   "MegaMoEV2: fuse Dispatch, GEMM1, GEMM2 and Combine into one kernel"
 *     (Technical Details): dispatch of top-k (token, expert, weight) routes,
 *     GEMM1, GEMM2 and a combine that skips invalid (-1) top-k slots; compact
 *     dispatch packs tokens in a prepare pass, fixed-slot writes each route
 *     into a per-expert slot with no prepare pass ("AITER MegaMoEV2 ... two
 *     dispatch schemes", page description).
 *   "full-expert DeepSeek V4.1 Flash MegaMoE tuning" (Summary): GEMM1 on the
 *     W13 experts, clamp-10 SwiGLU, FP8 quantisation of the intermediate,
 *     MXFP4 W2, weighted combine.
 *   "route before the rows move" (mono commit notes): the routed
 *     contributions are summed in f32 and rounded once.
 *
 * For every token t:
 *   out[t,:] = bf16( sum over k ascending, id local:
 *                    w[t,k] * W2_e . Q8( SwiGLU_clamp( W13_e . x_t ) ) )
 * with x, W13, W2 the MX-decoded values and Q8 the FP8 1x32 quantise /
 * dequantise of the intermediate.  orc_moe_layer_y8 also passes each
 * route's expert output row through Q8 (per 32 output columns) before the
 * weighted sum: the FP8 rows a rank with many rows sends to the combine
 * ("MegaMoEV2 ...", Technical Details, skewed routing, small input).
 * Readings where the pages are silent:
 *   - W13 rows 0..I-1 are the gate, I..2I-1 the up projection;
 *   - FP4 pairs: the low nibble holds the even K index;
 *   - FP8 is OCP E4M3FN (bias 7, no infinities, max 448);
 *   - the 1x32 exponent is floor(log2(amax)) - 8 (OCP MX rule for e4m3),
 *     clamped to [-127, 127]; an all-zero block gets exponent 0 (byte 127);
 *     scaled values round to nearest even and saturate at +-448;
 *   - gate' = min(g, gate_limit), up' = clamp(u, -up_limit, up_limit),
 *     h = gate' * sigmoid(gate') * up' (sigmoid in double, rounded to float);
 *   - every dot product accumulates in float32 in ascending index order;
 *   - an id of -1 is no expert; ids outside [0, E_total) are counted as
 *     invalid and skipped; ids of experts this GPU does not own are skipped.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_EXPORT __attribute__((visibility("default")))

typedef struct {
    int32_t T, H, I, K;
    int32_t E_total, expert_begin, E_local;
    int32_t dispatch_mode; /* 0 compact, 1 fixed-slot */
    int32_t capacity;      /* fixed-slot rows per expert */
    float gate_limit, up_limit;
} orc_shape;

/* ---------------------------------------------------------------------- */
/* MX element and scale codecs, from the format definitions.               */
/* ---------------------------------------------------------------------- */

/* e4m3 (OCP E4M3FN): sign | 4 exponent bits (bias 7) | 3 mantissa bits.
 * Exponent field 0 is subnormal: m/8 * 2^-6.  S.1111.111 is NaN. */
ORC_EXPORT float orc_e4m3_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return (float)(s ? -v : v);
}

/* e2m1 (OCP FP4): sign | 2 exponent bits (bias 1) | 1 mantissa bit.
 * Exponent field 0 is subnormal: m * 0.5. */
ORC_EXPORT float orc_e2m1_decode(uint8_t nib)
{
    int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
    double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return (float)(s ? -v : v);
}

/* E8M0: an unsigned biased exponent, 2^(b-127); 0xFF is NaN. */
ORC_EXPORT float orc_e8m0_decode(uint8_t b)
{
    if (b == 0xFF)
        return NAN;
    return (float)ldexp(1.0, (int)b - 127);
}

/* Nearest e4m3 value to v, ties to the even mantissa; magnitudes at or
 * above 448 saturate to 448; NaN maps to 0x7F. */
ORC_EXPORT uint8_t orc_e4m3_encode(double v)
{
    uint8_t s;
    double a, q, r;
    int ex, E, code;
    if (isnan(v))
        return 0x7F;
    s = signbit(v) ? 0x80 : 0x00;
    a = fabs(v);
    if (a >= 448.0)
        return s | 0x7E;
    if (a < ldexp(1.0, -6)) {
        /* subnormal binade: spacing 2^-9; r == 8 is the smallest normal,
         * whose code is also 8 */
        r = nearbyint(a * 512.0);
        return s | (uint8_t)r;
    }
    frexp(a, &ex);       /* a = f * 2^ex, f in [0.5, 1) */
    E = ex - 1;          /* a in [2^E, 2^(E+1)), E in [-6, 8] */
    q = ldexp(a, 3 - E); /* in [8, 16): 1.mmm scaled by 8 */
    r = nearbyint(q);    /* round half to even */
    if (r == 16.0) {
        r = 8.0;
        E += 1;
    }
    code = ((E + 7) << 3) | ((int)r - 8);
    if (code > 0x7E)
        code = 0x7E;
    return s | (uint8_t)code;
}

/* float32 -> bfloat16 bits, round to nearest even (NaN stays quiet NaN). */
ORC_EXPORT uint16_t orc_bf16_encode(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

ORC_EXPORT float orc_bf16_decode(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* One 32-value block to MX FP8: exponent byte and e4m3 codes. */
ORC_EXPORT void orc_mx8_quant_block(const float *v, uint8_t *codes, uint8_t *scale)
{
    float amax = 0.0f;
    int i, ex, E;
    for (i = 0; i < 32; ++i)
        amax = fmaxf(amax, fabsf(v[i]));
    if (amax == 0.0f) {
        *scale = 127;
        for (i = 0; i < 32; ++i)
            codes[i] = 0;
        return;
    }
    frexpf(amax, &ex); /* amax in [2^(ex-1), 2^ex) */
    E = (ex - 1) - 8;
    if (E < -127)
        E = -127;
    if (E > 127)
        E = 127;
    *scale = (uint8_t)(E + 127);
    for (i = 0; i < 32; ++i)
        codes[i] = orc_e4m3_encode(ldexp((double)v[i], -E));
}

/* bf16 activation rows to MX FP8, the step in front of the layer
 * ("MegaMoEV2: fuse dispatch, GEMM1, GEMM2 and combine into one kernel",
 * Summary: the quant runs before the dispatch, fused with the layer for
 * small inputs, as a kernel of its own for large ones): each row's values
 * decoded from bf16 exactly, then every 32 consecutive values through
 * orc_mx8_quant_block, the same rule as the requant of the intermediate. */
ORC_EXPORT void orc_quant_mxfp8(const uint16_t *x, int64_t rows, int32_t H, uint8_t *codes,
                                uint8_t *scales)
{
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < rows; ++t) {
        float v[32];
        int32_t b, i;
        for (b = 0; b < H / 32; ++b) {
            for (i = 0; i < 32; ++i)
                v[i] = orc_bf16_decode(x[t * H + 32 * b + i]);
            orc_mx8_quant_block(v, codes + t * H + 32 * b, scales + t * (H / 32) + b);
        }
    }
}

/* float32 rows to MX FP8 by the same 1x32 rule: every 32 consecutive
 * values of a row through orc_mx8_quant_block (codes [rows, H], exponent
 * bytes [rows, H/32]). */
ORC_EXPORT void orc_quant_rows_f32(const float *y, int64_t rows, int32_t H, uint8_t *codes,
                                   uint8_t *scales)
{
    int64_t t;
    int32_t b;
    for (t = 0; t < rows; ++t)
        for (b = 0; b < H / 32; ++b)
            orc_mx8_quant_block(y + t * H + 32 * b, codes + t * H + 32 * b,
                                scales + t * (H / 32) + b);
}

/* Clamped SwiGLU of one (gate, up) pair. */
ORC_EXPORT float orc_swiglu(float g, float u, float gate_limit, float up_limit)
{
    float gc = fminf(g, gate_limit);
    float uc = fminf(fmaxf(u, -up_limit), up_limit);
    float silu = (float)((double)gc / (1.0 + exp(-(double)gc)));
    return silu * uc;
}

/* ---------------------------------------------------------------------- */
/* Dispatch                                                                */
/* ---------------------------------------------------------------------- */

/* Local expert of route slot r, or -1 (no expert / not local), or -2
 * (invalid id). */
static int route_expert(const orc_shape *s, int32_t id)
{
    int e;
    if (id == -1)
        return -1;
    if (id < 0 || id >= s->E_total)
        return -2;
    e = id - s->expert_begin;
    if (e < 0 || e >= s->E_local)
        return -1;
    return e;
}

ORC_EXPORT int64_t orc_row_capacity(const orc_shape *s)
{
    if (s->dispatch_mode == 1)
        return (int64_t)s->E_local * s->capacity;
    return (int64_t)s->T * s->K;
}

/*
 * Route filter and dispatch, slots visited in (t, k) order, r = t*K + k.
 * compact: counts = per-expert histogram, offsets = its exclusive scan
 *          (offsets[E_local] = total), rows of each expert in ascending r.
 * fixed:   each route claims the next slot of its expert; slot < capacity
 *          gives row e*capacity + slot, otherwise the route is dropped and
 *          counted; counts = claims (may exceed capacity);
 *          offsets[e] = e*capacity.
 * row_route[row] = r for every kept route (rows not written stay as given),
 * route_row[r] = row or -1.  status[0] = invalid ids, status[1] = dropped.
 */
ORC_EXPORT int orc_dispatch(const orc_shape *s, const int32_t *ids, int32_t *counts,
                            int32_t *offsets, int32_t *row_route, int32_t *route_row,
                            int32_t *status)
{
    int64_t nslots = (int64_t)s->T * s->K, r;
    int e;
    int32_t *fill;
    status[0] = status[1] = status[2] = status[3] = 0;
    for (e = 0; e < s->E_local; ++e)
        counts[e] = 0;
    for (r = 0; r < nslots; ++r) {
        e = route_expert(s, ids[r]);
        route_row[r] = -1;
        if (e == -2)
            status[0]++;
        if (e >= 0)
            counts[e]++;
    }
    if (s->dispatch_mode == 1) {
        fill = (int32_t *)calloc((size_t)s->E_local, sizeof(int32_t));
        for (e = 0; e <= s->E_local; ++e)
            offsets[e] = e * s->capacity;
        for (r = 0; r < nslots; ++r) {
            int slot;
            e = route_expert(s, ids[r]);
            if (e < 0)
                continue;
            slot = fill[e]++;
            if (slot < s->capacity) {
                int64_t row = (int64_t)e * s->capacity + slot;
                row_route[row] = (int32_t)r;
                route_row[r] = (int32_t)row;
            } else {
                status[1]++;
            }
        }
        free(fill);
        return 0;
    }
    offsets[0] = 0;
    for (e = 0; e < s->E_local; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    fill = (int32_t *)calloc((size_t)s->E_local, sizeof(int32_t));
    for (r = 0; r < nslots; ++r) {
        int32_t row;
        e = route_expert(s, ids[r]);
        if (e < 0)
            continue;
        row = offsets[e] + fill[e]++;
        row_route[row] = (int32_t)r;
        route_row[r] = row;
    }
    free(fill);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* One route through one expert                                            */
/* ---------------------------------------------------------------------- */

/* x row (H e4m3 codes, H/32 exponents) through local expert e:
 *   gu[j] = sum_h x[h] * W13[e, j, h],  j in [0, 2I)
 *   hv[i] = SwiGLU(gu[i], gu[I + i])
 *   (h_codes, h_scale) = MX FP8 of hv, per 32 along I
 *   y[n]  = sum_i hq[i] * W2[e, n, i],  n in [0, H)
 * Any of gu_out / h_codes / h_scale may be NULL. */
ORC_EXPORT void orc_expert_ffn_hv(const orc_shape *s, const uint8_t *xrow, const uint8_t *xsc,
                                  int e, const uint8_t *w13, const uint8_t *w13s,
                                  const uint8_t *w2, const uint8_t *w2s, float *gu_out,
                                  float *hv_out, uint8_t *h_codes, uint8_t *h_scale, float *y);

ORC_EXPORT void orc_expert_ffn(const orc_shape *s, const uint8_t *xrow, const uint8_t *xsc,
                               int e, const uint8_t *w13, const uint8_t *w13s,
                               const uint8_t *w2, const uint8_t *w2s, float *gu_out,
                               uint8_t *h_codes, uint8_t *h_scale, float *y)
{
    orc_expert_ffn_hv(s, xrow, xsc, e, w13, w13s, w2, w2s, gu_out, NULL, h_codes, h_scale, y);
}

/* As orc_expert_ffn, also returning the SwiGLU output before
 * requantisation (hv_out[I], may be NULL). */
ORC_EXPORT void orc_expert_ffn_hv(const orc_shape *s, const uint8_t *xrow, const uint8_t *xsc,
                                  int e, const uint8_t *w13, const uint8_t *w13s,
                                  const uint8_t *w2, const uint8_t *w2s, float *gu_out,
                                  float *hv_out, uint8_t *h_codes, uint8_t *h_scale, float *y)
{
    const int H = s->H, I = s->I;
    float *xd = (float *)malloc(sizeof(float) * (size_t)H);
    float *gu = (float *)malloc(sizeof(float) * 2 * (size_t)I);
    float *hv = (float *)malloc(sizeof(float) * (size_t)I);
    float *hq = (float *)malloc(sizeof(float) * (size_t)I);
    uint8_t *hc = (uint8_t *)malloc((size_t)I);
    uint8_t *hs = (uint8_t *)malloc((size_t)I / 32);
    int h, j, i, n, b;

    for (h = 0; h < H; ++h)
        xd[h] = orc_e4m3_decode(xrow[h]) * orc_e8m0_decode(xsc[h / 32]);

    for (j = 0; j < 2 * I; ++j) {
        const uint8_t *wr = w13 + ((size_t)e * 2 * I + j) * (size_t)(H / 2);
        const uint8_t *sr = w13s + ((size_t)e * 2 * I + j) * (size_t)(H / 32);
        float acc = 0.0f;
        for (h = 0; h < H; ++h) {
            uint8_t byte = wr[h / 2];
            uint8_t nib = (h & 1) ? (byte >> 4) : (byte & 15);
            float wv = orc_e2m1_decode(nib) * orc_e8m0_decode(sr[h / 32]);
            acc = acc + xd[h] * wv;
        }
        gu[j] = acc;
    }
    if (gu_out)
        memcpy(gu_out, gu, sizeof(float) * 2 * (size_t)I);

    for (i = 0; i < I; ++i)
        hv[i] = orc_swiglu(gu[i], gu[I + i], s->gate_limit, s->up_limit);
    if (hv_out)
        memcpy(hv_out, hv, sizeof(float) * (size_t)I);
    for (b = 0; b < I / 32; ++b) {
        orc_mx8_quant_block(hv + 32 * b, hc + 32 * b, hs + b);
        for (i = 32 * b; i < 32 * b + 32; ++i)
            hq[i] = orc_e4m3_decode(hc[i]) * orc_e8m0_decode(hs[b]);
    }
    if (h_codes)
        memcpy(h_codes, hc, (size_t)I);
    if (h_scale)
        memcpy(h_scale, hs, (size_t)I / 32);

    for (n = 0; n < H; ++n) {
        const uint8_t *wr = w2 + ((size_t)e * H + n) * (size_t)(I / 2);
        const uint8_t *sr = w2s + ((size_t)e * H + n) * (size_t)(I / 32);
        float acc = 0.0f;
        for (i = 0; i < I; ++i) {
            uint8_t byte = wr[i / 2];
            uint8_t nib = (i & 1) ? (byte >> 4) : (byte & 15);
            float wv = orc_e2m1_decode(nib) * orc_e8m0_decode(sr[i / 32]);
            acc = acc + hq[i] * wv;
        }
        y[n] = acc;
    }
    free(xd);
    free(gu);
    free(hv);
    free(hq);
    free(hc);
    free(hs);
}

/* ---------------------------------------------------------------------- */
/* The layer, token by token                                               */
/* ---------------------------------------------------------------------- */

/* Output rows of the tokens in tok[0..ntok) (all T tokens if tok is NULL)
 * into out[ntok, H] as bf16 bits.  Each route is evaluated on its own, in k
 * order; the weighted sum is kept in float32 and rounded once.  Fixed-slot
 * capacity is not modelled: callers check that no route overflowed. */
static int moe_layer(const orc_shape *s, const uint8_t *x, const uint8_t *xs,
                     const int32_t *ids, const float *tw, const uint8_t *w13,
                     const uint8_t *w13s, const uint8_t *w2, const uint8_t *w2s,
                     const int32_t *tok, int ntok, int y_fp8, uint16_t *out)
{
    const int H = s->H, K = s->K;
    int n_items = tok ? ntok : s->T;
    int it;
#pragma omp parallel for schedule(dynamic, 1)
    for (it = 0; it < n_items; ++it) {
        int t = tok ? tok[it] : it;
        float *o = (float *)calloc((size_t)H, sizeof(float));
        float *y = (float *)malloc(sizeof(float) * (size_t)H);
        uint8_t *yc = (uint8_t *)malloc((size_t)H);
        uint8_t *ys = (uint8_t *)malloc((size_t)H / 32);
        int k, n;
        for (k = 0; k < K; ++k) {
            int e = route_expert(s, ids[(size_t)t * K + k]);
            float w = tw[(size_t)t * K + k];
            if (e < 0)
                continue;
            orc_expert_ffn(s, x + (size_t)t * H, xs + (size_t)t * (H / 32), e, w13, w13s, w2,
                           w2s, NULL, NULL, NULL, y);
            if (y_fp8) {
                /* the route's row goes to the combine as MX FP8: quantise
                 * per 32 columns, then every value decoded exactly */
                orc_quant_rows_f32(y, 1, H, yc, ys);
                for (n = 0; n < H; ++n)
                    y[n] = orc_e4m3_decode(yc[n]) * orc_e8m0_decode(ys[n / 32]);
            }
            for (n = 0; n < H; ++n) {
                float p = w * y[n];
                o[n] = o[n] + p;
            }
        }
        for (n = 0; n < H; ++n)
            out[(size_t)it * H + n] = orc_bf16_encode(o[n]);
        free(o);
        free(y);
        free(yc);
        free(ys);
    }
    return 0;
}

ORC_EXPORT int orc_moe_layer(const orc_shape *s, const uint8_t *x, const uint8_t *xs,
                             const int32_t *ids, const float *tw, const uint8_t *w13,
                             const uint8_t *w13s, const uint8_t *w2, const uint8_t *w2s,
                             const int32_t *tok, int ntok, uint16_t *out)
{
    return moe_layer(s, x, xs, ids, tw, w13, w13s, w2, w2s, tok, ntok, 0, out);
}

/* The layer with each route's expert output row sent to the combine as MX
 * FP8 instead of float32 ("MegaMoEV2: fuse Dispatch, GEMM1, GEMM2 and
 * Combine into one kernel", Technical Details, skewed routing on the small
 * input: a rank with many rows or a large expert sends its GEMM2 rows to
 * the combine in the main path's 1x32 FP8 format instead of BF16).  Read
 * here as: the float32 row y of a route through orc_quant_rows_f32 (the
 * rule of the intermediate's requant, per 32 consecutive output columns),
 * then the decoded values take y's place in the same weighted float32 sum,
 * rounded once. */
ORC_EXPORT int orc_moe_layer_y8(const orc_shape *s, const uint8_t *x, const uint8_t *xs,
                                const int32_t *ids, const float *tw, const uint8_t *w13,
                                const uint8_t *w13s, const uint8_t *w2, const uint8_t *w2s,
                                const int32_t *tok, int ntok, uint16_t *out)
{
    return moe_layer(s, x, xs, ids, tw, w13, w13s, w2, w2s, tok, ntok, 1, out);
}

/* Per-route intermediates for step checks: for the routes r_list[0..n),
 * h codes [n, I], h exponents [n, I/32] and y [n, H] in float32. */
ORC_EXPORT int orc_routes_ffn_hv(const orc_shape *s, const uint8_t *x, const uint8_t *xs,
                                 const int32_t *ids, const uint8_t *w13, const uint8_t *w13s,
                                 const uint8_t *w2, const uint8_t *w2s, const int32_t *r_list,
                                 int n, float *hv, uint8_t *h_codes, uint8_t *h_scale, float *y);

ORC_EXPORT int orc_routes_ffn(const orc_shape *s, const uint8_t *x, const uint8_t *xs,
                              const int32_t *ids, const uint8_t *w13, const uint8_t *w13s,
                              const uint8_t *w2, const uint8_t *w2s, const int32_t *r_list,
                              int n, uint8_t *h_codes, uint8_t *h_scale, float *y)
{
    return orc_routes_ffn_hv(s, x, xs, ids, w13, w13s, w2, w2s, r_list, n, NULL, h_codes,
                             h_scale, y);
}

/* As orc_routes_ffn, also returning the pre-requantisation SwiGLU output
 * hv [n, I] (may be NULL). */
ORC_EXPORT int orc_routes_ffn_hv(const orc_shape *s, const uint8_t *x, const uint8_t *xs,
                                 const int32_t *ids, const uint8_t *w13, const uint8_t *w13s,
                                 const uint8_t *w2, const uint8_t *w2s, const int32_t *r_list,
                                 int n, float *hv, uint8_t *h_codes, uint8_t *h_scale, float *y)
{
    const int H = s->H, I = s->I, K = s->K;
    int i, bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : bad)
    for (i = 0; i < n; ++i) {
        int r = r_list[i], t = r / K;
        int e = route_expert(s, ids[r]);
        if (e < 0) {
            bad++;
            continue;
        }
        orc_expert_ffn_hv(s, x + (size_t)t * H, xs + (size_t)t * (H / 32), e, w13, w13s, w2,
                          w2s, NULL, hv ? hv + (size_t)i * I : NULL, h_codes + (size_t)i * I,
                          h_scale + (size_t)i * (I / 32), y + (size_t)i * H);
    }
    return bad ? -1 : 0;
}

/* ---------------------------------------------------------------------- */
/* Single steps on given inputs                                            */
/* ---------------------------------------------------------------------- */

/* GEMM2 of given MX FP8 rows: row i holds h codes [I] and exponents [I/32]
 * and belongs to local expert experts[i]; y[i, n] = sum_i' hq * W2[e, n, i']
 * in float32, ascending i'. */
ORC_EXPORT int orc_gemm2_rows(const orc_shape *s, const uint8_t *h_codes, const uint8_t *h_scale,
                              const int32_t *experts, int n, const uint8_t *w2,
                              const uint8_t *w2s, float *y)
{
    const int H = s->H, I = s->I;
    int r, bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : bad)
    for (r = 0; r < n; ++r) {
        const uint8_t *hc = h_codes + (size_t)r * I;
        const uint8_t *hs = h_scale + (size_t)r * (I / 32);
        float *hq = (float *)malloc(sizeof(float) * (size_t)I);
        int e = experts[r], i, col;
        if (e < 0 || e >= s->E_local) {
            bad++;
            free(hq);
            continue;
        }
        for (i = 0; i < I; ++i)
            hq[i] = orc_e4m3_decode(hc[i]) * orc_e8m0_decode(hs[i / 32]);
        for (col = 0; col < H; ++col) {
            const uint8_t *wr = w2 + ((size_t)e * H + col) * (size_t)(I / 2);
            const uint8_t *sr = w2s + ((size_t)e * H + col) * (size_t)(I / 32);
            float acc = 0.0f;
            for (i = 0; i < I; ++i) {
                uint8_t byte = wr[i / 2];
                uint8_t nib = (i & 1) ? (byte >> 4) : (byte & 15);
                acc = acc + hq[i] * (orc_e2m1_decode(nib) * orc_e8m0_decode(sr[i / 32]));
            }
            y[(size_t)r * H + col] = acc;
        }
        free(hq);
    }
    return bad ? -1 : 0;
}

/* Combine of given MX FP8 rows (codes [R, H], exponent bytes [R, H/32]):
 * as orc_combine on the decoded values, each decoded exactly in float32
 * (e4m3 value times 2^(byte - 127)). */
ORC_EXPORT int orc_combine_fp8(const orc_shape *s, const float *tw, const int32_t *route_row,
                               const uint8_t *y_codes, const uint8_t *y_scale, uint16_t *out)
{
    const int H = s->H, K = s->K;
    int t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < s->T; ++t) {
        int n, k;
        for (n = 0; n < H; ++n) {
            float o = 0.0f;
            for (k = 0; k < K; ++k) {
                int32_t row = route_row[(size_t)t * K + k];
                float v, p;
                if (row < 0)
                    continue;
                v = orc_e4m3_decode(y_codes[(size_t)row * H + n]) *
                    orc_e8m0_decode(y_scale[(size_t)row * (H / 32) + n / 32]);
                p = tw[(size_t)t * K + k] * v;
                o = o + p;
            }
            out[(size_t)t * H + n] = orc_bf16_encode(o);
        }
    }
    return 0;
}

/* Combine of given float32 rows y[R, H]: out[t] = bf16(sum over k
 * ascending with route_row >= 0 of w[t,k] * y[route_row]) in float32. */
ORC_EXPORT int orc_combine(const orc_shape *s, const float *tw, const int32_t *route_row,
                           const float *y, uint16_t *out)
{
    const int H = s->H, K = s->K;
    int t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < s->T; ++t) {
        int n, k;
        for (n = 0; n < H; ++n) {
            float o = 0.0f;
            for (k = 0; k < K; ++k) {
                int32_t row = route_row[(size_t)t * K + k];
                float p;
                if (row < 0)
                    continue;
                p = tw[(size_t)t * K + k] * y[(size_t)row * H + n];
                o = o + p;
            }
            out[(size_t)t * H + n] = orc_bf16_encode(o);
        }
    }
    return 0;
}
