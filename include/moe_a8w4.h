/*
 * moe_a8w4.h -- C ABI of one GPU's share of an a8w4 MoE expert layer on
 * MI355X (gfx950).
 *
 * The layer ("MegaMoEV2: fuse Dispatch, GEMM1, GEMM2 and Combine into one
 * kernel", Technical Details; "full-expert DeepSeek V4.1 Flash MegaMoE
 * tuning", Summary) takes top-k routes (token, expert id, weight), keeps the
 * routes whose expert this GPU owns, groups them into per-expert row
 * segments (dispatch), runs each row through its expert -- GEMM1 with the
 * gate/up weights W13, a clamped SwiGLU, FP8 1x32 requantisation of the
 * intermediate, GEMM2 with W2 -- and sums each token's routed rows weighted
 * by its routing weights (combine), skipping -1 slots.
 *
 * Formats (all buffers row-major and contiguous):
 *   FP8   OCP e4m3 (E4M3FN) codes, one byte each.
 *   MXFP4 OCP E2M1 codes, two per byte, the low nibble holding the even index.
 *   E8M0  one unsigned exponent byte (value 2^(b-127)) per 32 consecutive
 *         elements along the contraction dimension (x, h: along H or I;
 *         W13, W2: along their K).
 *   BF16  raw 16-bit patterns.
 *
 * Buffers (T tokens, K slots per token, E = E_local experts, R = rows):
 *   x_fp8     [T, H]        x_scale   [T, H/32]
 *   topk_ids  int32 [T, K]  global expert ids; -1 = no expert
 *   topk_w    float [T, K]  routing weights (a -1 slot's weight is ignored)
 *   w13       [E, 2I, H/2]  rows 0..I-1 gate, rows I..2I-1 up
 *   w13_scale [E, 2I, H/32]
 *   w2        [E, H, I/2]   w2_scale [E, H, I/32]
 *   out_bf16  [T, H]
 * Dispatch results (R = moe_row_capacity(shape)):
 *   counts    int32 [E]     routes kept for each expert (fixed-slot: routes
 *                           that asked for a slot, which may exceed capacity)
 *   offsets   int32 [E+1]   first row of each expert's segment; compact:
 *                           exclusive scan of counts, offsets[E] = rows used;
 *                           fixed-slot: e * capacity
 *   row_route int32 [R]     route slot r = t*K + k held by each row; rows
 *                           outside every segment's used part are not written
 *   route_row int32 [T*K]   row of each route slot, or -1 when the slot is
 *                           -1, not local, invalid or dropped
 *   status    int32 [4]     [0] ids outside [-1, E_total) (skipped),
 *                           [1] fixed-slot routes dropped for capacity,
 *                           [2] persistent-layer waits that gave up (the
 *                               layer's output is then not valid),
 *                           [3] zero; the dispatch writes all four
 * Intermediates, indexed by row:
 *   h_fp8 [R, I], h_scale [R, I/32], y_bf16 [R, H] (bf16 bit patterns),
 *   or y_fp8 [R, H] + y_scale [R, H/32] (MX FP8 rows, along H)
 *
 * Rows inside a compact segment are in ascending r (a stable scatter);
 * inside a fixed-slot segment their order is unspecified.
 *
 * Alignment: the FP8, MXFP4 and E8M0 arrays (x_fp8, x_scale, w13,
 * w13_scale, w2, w2_scale, h_fp8, h_scale), y_bf16 and out_bf16 must start on
 * a 16-byte boundary (PyTorch allocations do); a misaligned one is refused
 * with MOE_EINVAL.
 *
 * Ownership: the caller owns every buffer; pointers are device pointers
 * unless stated.  The library allocates nothing in these calls and keeps no
 * pointer after a call returns.  All calls are asynchronous on `stream`
 * (a hipStream_t; NULL is the null stream) and never synchronise, so they
 * can be captured into a HIP graph.
 *
 * Errors: every argument check runs before the first launch; a refused call
 * returns a negative code and leaves every buffer untouched.  Device-side
 * anomalies (an id outside [-1, E_total), a fixed-slot overflow) never
 * fault: the route is skipped and counted in status.
 */
#ifndef MOE_A8W4_H
#define MOE_A8W4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_EINVAL (-1)     /* null or misaligned pointer, negative size, bad enum */
#define MOE_ENOTSUP (-2)    /* shape outside what the kernels support */
#define MOE_EWORKSPACE (-3) /* workspace missing or too small */
#define MOE_EHIP (-4)       /* a HIP launch or query failed */
#define MOE_ESCRATCH (-5)   /* moe_forward_static: shape too large for its scratch */

#define MOE_DISPATCH_COMPACT 0    /* histogram, scan, stable scatter */
#define MOE_DISPATCH_FIXED_SLOT 1 /* atomic claim into per-expert capacity */

/* Format of the expert output rows y between GEMM2 and the combine. */
#define MOE_Y_BF16 0 /* bf16 rows (default) */
#define MOE_Y_FP8 1  /* MX FP8 rows: e4m3 codes + one E8M0 byte per 32 columns */
#define MOE_Y_AUTO 2 /* FP8 where the rows per local expert are many, else bf16 */

typedef struct moe_shape {
    int32_t T;             /* source tokens (0 is a valid no-op); T*H < 2^32 */
    int32_t H;             /* hidden size, a multiple of 128 */
    int32_t I;             /* expert intermediate size, a multiple of 128;
                              I*H < 2^32 */
    int32_t K;             /* top-k slots per token, 1..8 */
    int32_t E_total;       /* experts in the model */
    int32_t expert_begin;  /* first global id owned here */
    int32_t E_local;       /* experts owned here, 1..512 */
    int32_t dispatch_mode; /* MOE_DISPATCH_* */
    int32_t capacity;      /* fixed-slot rows per expert (>= 1 if fixed-slot) */
    float gate_limit;      /* gate' = min(gate, gate_limit)            (10) */
    float up_limit;        /* up'   = clamp(up, -up_limit, up_limit)   (10) */
} moe_shape;

/* Check a shape; MOE_OK or the code a call with it would return. */
int moe_check_shape(const moe_shape *shape);

/* Rows of the dispatch buffers: T*K (compact) or E_local*capacity. */
int64_t moe_row_capacity(const moe_shape *shape);

/* Device scratch bytes moe_dispatch needs (0 for small T). */
size_t moe_dispatch_workspace_size(const moe_shape *shape);

/* Device scratch bytes moe_forward needs (dispatch results, h, y, and the
 * MX FP8 activations of moe_forward_bf16). */
size_t moe_workspace_size(const moe_shape *shape);

/* Zero the persistent layer's counters at the start of a moe_forward
 * workspace (its first 4096 bytes; one small launch on `stream`): needed
 * once before the first moe_forward_persistent call on a workspace whose
 * memory was not zero-filled.  MOE_EWORKSPACE for a null, short or
 * misaligned workspace. */
int moe_workspace_init(void *workspace, size_t workspace_bytes, void *stream);

/* Byte offset inside the moe_forward workspace of the dispatch's int32[4]
 * status array (see "status" above), which the forward entry points leave
 * there for the caller to read; -1 for a refused shape. */
int64_t moe_workspace_status_offset(const moe_shape *shape);

/*
 * Dispatch ("AITER MegaMoEV2 ... two dispatch schemes": compact packs the
 * routes in a prepare pass; fixed-slot writes each route straight into a
 * per-expert slot).  Reads topk_ids; writes counts, offsets, row_route,
 * route_row and status.  A slot is local when its id is in
 * [expert_begin, expert_begin + E_local).  workspace may be NULL when
 * moe_dispatch_workspace_size() is 0.
 */
int moe_dispatch(const moe_shape *shape, const int32_t *topk_ids, int32_t *counts,
                 int32_t *offsets, int32_t *row_route, int32_t *route_row, int32_t *status,
                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * moe_dispatch for a padded batch: *num_valid_tokens (a device int32, read
 * by the kernels, so a captured graph follows the value written before each
 * replay) is the count of real tokens; rows t >= that count (clamped to
 * [0, T]) are padding and every slot of theirs is treated as -1: no route,
 * not counted as invalid, route_row = -1 ("feat(moe): route before the rows
 * move; per-pass real row counts", Per-pass real row counts: the count
 * reaches every routing kernel and replaces the pad-row mask).
 */
int moe_dispatch_valid(const moe_shape *shape, const int32_t *topk_ids,
                       const int32_t *num_valid_tokens, int32_t *counts, int32_t *offsets,
                       int32_t *row_route, int32_t *route_row, int32_t *status, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * GEMM1 + clamped SwiGLU + FP8 1x32 requantisation ("full-expert DeepSeek
 * V4.1 Flash MegaMoE tuning", Summary: W13, clamp-10 SwiGLU, FP8
 * intermediate quantisation).  For every used row of every expert segment:
 *   gu[j] = sum_h x[t,h] * W13[e,j,h], t = row_route[row] / K
 *   h[i]  = min(gu[i], gate_limit) * sigmoid(min(gu[i], gate_limit))
 *           * clamp(gu[I+i], -up_limit, up_limit)
 * then per 32 columns the exponent floor(log2(amax)) - 8 (byte 127 for an
 * all-zero block) and e4m3 codes rounded to nearest even, saturating at 448.
 * Writes h_fp8 / h_scale rows of used rows only.
 */
int moe_gemm1_swiglu(const moe_shape *shape, const uint8_t *x_fp8, const uint8_t *x_scale,
                     const int32_t *counts, const int32_t *offsets, const int32_t *row_route,
                     const uint8_t *w13, const uint8_t *w13_scale, uint8_t *h_fp8,
                     uint8_t *h_scale, void *stream);

/*
 * GEMM2 (MXFP4 W2; "MegaMoEV2 ...", Technical Details: the expert output
 * rows are BF16): y[row, n] = bf16(sum_i h[row,i] * W2[e,n,i]), the sum in
 * float32, rounded to nearest even, for every used row (y_bf16 is
 * [row capacity, H] bf16 bit patterns).  Writes y rows of used rows only.
 */
int moe_gemm2(const moe_shape *shape, const uint8_t *h_fp8, const uint8_t *h_scale,
              const int32_t *counts, const int32_t *offsets, const uint8_t *w2,
              const uint8_t *w2_scale, uint16_t *y_bf16, void *stream);

/*
 * GEMM2 with MX FP8 output rows ("MegaMoEV2 ...", Technical Details,
 * skewed routing, small input: a rank with many rows or a large expert
 * sends its GEMM2 rows to the combine in the main path's 1x32 FP8 format
 * instead of BF16).  The same float32 sums as moe_gemm2, then per 32
 * consecutive columns of a row the requant's rule (exponent
 * floor(log2(amax)) - 8 clamped to [-127, 127], byte 127 for an all-zero
 * block, e4m3 codes rounded to nearest even, saturating at 448), with no
 * bf16 rounding in between.  y_fp8 is [row capacity, H] e4m3 (16-byte
 * aligned), y_scale [row capacity, H/32] exponent bytes; rows of used rows
 * only are written.  Lossy against moe_gemm2: a value moves by up to 1/8 of
 * its block's largest magnitude.
 */
int moe_gemm2_fp8(const moe_shape *shape, const uint8_t *h_fp8, const uint8_t *h_scale,
                  const int32_t *counts, const int32_t *offsets, const uint8_t *w2,
                  const uint8_t *w2_scale, uint8_t *y_fp8, uint8_t *y_scale, void *stream);

/*
 * Activation quant in front of the layer ("MegaMoEV2: fuse dispatch, GEMM1,
 * GEMM2 and combine into one kernel", Summary: the large-input path runs it
 * as its own kernel on the caller's stream): bf16 rows x_bf16[T, H] to e4m3
 * codes x_fp8[T, H] and E8M0 exponents x_scale[T, H/32], one exponent per
 * 32 consecutive values of a row, by the same 1x32 rule as the requant of h:
 * exponent floor(log2(amax)) - 8 clamped to [-127, 127], values divided by
 * 2^exponent, rounded to nearest even, saturated at +-448; a block whose
 * amax is zero gets byte 127 and +0 codes.  Exact: the codes are a function
 * of the bf16 bits only.  x_bf16 and x_fp8 16-byte aligned; T = 0 is a
 * no-op.  Finite inputs (a NaN makes its block's codes unspecified).
 */
int moe_quant_mxfp8(const moe_shape *shape, const uint16_t *x_bf16, uint8_t *x_fp8,
                    uint8_t *x_scale, void *stream);

/*
 * Combine ("MegaMoEV2 ...": the combine skips invalid (-1) top-k slots;
 * "route before the rows move": routed contributions summed in f32 and
 * rounded once).  For every token t:
 *   out[t,:] = bf16( sum over k = 0..K-1 with route_row[t*K+k] >= 0 of
 *                    topk_w[t,k] * y_bf16[route_row[t*K+k], :] )
 * in float32 (each y value widened exactly), k ascending, each term a
 * product then an add; a token with no kept route gets +0.
 */
int moe_combine(const moe_shape *shape, const float *topk_w, const int32_t *route_row,
                const uint16_t *y_bf16, uint16_t *out_bf16, void *stream);

/*
 * Combine of MX FP8 rows (as moe_gemm2_fp8 writes them; "MegaMoEV2 ...",
 * Technical Details: the combine reads both formats): moe_combine with
 * every y value decoded exactly, e4m3 value times 2^(y_scale byte - 127).
 * y_fp8 and out_bf16 16-byte aligned; y rows read only through route_row.
 */
int moe_combine_fp8(const moe_shape *shape, const float *topk_w, const int32_t *route_row,
                    const uint8_t *y_fp8, const uint8_t *y_scale, uint16_t *out_bf16,
                    void *stream);

/*
 * The y format a layer call takes for y_format (MOE_Y_BF16, MOE_Y_FP8 or
 * MOE_Y_AUTO): MOE_Y_AUTO becomes MOE_Y_FP8 when the expected rows per
 * local expert under uniform routing, T*K/E_total, exceed 96 (where the
 * tile rule takes tiles of 128 rows or more, whose weights are read through
 * the cache: the pages pair FP8 rows with cached weights), else MOE_Y_BF16.
 * Host-known sizes only, never device data.  Returns the format, or
 * MOE_EINVAL for another value (or moe_check_shape's error).
 */
int moe_resolve_y_format(const moe_shape *shape, int32_t y_format);

/*
 * The whole layer ("MegaMoEV2: fuse Dispatch, GEMM1, GEMM2 and Combine into
 * one kernel", Technical Details: dispatch, the two expert GEMMs and the
 * combine as one call on one stream; "full-expert DeepSeek V4.1 Flash
 * MegaMoE tuning", Summary: W13 GEMM, clamp-10 SwiGLU, FP8 requant, W2 GEMM,
 * weighted combine): for every token t,
 *   out[t,:] = bf16( sum over k ascending with a local id of
 *                    topk_w[t,k] * W2_e . Q8( SwiGLU( W13_e . x_t ) ) )
 * computed as moe_dispatch, moe_gemm1_swiglu, moe_gemm2 and moe_combine in
 * that order (the result is bit-identical to calling them), with the
 * dispatch results and intermediates in `workspace` (>=
 * moe_workspace_size(shape) bytes, 256-byte aligned; its contents are
 * scratch, nothing in it needs clearing).  The kernel of each step is chosen
 * from host-known sizes only.  Calls that overlap on one workspace race.
 */
int moe_forward(const moe_shape *shape, const uint8_t *x_fp8, const uint8_t *x_scale,
                const int32_t *topk_ids, const float *topk_w, const uint8_t *w13,
                const uint8_t *w13_scale, const uint8_t *w2, const uint8_t *w2_scale,
                uint16_t *out_bf16, void *workspace, size_t workspace_bytes, void *stream);

/*
 * The same layer in one persistent launch ("MegaMoEV2 ...", Technical
 * Details, large input: dispatch, GEMM1, GEMM2 and combine fused into one
 * persistent kernel that overlaps the stages; skewed routing handled inside
 * the kernel, with no host sync).  Every workgroup of the grid (the device's
 * CUs times the kernel's occupancy, all resident at once) dispatches a slice
 * of the route slots, meets the others at a grid barrier, takes GEMM1 and
 * GEMM2 tickets from the work queue of the XCD it runs on (a GEMM2 item of a
 * row chunk waits until every GEMM1 item of that chunk is done; h passes
 * between them through that XCD's L2; tickets cover blocks of row chunks x
 * weight tiles, so a large expert's weight tile serves several chunks in
 * turn), and after a last barrier combines tokens.  Same arguments and
 * result as moe_forward (identical output bits).
 *
 * The first 1024 int32 words (4096 bytes) of `workspace` hold
 * the kernel's counters: they must be zero before the first persistent call
 * on a workspace (moe_workspace_init, or a zero-filled allocation), and
 * every call leaves them zero when it ends, also after a wait gave up; the
 * four-launch entry points never touch them.  MOE_ENOTSUP for shapes it
 * does not cover (H or I below 512, or a tuned table giving GEMM1 and GEMM2
 * different row tiles) and on a device whose CU count is not that of 1, 2,
 * 4 or 8 MI355X XCDs.  The grid barriers need the whole grid resident: with
 * other work occupying the device some workgroups may start late.  Every
 * wait is bounded; one that gives up counts in status[2] of the workspace
 * (moe_workspace_status_offset) and sends its workgroup to the end without
 * touching memory it has not been handed, and the output is then not valid.
 * MOE_PERSISTENT_MAX_POLLS in the environment (read at every launch) lowers
 * the bound, which tests use to force the timeouts.  Calls that overlap on
 * one workspace race.
 */
int moe_forward_persistent(const moe_shape *shape, const uint8_t *x_fp8, const uint8_t *x_scale,
                           const int32_t *topk_ids, const float *topk_w, const uint8_t *w13,
                           const uint8_t *w13_scale, const uint8_t *w2, const uint8_t *w2_scale,
                           uint16_t *out_bf16, void *workspace, size_t workspace_bytes,
                           void *stream);

/*
 * moe_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments and result as moe_forward without the workspace, which
 * is a file-scope device array of moe_static_scratch_bytes() (128 MiB)
 * inside the library instead.  Each GPU the library runs on holds its own
 * copy of that array until the process ends; the first call on a device
 * looks up its address there.  The call allocates nothing and launches the
 * kernels of moe_forward on `stream`.  Shapes whose workspace
 * (moe_forward_static_need) exceeds the array are refused with
 * MOE_ESCRATCH before any launch: the V4 shape (H 7168, I 3072, 48 local
 * experts) fits up to 159 fixed slots per expert, or 1,277 tokens with
 * compact dispatch.  Every call on one GPU shares that GPU's array (no part of which
 * needs clearing: each call writes what it reads), so calls that overlap
 * on one GPU -- on two streams, or from two threads -- race.
 */
int moe_forward_static(const moe_shape *shape, const uint8_t *x_fp8, const uint8_t *x_scale,
                       const int32_t *topk_ids, const float *topk_w, const uint8_t *w13,
                       const uint8_t *w13_scale, const uint8_t *w2, const uint8_t *w2_scale,
                       uint16_t *out_bf16, void *stream);

/* Bytes of moe_forward_static's scratch array. */
size_t moe_static_scratch_bytes(void);

/* Scratch bytes moe_forward_static needs for a shape (0 for a refused
 * shape); the call is refused when this exceeds moe_static_scratch_bytes(). */
size_t moe_forward_static_need(const moe_shape *shape);

/*
 * The layer from bf16 activations (the pages' small-input path fuses the
 * quant with the layer, the large-input path runs it first on the same
 * stream): moe_quant_mxfp8 of x_bf16 into the workspace, then moe_forward
 * on those codes.  Where the dispatch runs as one workgroup (at most 8,192
 * route slots) the quant shares its launch; otherwise it is a launch of its
 * own.  The output bits equal moe_forward's on moe_quant_mxfp8's codes.
 * Same workspace as moe_forward.
 */
int moe_forward_bf16(const moe_shape *shape, const uint16_t *x_bf16, const int32_t *topk_ids,
                     const float *topk_w, const uint8_t *w13, const uint8_t *w13_scale,
                     const uint8_t *w2, const uint8_t *w2_scale, uint16_t *out_bf16,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * The layer with every option: MX FP8 activations (x_fp8 + x_scale) or bf16
 * rows (x_bf16, quantised in the call as by moe_forward_bf16) -- exactly one
 * of the two; num_valid_tokens (device int32, or NULL for all T rows) as in
 * moe_dispatch_valid, so padding rows cost no expert work and get +0 output
 * rows; persistent != 0 takes moe_forward_persistent's launch (same
 * refusals); y_format (see moe_resolve_y_format) sends the expert output
 * rows to the combine as bf16 (MOE_Y_BF16, the result of moe_forward) or as
 * MX FP8 (moe_gemm2_fp8 then moe_combine_fp8 in the workspace's y area; a
 * lossy mode).  Same workspace as moe_forward.  w13_packed / w2_packed
 * (with their scale arrays; each pair may be given alone, or NULL) are
 * moe_pack_weights of w13 / w2: where the shape's GEMM takes a tile of 32
 * or 64 rows (moe_get_tile_config) it then runs the packed-weight kernel
 * on them, which gives the same output bits; elsewhere, and in the
 * persistent launch, they are not read.  The plain arrays are still
 * required.
 */
typedef struct {
    const uint8_t *x_fp8;             /* [T, H] e4m3, or NULL */
    const uint8_t *x_scale;           /* [T, H/32] E8M0, or NULL */
    const uint16_t *x_bf16;           /* [T, H] bf16, or NULL */
    const int32_t *topk_ids;          /* [T, K] */
    const float *topk_w;              /* [T, K] */
    const uint8_t *w13;               /* [E_local, 2I, H/2] */
    const uint8_t *w13_scale;         /* [E_local, 2I, H/32] */
    const uint8_t *w2;                /* [E_local, H, I/2] */
    const uint8_t *w2_scale;          /* [E_local, H, I/32] */
    uint16_t *out_bf16;               /* [T, H] */
    const int32_t *num_valid_tokens;  /* device int32, or NULL */
    int32_t persistent;
    int32_t y_format;                 /* MOE_Y_BF16 (0), MOE_Y_FP8 or MOE_Y_AUTO */
    const uint8_t *w13_packed;        /* moe_pack_weights(w13, N 2I, K H), or NULL */
    const uint8_t *w13_packed_scale;
    const uint8_t *w2_packed;         /* moe_pack_weights(w2, N H, K I), or NULL */
    const uint8_t *w2_packed_scale;
} moe_forward_args;

int moe_forward_ex(const moe_shape *shape, const moe_forward_args *args, void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * Weights packed for the packed-weight GEMMs ("full-expert DeepSeek
 * V4.1 Flash MegaMoE tuning", Changes and tuning: weight pipelining and the
 * B-matrix cache policy are among the knobs the pages search; this layout
 * is this library's own).  A weight array w [E, N, K/2] of MXFP4 codes with
 * exponents w_scale [E, N, K/32] (W13: N = 2I, K = H; W2: N = H, K = I) is
 * rewritten so that each 16-row group's 128-value K step is 1 KiB in the
 * scaled MFMA's operand order (lane l: row l mod 16, 16 code bytes from byte
 * 64 ks + 16 (l div 16) of the row) and its exponents four K steps to a
 * dword per lane:
 *   packed       [E][K/128][N/16][64 lanes][16 bytes]
 *   packed_scale [E][ceil(K/512)][N/16][64 lanes][4 bytes], byte j = the
 *                exponent of K step 4 q + j (zero past the last step).
 * One pass on `stream`, reading the inputs once; the caller owns every
 * buffer (moe_packed_codes_bytes / moe_packed_scales_bytes bytes, 16-byte
 * aligned).  MOE_EINVAL for E < 1, N not a multiple of 64, K not a multiple
 * of 128, E N K / 2 of 2^40 bytes or more, a NULL or misaligned pointer.
 * The packed copy is a second copy of the weights: pack once at load time.
 */
size_t moe_packed_codes_bytes(int32_t E, int32_t N, int32_t K);
size_t moe_packed_scales_bytes(int32_t E, int32_t N, int32_t K);
int moe_pack_weights(const uint8_t *w, const uint8_t *w_scale, int32_t E, int32_t N, int32_t K,
                     uint8_t *packed, uint8_t *packed_scale, void *stream);
/* The inverse: the logical arrays back from a packed pair (exponent bytes
 * past the last K step are ignored); the same sizes and refusals.  Packing
 * then unpacking gives back every byte. */
int moe_unpack_weights(const uint8_t *packed, const uint8_t *packed_scale, int32_t E, int32_t N,
                       int32_t K, uint8_t *w, uint8_t *w_scale, void *stream);

/*
 * moe_gemm1_swiglu and moe_gemm2 / moe_gemm2_fp8 on packed weights (the
 * packed-weight kernels moe_forward_ex runs when given them): the same
 * arguments and output bits, the weights replaced by moe_pack_weights of
 * w13 (N 2I, K H) or w2 (N H, K I).  moe_gemm2_packed writes bf16 rows
 * (y_bf16, with y_fp8 and y_scale NULL) or MX FP8 rows (y_fp8 and y_scale,
 * with y_bf16 NULL).  MOE_ENOTSUP where the shape's GEMM takes no packed
 * kernel (moe_get_tile_config gives other than 32 or 64 rows, or no tile).
 */
int moe_gemm1_swiglu_packed(const moe_shape *shape, const uint8_t *x_fp8,
                            const uint8_t *x_scale, const int32_t *counts,
                            const int32_t *offsets, const int32_t *row_route,
                            const uint8_t *w13_packed, const uint8_t *w13_packed_scale,
                            uint8_t *h_fp8, uint8_t *h_scale, void *stream);
int moe_gemm2_packed(const moe_shape *shape, const uint8_t *h_fp8, const uint8_t *h_scale,
                     const int32_t *counts, const int32_t *offsets, const uint8_t *w2_packed,
                     const uint8_t *w2_packed_scale, uint16_t *y_bf16, uint8_t *y_fp8,
                     uint8_t *y_scale, void *stream);

/*
 * Tuned tile table ("[FlyDSL] Add full-expert DeepSeek V4.1 Flash MegaMoE
 * tuning for gfx950", tuning: one kernel config per shape and token bucket,
 * a token count between two buckets taking the larger bucket, every
 * candidate checked against the reference config).  An entry names a GEMM
 * (1: GEMM1 + SwiGLU + requant, 2: GEMM2), the shape fields it applies to
 * (H, I, K, E_total, E_local exactly), the bucket's largest T, and the tile
 * of the LDS-tiled kernel: rows bm x weight rows bn, ku K steps per stage,
 * one of (32, 128, 2), (64, 128, 2), (64, 256, 1), (128, 128, 1),
 * (128, 256, 1), (256, 256, 1).  A call takes the entry of its GEMM and
 * shape with the smallest max_tokens >= T; with none, the built-in rule
 * (by the expected rows per expert T*K/E_total: 32-row tiles up to 16,
 * 64-row up to 96, else 128-row, and 256-row from 512).  Every
 * tile gives the same bits (the K order of each sum does not depend on it).  The table applies where the tiled kernels run (H or I at
 * least 512); an entry whose N tile does not divide the output columns
 * (GEMM1: I by bn/2, GEMM2: H by bn) is passed over.
 */
typedef struct {
    int32_t gemm;
    int32_t H, I, K, E_total, E_local;
    int32_t max_tokens;
    int32_t bm, bn, ku;
} moe_tile_entry;

/* Replace the table with n entries (copied; n = 0 clears it).  MOE_EINVAL
 * for an unknown tile or GEMM.  Takes effect for launches issued after it
 * returns; safe to call while other threads launch. */
int moe_set_tile_table(const moe_tile_entry *entries, int32_t n);

/* The tile a launch of GEMM `gemm` (1 or 2) with this shape would take, in
 * out->bm, bn, ku (the other fields copied from the shape); MOE_ENOTSUP where
 * the register-streaming kernels serve the shape. */
int moe_get_tile_config(const moe_shape *shape, int32_t gemm, moe_tile_entry *out);

/* Static description of a return code. */
const char *moe_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* MOE_A8W4_H */
