"""Helpers of the GPU tests: upload synthetic cases and run the layer's
steps through the C ABI binding."""

from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import dispatch_grouped_gemm_amd as moe
import oracle
import synth

DEV = torch.device("cuda", 0)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


@functools.lru_cache(maxsize=2)
def cached_case(name: str):
    return synth.make_case(name)


def upload(case: dict) -> dict:
    return {k: dev(v) for k, v in case.items() if isinstance(v, np.ndarray)}


def shape_of(spec) -> moe.MoeShape:
    return moe.MoeShape.of(spec)


def run_dispatch(spec, ids_dev: torch.Tensor) -> moe.DispatchBuffers:
    shape = shape_of(spec)
    d = moe.alloc_dispatch(shape, DEV)
    moe.moe_dispatch(shape, ids_dev, d)
    return d


def run_steps(case: dict, g: dict | None = None) -> dict:
    """All four steps one after the other; returns device tensors."""
    spec = case["spec"]
    shape = shape_of(spec)
    g = g or upload(case)
    d = run_dispatch(spec, g["topk_ids"])
    R = max(moe.moe_row_capacity(shape), 1)
    h = torch.zeros((R, spec.I), dtype=torch.uint8, device=DEV)
    hs = torch.zeros((R, spec.I // 32), dtype=torch.uint8, device=DEV)
    y = torch.zeros((R, spec.H), dtype=torch.uint16, device=DEV)
    out = torch.zeros((spec.T, spec.H), dtype=torch.uint16, device=DEV)
    moe.moe_gemm1_swiglu(shape, g["x_fp8"], g["x_scale"], d, g["w13"], g["w13_scale"], h, hs)
    moe.moe_gemm2(shape, h, hs, d, g["w2"], g["w2_scale"], y)
    moe.moe_combine(shape, g["topk_w"], d.route_row, y, out)
    return dict(d=d, h=h, hs=hs, y=y, out=out)


def run_forward(case: dict, g: dict | None = None, ws: torch.Tensor | None = None,
                persistent: bool = False):
    spec = case["spec"]
    shape = shape_of(spec)
    g = g or upload(case)
    if ws is None:
        ws = moe.alloc_workspace(shape, DEV)
    out = torch.zeros((spec.T, spec.H), dtype=torch.uint16, device=DEV)
    moe.moe_forward(shape, g["x_fp8"], g["x_scale"], g["topk_ids"], g["topk_w"], g["w13"],
                    g["w13_scale"], g["w2"], g["w2_scale"], out, ws, persistent=persistent)
    return out


def bf16_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def sample_tokens(case: dict, n_routed: int = 6, n_empty: int = 2) -> np.ndarray:
    """Tokens spread over the batch: some with local routes, some without."""
    s = case["spec"]
    ids = case["topk_ids"]
    e = ids.astype(np.int64) - s.expert_begin
    loc = ((ids >= 0) & (ids < s.E_total) & (e >= 0) & (e < s.E_local)).any(axis=1)
    routed = np.nonzero(loc)[0]
    empty = np.nonzero(~loc)[0]
    pick = []
    if routed.size:
        pick += list(routed[np.linspace(0, routed.size - 1, min(n_routed, routed.size)).astype(int)])
    if empty.size:
        pick += list(empty[np.linspace(0, empty.size - 1, min(n_empty, empty.size)).astype(int)])
    return np.unique(np.array(pick, dtype=np.int64))


def log_parity(what: str, **fields):
    """Append one JSON record of a layer check to $MOE_PARITY_LOG (if set):
    the literal max|err|/RMS against the oracle and how many elements lie
    beyond 2e-2 * RMS(ref)."""
    import json
    import os
    path = os.environ.get("MOE_PARITY_LOG")
    if not path:
        return
    rec = {"check": what}
    rec.update({k: (float(v) if isinstance(v, (np.floating, float)) else
                    int(v) if isinstance(v, (np.integer, int)) else v)
                for k, v in fields.items()})
    with open(path, "a") as f:
        f.write(json.dumps(rec) + "\n")


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |v| (8 significant bits)."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def assert_layer_close(got_bits: np.ndarray, ref_bits: np.ndarray, what: str = ""):
    """Every element within 2e-2 * RMS(ref) of the oracle, except that where
    one bf16 step of the reference element is larger than that bound the
    element may differ by that one step (two float32 sums of the same terms
    in different orders can round to neighbouring bf16 values).  An all-zero
    reference demands exact zeros.  Returns max|err| / RMS (literal)."""
    got = bf16_f64(got_bits)
    ref = bf16_f64(ref_bits)
    rms = float(np.sqrt((ref ** 2).mean())) if ref.size else 0.0
    if rms == 0.0:
        assert not np.any(got), what + ": reference is zero, output is not"
        return 0.0
    err = np.abs(got - ref)
    allowed = np.maximum(2e-2 * rms, bf16_ulp(ref))
    bad = err > allowed
    lit = float(err.max()) / rms
    over = int((err > 2e-2 * rms).sum())
    say("%s: %d of %d elements differ, max|err|/RMS %.4g, RMS %.4g, beyond 2e-2*RMS %d, "
        "over the bar %d" % (what, int((got != ref).sum()), got.size, lit, rms, over,
                             int(bad.sum())))
    log_parity(what, elements=got.size, differ=int((got != ref).sum()), max_err_over_rms=lit,
               beyond_2e2_rms=over)
    assert not bad.any(), "%s: %d elements beyond max(2e-2 * RMS, 1 bf16 step), worst %.4g * RMS" % (
        what, int(bad.sum()), float((err - allowed).max() + 2e-2 * rms) / rms)
    return lit


_E4M3 = None


def e4m3_values() -> np.ndarray:
    global _E4M3
    if _E4M3 is None:
        import oracle
        _E4M3 = np.array([oracle.e4m3_decode(c) for c in range(256)], np.float64)
    return _E4M3


def dequant_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    return e4m3_values()[codes] * np.exp2(np.repeat(scales.astype(np.float64) - 127, 32, axis=1))


def e4m3_step(v: np.ndarray, E: np.ndarray) -> np.ndarray:
    """Spacing of the e4m3 values (scaled by 2^E) at |v|: 2^(E - 9) in the
    subnormal range below 2^(E - 6), else 2^(E + b - 3) for the binade
    2^b <= |v| / 2^E (b at most 8, where values saturate at 448)."""
    a = np.abs(v) * np.exp2(-E)
    b = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return np.exp2(E + np.minimum(b, 8) - 3)


def y8_moves_allowed(bound: np.ndarray, y: np.ndarray, E: np.ndarray) -> float:
    """How many FP8 y codes may move when each float32 sum may be off by
    its MFMA bound: a code moves only if its sum lies within that error of a
    rounding midpoint, at most min(1, 2 b / s) per code (s the e4m3 step)."""
    return float(np.minimum(1.0, 2.0 * bound / e4m3_step(y, E)).sum())


def gemm1_mfma_bound(case: dict, routes: np.ndarray) -> np.ndarray:
    """How far the GPU's pre-quantisation value of h may lie from the
    oracle's, per route slot and column [n, I]: inside one 32-value K block
    the scaled MFMA aligns the products to the largest and keeps about 14
    bits below it, so a block sum is off by at most 32 * 2^-14 of its largest
    term, in total at most 2^-9 * sum|x * w| for the gate sum g and the up
    sum u; carried through the clamped SwiGLU (|d silu / dg| <= 1.1).  The
    bound matters only where the sums cancel."""
    from dense_ref import dec_fp4_rows, dec_fp8_rows
    spec = case["spec"]
    routes = np.asarray(routes, dtype=np.int64)
    I = spec.I
    toks = routes // spec.K
    eids = case["topk_ids"].reshape(-1)[routes].astype(np.int64) - spec.expert_begin
    x = dec_fp8_rows(case["x_fp8"][toks], case["x_scale"][toks])
    g = np.zeros((routes.size, I))
    u = np.zeros((routes.size, I))
    ag = np.zeros((routes.size, I))
    au = np.zeros((routes.size, I))
    for e in np.unique(eids):
        sel = eids == e
        W = dec_fp4_rows(case["w13"][e], case["w13_scale"][e])
        g[sel] = x[sel] @ W[:I].T
        u[sel] = x[sel] @ W[I:].T
        ag[sel] = np.abs(x[sel]) @ np.abs(W[:I]).T
        au[sel] = np.abs(x[sel]) @ np.abs(W[I:]).T
    gc = np.minimum(g, spec.gate_limit)
    uc = np.clip(u, -spec.up_limit, spec.up_limit)
    with np.errstate(over="ignore"):
        silu = gc / (1.0 + np.exp(-gc))
    return 1.1 * np.abs(uc) * 2.0 ** -9 * ag + np.abs(silu) * 2.0 ** -9 * au


def run_steps_y8(case: dict, g: dict | None = None) -> dict:
    """The four steps with MX FP8 y rows (moe_gemm2_fp8, moe_combine_fp8)."""
    spec = case["spec"]
    shape = shape_of(spec)
    g = g or upload(case)
    d = run_dispatch(spec, g["topk_ids"])
    R = max(moe.moe_row_capacity(shape), 1)
    h = torch.zeros((R, spec.I), dtype=torch.uint8, device=DEV)
    hs = torch.zeros((R, spec.I // 32), dtype=torch.uint8, device=DEV)
    yc = torch.zeros((R, spec.H), dtype=torch.uint8, device=DEV)
    ys = torch.zeros((R, spec.H // 32), dtype=torch.uint8, device=DEV)
    out = torch.zeros((spec.T, spec.H), dtype=torch.uint16, device=DEV)
    moe.moe_gemm1_swiglu(shape, g["x_fp8"], g["x_scale"], d, g["w13"], g["w13_scale"], h, hs)
    moe.moe_gemm2_fp8(shape, h, hs, d, g["w2"], g["w2_scale"], yc, ys)
    moe.moe_combine_fp8(shape, g["topk_w"], d.route_row, yc, ys, out)
    return dict(d=d, h=h, hs=hs, yc=yc, ys=ys, out=out)


def check_layer(case: dict, tokens: np.ndarray, out_bits: np.ndarray, steps: dict,
                what: str = "", max_flip_rate: float = 1e-3):
    """The layer output of `tokens` against the oracle.

    The FP8 requantisation of the intermediate is an integer decision taken
    from float32 sums: the GPU sums each 32-term K block inside the MFMA
    (about 14 bits below its largest product), the oracle sums sequentially,
    so a value that sits at an e4m3 rounding boundary may round the other
    way.  Such a flip is accepted when the GPU code is a valid rounding of
    the oracle's own pre-quantisation value (within one e4m3 step of it, plus
    the MFMA summation bound where the GEMM1 sums cancel) and flips are rare; its effect on the output, |w| * |W2[:, i]| * |step|
    (float64, oracle-decoded W2), is added to that token's allowance.

    The GPU keeps y in bf16 (the pages' expert output rows) where the oracle
    keeps float32: each kept route adds |w| * half a bf16 step of its y value
    to the allowance of its token.  Every other difference must be within
    max(2e-2 * RMS(ref), one bf16 step).

    With MX FP8 y rows (steps holding "yc" and "ys") the reference is the
    oracle's FP8-y layer; each y code that moved adds |w| * |its value
    change| to the token's allowance instead of the half bf16 step, and
    must lie within one e4m3 step (larger block scale) of the oracle's
    float32 y, widened by the MFMA bound of its sum and the effect of the
    route's requant flips; moved y codes are held to max_flip_rate in the
    routes without a requant flip."""
    from dense_ref import dec_fp4_rows, dec_fp8_rows
    import oracle
    spec = case["spec"]
    K = spec.K
    y8 = "yc" in steps
    tokens = np.asarray(tokens, dtype=np.int64)
    ref_bits = oracle.moe_layer(case, tokens, y_fp8=y8)
    rr = host(steps["d"].route_row).reshape(spec.T, K)
    slots = [(i, t * K + k) for i, t in enumerate(tokens) for k in range(K) if rr[t, k] >= 0]
    allowance = np.zeros((tokens.size, spec.H))
    n_codes = n_flips = 0
    y8_codes = y8_moved = y8_moved_all = 0
    y8_allowed = 0.0
    w2abs = {}
    if slots:
        routes = np.array([r for _, r in slots], np.int64)
        orc = oracle.routes_ffn(case, routes)
        rows = rr.reshape(-1)[routes]
        hq_gpu = dequant_rows(host(steps["h"])[rows], host(steps["hs"])[rows])
        hq_ref = dequant_rows(orc["h_codes"], orc["h_scale"])
        hv = orc["hv"].astype(np.float64)
        yabs = np.abs(orc["y"].astype(np.float64))
        flips = hq_gpu != hq_ref
        n_codes, n_flips = flips.size, int(flips.sum())
        # a valid rounding: within one e4m3 step (1/8 of the larger magnitude,
        # or a subnormal step of the block) of the oracle's own value
        blk = np.repeat(orc["h_scale"].astype(np.float64) - 127, 32, axis=1)
        step = np.maximum(np.abs(hq_gpu), np.abs(hq_ref)) / 8 + np.exp2(blk - 9)
        far = flips & (np.abs(hq_gpu - hv) > step * 1.0001)
        if far.any():
            sel = np.nonzero(far.any(axis=1))[0]
            dh = gemm1_mfma_bound(case, routes[sel])
            ok = np.abs(hq_gpu[sel] - hv[sel]) <= (step[sel] + dh) * 1.0001
            assert ok[far[sel]].all(), what + ": invalid code"
        ids = case["topk_ids"].reshape(-1)
        w = case["topk_w"].reshape(-1)
        if y8:
            yg = dequant_rows(host(steps["yc"])[rows], host(steps["ys"])[rows])
            rc, rs = oracle.quant_rows_f32(orc["y"])
            yr = dequant_rows(rc, rs)
            ymoved = yg != yr
            Eg = np.repeat(host(steps["ys"])[rows].astype(np.float64) - 127, 32, axis=1)
            Er = np.repeat(rs.astype(np.float64) - 127, 32, axis=1)
        for j, (i, r) in enumerate(slots):
            e = int(ids[r]) - spec.expert_begin
            cols = np.nonzero(flips[j])[0]
            dy = np.zeros(spec.H)
            if cols.size:
                W2c = dec_fp4_rows(case["w2"][e], case["w2_scale"][e])[:, cols]
                dy = np.abs(W2c) @ np.abs(hq_gpu[j, cols] - hq_ref[j, cols])
                allowance[i] += abs(float(w[r])) * dy
            if not y8:
                allowance[i] += abs(float(w[r])) * bf16_ulp(yabs[j] * (1 + 2.0 ** -7)) / 2
                continue
            mc = np.nonzero(ymoved[j])[0]
            y8_moved_all += mc.size
            if cols.size == 0:
                # no requant flip in this route: its moved y codes count
                # against what the MFMA bound of its sums allows
                y8_codes += spec.H
                y8_moved += mc.size
                if e in w2abs:
                    W2e = w2abs[e]
                else:
                    W2e = np.abs(dec_fp4_rows(case["w2"][e], case["w2_scale"][e]))
                    if spec.H * spec.I <= 1 << 22:
                        w2abs[e] = W2e
                y8_allowed += y8_moves_allowed(2.0 ** -12 * (W2e @ np.abs(hq_gpu[j])),
                                               orc["y"][j].astype(np.float64), Er[j])
            if mc.size == 0:
                continue
            allowance[i, mc] += abs(float(w[r])) * np.abs(yg[j, mc] - yr[j, mc])
            # each moved code: one e4m3 step of the oracle's value at the
            # larger block scale, widened by the MFMA bound of its sum and
            # the requant flips' effect
            W2m = np.abs(dec_fp4_rows(case["w2"][e][mc], case["w2_scale"][e][mc]))
            mfma = 2.0 ** -12 * (W2m @ np.abs(hq_gpu[j]))
            yo = orc["y"][j, mc].astype(np.float64)
            E = np.maximum(Eg[j, mc], Er[j, mc])
            slack = mfma + dy[mc]
            step = (np.maximum(np.abs(yg[j, mc]), np.abs(yo) + slack) / 8 + np.exp2(E - 9)
                    + np.maximum(np.abs(yo) + slack - 448.0 * np.exp2(Eg[j, mc]), 0))
            assert (np.abs(yg[j, mc] - yo) <= (step + slack) * 1.0001).all(), \
                what + ": a y code is not a rounding of the oracle's y"
    got = bf16_f64(out_bits)
    ref = bf16_f64(ref_bits)
    rms = float(np.sqrt((ref ** 2).mean())) if ref.size else 0.0
    if rms == 0.0:
        assert not np.any(got), what + ": reference is zero, output is not"
        return 0.0
    err = np.abs(got - ref)
    bar = np.maximum(2e-2 * rms, bf16_ulp(ref))
    beyond = err > bar + allowance * 1.0001 + 1e-6 * rms
    lit = float(err.max()) / rms
    over = int((err > 2e-2 * rms).sum())
    say("%s: %d tokens, %d routes, %d of %d elements differ, max|err|/RMS %.4g (RMS %.4g), "
        "beyond 2e-2*RMS %d; requant flips %d of %d codes; beyond the bar without a flip to "
        "explain it: %d" % (what, tokens.size, len(slots), int((got != ref).sum()), got.size, lit,
                            rms, over, n_flips, n_codes, int(beyond.sum())))
    extra = {}
    if y8:
        say("  FP8 y rows: %d y codes moved; in the routes without a requant flip %d of %d "
            "(the MFMA bound allows %.1f)" % (y8_moved_all, y8_moved, y8_codes, y8_allowed))
        extra = dict(y_fp8=1, y8_codes_no_requant_flip=y8_codes, y8_moved=y8_moved_all,
                     y8_moved_no_requant_flip=y8_moved, y8_moves_allowed=y8_allowed)
    log_parity(what, tokens=tokens.size, routes=len(slots), elements=got.size,
               differ=int((got != ref).sum()), max_err_over_rms=lit, beyond_2e2_rms=over,
               requant_flips=n_flips, requant_codes=n_codes, **extra)
    assert not beyond.any(), what + ": elements beyond the bar"
    if n_codes:
        assert n_flips <= max(4, max_flip_rate * n_codes), what + ": too many requant flips"
    if y8_codes:
        assert y8_moved <= y8_allowed, what + ": more moved y codes than the MFMA bound allows"
    return lit


def check_dispatch(spec, ids: np.ndarray, d, num_valid=None):
    """GPU dispatch buffers against the oracle: compact bit-exact, fixed-slot
    as sets of routes per expert segment."""
    ref = oracle.dispatch(spec, ids, num_valid=num_valid)
    counts, offsets, status = host(d.counts), host(d.offsets), host(d.status)
    np.testing.assert_array_equal(counts, ref["counts"])
    np.testing.assert_array_equal(offsets, ref["offsets"])
    np.testing.assert_array_equal(status, ref["status"])
    rr = host(d.route_row)[:spec.T * spec.K]
    row_route = host(d.row_route)
    if spec.dispatch_mode == 0:
        total = int(offsets[-1])
        np.testing.assert_array_equal(row_route[:total], ref["row_route"][:total])
        np.testing.assert_array_equal(rr, ref["route_row"])
    else:
        C = spec.capacity
        for e in range(spec.E_local):
            kept = min(int(counts[e]), C)
            seg = row_route[e * C:e * C + kept]
            refseg = ref["row_route"][e * C:e * C + kept]
            if counts[e] <= C:
                np.testing.assert_array_equal(np.sort(seg), np.sort(refseg))
            else:
                # an overflowing segment holds `kept` distinct routes, each a
                # valid slot of this expert (which of them win is a race)
                assert len(set(seg.tolist())) == kept
                eff = ids if num_valid is None else oracle.pad_rows(ids, num_valid)
                mine = np.nonzero(eff.reshape(-1) == spec.expert_begin + e)[0]
                assert np.isin(seg, mine).all(), e
            assert (row_route[e * C + kept:(e + 1) * C] == -1).all()  # untouched
        kept_r = np.nonzero(rr >= 0)[0]
        np.testing.assert_array_equal(row_route[rr[kept_r]], kept_r)
        assert ((rr >= 0) == (ref["route_row"] >= 0)).all() or status[1] > 0
    return ref


def boundary_tokens(case: dict, d, route_budget: int = 160, bms=(32, 64, 128, 256),
                    seed: int = 0) -> np.ndarray:
    """Tokens whose routes sit at the edges of the row tiles the GEMMs cut
    (first and last row of a tile of every row count in `bms`, the last row
    of each expert's segment), the most loaded expert first, then the other
    experts in turn, until the tokens hold about `route_budget` local routes;
    plus two tokens without a local route.  `d` holds the GPU's dispatch
    buffers (checked against the oracle's elsewhere)."""
    spec = case["spec"]
    K = spec.K
    rng = np.random.default_rng(seed)
    counts, offsets = host(d.counts), host(d.offsets)
    row_route = host(d.row_route)
    used = np.minimum(counts, spec.capacity) if spec.dispatch_mode == 1 else counts
    ids = case["topk_ids"]
    e_of = ids.astype(np.int64) - spec.expert_begin
    loc = (ids >= 0) & (ids < spec.E_total) & (e_of >= 0) & (e_of < spec.E_local)
    per_tok = loc.sum(axis=1)
    rows_by_expert = []
    for e in np.argsort(-used, kind="stable"):
        n = int(used[e])
        if n == 0:
            continue
        cand = [n - 1]
        for bm in bms:
            tiles = (n + bm - 1) // bm
            picks = {0, tiles - 1}
            if tiles > 2:
                picks.add(int(rng.integers(1, tiles - 1)))
            for c in sorted(picks):
                cand += [c * bm, min((c + 1) * bm, n) - 1]
        rows_by_expert.append([int(offsets[e]) + r for r in dict.fromkeys(cand)])
    toks, routes = [], 0
    depth = 0
    while routes < route_budget and any(depth < len(r) for r in rows_by_expert):
        for rows in rows_by_expert:
            if depth < len(rows) and routes < route_budget:
                t = int(row_route[rows[depth]]) // K
                if t not in toks:
                    toks.append(t)
                    routes += int(per_tok[t])
        depth += 1
    empty = np.nonzero(per_tok == 0)[0]
    if empty.size:
        toks += [int(empty[0]), int(empty[-1])]
    return np.unique(np.array(toks, dtype=np.int64))


CANARY = 0x5A


def with_canary(t: torch.Tensor, nbytes: int = 4096):
    """(view, guard): `view` is t's shape over a buffer `nbytes` longer whose
    tail holds the canary byte; guard() asserts the tail is untouched."""
    n = t.numel() * t.element_size()
    buf = torch.full((n + nbytes,), CANARY, dtype=torch.uint8, device=t.device)
    buf[:n].copy_(t.reshape(-1).view(torch.uint8) if n else buf[:0])
    view = buf[:n].view(t.dtype).reshape(t.shape)

    def guard(what=""):
        tail = buf[n:].cpu().numpy()
        assert (tail == CANARY).all(), "%s: %d bytes written past the end" % (
            what, int((tail != CANARY).sum()))
    return view, guard
