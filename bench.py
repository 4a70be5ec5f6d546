#!/usr/bin/env python3
"""Benchmark of one GPU's share of the a8w4 MoE expert layer on MI355X.

A step is one moe_forward (dispatch, GEMM1 + SwiGLU + FP8 requant, GEMM2,
combine) over one synthetic batch whose inputs and weights are already
resident in HBM.  The layer is captured once in a HIP graph and replayed;
W warmup replays, then exactly K timed replays between two device
synchronisations.

Reported (one JSON line):
  value        routed TFLOP/s (6*H*I FLOP per valid local route / step time)
               on a workload whose GEMMs are MFMA-bound (above the ridge
               point of 5.0 PFLOP/s over 8 TB/s), else weight GB/s
               (touched-expert W13+W2 bytes per step / step time)
  us_per_layer, routed_tflops, weight_gbps, hbm_frac (all algorithmic bytes
  / 8 TB/s), mfma_frac (routed FLOP / 5.0 PFLOP/s dense FP8)
  roofline     the dominant kernel (GEMM1 + SwiGLU + requant): its
               algorithmic bytes (HBM-bound workloads) or FLOP (MFMA-bound,
               above the ridge point) per launch / its mean launch time, the
               time taken with HIP events on the launch stream over K
               back-to-back launches of the four steps; traffic = its HBM
               bytes per launch from the rocprofv3 counter summary
  cpu_baseline the CPU oracle timed on a bounded sample of the same batch
               (whole tokens), scaled to the full batch by its routes
  cold         the same replay with the caches cold: before each replay a
               512 MiB buffer (twice the 256 MB Infinity Cache) is written,
               outside the timed span; each replay is timed alone with HIP
               events; median and spread over the replays
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("MoE layer µs + routed TFLOP/s + weight GB/s, fraction of roofline, "
          "1 MI355X")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, TFLOP/s
# the largest single-GPU workload: V4 prefill share, 8 x 8192 source tokens
DEFAULT_WORKLOAD = "v4_prefill_t65536_uniform"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-routes", type=int, default=128,
                   help="routes in the oracle's timed sample")
    p.add_argument("--kernel-iters", type=int, default=0,
                   help="launches per kernel for the roofline timing (default: steps)")
    p.add_argument("--cold-steps", type=int, default=20,
                   help="replays timed one by one after a 512 MiB cache flush (0: skip)")
    p.add_argument("--bf16-input", action="store_true",
                   help="time moe_forward_bf16: the layer from bf16 activation rows, their "
                        "MX FP8 quant included in the step")
    p.add_argument("--persistent", action="store_true",
                   help="time moe_forward_persistent (the whole layer in one persistent "
                        "launch)")
    p.add_argument("--packed", action="store_true",
                   help="pack W13 and W2 once with moe_pack_weights (before timing) and time "
                        "moe_forward_ex on the packed copies: the packed-weight GEMMs where "
                        "the tile rule takes 32- or 64-row tiles, the same bits")
    p.add_argument("--y-format", choices=["bf16", "fp8", "auto"], default="bf16",
                   help="expert output rows between GEMM2 and the combine: bf16 (the exact "
                        "layer, default), MX FP8 (a lossy option), or the size rule")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="instead of the layer, time a plain device copy of this many MiB "
                        "(the reference size for the HBM byte counters)")
    return p.parse_args()


def copy_reference(args):
    """A plain copy of known size: N bytes read and N bytes written per launch."""
    import torch
    n = args.copy_mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    s = (time.perf_counter() - t0) / args.steps
    print(json.dumps({"copy_bytes": n, "read_kib": n // 1024, "write_kib": n // 1024,
                      "us_per_copy": round(s * 1e6, 2),
                      "gbs": round(2 * n / s / 1e9, 1)}), flush=True)


def kernel_sources_digest() -> str:
    """sha256 over the HIP sources of the library (names and bytes)."""
    import hashlib
    d = os.path.join(ROOT, "dispatch_grouped_gemm_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".hpp", ".h")):
            h.update(name.encode())
            with open(os.path.join(d, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload: str, packed: bool = False):
    """HBM bytes per launch of the dominant kernel, from the rocprofv3 counter
    summary of this workload (with packed weights: <workload>_packed) under
    profiles/, or None when there is none or the kernel sources have changed
    since it was taken."""
    path = os.path.join(ROOT, "profiles", workload + ("_packed" if packed else "") + ".md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.split(":", 1)[0].strip() in (
                    "traffic_bytes_per_launch", "source_sha256", "traffic_kernel"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("source_sha256") != kernel_sources_digest():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def gemm1_algorithmic_bytes(spec, work) -> int:
    """What GEMM1 must read by the layer's own accounting (intermediates are
    implementation traffic and not counted): the W13 codes + exponents of
    each touched expert and the MX FP8 x row of each token with a local
    route."""
    H, I = spec.H, spec.I
    w13 = work["touched"] * (2 * I * H // 2 + 2 * I * H // 32)
    xin = work["tokens_with_route"] * (H + H // 32)
    return w13 + xin


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.copy_mib:
        copy_reference(args)
        return

    import torch

    import dispatch_grouped_gemm_amd as moe
    import synth

    dev = torch.device("cuda", 0)
    spec_name = args.workload
    case = synth.make_case(spec_name)
    spec = case["spec"]
    work = synth.algorithmic_work(case)
    shape = moe.MoeShape.of(spec)
    g = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev)
         for k, v in case.items() if isinstance(v, np.ndarray)}
    ws = moe.alloc_workspace(shape, dev)
    out = torch.zeros((spec.T, spec.H), dtype=torch.uint16, device=dev)

    y_format = {"bf16": moe.Y_BF16, "fp8": moe.Y_FP8, "auto": moe.Y_AUTO}[args.y_format]
    y8 = moe.moe_resolve_y_format(shape, y_format) == moe.Y_FP8

    pk = None
    if args.packed:
        pk = moe.pack_layer_weights(g["w13"], g["w13_scale"], g["w2"], g["w2_scale"])
        torch.cuda.synchronize()
    packed_gemm = [pk is not None and moe.get_tile_config(shape, k) is not None
                   and moe.get_tile_config(shape, k)["bm"] in (32, 64) for k in (1, 2)]

    def forward(stream=None):
        if y_format != moe.Y_BF16 or (args.bf16_input and args.persistent) or pk is not None:
            xa = (dict(x_bf16=g["x_bf16"]) if args.bf16_input
                  else dict(x_fp8=g["x_fp8"], x_scale=g["x_scale"]))
            moe.moe_forward_ex(shape, g["topk_ids"], g["topk_w"], g["w13"], g["w13_scale"],
                               g["w2"], g["w2_scale"], out, ws, persistent=args.persistent,
                               y_format=y_format, stream=stream, packed=pk, **xa)
            return
        if args.bf16_input:
            moe.moe_forward_bf16(shape, g["x_bf16"], g["topk_ids"], g["topk_w"], g["w13"],
                                 g["w13_scale"], g["w2"], g["w2_scale"], out, ws, stream=stream)
            return
        moe.moe_forward(shape, g["x_fp8"], g["x_scale"], g["topk_ids"], g["topk_w"], g["w13"],
                        g["w13_scale"], g["w2"], g["w2_scale"], out, ws, stream=stream,
                        persistent=args.persistent)

    # ---- whole layer: graph replays ---------------------------------------------
    forward()
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        forward(stream=torch.cuda.current_stream())
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps

    # ---- whole layer with cold caches: flush, then one timed replay ---------------
    cold = None
    if args.cold_steps > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        st0 = torch.cuda.current_stream()
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.cold_steps)]
        for a, b in cev:
            flush.fill_(1)
            a.record(st0)
            graph.replay()
            b.record(st0)
        torch.cuda.synchronize()
        cus = np.array([a.elapsed_time(b) * 1e3 for a, b in cev])
        cold = {"us_per_layer": round(float(np.median(cus)), 2),
                "min": round(float(cus.min()), 2), "max": round(float(cus.max()), 2),
                "replays": args.cold_steps, "flush_mib": 512}
        del flush

    # ---- per-kernel times: the four steps back to back on one stream --------------
    d = moe.alloc_dispatch(shape, dev)
    R = max(moe.moe_row_capacity(shape), 1)
    h = torch.empty((R, spec.I), dtype=torch.uint8, device=dev)
    hs = torch.empty((R, spec.I // 32), dtype=torch.uint8, device=dev)
    y = torch.empty((R, spec.H), dtype=torch.uint16, device=dev)
    y8c = torch.empty((R, spec.H), dtype=torch.uint8, device=dev) if y8 else None
    y8s = torch.empty((R, spec.H // 32), dtype=torch.uint8, device=dev) if y8 else None
    st = torch.cuda.current_stream()
    iters = args.kernel_iters or args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(iters)]
    xq = torch.empty((spec.T, spec.H), dtype=torch.uint8, device=dev)
    xqs = torch.empty((spec.T, spec.H // 32), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2e8))   # keep the GPU busy while the launches are queued
    for i in range(iters):
        e = ev[i]
        e[5].record(st)
        if args.bf16_input:
            moe.moe_quant_mxfp8(shape, g["x_bf16"], xq, xqs, stream=st)
        e[0].record(st)
        moe.moe_dispatch(shape, g["topk_ids"], d, stream=st)
        e[1].record(st)
        if packed_gemm[0]:
            moe.moe_gemm1_swiglu_packed(shape, g["x_fp8"], g["x_scale"], d, pk, h, hs, stream=st)
        else:
            moe.moe_gemm1_swiglu(shape, g["x_fp8"], g["x_scale"], d, g["w13"], g["w13_scale"],
                                 h, hs, stream=st)
        e[2].record(st)
        if packed_gemm[1]:
            if y8:
                moe.moe_gemm2_packed(shape, h, hs, d, pk, y_fp8=y8c, y_scale=y8s, stream=st)
            else:
                moe.moe_gemm2_packed(shape, h, hs, d, pk, y_bf16=y, stream=st)
        elif y8:
            moe.moe_gemm2_fp8(shape, h, hs, d, g["w2"], g["w2_scale"], y8c, y8s, stream=st)
        else:
            moe.moe_gemm2(shape, h, hs, d, g["w2"], g["w2_scale"], y, stream=st)
        e[3].record(st)
        if y8:
            moe.moe_combine_fp8(shape, g["topk_w"], d.route_row, y8c, y8s, out, stream=st)
        else:
            moe.moe_combine(shape, g["topk_w"], d.route_row, y, out, stream=st)
        e[4].record(st)
    torch.cuda.synchronize()
    names = ["dispatch", "gemm1_swiglu", "gemm2", "combine"]
    kern_us = {n: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(iters)]))
               * 1e3 for j, n in enumerate(names)}
    if args.bf16_input:
        # the quant as a launch of its own (inside the layer it shares the
        # dispatch launch where the dispatch is one workgroup)
        kern_us = {"quant": float(np.mean([ev[i][5].elapsed_time(ev[i][0])
                                           for i in range(iters)])) * 1e3, **kern_us}
    status = d.status.cpu().numpy()

    us = ms_per_step * 1e3
    t_s = ms_per_step * 1e-3
    weight_gbs = work["weight_bytes"] / t_s / 1e9
    tflops = work["flop"] / t_s / 1e12
    g1_bytes = gemm1_algorithmic_bytes(spec, work)
    g1_flop = 4.0 * spec.H * spec.I * work["routes"]
    g1_s = kern_us["gemm1_swiglu"] * 1e-6
    # GEMM1 is bound by HBM below the ridge point of the FP8 MFMA peak and
    # HBM bandwidth (625 FLOP/byte), by the MFMA above it
    if g1_flop / g1_bytes > FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        roof = {"bound": "mfma", "kernel": "gemm1_swiglu",
                "achieved": round(g1_flop / g1_s / 1e12, 1), "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(g1_flop / g1_s / 1e12 / FP8_PEAK_TFLOPS, 4),
                "flop_per_launch": int(g1_flop)}
    else:
        roof = {"bound": "hbm", "kernel": "gemm1_swiglu",
                "achieved": round(g1_bytes / g1_s / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(g1_bytes / g1_s / 1e9 / HBM_PEAK_GBS, 4)}
    roof["traffic"] = recorded_traffic(spec_name, packed_gemm[0])
    roof["bytes_per_launch"] = int(g1_bytes)
    mfma_bound = roof["bound"] == "mfma"
    result = {
        "metric": METRIC,
        "value": round(tflops, 2) if mfma_bound else round(weight_gbs, 2),
        "unit": "TFLOP/s" if mfma_bound else "GB/s",
        "value_is": "routed TFLOP/s" if mfma_bound else "weight GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 x fp4e2m1, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": spec_name, "T": spec.T, "H": spec.H, "I": spec.I,
                   "K": spec.K, "E_total": spec.E_total, "E_local": spec.E_local,
                   "dispatch": "fixed-slot" if spec.dispatch_mode else "compact",
                   "capacity": spec.capacity, "routes": work["routes"],
                   "touched_experts": work["touched"],
                   "forward": "persistent" if args.persistent else "four launches",
                   "y_rows": "MX FP8" if y8 else "bf16",
                   "weights": ("packed (moe_pack_weights, once before timing); GEMMs on "
                               "them: %s" % ",".join(n for n, k in zip(("1", "2"), packed_gemm)
                                                     if k) or "none") if pk is not None
                   else "as given",
                   "input": "bf16 rows, quantised in the step" if args.bf16_input
                   else "MX FP8 rows"},
        "us_per_layer": round(us, 2),
        "routed_tflops": round(tflops, 3),
        "weight_gbps": round(weight_gbs, 2),
        "hbm_frac": round(work["bytes"] / t_s / 1e9 / HBM_PEAK_GBS, 4),
        "mfma_frac": round(tflops / FP8_PEAK_TFLOPS, 5),
        "kernel_us": {k: round(v, 2) for k, v in kern_us.items()},
        "dispatch_status": status.tolist(),
        "roofline": roof,
    }
    if cold is not None:
        cold["weight_gbps"] = round(work["weight_bytes"] / (cold["us_per_layer"] * 1e-6) / 1e9, 2)
        result["cold"] = cold

    if not args.no_cpu_baseline:
        import oracle
        ids = case["topk_ids"]
        e = ids.astype(np.int64) - spec.expert_begin
        loc = (ids >= 0) & (ids < spec.E_total) & (e >= 0) & (e < spec.E_local)
        per_tok = loc.sum(axis=1)
        toks = np.nonzero(per_tok)[0]
        rng = np.random.default_rng(0)
        rng.shuffle(toks)
        take = toks[np.cumsum(per_tok[toks]) <= args.cpu_routes]
        if take.size == 0:
            take = toks[:1]
        n_routes = int(per_tok[take].sum())
        omp_env = os.environ.get("OMP_NUM_THREADS")
        threads = int(omp_env or os.cpu_count() or 1)
        threads = max(1, min(threads, take.size))
        os.environ["OMP_NUM_THREADS"] = str(threads)
        oracle.lib()
        c0 = time.perf_counter()
        oracle.moe_layer(case, np.sort(take))
        cpu_s = time.perf_counter() - c0
        full_s = cpu_s * work["routes"] / max(n_routes, 1)
        full_us = full_s * 1e6
        result["cpu_baseline"] = {
            "value": (round(work["flop"] / full_s / 1e12, 6) if mfma_bound
                      else round(work["weight_bytes"] / full_s / 1e9, 4)),
            "unit": result["unit"], "cores": threads, "kind": "oracle",
            "us_per_layer": round(full_us, 1),
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "omp_num_threads": omp_env,
            "sample": "%d whole tokens holding %d of the batch's %d routes, %.2f s wall on %d "
                      "threads; time scaled by routes to the full batch (%.1f s)" % (
                          take.size, n_routes, work["routes"], cpu_s, threads, full_s)}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
