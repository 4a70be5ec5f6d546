"""Tile tuner for the expert GEMMs: one tile per (GEMM, shape, token bucket).

For each shape and each bucket's token count it draws a batch of synthetic
inputs on the GPU (bf16 N(0,1) activations quantised by moe_quant_mxfp8,
uniform random E2M1 weights with E8M0 exponents 2^-6..2^-3, top-k routing of
random scores), dispatches it once, then times every compiled tile of GEMM1
and of GEMM2 on it and keeps the fastest.  Every candidate's output is first
checked against the output of the built-in rule's tile (the reference
config): GEMM1's h codes and exponents, GEMM2's bf16 rows, relative L2
distance at most 1e-3 ("[FlyDSL] Add full-expert DeepSeek V4.1 Flash
MegaMoE tuning for gfx950", tuning: one config per shape and bucket, every
candidate checked against the reference config).  The tiles share the K
order of every sum, so the check finds identical bits in practice.

    python -m dispatch_grouped_gemm_amd.tune \\
        --shape H=7168,I=3072,K=6,E_total=384,E_local=48 \\
        --tokens 128,1024,2048,65536 --out tile_table.json

The JSON file is read back with ``dispatch_grouped_gemm_amd.load_tile_table``.
"""

from __future__ import annotations

import argparse
import json
import sys

import torch

import dispatch_grouped_gemm_amd as moe

TILES = [(32, 128, 2), (64, 128, 2), (64, 256, 1), (128, 128, 1), (128, 256, 1), (256, 256, 1)]


def parse_shape(text: str) -> dict:
    kv = dict(p.split("=") for p in text.split(","))
    out = {k: int(v) for k, v in kv.items()}
    for k in ("H", "I", "K", "E_total", "E_local"):
        if k not in out:
            raise SystemExit("--shape needs %s" % k)
    return out


def draw(shape: moe.MoeShape, dev, seed: int, pad_frac: float = 0.0) -> dict:
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    T, H, I, K, E, EL = shape.T, shape.H, shape.I, shape.K, shape.E_total, shape.E_local
    xb = torch.randn((T, H), generator=g, device=dev).to(torch.bfloat16)
    xq = torch.empty((T, H), dtype=torch.uint8, device=dev)
    xs = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
    moe.moe_quant_mxfp8(shape, xb, xq, xs)
    scores = torch.rand((T, E), generator=g, device=dev)
    ids = scores.topk(K, dim=1).indices.to(torch.int32).contiguous()
    npad = int(round(pad_frac * T * K))
    if npad:
        # -1 slots, uniform without replacement (the routing of padded ranks)
        flat = torch.randperm(T * K, generator=g, device=dev)[:npad]
        ids.view(-1)[flat] = -1

    def codes(*size):
        return torch.randint(0, 256, size, generator=g, device=dev, dtype=torch.uint8)

    def exps(*size):
        return torch.randint(121, 125, size, generator=g, device=dev, dtype=torch.uint8)

    return dict(x=xq, xs=xs, ids=ids, w13=codes(EL, 2 * I, H // 2), w13s=exps(EL, 2 * I, H // 32),
                w2=codes(EL, H, I // 2), w2s=exps(EL, H, I // 32))


def run(shape, d, inp, gemm, out):
    if gemm == 1:
        moe.moe_gemm1_swiglu(shape, inp["x"], inp["xs"], d, inp["w13"], inp["w13s"], out[0], out[1])
    else:
        moe.moe_gemm2(shape, out[0], out[1], d, inp["w2"], inp["w2s"], out[2])


def rel_l2(a: torch.Tensor, b: torch.Tensor) -> float:
    a = a.double()
    b = b.double()
    den = float(torch.linalg.vector_norm(b))
    return float(torch.linalg.vector_norm(a - b)) / (den if den > 0 else 1.0)


def dequant(codes: torch.Tensor, scales: torch.Tensor) -> torch.Tensor:
    v = codes.view(torch.float8_e4m3fn).to(torch.float64)
    e = torch.pow(2.0, scales.to(torch.float64) - 127.0)
    return v * e.repeat_interleave(32, dim=1)


def tune_bucket(base: dict, T: int, mode: int, capacity: int, iters: int, dev,
                pad_frac: float = 0.0) -> list:
    shape = moe.MoeShape(T=T, H=base["H"], I=base["I"], K=base["K"], E_total=base["E_total"],
                         E_local=base["E_local"], dispatch_mode=mode, capacity=capacity)
    inp = draw(shape, dev, seed=T, pad_frac=pad_frac)
    d = moe.alloc_dispatch(shape, dev)
    moe.moe_dispatch(shape, inp["ids"], d)
    R = max(moe.moe_row_capacity(shape), 1)
    entries = []
    for gemm in (1, 2):
        moe.set_tile_table([])
        if moe.get_tile_config(shape, gemm) is None:
            continue
        bufs = lambda: [torch.zeros((R, shape.I), dtype=torch.uint8, device=dev),
                        torch.zeros((R, shape.I // 32), dtype=torch.uint8, device=dev),
                        torch.zeros((R, shape.H), dtype=torch.uint16, device=dev)]
        ref = bufs()
        run(shape, d, inp, 1, ref)          # GEMM2 reads the reference h
        if gemm == 2:
            run(shape, d, inp, 2, ref)
        torch.cuda.synchronize()
        best = None
        for bm, bn, ku in TILES:
            e = dict(gemm=gemm, H=shape.H, I=shape.I, K=shape.K, E_total=shape.E_total,
                     E_local=shape.E_local, max_tokens=T, bm=bm, bn=bn, ku=ku)
            moe.set_tile_table([e])
            got = moe.get_tile_config(shape, gemm)
            if got is None or (got["bm"], got["bn"], got["ku"]) != (bm, bn, ku):
                # the N tile does not divide the output columns: passed over
                print("  gemm%d tile %s does not apply to this shape" % (gemm, (bm, bn, ku)))
                continue
            out = bufs()
            if gemm == 2:
                out[0].copy_(ref[0])
                out[1].copy_(ref[1])
            run(shape, d, inp, gemm, out)
            torch.cuda.synchronize()
            # rows no route fills stay zero in both
            if gemm == 1:
                err = rel_l2(dequant(out[0], out[1]), dequant(ref[0], ref[1]))
            else:
                err = rel_l2(out[2].view(torch.bfloat16), ref[2].view(torch.bfloat16))
            if not err <= 1e-3:
                print("  gemm%d tile %s rejected: rel-L2 %.3g" % (gemm, (bm, bn, ku), err))
                continue
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            for _ in range(3):
                run(shape, d, inp, gemm, out)
            ev[0].record()
            for _ in range(iters):
                run(shape, d, inp, gemm, out)
            ev[1].record()
            torch.cuda.synchronize()
            us = ev[0].elapsed_time(ev[1]) * 1e3 / iters
            print("  T=%d gemm%d tile %s: %.1f us (rel-L2 %.1g)" % (T, gemm, (bm, bn, ku), us, err),
                  flush=True)
            if best is None or us < best[0]:
                best = (us, e)
        moe.set_tile_table([])
        if best is not None:
            entries.append(best[1])
    return entries


def main(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--shape", action="append", required=True,
                   help="H=..,I=..,K=..,E_total=..,E_local=.. (repeatable)")
    p.add_argument("--tokens", required=True, help="bucket token counts, comma separated")
    p.add_argument("--fixed-capacity", type=int, default=0,
                   help="tune fixed-slot dispatch with this capacity (default: compact)")
    p.add_argument("--pad-frac", type=float, default=0.0,
                   help="fraction of top-k slots set to -1 in the drawn routing")
    p.add_argument("--iters", type=int, default=10)
    p.add_argument("--out", required=True)
    args = p.parse_args(argv)
    dev = torch.device("cuda", 0)
    entries = []
    for text in args.shape:
        base = parse_shape(text)
        for T in sorted(int(t) for t in args.tokens.split(",")):
            print("shape %s T=%d" % (text, T), flush=True)
            mode = 1 if args.fixed_capacity else 0
            entries += tune_bucket(base, T, mode, args.fixed_capacity, args.iters, dev,
                                   args.pad_frac)
    with open(args.out, "w") as f:
        json.dump({"entries": entries}, f, indent=1)
    print("wrote %d entries to %s" % (len(entries), args.out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
