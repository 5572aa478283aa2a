#!/usr/bin/env python3
"""Benchmark: Cassandra draft GEMV on one Llama-3-8B-shaped decoder layer, bs=1.

One step = the draft GEMVs of one decode step of the layer, i.e. the four
fused projections q|k|v (6144x4096), o (4096x4096), gate|up (28672x4096) and
down (4096x14336), each a cass_draft_gemv call that streams the speculation
bytes of that matrix from HBM.  Steps rotate over `--copies` distinct encoded
layers so the bytes come from HBM, not from the 256 MB last-level cache.

Prints ONE JSON line: value = speculation-stream bytes / second over the timed
steps (GB/s), plus the roofline of the GEMV kernel (HIP events around every
launch), per-row timings of the other hot-path calls (encode, verify GEMM N=5,
reconstruct, draft decode) and the CPU oracle timed on a row sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MATS = ("qkv", "o", "gu", "down")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--keep", type=float, default=0.3)
    ap.add_argument("--mant", type=int, default=3)
    ap.add_argument("--block", type=int, default=256)
    ap.add_argument("--copies", type=int, default=8)
    ap.add_argument("--sweep", action="store_true", help="also time the 3x3 keep x mant grid")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def torch_layer(torch, shapes, gen, sigma=0.02, outlier_frac=0.01):
    """A further seeded layer drawn on the GPU (torch generator), same recipe:
    N(0, sigma^2) rounded to bf16, 1% of input columns x10."""
    out = {}
    parts = {}
    for name, (r, c) in shapes.items():
        a = torch.randn((r, c), generator=gen, device="cuda", dtype=torch.float32) * sigma
        cols = torch.randperm(c, generator=gen, device="cuda")[: int(round(outlier_frac * c))]
        a[:, cols] *= 10.0
        parts[name] = a.to(torch.bfloat16).view(torch.int16)
        del a
    out["qkv"] = torch.cat([parts["q"], parts["k"], parts["v"]], 0)
    out["o"] = parts["o"]
    out["gu"] = torch.cat([parts["gate"], parts["up"]], 0)
    out["down"] = parts["down"]
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the draft GEMV streams one GPU's share of the "
              "weights and needs no collective; run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_level_weight_amd as cass
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cass.lib()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    dev16 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).cuda()

    # ---- inputs: layer 0 from the numpy recipe, further copies from a seeded torch generator
    t0 = time.time()
    layer0 = synth.fused_layer(synth.LLAMA3_8B, config=2, layer=0, outlier_frac=0.01)
    layers = [{k: dev16(v) for k, v in layer0.items()}]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2_000_001)
    for _ in range(1, args.copies):
        layers.append(torch_layer(torch, synth.LLAMA3_8B, gen))
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s")

    def encode_layer(L, keep, mant, ws):
        return {n: cass.encode(L[n], synth.keep_count(keep, L[n].shape[1]), mant,
                               block=args.block, ws=ws) for n in MATS}

    ws = torch.empty(cass.cass_encode_ws_bytes(28672, 4096, cass._params(1, 3, args.block, 1)),
                     dtype=torch.uint8, device="cuda")
    t0 = time.time()
    encs = [encode_layer(L, args.keep, args.mant, ws) for L in layers]
    torch.cuda.synchronize()
    enc_s = time.time() - t0
    log(f"encoded {len(encs)} layers in {enc_s:.1f}s")

    # activations (bs=1): x for q|k|v and gate|up (hidden 4096), o input (4096), down input (14336)
    xs = {n: dev16(synth.activations(1, layer0[n].shape[1], 2, t0=i)) for i, n in enumerate(MATS)}
    ys = {n: torch.empty((1, layer0[n].shape[0]), dtype=torch.float32, device="cuda") for n in MATS}
    spec_bytes = {n: encs[0][n].spec_bytes for n in MATS}
    step_bytes_each = [sum(e[n].spec_bytes for n in MATS) for e in encs]

    def step(i, events=None):
        e = encs[i % len(encs)]
        for j, n in enumerate(MATS):
            if events is not None:
                events[j][0].record(stream)
            cass.cass_draft_gemv(e[n].desc, xs[n], ys[n], stream)
            if events is not None:
                events[j][1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region 1: whole steps, back to back
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    total_bytes = sum(step_bytes_each[i % len(encs)] for i in range(args.steps))
    value = total_bytes / (total_ms * 1e-3) / 1e9

    # timed region 2: HIP events around every GEMV launch (kernel durations)
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in MATS]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, ev[i])
    torch.cuda.synchronize()
    kern_ms = {n: [] for n in MATS}
    kern_bytes = 0  # speculation bytes
    alg_bytes = 0   # + x read (2*cols) + y written (4*rows)
    for i in range(args.steps):
        for j, n in enumerate(MATS):
            kern_ms[n].append(ev[i][j][0].elapsed_time(ev[i][j][1]))
            e = encs[i % len(encs)][n]
            kern_bytes += e.spec_bytes
            alg_bytes += e.spec_bytes + 2 * e.cols + 4 * e.rows
    sum_ms = sum(sum(v) for v in kern_ms.values())
    kernel_gbs = kern_bytes / (sum_ms * 1e-3) / 1e9
    per_matrix = {n: {"spec_MB": spec_bytes[n] / 1e6,
                      "avg_us": 1e3 * float(np.mean(kern_ms[n])),
                      "GB_s": spec_bytes[n] / (float(np.mean(kern_ms[n])) * 1e-3) / 1e9}
                  for n in MATS}
    avg_launch_ms = sum_ms / (args.steps * len(MATS))
    avg_launch_bytes = alg_bytes / (args.steps * len(MATS))

    # ---- the other hot-path calls, timed on layer 0
    rows = {}

    def time_call(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    X5 = {n: dev16(synth.activations(5, layer0[n].shape[1], 2, t0=10 + i)) for i, n in enumerate(MATS)}
    Y5 = {n: torch.empty((5, layer0[n].shape[0]), dtype=torch.float32, device="cuda") for n in MATS}
    e0 = encs[0]
    ver_ms = sum(time_call(lambda n=n: cass.cass_verify_gemm(e0[n].desc, X5[n], Y5[n], stream))
                 for n in MATS)
    both_bytes = sum(e0[n].spec_bytes + e0[n].verif_bytes for n in MATS)
    rows["verify_gemm_n5"] = {"ms_per_layer": ver_ms, "GB_s": both_bytes / (ver_ms * 1e-3) / 1e9,
                              "spec_plus_verif_MB": both_bytes / 1e6}
    out = {n: torch.empty_like(layers[0][n]) for n in MATS}
    rec_ms = sum(time_call(lambda n=n: cass.cass_reconstruct(e0[n].desc, out[n], stream), 3)
                 for n in MATS)
    rows["reconstruct"] = {"ms_per_layer": rec_ms,
                           "GB_s_read": both_bytes / (rec_ms * 1e-3) / 1e9}
    dd_ms = sum(time_call(lambda n=n: cass.cass_draft_decode(e0[n].desc, out[n], stream), 3)
                for n in MATS)
    rows["draft_decode"] = {"ms_per_layer": dd_ms}
    for n in MATS:  # exactness of the decoded layer on the device
        cass.cass_reconstruct(e0[n].desc, out[n], stream)
    torch.cuda.synchronize()
    exact = all(torch.equal(out[n], layers[0][n]) for n in MATS)
    t0 = time.time()
    encode_layer(layers[0], args.keep, args.mant, ws)
    torch.cuda.synchronize()
    rows["encode"] = {"ms_per_layer": 1e3 * (time.time() - t0),
                      "note": "two host synchronisations per tensor (histograms, sizes)"}
    n_values = sum(layers[0][n].numel() for n in MATS)
    bits_per_value = sum(spec_bytes.values()) * 8 / n_values

    sweep = None
    if args.sweep:
        sweep = {}
        for keep in (0.5, 0.3, 0.2):
            for mant in (2, 3, 4):
                e = encode_layer(layers[0], keep, mant, ws)
                b = sum(e[n].spec_bytes for n in MATS)
                ms = sum(time_call(lambda n=n: cass.cass_draft_gemv(e[n].desc, xs[n], ys[n], stream), 20)
                         for n in MATS)
                sweep[f"keep{keep}_m{mant}"] = {"spec_MB": b / 1e6, "GB_s": b / (ms * 1e-3) / 1e9,
                                               "bits_per_value": b * 8 / n_values}
                del e

    # ---- CPU oracle on a row sample of layer 0
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = max(1, min(16, os.cpu_count() or 1))
        sample = {}
        for n in MATS:
            w = layer0[n][::16]
            sample[n] = oracle.encode(w, synth.keep_count(args.keep, w.shape[1]), args.mant,
                                      block=args.block)[0]
        xh = {n: synth.activations(1, layer0[n].shape[1], 2, t0=i) for i, n in enumerate(MATS)}
        done_bytes, t_start = 0, time.time()
        while True:
            for n in MATS:
                oracle.product(sample[n], xh[n], threads=threads)
                done_bytes += sample[n].size
            if time.time() - t_start >= args.cpu_seconds:
                break
        dt = time.time() - t_start
        cpu = {"value": done_bytes / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": "every 16th row of each fused matrix of layer 0, encoded by the oracle; "
                         "oracle draft product (decode + fp64 multiply-accumulate) repeated for "
                         f"{dt:.1f}s"}

    result = {
        "metric": "draft GEMV GB/s on compressed bytes & % HBM peak, 8B-shape layer bs=1",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "Llama-3-8B-shaped decoder layer, draft GEMV bs=1 over q|k|v 6144x4096, "
                        "o 4096x4096, gate|up 28672x4096, down 4096x14336",
            "format": "Cassandra-1 unary exponents", "keep": args.keep, "mant_bits": args.mant,
            "block": args.block, "batch": 1, "layer_copies": len(encs),
            "spec_MB_per_layer": round(sum(spec_bytes.values()) / 1e6, 3),
            "spec_bits_per_value": round(bits_per_value, 4),
        },
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s_equiv_layer": round(1e3 / ms_per_step, 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(avg_launch_bytes / (avg_launch_ms * 1e-3) / 1e9, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(avg_launch_bytes / (avg_launch_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": None,
            "kernel": "k_draft_gemv_c1<1>",
            "avg_launch_us": round(avg_launch_ms * 1e3, 3),
            "algorithmic_bytes_per_launch": round(avg_launch_bytes),
        },
        "per_matrix": {n: {k: round(v, 3) for k, v in d.items()} for n, d in per_matrix.items()},
        "kernel_sum_GB_s": round(kernel_gbs, 2),
        "rows": rows,
        "reconstruct_exact": exact,
        "cpu_baseline": cpu,
    }
    if sweep is not None:
        result["sweep"] = sweep
    print(json.dumps(result))


if __name__ == "__main__":
    main()
