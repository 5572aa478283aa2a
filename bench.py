#!/usr/bin/env python3
"""Benchmark of the Cassandra hot path on one MI355X.

Headline (the printed `value`): draft GEMV throughput on the speculation
(compressed) bytes of one Llama-3-8B-shaped decoder layer at batch 1, keep 0.3,
3 mantissa bits, Cassandra-1.  One step = the draft GEMVs of one decode step of
the layer: the fused projections q|k|v (6144x4096), o (4096x4096), gate|up
(28672x4096) and down (4096x14336), each one cass_draft_gemv call.  Steps
rotate over --copies distinct encoded layers so the bytes come from HBM, not
from the 256 MB last-level cache.

The same JSON line also carries the roofline of the GEMV kernel (HIP events
around every launch), the other hot-path calls (encode, verification GEMM for
5 tokens, reconstruction, draft decode), the keep x mantissa sweep, the
32-layer stack (tokens/s-equivalent), the compressed KV cache at 32K / 64K
context (append latency, draft and verification attention), the Qwen3-4B
Cassandra-2 stack at batch 2 with its 128K-token Cassandra-2 KV cache, and the
CPU oracle timed on a row sample.

Modes for profiling: --mode gemv runs only the timed GEMV steps; --mode exact
runs the verification GEMM (N = 5) and the reconstruction of each matrix; --mode copy
runs a plain 1 GiB device copy (to calibrate the HBM byte counters); --mode spec
runs only the speculative step over the 32-layer stack (and, without
--no-extras, the dense bf16 context); --mode mxt compares Cassandra-2 with
a lossless and with an MX-quantised target on one Qwen3-4B-shaped layer;
--mode codecs compares the exponent codes (Huffman, unary) and their decoders;
--mode superblock compares the superblock metadata layout with the flat one.
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
    ap.add_argument("--mode", choices=("full", "gemv", "exact", "copy", "spec", "mxt", "codecs",
                                       "superblock", "kv"), default="full")
    ap.add_argument("--no-extras", action="store_true", help="headline and CPU baseline only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def torch_layer(torch, shapes, gen, sigma=0.02, outlier_frac=0.01):
    """A further seeded layer drawn on the GPU with torch's generator, same
    recipe: N(0, sigma^2) rounded to bf16, round(1%) of input columns x10."""
    parts = {}
    for name, (r, c) in shapes.items():
        a = torch.randn((r, c), generator=gen, device="cuda", dtype=torch.float32) * sigma
        n_out = int(round(outlier_frac * c))
        if n_out:
            cols = torch.randperm(c, generator=gen, device="cuda")[:n_out]
            a[:, cols] *= 10.0
        parts[name] = a.to(torch.bfloat16).view(torch.int16)
        del a
    return {"qkv": torch.cat([parts["q"], parts["k"], parts["v"]], 0), "o": parts["o"],
            "gu": torch.cat([parts["gate"], parts["up"]], 0), "down": parts["down"]}


class Timer:
    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def ms(self, fn, reps=10, warm=1):
        torch = self.torch
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(self.stream)
        for _ in range(reps):
            fn()
        b.record(self.stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU (the path shards by rows with no exchange besides "
              "an all-gather of outputs); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_level_weight_amd as cass
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cass.lib()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    timer = Timer(torch, stream)
    dev16 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).cuda()

    if args.mode == "copy":
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy", "bytes": 1 << 30}))
        return

    if args.mode == "superblock":
        gen = torch.Generator(device="cuda")
        gen.manual_seed(2_000_001)
        L = torch_layer(torch, synth.LLAMA3_8B, gen)
        xs = {n: dev16(synth.activations(1, L[n].shape[1], 2, t0=i)) for i, n in enumerate(MATS)}
        print(json.dumps({"mode": "superblock", "superblock_metadata_llama8b_layer":
                          run_superblock(torch, cass, timer, stream, L, xs)}))
        return

    if args.mode == "codecs":
        gen = torch.Generator(device="cuda")
        gen.manual_seed(2_000_001)
        L = torch_layer(torch, synth.LLAMA3_8B, gen)
        print(json.dumps({"mode": "codecs", "exponent_codecs_llama8b_layer":
                          run_prefix_codecs(torch, cass, timer, stream, L)}))
        return

    if args.mode == "mxt":
        print(json.dumps({"mode": "mxt", "c2_mx_target_qwen3_4b_layer":
                          run_mx_target(torch, cass, synth, timer, stream, dev16)}))
        return

    if args.mode == "kv":
        # one layer's Cassandra-1 KV cache at 32K tokens (8 KV heads x 128, 32
        # query heads): single-token appends, draft attention, a 5-token append
        # and verification attention, each repeated (for kernel traces and
        # counters)
        print(json.dumps({"mode": "kv", "kv_llama8b_32k": run_kv_profile(torch, cass, synth, dev16,
                                                                           args.steps)}))
        return

    if args.mode == "spec":
        # the speculative step over 32 layers and the dense context, nothing else
        gen = torch.Generator(device="cuda")
        gen.manual_seed(2_000_001)
        ws = torch.empty(cass.cass_encode_ws_bytes(28672, 4096, cass._params(1, 3, args.block, 1)),
                         dtype=torch.uint8, device="cuda")
        stack = []
        for _ in range(32):
            L = torch_layer(torch, synth.LLAMA3_8B, gen)
            stack.append({n: cass.encode(L[n], synth.keep_count(0.3, L[n].shape[1]), 3,
                                         block=args.block, ws=ws) for n in L})
            del L
        torch.cuda.synchronize()
        log("stack encoded")
        res = {"mode": "spec", "spec_step_llama8b": run_spec_step(torch, cass, synth, stack, dev16)}
        del stack
        torch.cuda.empty_cache()
        if not args.no_extras:
            res["dense_bf16_llama8b_context"] = run_dense_stack(torch, synth)
        print(json.dumps(res))
        return

    # ---- inputs: layer 0 from the numpy recipe, further copies from torch's generator
    t0 = time.time()
    layer0 = synth.fused_layer(synth.LLAMA3_8B, config=2, layer=0, outlier_frac=0.01)
    layers = [{k: dev16(v) for k, v in layer0.items()}]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2_000_001)
    for _ in range(1, args.copies):
        layers.append(torch_layer(torch, synth.LLAMA3_8B, gen))
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s")

    ws = torch.empty(cass.cass_encode_ws_bytes(28672, 4096, cass._params(1, 3, args.block, 1)),
                     dtype=torch.uint8, device="cuda")

    def encode_layer(L, keep, mant, fmt=cass.CASS_FMT_C1_UNARY):
        return {n: cass.encode(L[n], synth.keep_count(keep, L[n].shape[1]), mant,
                               block=args.block, fmt=fmt, ws=ws) for n in L}

    encs = [encode_layer(L, args.keep, args.mant) for L in layers]
    n_copies = len(encs)
    torch.cuda.synchronize()
    log(f"encoded {len(encs)} layers")

    if args.mode == "exact":
        # verification GEMM (N = 5) and exact reconstruction of each matrix, steps rotating copies
        X5 = {n: dev16(synth.activations(5, layer0[n].shape[1], 2, t0=10 + i))
              for i, n in enumerate(MATS)}
        Y5 = {n: torch.empty((5, layer0[n].shape[0]), dtype=torch.float32, device="cuda") for n in MATS}
        outb = {n: torch.empty_like(layers[0][n]) for n in MATS}
        for i in range(args.warmup + args.steps):
            e = encs[i % len(encs)]
            for n in MATS:
                cass.cass_verify_gemm(e[n].desc, X5[n], Y5[n], stream)
            for n in MATS:
                cass.cass_reconstruct(e[n].desc, outb[n], stream)
        torch.cuda.synchronize()
        # algorithmic bytes per call: both streams read; X read and Y written (verification),
        # the bf16 tensor written (reconstruction)
        e0 = encs[0]
        print(json.dumps({"mode": "exact", "steps": args.steps, "bytes": {
            n: {"spec": e0[n].spec_bytes, "verif": e0[n].verif_bytes,
                "verify_gemm": e0[n].spec_bytes + e0[n].verif_bytes + 5 * 2 * e0[n].cols + 5 * 4 * e0[n].rows,
                "reconstruct": e0[n].spec_bytes + e0[n].verif_bytes + 2 * e0[n].rows * e0[n].cols}
            for n in MATS}}))
        return

    xs = {n: dev16(synth.activations(1, layer0[n].shape[1], 2, t0=i)) for i, n in enumerate(MATS)}
    ys = {n: torch.empty((1, layer0[n].shape[0]), dtype=torch.float32, device="cuda") for n in MATS}
    spec_bytes = {n: encs[0][n].spec_bytes for n in MATS}

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
    # timed region: whole steps back to back
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    total_bytes = sum(sum(encs[i % len(encs)][n].spec_bytes for n in MATS) for i in range(args.steps))
    value = total_bytes / (total_ms * 1e-3) / 1e9
    if args.mode == "gemv":
        print(json.dumps({"mode": "gemv", "value": round(value, 2), "unit": "GB/s",
                          "ms_per_step": round(ms_per_step, 5)}))
        return

    # kernel durations: HIP events around every GEMV launch
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in MATS]
          for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, ev[i])
    torch.cuda.synchronize()
    kern_ms = {n: [] for n in MATS}
    alg_bytes = 0  # speculation bytes + x read (2*cols) + y written (4*rows)
    for i in range(args.steps):
        for j, n in enumerate(MATS):
            kern_ms[n].append(ev[i][j][0].elapsed_time(ev[i][j][1]))
            e = encs[i % len(encs)][n]
            alg_bytes += e.spec_bytes + 2 * e.cols + 4 * e.rows
    sum_ms = sum(sum(v) for v in kern_ms.values())
    n_launch = args.steps * len(MATS)
    layer_ms = [sum(kern_ms[n][i] for n in MATS) for i in range(args.steps)]
    step_pct = {f"p{q}": round(float(np.percentile(layer_ms, q)) * 1e3, 2) for q in (10, 50, 90)}
    ceiling = read_ceiling(torch, cass, stream)
    # the kernel's mean launch time over the timed region (HIP events on the
    # launch stream around all steps; launches are back to back)
    avg_launch_ms = total_ms / (args.steps * len(MATS))
    achieved = alg_bytes / n_launch / (avg_launch_ms * 1e-3) / 1e9
    trace = trace_summary()
    per_matrix = {n: {"spec_MB": round(spec_bytes[n] / 1e6, 3),
                      "avg_us": round(1e3 * float(np.mean(kern_ms[n])), 2),
                      "GB_s": round(spec_bytes[n] / (float(np.mean(kern_ms[n])) * 1e-3) / 1e9, 1)}
                  for n in MATS}
    n_values = sum(layers[0][n].numel() for n in MATS)
    bits_per_value = sum(spec_bytes.values()) * 8 / n_values

    extras = {}
    if not args.no_extras:
        extras = run_extras(args, torch, cass, synth, timer, stream, layers, encs, layer0,
                            encode_layer, xs, ys, dev16, gen, n_values)

    cpu = cpu1 = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, synth, layer0)
        cpu1 = cpu_baseline(args, synth, layer0, threads=1, seconds=max(2.0, args.cpu_seconds / 3))

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
            "block": args.block, "batch": 1, "layer_copies": n_copies,
            "spec_MB_per_layer": round(sum(spec_bytes.values()) / 1e6, 3),
            "spec_bits_per_value": round(bits_per_value, 4),
        },
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "hbm_read_ceiling": ceiling,
        "pct_of_read_ceiling": round(100 * value / ceiling["GB_s"], 2),
        "layer_us_by_events": step_pct,
        "tokens_per_s_equiv_layer": round(1e3 / ms_per_step, 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_from_profile(),
            "kernel": trace["kernel"],
            "avg_launch_us": round(avg_launch_ms * 1e3, 3),
            "avg_launch_us_per_launch_events": round(sum_ms / n_launch * 1e3, 3),
            "profile_avg_launch_us": trace["avg_us"],
            "profile_on_current_sources": trace["sources_match"],
            "algorithmic_bytes_per_launch": round(alg_bytes / n_launch),
        },
        "valu_ceiling": valu_from_profile(step_pct["p50"]),
        "per_matrix": per_matrix,
        "cpu_baseline": cpu,
        "cpu_baseline_1core": cpu1,
    }
    result["inputs_sha256"] = input_digest([layers[0][n] for n in MATS] + [xs[n] for n in MATS])
    if not args.no_extras:
        result["worked_config_1024_cache_resident"] = cache_resident_row(torch, cass, synth, dev16,
                                                                         timer, stream)
    result.update(extras)
    print(json.dumps(result))


def profile_fields(name):
    """Key: value lines of a committed counter summary under profiles/, when it
    was taken on the current kernel sources (sha256 of the listed files); else
    None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    try:
        h = hashlib.sha256()
        for f in fields["sources"].split():
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if h.hexdigest() != fields["sources_sha256"]:
            return None
    except (KeyError, OSError):
        return None
    return fields


def traffic_from_profile():
    """HBM bytes per GEMV launch from the committed counter summary (FETCH_SIZE +
    WRITE_SIZE, calibrated on a device copy), when it was taken on the current
    kernel sources; else null."""
    f = profile_fields("draft_gemv_llama8b_layer_traffic.txt")
    try:
        return int(f["traffic_bytes_per_launch"]) if f else None
    except (KeyError, ValueError):
        return None


def valu_from_profile(layer_us):
    """The secondary (VALU issue) ceiling of the GEMV from the committed SQ
    counter summary: lane instructions per kept value and the time the layer's
    VALU instructions need at one wave64 instruction per 4 cycles per SIMD
    (256 CUs x 4 SIMDs, 2.4 GHz, i.e. 39.3 T lane-ops/s); null when the
    counters were taken on other kernel sources."""
    f = profile_fields("draft_gemv_llama8b_layer_sq_counters.txt")
    try:
        floor = float(f["valu_issue_floor_us_per_layer"])
        return {"lane_instr_per_kept_value": float(f["valu_lane_instr_per_kept_value"]),
                "issue_floor_us_per_layer": floor, "peak_lane_ops_per_s": 39.3e12,
                "frac_of_layer_time": round(floor / layer_us, 3)}
    except (TypeError, KeyError, ValueError):
        return None


def run_extras(args, torch, cass, synth, timer, stream, layers, encs, layer0, encode_layer,
               xs, ys, dev16, gen, n_values):
    out = {}
    e0 = encs[0]
    # ---- other calls on the 8B layer
    X5 = {n: dev16(synth.activations(5, layer0[n].shape[1], 2, t0=10 + i)) for i, n in enumerate(MATS)}
    Y5 = {n: torch.empty((5, layer0[n].shape[0]), dtype=torch.float32, device="cuda") for n in MATS}
    both = sum(e0[n].spec_bytes + e0[n].verif_bytes for n in MATS)
    ver_ms = sum(timer.ms(lambda n=n: cass.cass_verify_gemm(e0[n].desc, X5[n], Y5[n], stream))
                 for n in MATS)
    rows = {"verify_gemm_n5": {"ms_per_layer": round(ver_ms, 4),
                               "GB_s": round(both / (ver_ms * 1e-3) / 1e9, 1),
                               "pct_hbm_peak": round(100 * both / (ver_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                               "spec_plus_verif_MB": round(both / 1e6, 2)}}
    outb = {n: torch.empty_like(layers[0][n]) for n in MATS}
    rec_ms = sum(timer.ms(lambda n=n: cass.cass_reconstruct(e0[n].desc, outb[n], stream), 3)
                 for n in MATS)
    out_b = sum(2 * layers[0][n].numel() for n in MATS)
    rows["reconstruct"] = {"ms_per_layer": round(rec_ms, 4),
                           "GB_s_read": round(both / (rec_ms * 1e-3) / 1e9, 1),
                           "pct_hbm_peak_read_plus_write":
                               round(100 * (both + out_b) / (rec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}
    dd_ms = sum(timer.ms(lambda n=n: cass.cass_draft_decode(e0[n].desc, outb[n], stream), 3)
                for n in MATS)
    rows["draft_decode"] = {"ms_per_layer": round(dd_ms, 4)}
    for n in MATS:
        cass.cass_reconstruct(e0[n].desc, outb[n], stream)
    torch.cuda.synchronize()
    rows["reconstruct_exact"] = all(torch.equal(outb[n], layers[0][n]) for n in MATS)
    del outb
    t0 = time.time()
    encode_layer(layers[0], args.keep, args.mant)
    torch.cuda.synchronize()
    rows["encode"] = {"ms_per_layer": round(1e3 * (time.time() - t0), 2),
                      "note": "two host synchronisations per tensor (histograms, sizes)"}
    out["rows"] = rows
    out["exponent_codecs_llama8b_layer"] = run_prefix_codecs(torch, cass, timer, stream, layers[0])
    log("codecs done")
    out["superblock_metadata_llama8b_layer"] = run_superblock(torch, cass, timer, stream, layers[0], xs)
    log("superblock done")

    # ---- keep x mantissa sweep (layer 0)
    sweep = {}
    for keep in (0.5, 0.3, 0.2):
        for mant in (2, 3, 4):
            e = encode_layer(layers[0], keep, mant)
            b = sum(e[n].spec_bytes for n in MATS)
            ms = sum(timer.ms(lambda n=n: cass.cass_draft_gemv(e[n].desc, xs[n], ys[n], stream), 20)
                     for n in MATS)
            sweep[f"keep{keep}_m{mant}"] = {"spec_MB": round(b / 1e6, 2),
                                           "GB_s": round(b / (ms * 1e-3) / 1e9, 1),
                                           "bits_per_value": round(b * 8 / n_values, 4)}
            del e
    out["sweep"] = sweep
    out["sweep_min_GB_s"] = min(v["GB_s"] for v in sweep.values())
    del encs[1:]
    del layers[1:]
    torch.cuda.empty_cache()
    log("sweep done")

    # ---- 32-layer stack: one draft step (4 GEMVs per layer) and one N=5 verify pass
    stack = []
    for li in range(32):
        L = torch_layer(torch, synth.LLAMA3_8B, gen)
        stack.append(encode_layer(L, 0.3, 3))
        del L
    torch.cuda.synchronize()
    sb = sum(e[n].spec_bytes for e in stack for n in MATS)
    vb = sum(e[n].verif_bytes for e in stack for n in MATS)
    draft_ms = timer.ms(lambda: [cass.cass_draft_gemv(e[n].desc, xs[n], ys[n], stream)
                                 for e in stack for n in MATS], 5)
    verify_ms = timer.ms(lambda: [cass.cass_verify_gemm(e[n].desc, X5[n], Y5[n], stream)
                                  for e in stack for n in MATS], 2)
    out["stack32_llama8b"] = {
        "draft_step_ms": round(draft_ms, 3), "tokens_per_s_equiv": round(1e3 / draft_ms, 1),
        "draft_GB_s": round(sb / (draft_ms * 1e-3) / 1e9, 1), "spec_GB": round(sb / 1e9, 3),
        "verify_n5_ms": round(verify_ms, 3), "spec_plus_verif_GB": round((sb + vb) / 1e9, 3),
        "note": "linear layers only (4 fused GEMVs per layer), keep 0.3, m=3, Cassandra-1"}
    out["spec_step_llama8b"] = run_spec_step(torch, cass, synth, stack, dev16)
    del stack
    torch.cuda.empty_cache()
    log("spec step done")
    out["dense_bf16_llama8b_context"] = run_dense_stack(torch, synth)
    torch.cuda.empty_cache()
    log("stack done")

    # ---- Qwen3-4B-shaped 36-layer stack, Cassandra-2 (MX-32), batch 2
    x2 = {n: None for n in MATS}
    qstack = []
    for li in range(36):
        L = torch_layer(torch, synth.QWEN3_4B, gen, outlier_frac=0.0)
        qstack.append(encode_layer(L, 0.3, 3, fmt=cass.CASS_FMT_C2_MX32))
        if li == 0:
            for i, n in enumerate(MATS):
                x2[n] = dev16(synth.activations(2, L[n].shape[1], 5, t0=2 * i))
        del L
    y2 = {n: torch.empty((2, qstack[0][n].rows), dtype=torch.float32, device="cuda") for n in MATS}
    qb = sum(e[n].spec_bytes for e in qstack for n in MATS)
    q_ms = timer.ms(lambda: [cass.cass_draft_gemv(e[n].desc, x2[n], y2[n], stream)
                             for e in qstack for n in MATS], 5)
    out["stack36_qwen3_4b_c2_bs2"] = {
        "draft_step_ms": round(q_ms, 3), "GB_s": round(qb / (q_ms * 1e-3) / 1e9, 1),
        "spec_GB": round(qb / 1e9, 3), "tokens_per_s_equiv_bs2": round(2e3 / q_ms, 1),
        "spec_bits_per_value": round(qb * 8 / (36 * sum(int(np.prod(s)) for s in synth.QWEN3_4B.values())), 4)}
    del qstack
    torch.cuda.empty_cache()
    log("qwen done")
    out["c2_mx_target_qwen3_4b_layer"] = run_mx_target(torch, cass, synth, timer, stream, dev16)
    torch.cuda.empty_cache()
    log("mx target done")

    # ---- KV cache at 32K / 64K context (8 KV heads x 128, 32 query heads)
    kvres = {}
    for T in (32768, 65536):
        H, Hq, keep, mant, nq = 8, 32, 38, 3, 5
        Kt = synth.kv_tensor(T + nq, H, 128, 1_000_000 * 4 + 7)
        Vt = synth.kv_tensor(T + nq, H, 128, 1_000_000 * 4 + 8)
        cache = cass.KvCache(H, 128, keep, mant, max_tokens=T + nq + 64)
        pre = T - 64
        cache.append(dev16(Kt[:pre]), dev16(Vt[:pre]))
        torch.cuda.synchronize()
        tokK = [dev16(Kt[t:t + 1]) for t in range(pre, T)]
        tokV = [dev16(Vt[t:t + 1]) for t in range(pre, T)]
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(64):
            cache.append(tokK[i], tokV[i])
        b.record(stream)
        torch.cuda.synchronize()
        app_us = a.elapsed_time(b) * 1e3 / 64
        app_gpu_us = append_graph_us(torch, cache, tokK, tokV)
        q1 = dev16(synth.activations(Hq, 128, 4, t0=T))
        wsa = torch.empty(cass.cass_kv_attn_ws_bytes(cache.kv, nq, Hq), dtype=torch.uint8, device="cuda")
        o1 = torch.empty((Hq, 128), dtype=torch.float32, device="cuda")
        d_ms = timer.ms(lambda: cass.cass_kv_draft_attn(cache.kv, q1, 1 / np.sqrt(128), o1, wsa, stream), 5)
        cache.append(dev16(Kt[T:T + nq]), dev16(Vt[T:T + nq]))
        qv = dev16(np.stack([synth.activations(Hq, 128, 5, t0=T + i) for i in range(nq)]))
        ov = torch.empty((nq, Hq, 128), dtype=torch.float32, device="cuda")
        wsv = torch.empty(cass.cass_kv_attn_ws_bytes(cache.kv, nq, Hq), dtype=torch.uint8, device="cuda")
        v_ms = timer.ms(lambda: cass.cass_kv_verify_attn(cache.kv, qv, 1 / np.sqrt(128), ov, wsv, stream), 3)
        tokens, flags = cass.cass_kv_status(cache.kv)
        # bytes the draft attention reads over T tokens: per K|V stream the keep
        # bitmap, the code offsets, the sign+mantissa fields and the used code bits
        st = cache.state.cpu().numpy().view(np.int64)
        code_bytes = sum(int(st[2 + 2 * s]) for s in range(2 * H)) / 8
        attn_bytes = 2 * H * T * (128 / 8 + 4 + keep * (1 + mant) / 8) + code_bytes * T / tokens
        kvres[f"T{T}"] = {"append_1tok_us": round(app_gpu_us, 2),
                          "append_1tok_us_eager": round(app_us, 2),
                          "draft_attn_us": round(d_ms * 1e3, 1),
                          "draft_attn_spec_MB": round(attn_bytes / 1e6, 2),
                          "draft_attn_GB_s": round(attn_bytes / (d_ms * 1e-3) / 1e9, 1),
                          "verify_attn_n5_us": round(v_ms * 1e3, 1), "tokens": tokens,
                          "overflow": bool(flags & cass.CASS_KV_FLAG_OVERFLOW)}
        del cache, Kt, Vt
        torch.cuda.empty_cache()
    out["kv_cache"] = kvres
    log("kv done")

    # ---- Qwen3-4B-shaped KV at 128K tokens, Cassandra-2 (one layer timed)
    T, H, Hq, keep, mant = 131072, 8, 32, 38, 3
    Kt = synth.kv_tensor(T, H, 128, 1_000_000 * 5 + 7)
    Vt = synth.kv_tensor(T, H, 128, 1_000_000 * 5 + 8)
    cache = cass.KvCache(H, 128, keep, mant, max_tokens=T + 64, fmt=cass.CASS_FMT_C2_MX32)
    cache.append(dev16(Kt[:T - 64]), dev16(Vt[:T - 64]))
    torch.cuda.synchronize()
    tokK = [dev16(Kt[t:t + 1]) for t in range(T - 64, T)]
    tokV = [dev16(Vt[t:t + 1]) for t in range(T - 64, T)]
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(64):
        cache.append(tokK[i], tokV[i])
    b.record(stream)
    torch.cuda.synchronize()
    app_eager_us = a.elapsed_time(b) * 1e3 / 64
    app_gpu_us = append_graph_us(torch, cache, tokK, tokV)
    q1 = dev16(synth.activations(Hq, 128, 5, t0=T))
    wsa = torch.empty(cass.cass_kv_attn_ws_bytes(cache.kv, 1, Hq), dtype=torch.uint8, device="cuda")
    o1 = torch.empty((Hq, 128), dtype=torch.float32, device="cuda")
    d_ms = timer.ms(lambda: cass.cass_kv_draft_attn(cache.kv, q1, 1 / np.sqrt(128), o1, wsa, stream), 3)
    tokens, flags = cass.cass_kv_status(cache.kv)
    # draft attention reads, per K|V stream and token: bitmap, shared exponents, fields
    attn_bytes = 2 * H * T * (128 / 8 + 128 / 32 + keep * (2 + mant) / 8)
    out["kv_cache_qwen3_4b_c2_128k"] = {
        "append_1tok_us": round(app_gpu_us, 2), "append_1tok_us_eager": round(app_eager_us, 2),
        "draft_attn_us": round(d_ms * 1e3, 1), "draft_attn_spec_MB": round(attn_bytes / 1e6, 2),
        "draft_attn_GB_s": round(attn_bytes / (d_ms * 1e-3) / 1e9, 1), "tokens": tokens,
        "overflow": bool(flags & cass.CASS_KV_FLAG_OVERFLOW),
        "spec_MB_per_layer": round(cache.spec.numel() / 1e6, 1),
        "verif_MB_per_layer": round(cache.verif.numel() / 1e6, 1),
        "bf16_MB_per_layer": round(2 * T * H * 128 * 2 / 1e6, 1)}
    del cache, Kt, Vt
    torch.cuda.empty_cache()
    log("qwen kv done")
    return out


def run_kv_profile(torch, cass, synth, dev16, steps, T=32768):
    """The KV calls of one Cassandra-1 layer at T tokens, `steps` times each,
    with their algorithmic bytes per call (what each kernel must read)."""
    H, Hq, keep, mant, nq = 8, 32, 38, 3, 5
    Kt = synth.kv_tensor(T + nq + steps, H, 128, 1_000_000 * 4 + 7)
    Vt = synth.kv_tensor(T + nq + steps, H, 128, 1_000_000 * 4 + 8)
    cache = cass.KvCache(H, 128, keep, mant, max_tokens=T + nq + steps + 8)
    cache.append(dev16(Kt[:T]), dev16(Vt[:T]))
    q1 = dev16(synth.activations(Hq, 128, 4, t0=T))
    qv = dev16(np.stack([synth.activations(Hq, 128, 5, t0=T + i) for i in range(nq)]))
    o1 = torch.empty((Hq, 128), dtype=torch.float32, device="cuda")
    ov = torch.empty((nq, Hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(cass.cass_kv_attn_ws_bytes(cache.kv, nq, Hq) * 2, dtype=torch.uint8,
                     device="cuda")
    torch.cuda.synchronize()
    st = cache.state.cpu().numpy().view(np.int64)
    code_bits = [int(st[2 + 2 * s]) for s in range(2 * H)], [int(st[3 + 2 * s]) for s in range(2 * H)]
    tk = [dev16(Kt[t:t + 1]) for t in range(T, T + steps)]
    tv = [dev16(Vt[t:t + 1]) for t in range(T, T + steps)]
    for i in range(steps):  # single-token appends (the one-launch path)
        cache.append(tk[i], tv[i])
    for _ in range(steps):
        cass.cass_kv_draft_attn(cache.kv, q1, 1 / np.sqrt(128), o1, ws)
    cache.append(dev16(Kt[T + steps:T + steps + nq]), dev16(Vt[T + steps:T + steps + nq]))
    for _ in range(steps):
        cass.cass_kv_verify_attn(cache.kv, qv, 1 / np.sqrt(128), ov, ws)
    torch.cuda.synchronize()
    tokens = cache.tokens
    # per K|V stream and token: keep words 16 B, code offset 4 B, fields k(1+m)/8 B; the used
    # code bits; the verification side adds low mantissas k(7-m)/8 B, pruned bytes D-k, its
    # offset 4 B and its code bits
    spec_b = 2 * H * tokens * (16 + 4 + keep * (1 + mant) / 8) + sum(code_bits[0]) / 8
    verif_b = 2 * H * tokens * (keep * (7 - mant) / 8 + (128 - keep) + 4) + sum(code_bits[1]) / 8
    return {"tokens": tokens, "steps": steps,
            "draft_attn_bytes_per_call": round(spec_b),
            "verify_attn_bytes_per_call": round(spec_b + verif_b)}


def append_graph_us(torch, cache, tokK, tokV, n=16, reps=7):
    """GPU time of one single-token append: HIP graphs of n and of n/2
    single-token appends, each followed by a truncation back to the starting
    length; the difference of their replay times over n/2.  Graph replays run
    back to back on the GPU, so host time (the binding's per-call cost, which
    bounds the eager figure) does not enter."""
    base = cache.tokens

    def body(k):
        s = torch.cuda.current_stream()
        for i in range(k):
            cache.append(tokK[i], tokV[i], s)
        cache.truncate(base, s)

    def replay_ms(g):
        ms = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        return float(np.median(ms))

    t = []
    for k in (n, n // 2):
        body(k)  # warm: workspace sized, kernels loaded
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            body(k)
        torch.cuda.synchronize()
        t.append(replay_ms(g))
        del g
    return (t[0] - t[1]) * 1e3 / (n - n // 2)


def run_mx_target(torch, cass, synth, timer, stream, dev16):
    """Cassandra-2 with a lossless target (format 2) against Cassandra-2 with
    an MX-quantised target (format 3) on one Qwen3-4B-shaped layer (keep 0.3,
    m = 3): stream sizes, verification GEMM (N = 5) and reconstruction time,
    and how far the quantised target's products move from the exact ones."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5_000_001)
    L = torch_layer(torch, synth.QWEN3_4B, gen, outlier_frac=0.0)
    res = {"layer": "Qwen3-4B-shaped q|k|v 6144x2560, o 2560x4096, gate|up 19456x2560, "
                    "down 2560x9728; keep 0.3, m 3"}
    n_values = sum(L[n].numel() for n in MATS)
    X5 = {n: dev16(synth.activations(5, L[n].shape[1], 5, t0=20 + i)) for i, n in enumerate(MATS)}
    Y = {}
    for fmt, name in ((cass.CASS_FMT_C2_MX32, "lossless_target"),
                      (cass.CASS_FMT_C2_MX_TARGET, "mx_target")):
        enc = {n: cass.encode(L[n], synth.keep_count(0.3, L[n].shape[1]), 3, fmt=fmt) for n in MATS}
        Y[name] = {n: torch.empty((5, enc[n].rows), dtype=torch.float32, device="cuda") for n in MATS}
        outb = {n: torch.empty_like(L[n]) for n in MATS}
        ver_ms = sum(timer.ms(lambda n=n: cass.cass_verify_gemm(enc[n].desc, X5[n], Y[name][n], stream), 3)
                     for n in MATS)
        rec_ms = sum(timer.ms(lambda n=n: cass.cass_reconstruct(enc[n].desc, outb[n], stream), 3)
                     for n in MATS)
        for n in MATS:
            cass.cass_verify_gemm(enc[n].desc, X5[n], Y[name][n], stream)
        sb = sum(enc[n].spec_bytes for n in MATS)
        vb = sum(enc[n].verif_bytes for n in MATS)
        res[name] = {"spec_bits_per_value": round(8 * sb / n_values, 4),
                     "verif_bits_per_value": round(8 * vb / n_values, 4),
                     "verify_n5_ms_per_layer": round(ver_ms, 4),
                     "verify_GB_s": round((sb + vb) / (ver_ms * 1e-3) / 1e9, 1),
                     "reconstruct_ms_per_layer": round(rec_ms, 4)}
        if fmt == cass.CASS_FMT_C2_MX32:
            torch.cuda.synchronize()
            res[name]["reconstruct_exact"] = all(torch.equal(outb[n], L[n]) for n in MATS)
        else:
            # the quantised target's deviation from the original weights
            torch.cuda.synchronize()
            num = den = 0.0
            for n in MATS:
                wt = outb[n].view(torch.bfloat16).float()
                wo = L[n].view(torch.bfloat16).float()
                num += float((wt - wo).abs().sum())
                den += float(wo.abs().sum())
            res[name]["weight_rel_l1_change"] = round(num / den, 6)
        del enc, outb
    dev_max = 0.0
    for n in MATS:
        a, b = Y["mx_target"][n], Y["lossless_target"][n]
        dev_max = max(dev_max, float(((a - b).abs() / b.abs().clamp_min(1e-30)).median()))
    res["verify_output_median_rel_change"] = round(dev_max, 6)
    return res


def run_prefix_codecs(torch, cass, timer, stream, layer, keep=0.3):
    """The exponent codes compared on one Llama-3-8B-shaped layer's kept
    exponents (top 30 % by magnitude per row) and pruned exponents (the rest),
    each sequence coded both ways: bits per exponent of a 12-bit-limited
    canonical Huffman code and of the frequency-ranked unary code against the
    entropy, and how fast each decoder turns the stream back into exponents."""
    kept, pruned = [], []
    for n in MATS:
        w = layer[n]
        a = (w & 0x7FFF).to(torch.int32)  # magnitude order of bf16 patterns
        k = max(1, int(round(keep * w.shape[1])))
        thr = torch.topk(a, k, dim=1).values[:, -1:]
        e = ((w.to(torch.int32) >> 7) & 0xFF).to(torch.uint8)
        kept.append(e[a >= thr])
        pruned.append(e[a < thr])
    out = {"kept": codec_compare(torch, cass, timer, stream, torch.cat(kept))}
    del kept
    out["pruned"] = codec_compare(torch, cass, timer, stream, torch.cat(pruned))
    return out


def codec_compare(torch, cass, timer, stream, sym):
    sym = sym[: sym.numel() // 16 * 16].contiguous()
    n = sym.numel()
    hist = torch.bincount(sym.to(torch.int64), minlength=256).cpu().numpy().astype(np.uint64)
    p = hist[hist > 0].astype(np.float64) / n
    res = {"symbols": n, "entropy_bits": round(float(-(p * np.log2(p)).sum()), 4),
           "distinct": int((hist > 0).sum())}
    block = 256
    codes = [("huffman12", cass.cass_prefix_code_huffman(hist, 12))]
    if res["distinct"] <= 32:  # unary codes of ranks past 31 exceed 32 bits
        codes.append(("unary", cass.cass_prefix_code_unary(hist)))
    blkoff = torch.empty(((n + block - 1) // block,), dtype=torch.int32, device="cuda")
    for name, code in codes:
        bits = cass.cass_prefix_stream_bits(code, hist)
        sb = ((bits + 7) // 8 + 15) // 16 * 16 + 16
        st = torch.empty((sb,), dtype=torch.uint8, device="cuda")
        enc_ms = timer.ms(lambda: cass.cass_prefix_encode(code, sym, block, st, blkoff, stream), 3)
        ws = torch.empty((cass.cass_prefix_decode_ws_bytes(sb),), dtype=torch.uint8, device="cuda")
        out = torch.empty_like(sym)
        row = {"bits_per_exponent": round(bits / n, 4), "max_len": code.max_len,
               "encode_ms": round(enc_ms, 3)}
        methods = [("table", cass.CASS_PREFIX_TABLE)] if code.max_len <= 12 else []
        if name == "unary":
            methods += [("serial", cass.CASS_PREFIX_UNARY_SERIAL),
                        ("parallel", cass.CASS_PREFIX_UNARY_PARALLEL)]
        for mname, m in methods:
            ms = timer.ms(lambda: cass.cass_prefix_decode(code, st, blkoff, n, block, m, out, ws,
                                                          stream), 5)
            torch.cuda.synchronize()
            row[f"decode_{mname}"] = {"ms": round(ms, 3), "Gexp_s": round(n / (ms * 1e-3) / 1e9, 2),
                                      "stream_GB_s": round(sb / (ms * 1e-3) / 1e9, 1),
                                      "exact": bool(torch.equal(out, sym))}
        res[name] = row
        del st, ws, out
    return res


def run_superblock(torch, cass, timer, stream, layer, xs):
    """Cassandra-1 with superblock metadata (format 4) against the flat
    metadata (format 1) on one Llama-3-8B-shaped layer (keep 0.3, m 3):
    speculation bits per value, metadata bits per value, and the draft GEMV
    time per layer of both formats on the default (balanced) kernel and on the
    per-thread stream-reader kernel."""
    import synth
    res = {}
    n_values = sum(layer[n].numel() for n in MATS)
    enc = {}
    for fmt, name in ((cass.CASS_FMT_C1_UNARY, "flat"), (cass.CASS_FMT_C1_SUPERBLOCK, "superblock")):
        enc[name] = {n: cass.encode(layer[n], synth.keep_count(0.3, layer[n].shape[1]), 3, fmt=fmt)
                     for n in MATS}
        sb = sum(enc[name][n].spec_bytes for n in MATS)
        meta = 0
        for n in MATS:
            meta += sum(int(enc[name][n].plan.spec_len[i]) for i in (2, 3, 4))
        res[name] = {"spec_bits_per_value": round(8 * sb / n_values, 4),
                     "metadata_bits_per_value": round(8 * meta / n_values, 4)}
    cass.cass_set_option("gemv_path", 2)
    try:
        for name in ("flat", "superblock"):
            e = enc[name]
            ms = sum(timer.ms(lambda n=n: cass.cass_draft_gemv(e[n].desc, xs[n], ys_of(torch, e[n]),
                                                               stream), 10) for n in MATS)
            res[name]["draft_gemv_direct_kernel_ms_per_layer"] = round(ms, 4)
    finally:
        cass.cass_set_option("gemv_path", 0)
    for name in ("flat", "superblock"):
        e = enc[name]
        ms = sum(timer.ms(lambda n=n: cass.cass_draft_gemv(e[n].desc, xs[n], ys_of(torch, e[n]),
                                                           stream), 20) for n in MATS)
        res[name]["draft_gemv_default_kernel_ms_per_layer"] = round(ms, 4)
        res[name]["draft_gemv_default_GB_s"] = round(
            sum(e[n].spec_bytes for n in MATS) / (ms * 1e-3) / 1e9, 1)
    res["spec_bytes_saved_pct"] = round(
        100 * (1 - res["superblock"]["spec_bits_per_value"] / res["flat"]["spec_bits_per_value"]), 3)
    del enc
    return res


_ys = {}


def ys_of(torch, e):
    key = e.rows
    if key not in _ys:
        _ys[key] = torch.empty((1, e.rows), dtype=torch.float32, device="cuda")
    return _ys[key]


def graph_ms(torch, g, reps):
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g.replay()
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def run_spec_step(torch, cass, synth, stack, dev16, T=32768, k=4):
    """One self-speculative step over the 32 encoded layers, each with its own
    compressed KV cache at T tokens (8 KV heads x 128, 32 query heads): k draft
    passes (draft GEMVs, one-token KV append, draft attention) and one
    verification pass of k+1 tokens (verification GEMMs, KV append,
    verification attention), acceptance stubbed."""
    from bit_level_weight_amd.spec_step import SpecStep, draw_accepted, expected_tokens
    H, Hq, D, kk, mant = 8, 32, 128, 38, 3
    Kd = dev16(synth.kv_tensor(T, H, D, 7_000_001))
    Vd = dev16(synth.kv_tensor(T, H, D, 7_000_002))
    caches = []
    for _ in stack:
        c = cass.KvCache(H, D, kk, mant, max_tokens=T + 64)
        c.append(Kd, Vd)
        caches.append(c)
    del Kd, Vd
    st = SpecStep(stack, caches, Hq, k=k, seed=11)
    torch.cuda.synchronize()
    res = {"context_tokens": T, "k": k, "layers": len(stack), "kv": "Cassandra-1 keep 38/128 m3"}
    # eager (host-driven calls), fixed context
    st.run("step")
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(3):
        st.run("step")
    b.record()
    torch.cuda.synchronize()
    res["step_ms_eager"] = round(a.elapsed_time(b) / 3, 3)
    # HIP graphs of the whole step and of its two phases
    for phase in ("step", "draft", "verify"):
        g = st.capture(phase)
        res[f"{phase}_ms_graph"] = round(graph_ms(torch, g, 5 if phase != "step" else 5), 3)
        del g
    step_ms = res["step_ms_graph"]
    res["tokens_per_s_equiv"] = {f"alpha{al}": round(1e3 * expected_tokens(al, k) / step_ms, 1)
                                 for al in (0.74, 0.80, 0.91)}
    res["expected_tokens_per_step"] = {f"alpha{al}": round(expected_tokens(al, k), 4)
                                       for al in (0.74, 0.80, 0.91)}
    # the loop with drawn acceptance (alpha 0.8): the context grows by the kept tokens
    rng = np.random.default_rng(1234)
    made = 0
    a.record()
    for _ in range(8):
        made += st.step(draw_accepted(rng, 0.8, k))
    b.record()
    torch.cuda.synchronize()
    res["drawn_alpha0.8_eager"] = {"steps": 8, "tokens": made,
                                   "tokens_per_s": round(made / (a.elapsed_time(b) * 1e-3), 1),
                                   "final_context": st.tokens()}
    res["note"] = ("activations between the linear maps, queries and new K/V are resident "
                   "synthetic bf16; norms, rotary embedding, gated activation and LM head not run")
    del st, caches
    return res


def run_dense_stack(torch, synth, nl=32):
    """Context only: the same 32-layer linear stack as dense bf16 weights,
    torch.nn.functional.linear (the vendor BLAS) at batch 1 and 5, in a graph."""
    import torch.nn.functional as F
    shapes = {"qkv": (6144, 4096), "o": (4096, 4096), "gu": (28672, 4096), "down": (4096, 14336)}
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3_000_001)
    Ws = [{m: (torch.randn(r, c, generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
           for m, (r, c) in shapes.items()} for _ in range(nl)]
    res = {}
    for n in (1, 5):
        xs = {m: torch.randn(n, c, generator=gen, device="cuda").to(torch.bfloat16)
              for m, (r, c) in shapes.items()}
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for L in Ws:
                for m in shapes:
                    F.linear(xs[m], L[m])
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            ys = [F.linear(xs[m], L[m]) for L in Ws for m in shapes]
        ms = graph_ms(torch, g, 10)
        byts = sum(2 * r * c for r, c in shapes.values()) * nl
        res[f"bs{n}"] = {"ms": round(ms, 3), "GB_s": round(byts / (ms * 1e-3) / 1e9, 1)}
        del g, ys
    res["tokens_per_s_bs1"] = round(1e3 / res["bs1"]["ms"], 1)
    res["note"] = "dense bf16 linear maps only (no attention), measured as context, not a target"
    del Ws
    return res


def read_ceiling(torch, cass, stream):
    """Achievable HBM read rate on this GPU: the library's streaming-read kernel
    (cass_stream_read: 16-byte nontemporal loads, four in flight per lane, one
    word per workgroup written) over 2 GiB, best of 6; a 1 GiB device copy as
    context (bytes read plus bytes written)."""
    t = torch.ones(1 << 29, dtype=torch.float32, device="cuda")
    fold = torch.empty((cass.CASS_STREAM_READ_BLOCKS,), dtype=torch.int32, device="cuda")
    best = None
    for _ in range(6):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        cass.cass_stream_read(t, fold, stream)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None else min(best, ms)
    gbs = t.numel() * 4 / (best * 1e-3) / 1e9
    src = t.view(torch.uint8)[: 1 << 30]
    dst = torch.empty_like(src)
    cbest = None
    for _ in range(6):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        cbest = ms if cbest is None else min(cbest, ms)
    copy_gbs = 2 * src.numel() / (cbest * 1e-3) / 1e9
    del t, src, dst
    torch.cuda.empty_cache()
    return {"GB_s": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "kernel": "k_stream_read (cass_stream_read) over 2 GiB, best of 6",
            "copy_read_plus_write_GB_s": round(copy_gbs, 1),
            "copy_pct_hbm_peak": round(100 * copy_gbs / HBM_PEAK_GBS, 2)}


def host_facts():
    """nproc and the CPU model of the host the benchmark runs on."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model}


def input_digest(tensors):
    """SHA-256 over the bytes of the generated inputs, in order."""
    import hashlib
    h = hashlib.sha256()
    for t in tensors:
        h.update(t.cpu().numpy().tobytes())
    return h.hexdigest()


def trace_summary():
    """Kernel name and mean launch time of the GEMV from the committed
    rocprofv3 kernel-trace summary, and whether it was taken on the current
    kernel sources."""
    path = os.path.join(ROOT, "profiles", "draft_gemv_llama8b_layer_kernel_trace.txt")
    out = {"kernel": None, "avg_us": None, "sources_match": False}
    if not os.path.exists(path):
        return out
    f = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            f[k.strip()] = v.strip()
    out["kernel"] = f.get("kernel")
    try:
        out["avg_us"] = float(f["gemv_avg_launch_us"])
    except (KeyError, ValueError):
        pass
    out["sources_match"] = profile_fields("draft_gemv_llama8b_layer_kernel_trace.txt") is not None
    return out


def cache_resident_row(torch, cass, synth, dev16, timer, stream):
    """The 1024 x 1024 worked configuration (keep 0.5, m 3, Cassandra-1): it
    fits in the last-level cache, so its rate is not an HBM figure."""
    w = synth.weight(1024, 1024, 1_000_001)
    enc = cass.encode(dev16(w), 512, 3)
    x = dev16(synth.activations(1, 1024, 1))
    y = torch.empty((1, 1024), dtype=torch.float32, device="cuda")
    X = dev16(synth.activations(5, 1024, 1, t0=1))
    Y = torch.empty((5, 1024), dtype=torch.float32, device="cuda")
    out = torch.empty((1024, 1024), dtype=torch.int16, device="cuda")
    g = timer.ms(lambda: cass.cass_draft_gemv(enc.desc, x, y, stream), 50)
    v = timer.ms(lambda: cass.cass_verify_gemm(enc.desc, X, Y, stream), 20)
    r = timer.ms(lambda: cass.cass_reconstruct(enc.desc, out, stream), 20)
    return {"note": "cache-resident (1024 x 1024 bf16, 0.3 MB of speculation bytes): not an HBM rate",
            "spec_bytes": enc.spec_bytes, "draft_gemv_us": round(g * 1e3, 2),
            "draft_gemv_GB_s": round(enc.spec_bytes / (g * 1e-3) / 1e9, 1),
            "verify_gemm_n5_us": round(v * 1e3, 2), "reconstruct_us": round(r * 1e3, 2)}


def cpu_baseline(args, synth, layer0, threads=None, seconds=None):
    """The oracle's draft product on a row sample, on the host's cores: 16
    threads (the host share of one GPU of this machine) or fewer if the host
    has fewer."""
    import oracle
    threads = threads or max(1, min(16, os.cpu_count() or 1))
    seconds = seconds or args.cpu_seconds
    sample = {}
    for n in MATS:
        w = layer0[n][::16]
        sample[n] = oracle.encode(w, synth.keep_count(args.keep, w.shape[1]), args.mant,
                                  block=args.block)[0]
    xh = {n: synth.activations(1, layer0[n].shape[1], 2, t0=i) for i, n in enumerate(MATS)}
    done, t_start = 0, time.time()
    while True:
        for n in MATS:
            oracle.product(sample[n], xh[n], threads=threads)
            done += sample[n].size
        if time.time() - t_start >= seconds:
            break
    dt = time.time() - t_start
    return {"value": round(done / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "host": host_facts(),
            "sample": "every 16th row of each fused matrix of layer 0, encoded by the oracle; the "
                      "oracle's draft product (decode + fp64 multiply-accumulate) repeated for "
                      f"{dt:.1f} s"}


if __name__ == "__main__":
    main()
