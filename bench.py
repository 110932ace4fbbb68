#!/usr/bin/env python3
"""Benchmark: one 48-layer hybrid decode step (append + split-KV decode per layer).

Workload (synthetic, seeded): batch 32, per-sequence context uniform on [1, 16384];
layers at 0-based index l with l % 6 == 5 are global (16 query heads on 1 KV head,
K = V, head_dim 512, linear cache of 16384 positions, full causal), every other layer
is sliding (16 query heads on 8 KV heads, head_dim 256, bf16 ring of W = w = 1024),
no soft-cap, query scale 1/sqrt(head_dim).  Each step appends the current token
(position ctx - 1) to every layer's cache and then attends with q_pos = ctx - 1.

Prints ONE JSON line.  `value` is effective KV GB/s of the whole step: algorithmic
bytes (valid K rows, plus V rows unless K = V, plus q, out, the int inputs, and the
append's reads and writes) divided by the step time, with every input resident in
HBM.  `roofline` is for the dominant kernel (the sliding-layer fused append + decode,
40 of the 48 launches), timed with HIP events around back-to-back launches of it on the
stream it runs on.
`cpu_baseline` times the fp64 oracle on a bounded sample of the same workload.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
HBM_PEAK_GBPS = 8000.0
METRIC = "decode attention effective KV GB/s and % of HBM peak; layer-tokens/sec"


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--graph", action="store_true", help="replay the step as a HIP graph")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="first run a 1 GiB device-to-device copy (counter calibration)")
    p.add_argument("--summarize-trace", metavar="KERNEL_STATS_CSV",
                   help="print a summary of a rocprofv3 --stats kernel_stats.csv and exit")
    p.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="print the HBM traffic summary of two rocprofv3 --pmc runs and exit")
    p.add_argument("--counter-kernel", default="",
                   help="with --summarize-counters: kernel name substring (default: the "
                        "dominant sliding decode kernel)")
    p.add_argument("--summarize-sq", nargs="+", metavar="PMC_CSV",
                   help="print per-kernel SQ counter averages of rocprofv3 --pmc runs and exit")
    p.add_argument("--command", default="", help="command line recorded in summaries")
    p.add_argument("--step-only", action="store_true",
                   help="48-layer step: leave out the single-layer lines (counter runs that "
                        "must see the step's launches only)")
    p.add_argument("--workload", default="hybrid48",
                   choices=sorted(SINGLE_LAYER) + ["hybrid48", "hybrid48_rope"],
                   help="hybrid48: the 48-layer step (default); hybrid48_rope: the same step "
                        "with the rotary embedding fused into each append; others: one layer")
    return p.parse_args()


# Single-layer workloads measured with --workload (the default line is the 48-layer step).
SINGLE_LAYER = {"g3_1b_sliding": "G3_1B_SLIDING", "hd128_sliding": "HD128_SLIDING",
                "g4_12b_sliding": "G4_12B_SLIDING",
                "g4_12b_global": "G4_12B_GLOBAL", "spec_decode_sliding": "SPEC_DECODE_SLIDING",
                "fp8_sliding": "FP8_SLIDING", "fp8_global": "FP8_GLOBAL",
                "fp8_spec_decode_sliding": "FP8_SPEC_DECODE_SLIDING"}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def valid_keys(g, ctx):
    """Keys a row attends to at q_pos = ctx - 1: the newest min(ctx, w) positions for a
    sliding layer (ring of W >= w slots), all ctx positions for a full-causal layer."""
    import numpy as np
    return np.minimum(ctx, g.window) if g.window > 0 else ctx.copy()


def layer_bytes(g, B, ctx):
    """Algorithmic bytes of one layer: decode reads + writes, append reads + writes."""
    n = valid_keys(g, ctx).astype("int64")
    tensors = 1 if g.k_eq_v else 2
    kv = int(n.sum()) * g.num_kv_heads * g.head_dim * 2 * tensors
    q = B * g.num_q_heads * g.head_dim * 2
    out = B * g.num_q_heads * g.head_dim * 4
    ints = 2 * B * 4
    append = 2 * B * g.num_kv_heads * g.head_dim * 2 * tensors + B * 4
    return {"kv": kv, "decode": kv + q + out + ints, "append": append}


def read_traffic(kernel_tag):
    """Counter-measured HBM bytes per launch from profiles/, or None when absent or when
    the kernel sources changed since the counters were taken."""
    path = os.path.join(PROFILES, f"hbm_traffic_{kernel_tag}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    rels = kv.get("sources", "").split()
    if not rels or kv.get("sources_sha256") != sources_digest(rels):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# Sources whose change invalidates counter-measured traffic of a kernel (by name).
_CSRC = "decode_attention_split_amd/csrc/"
TRAFFIC_SOURCES = {
    "decode_valu_kernel": [_CSRC + f for f in ["decode_valu_impl.h", "decode_valu_d256.hip",
                                               "ga_device.h", "ga_internal.h", "ga_rope.h",
                                               "ga_quant.h", "api.hip"]],
    "decode_mfma_kernel": [_CSRC + f for f in ["decode_mfma.hip", "ga_mfma.h", "ga_device.h",
                                               "ga_internal.h", "api.hip"]],
}


def traffic_sources(kernel):
    for key, files in TRAFFIC_SOURCES.items():
        if key in kernel:
            return files
    raise KeyError(f"no source list for kernel {kernel}")
DOMINANT = "decode_valu_kernel<256, 2"
COPY_BYTES = 1 << 30
READ_BYTES = 1 << 30


def sources_digest(rels):
    import hashlib
    h = hashlib.sha256()
    for rel in rels:
        h.update(open(os.path.join(ROOT, rel), "rb").read())
    return h.hexdigest()


def summarize_trace(path, command):
    """Markdown summary of a rocprofv3 kernel_stats.csv (durations in microseconds)."""
    import csv
    rows = list(csv.DictReader(open(path)))
    print(f"# rocprofv3 kernel statistics\n\ncommand: `{command}`\n")
    print("| kernel | calls | avg us | min us | max us | share % |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        name = r["Name"].replace("|", "/")
        print(f"| `{name[:110]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
              f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
              f"{float(r['Percentage']):.2f} |")


def summarize_counters(fetch_csv, write_csv, command, kernel=""):
    """HBM bytes per launch of the dominant kernel (or of `kernel`) from FETCH_SIZE and
    WRITE_SIZE runs (KiB per dispatch), each scaled by what the counter reads for the 1 GiB
    calibration copy."""
    import csv

    def per_kernel(path, counter):
        # keyed by (kernel, grid size): the same kernel also serves other workloads of the
        # run (the single-layer lines), whose launches have other grids
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault((r["Kernel_Name"], int(r["Grid_Size"])), []).append(
                float(r["Counter_Value"]) * 1024.0)
        return vals

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")

    def calib(vals):
        copies = [v for k, vs in vals.items() if "copyBuffer" in k[0] for v in vs if v > 1e8]
        return COPY_BYTES / (sum(copies) / len(copies))

    f_scale, w_scale = calib(fetch), calib(write)
    # the timed workload's launches: the matching (kernel, grid) with the most dispatches
    dom = max((k for k in fetch if (kernel or DOMINANT) in k[0]),
              key=lambda k: len(fetch[k]), default=None)
    if dom is None or dom not in write:
        raise SystemExit(f"no dispatches of {kernel or DOMINANT} in both counter runs")
    f = sum(fetch[dom]) / len(fetch[dom])
    w = sum(write[dom]) / len(write[dom])
    what = "the dominant kernel" if not kernel else "one kernel"
    print(f"# HBM traffic of {what} (rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    print(f"command: {command}")
    print(f"kernel: {dom[0][:100]}")
    print(f"grid_size: {dom[1]} (dispatches: {len(fetch[dom])} fetch, {len(write[dom])} write)")
    print(f"fetch_calibration (1 GiB copy bytes / counter bytes): {f_scale:.4f}")
    print(f"write_calibration (1 GiB copy bytes / counter bytes): {w_scale:.4f}")
    print(f"fetch_bytes_per_launch: {f * f_scale:.0f}")
    print(f"write_bytes_per_launch: {w * w_scale:.0f}")
    print(f"hbm_bytes_per_launch: {f * f_scale + w * w_scale:.0f}")
    files = traffic_sources(dom[0])
    print(f"sources: {' '.join(files)}")
    print(f"sources_sha256: {sources_digest(files)}")


def summarize_sq(csvs, command):
    """Per-kernel averages (over dispatches, summed over the chip) of the SQ counters in
    rocprofv3 --pmc runs, with the ratios that say where waves spend their cycles."""
    import csv
    vals = {}
    for path in csvs:
        for r in csv.DictReader(open(path)):
            k = r["Kernel_Name"]
            if not k.startswith("void ga::") and not k.startswith("ga::"):
                continue
            k = f"{k[:100]}  (grid {r['Grid_Size']})"
            vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
    print("# SQ counters per dispatch (rocprofv3 --pmc, summed over the chip, averaged)")
    print(f"command: {command}")
    for k, cs in vals.items():
        avg = {c: sum(v) / len(v) for c, v in cs.items()}
        n = max(len(v) for v in cs.values())
        print(f"\nkernel: {k}  (dispatches per counter: {n})")
        for c in sorted(avg):
            print(f"  {c:28s} {avg[c]:.4g}")
        cyc = avg.get("SQ_WAVE_CYCLES")
        if cyc:
            ratio = lambda c: f"{avg[c] / cyc:.2f}" if c in avg else "n/a"
            print(f"  derived: waiting to issue (WAIT_INST_ANY / WAVE_CYCLES) "
                  f"{ratio('SQ_WAIT_INST_ANY')}; waiting on counters or barriers (WAIT_ANY / "
                  f"WAVE_CYCLES) {ratio('SQ_WAIT_ANY')}; VALU issue (ACTIVE_INST_VALU / "
                  f"WAVE_CYCLES) {ratio('SQ_ACTIVE_INST_VALU')}")
        if avg.get("SQ_INSTS_LDS"):
            print(f"  derived: LDS bank-conflict cycles per LDS instruction "
                  f"{avg.get('SQ_LDS_BANK_CONFLICT', 0) / avg['SQ_INSTS_LDS']:.2f}")
        if avg.get("SQ_INSTS_MFMA"):
            print(f"  derived: VALU instructions per MFMA "
                  f"{avg.get('SQ_INSTS_VALU', 0) / avg['SQ_INSTS_MFMA']:.1f}")


def main():
    args = parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.command)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.command, args.counter_kernel)
        return
    if args.summarize_sq:
        summarize_sq(args.summarize_sq, args.command)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the per-GPU workload is the whole step at its real shape)", file=sys.stderr)
        sys.exit(2)
    if args.workload not in ("hybrid48", "hybrid48_rope"):
        bench_single_layer(args)
        return
    import numpy as np
    import torch

    sys.path.insert(0, ROOT)
    from decode_attention_split_amd import api, synth
    from decode_attention_split_amd import workloads as wl
    from decode_attention_split_amd.hybrid import HybridKVCache

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rope = args.workload == "hybrid48_rope"
    w = wl.HYBRID_48_ROPE if rope else wl.HYBRID_48
    B, L = w.batch, w.num_layers

    # ---- inputs, resident in HBM before timing
    gen_cpu = synth.generator(w.seed)
    ctx = synth.uniform_int(gen_cpu, B, w.ctx_lo, w.ctx_hi).numpy().astype(np.int32)
    gdev = synth.generator(w.seed, device=dev)

    def fill(li, name, shape):
        return synth.normal_bf16(gdev, shape, device=dev)

    t0 = time.time()
    cache = HybridKVCache(w.layers, B, w.ctx_hi, device=dev, fill=fill)
    qs = [synth.normal_bf16(gdev, (B, g.num_q_heads, g.head_dim), device=dev) for g in w.layers]
    k_new = [synth.normal_bf16(gdev, (B, g.num_kv_heads, g.head_dim), device=dev)
             for g in w.layers]
    v_new = [None if g.k_eq_v else synth.normal_bf16(gdev, (B, g.num_kv_heads, g.head_dim),
                                                     device=dev) for g in w.layers]
    outs = [torch.empty((B, g.num_q_heads, g.head_dim), dtype=torch.float32, device=dev)
            for g in w.layers]
    ctx_t = torch.from_numpy(ctx).to(dev)
    qpos_t = ctx_t - 1
    pos_t = ctx_t - 1
    torch.cuda.synchronize()
    log(f"inputs ready: {cache.bytes() / 2**30:.2f} GiB of caches in {time.time() - t0:.1f}s")

    if args.calibrate_copy:
        src = torch.ones((COPY_BYTES // 4,), dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    per_layer = [layer_bytes(g, B, ctx) for g in w.layers]
    if rope:  # the fused rotary pass also reads q and writes the rotated q
        for g, x in zip(w.layers, per_layer):
            x["append"] += 2 * B * g.num_q_heads * g.head_dim * 2
    step_bytes = sum(x["decode"] + x["append"] for x in per_layer)
    q_rot = [torch.empty_like(q) for q in qs] if rope else None
    sliding = [i for i, g in enumerate(w.layers) if not g.k_eq_v]

    stream = torch.cuda.current_stream()

    def step():
        if rope:  # per layer: rotary + append + decode in one call (see HybridKVCache.step)
            cache.step(qs, k_new, v_new, pos_t, ctx_t, qpos_t, outs, q_rot=q_rot)
            return
        # per layer, one launch: append the current token to the cache and attend
        for li in range(L):
            cache.decode_append(li, qs[li], k_new[li], v_new[li], pos_t, ctx_t, qpos_t,
                                out=outs[li])

    graph = None
    if args.graph:
        step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()

    def run_step():
        if graph is not None:
            graph.replay()
        else:
            step()

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()

    # ---- timed region: K steps
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        run_step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = e0.elapsed_time(e1) / args.steps
    log(f"step: {ms_step:.4f} ms (wall {wall * 1e3 / args.steps:.4f} ms)")

    # ---- dominant kernel: the sliding-layer fused append + decode, launched back to back
    # for every sliding layer of the step, bracketed by one event pair on its stream (an
    # event pair around each launch would add its own overhead to every launch).
    kern_steps = max(1, args.steps)
    k0 = torch.cuda.Event(enable_timing=True)
    k1 = torch.cuda.Event(enable_timing=True)
    tables = cache.rope_tables(pos_t) if rope else {}
    torch.cuda.synchronize()
    k0.record(stream)
    for _ in range(kern_steps):
        for li in sliding:
            if rope:
                g = w.layers[li]
                cache.decode_rope_append(li, qs[li], q_rot[li], k_new[li], v_new[li], pos_t,
                                         ctx_t, qpos_t,
                                         tables[(g.rope_base, g.rotary_dim, g.head_dim)],
                                         out=outs[li])
            else:
                cache.decode_append(li, qs[li], k_new[li], v_new[li], pos_t, ctx_t, qpos_t,
                                    out=outs[li])
    k1.record(stream)
    torch.cuda.synchronize()
    n_launch = kern_steps * len(sliding)
    kern_ms = k0.elapsed_time(k1) / n_launch
    kern_bytes = float(np.mean([per_layer[li]["decode"] + per_layer[li]["append"]
                                for li in sliding]))
    kern_gbps = kern_bytes / (kern_ms * 1e-3) / 1e9
    log(f"sliding decode kernel: {kern_ms * 1e3:.2f} us avg over {n_launch} launches, "
        f"{kern_gbps:.1f} GB/s")

    extras = step_variants(args, step, stream, cache, qs, ctx_t, qpos_t, outs, L,
                           sum(x["decode"] for x in per_layer), graph is not None)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    extras["pct_of_read_ceiling"] = round(100.0 * value / extras["read_ceiling_gbps"], 2)
    kern_read_us = same_size_read_us(int(kern_bytes), stream)
    log(f"a streaming read of the sliding kernel's bytes: {kern_read_us:.2f} us")
    if not rope and not args.step_only:
        extras["single_layer_workloads"] = gated_layers(args)
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": ("rotary embedding fused with the append, then decode, per layer "
                         "(sliding base 1e4 over 256, global base 1e6 over 128); " if rope
                         else "") +
                        "48-layer hybrid decode step (append + decode per layer): 40 sliding "
                        "layers 16q/8kv hd256 ring w=W=1024 + 8 global layers 16q/1kv K=V "
                        "hd512 linear C=16384 at l%6==5; batch 32; ctx U[1,16384] seed 5; "
                        "no softcap; scale 1/sqrt(hd)",
            "batch": B, "layers": L, "ctx_mean": float(ctx.mean()),
            "accumulate": "fp32", "graph": bool(args.graph),
            "algorithmic_bytes_per_step": int(step_bytes),
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "layer_tokens_per_s": round(B * L / (ms_step * 1e-3), 1),
        "roofline": {
            "kernel": ("sliding-layer fused RoPE + append + decode" if rope else
                       "sliding-layer fused append + decode") +
                      " (hd256, 16q/8kv, ring 1024), per launch",
            "bound": "hbm",
            "achieved": round(kern_gbps, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(kern_gbps / HBM_PEAK_GBPS, 4),
            "traffic": read_traffic("sliding_rope_decode_hybrid48" if rope
                                    else "sliding_decode_hybrid48"),
            "bytes_per_launch": int(kern_bytes),
            "avg_launch_us": round(kern_ms * 1e3, 3),
            "same_size_read_us": round(kern_read_us, 3),
            "frac_of_same_size_read": round(kern_read_us / (kern_ms * 1e3), 4),
        },
    }

    result["extras"] = extras
    if not args.no_cpu_baseline:
        # (with the rotary embedding the decode read the rotated q of each layer)
        result["cpu_baseline"], result["oracle_check"] = cpu_baseline(
            cache, q_rot if rope else qs, outs, ctx, w, per_layer, args.cpu_seconds)
    # release the device memory before the line is printed, so the process ends promptly
    del cache, qs, k_new, v_new, outs, q_rot, graph
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    print(json.dumps(result), flush=True)


def gated_layers(args):
    """The single-layer workloads with a bandwidth target besides the 48-layer step (the
    Gemma-4-12B sliding and global layers), each timed as its own fused append + decode
    launch over rotating cache copies: us per launch, algorithmic bytes, GB/s and the
    fraction of the 8 TB/s peak."""
    import torch
    from decode_attention_split_amd import workloads as wl
    res = {}
    for name, w in [("g4_12b_sliding", wl.G4_12B_SLIDING), ("g4_12b_global", wl.G4_12B_GLOBAL)]:
        r = time_single_layer(w, max(10, args.steps), max(3, args.warmup))
        gbps = r["bytes"] / (r["ms"] * 1e-3) / 1e9
        torch.cuda.empty_cache()
        read_us = same_size_read_us(int(r["bytes"]), torch.cuda.current_stream())
        log(f"{name}: {r['ms'] * 1e3:.2f} us per launch, {gbps:.1f} GB/s; a streaming read of "
            f"the same bytes {read_us:.2f} us")
        res[name] = {"workload": w.name, "us_per_launch": round(r["ms"] * 1e3, 3),
                     "algorithmic_bytes": int(r["bytes"]), "gbps": round(gbps, 1),
                     "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
                     "same_size_read_us": round(read_us, 3),
                     "frac_of_same_size_read": round(read_us / (r["ms"] * 1e3), 4),
                     "graph_us_per_launch": round(r["ms_graph"] * 1e3, 3)}
        torch.cuda.empty_cache()
    return res


def step_variants(args, step, stream, cache, qs, ctx_t, qpos_t, outs, L, decode_bytes, graphed):
    """Besides the timed step: its per-step time distribution, the step without the append
    (decode over the resident caches only), the step replayed as a HIP graph, and the read
    ceiling measured on the same GPU (gemma_stream_read over 1 GiB), each after the main
    measurement."""
    import numpy as np
    import torch
    n = max(1, args.steps)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(n):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(n)])

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    def decode_only():
        for li in range(L):
            cache.decode(li, qs[li], ctx_t, qpos_t, out=outs[li])

    ms_decode = timed(decode_only)
    ms_graph = None
    if not graphed:
        step()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        ms_graph = timed(g.replay)
        del g
    read_gbps = read_ceiling(stream, qs[0].device, n)
    log(f"step p10/p50/p90 {np.percentile(per, [10, 50, 90]).round(4).tolist()} ms; decode only "
        f"{ms_decode:.4f} ms; graph {ms_graph} ms; read ceiling {read_gbps:.0f} GB/s")
    return {
        "step_ms_p10_p50_p90": [round(float(x), 5) for x in np.percentile(per, [10, 50, 90])],
        "decode_only_ms_per_step": round(ms_decode, 5),
        "decode_only_gbps": round(decode_bytes / (ms_decode * 1e-3) / 1e9, 2),
        "graph_ms_per_step": None if ms_graph is None else round(ms_graph, 5),
        "read_ceiling_gbps": round(read_gbps, 1),
    }


def read_ceiling(stream, device, reps):
    """The practical read ceiling on this GPU: gemma_stream_read (the decode kernels' own
    16-byte non-temporal loads, 16 in flight per wave, four waves per CU) over two 1 GiB
    buffers read in turn (8x the 256 MB Infinity Cache), timed with HIP events."""
    import torch
    from decode_attention_split_amd import api
    bufs = [torch.ones((READ_BYTES // 4,), dtype=torch.float32, device=device) for _ in range(2)]
    sink = api.stream_read(bufs[0])
    for i in range(2):
        api.stream_read(bufs[i % 2], sink)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = max(4, reps)
    a.record(stream)
    for i in range(reps):
        api.stream_read(bufs[i % 2], sink)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del bufs, sink
    return READ_BYTES / (ms * 1e-3) / 1e9


def same_size_read_us(nbytes, stream, reps=20):
    """gemma_stream_read over nbytes (rounded down to whole KiB), rotating over buffers of
    that size that together pass 1 GiB, launched back to back like the decode: the
    streaming-read time of a launch that moves the same bytes, ramp and drain included
    (a launch's fixed cost weighs more the fewer bytes it moves)."""
    import torch
    from decode_attention_split_amd import api
    nbytes = nbytes // 1024 * 1024
    n = max(2, -(-(READ_BYTES + nbytes) // nbytes))
    bufs = [torch.ones((nbytes // 4,), dtype=torch.float32, device="cuda") for _ in range(n)]
    sink = api.stream_read(bufs[0])
    for i in range(n):
        api.stream_read(bufs[i], sink)
    torch.cuda.synchronize()
    reps = max(reps, 2 * n)
    batches = []
    for _ in range(5):  # the median of five batches of back-to-back launches
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(reps):
            api.stream_read(bufs[i % n], sink)
        b.record(stream)
        torch.cuda.synchronize()
        batches.append(a.elapsed_time(b) / reps * 1e3)
    us = sorted(batches)[2]
    del bufs, sink
    torch.cuda.empty_cache()
    return us


def time_single_layer(w, steps, warmup, keep=False):
    """Fused append + decode of one single-token bf16 layer workload, rotating over enough
    cache copies (>= 1 GiB in all) that no launch finds its keys in the 256 MB Infinity
    Cache.  Returns the time per launch and the algorithmic bytes; with keep, also the
    inputs of the first copy (for the oracle)."""
    import numpy as np
    import torch
    from decode_attention_split_amd import api, synth

    dev = torch.device("cuda:0")
    g = w.layers[0]
    B = w.batch
    gen_cpu = synth.generator(w.seed)
    ctx = synth.uniform_int(gen_cpu, B, w.ctx_lo, w.ctx_hi).numpy().astype(np.int32)
    gdev = synth.generator(w.seed, device=dev)
    cache_shape = (B, g.num_kv_heads, g.capacity, g.head_dim)
    cache_bytes = int(np.prod(cache_shape)) * 2 * (1 if g.k_eq_v else 2)
    copies = int(min(128, max(2, math.ceil((1 << 30) / cache_bytes))))
    sets = []
    for _ in range(copies):
        q = synth.normal_bf16(gdev, (B, g.num_q_heads, g.head_dim), device=dev)
        k = synth.normal_bf16(gdev, cache_shape, device=dev)
        v = None if g.k_eq_v else synth.normal_bf16(gdev, cache_shape, device=dev)
        sets.append((q, k, v))
    k_new = synth.normal_bf16(gdev, (B, g.num_kv_heads, g.head_dim), device=dev)
    v_new = None if g.k_eq_v else synth.normal_bf16(gdev, k_new.shape, device=dev)
    out = torch.empty((B, g.num_q_heads, g.head_dim), dtype=torch.float32, device=dev)
    ctx_t = torch.from_numpy(ctx).to(dev)
    pos_t = ctx_t - 1
    max_ctx = w.ctx_hi if g.kind == api.RING else g.capacity
    shape = api.make_shape(B, g.num_q_heads, g.num_kv_heads, g.head_dim, g.capacity, g.kind,
                           max_ctx)
    ws = torch.empty((max(1, api.workspace_bytes(shape, g.window)),), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        q, k, v = sets[i % copies]
        api.decode_append(q, k, v, k_new, v_new, pos_t, ctx_t, pos_t, g.window, g.softcap,
                          g.q_scale, g.kind, out=out, workspace=ws, max_ctx=max_ctx)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        step(warmup + i)  # (the rotation goes on: the timed launches find cold copies)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # The same launches recorded once as a HIP graph and replayed: the GPU time without
    # the Python binding's per-call host time, which a small layer's launch does not hide.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            step(i)
    graph.replay()
    torch.cuda.synchronize()
    reps = 5
    e0.record(stream)
    for _ in range(reps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_graph = e0.elapsed_time(e1) / (reps * steps)
    del graph
    lb = layer_bytes(g, B, ctx)
    res = {"ms": ms, "ms_graph": ms_graph, "bytes": lb["decode"] + lb["append"], "ctx": ctx,
           "copies": copies}
    if keep:
        res["inputs"] = sets[0]
    del sets, ws, out
    return res


def bench_single_layer(args):
    """One layer type: fused append + decode of its workload, rotating over enough cache
    copies (>= 1 GiB in all) that no launch finds its keys in the 256 MB Infinity Cache."""
    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    from decode_attention_split_amd import api, synth
    from decode_attention_split_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = getattr(wl, SINGLE_LAYER[args.workload])
    if w.kv_dtype == "fp8":
        return bench_fp8(args, w)
    if w.tokens > 1:
        return bench_multi_token(args, w)
    g = w.layers[0]
    B = w.batch
    r = time_single_layer(w, args.steps, args.warmup, keep=not args.no_cpu_baseline)
    ms_eager, nbytes, ctx, copies = r["ms"], r["bytes"], r["ctx"], r["copies"]
    # a layer whose launches the host cannot issue as fast as the GPU runs them is reported
    # at its GPU time (graph replay); either way both figures go into the line
    ms = min(ms_eager, r["ms_graph"])
    gbps = nbytes / (ms * 1e-3) / 1e9
    log(f"{w.name}: {ms * 1e3:.2f} us per launch, {gbps:.1f} GB/s, {copies} cache copies "
        f"(eager {ms_eager * 1e3:.2f} us, graph replay {r['ms_graph'] * 1e3:.2f} us)")
    result = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name + " (one layer: fused append + decode)", "batch": B,
                   "layers": 1, "ctx_mean": float(ctx.mean()), "accumulate": "fp32",
                   "algorithmic_bytes_per_step": int(nbytes), "cache_copies": copies,
                   "timing": "graph replay" if ms < ms_eager else "eager launches",
                   "eager_us_per_launch": round(ms_eager * 1e3, 3),
                   "graph_us_per_launch": round(r["ms_graph"] * 1e3, 3)},
        "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "layer_tokens_per_s": round(B / (ms * 1e-3), 1),
        "roofline": {"kernel": "fused append + decode, per launch", "bound": "hbm",
                     "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "bytes_per_launch": int(nbytes), "avg_launch_us": round(ms * 1e3, 3)},
    }
    if not args.no_cpu_baseline:
        import oracle
        q, k, v = r["inputs"]
        qb, kb, vb = synth.bits(q), synth.bits(k), None if v is None else synth.bits(v)
        threads = oracle.num_threads_default()
        rows, spent, done = 0, 0.0, 0
        chunk = 4
        while rows < B and spent < args.cpu_seconds:
            sl = slice(rows, min(B, rows + chunk))
            t0 = time.perf_counter()
            oracle.decode(qb[sl], kb[sl], None if vb is None else vb[sl], ctx[sl], ctx[sl] - 1,
                          g.window, g.softcap, g.q_scale, g.kind, nthreads=threads)
            spent += time.perf_counter() - t0
            done += layer_bytes(g, sl.stop - sl.start, ctx[sl])["decode"]
            rows = sl.stop
        result["cpu_baseline"] = {"value": round(done / spent / 1e9, 4), "unit": "GB/s",
                                  "cores": int(min(threads, rows * g.num_q_heads)),
                                  "kind": "oracle", "host": host_cpu(),
                                  "sample": f"rows 0-{rows - 1} of the layer (decode only), "
                                            f"{spent:.1f}s of oracle time"}
    print(json.dumps(result), flush=True)


def multi_token_bytes(g, B, T, ctx):
    """Algorithmic bytes of one multi-token step (T tokens per row at ctx - T .. ctx - 1):
    every key any token attends to, read once (the union of the T windows), plus q, out,
    the int inputs, and the append of T rows."""
    import numpy as np
    span = np.minimum(ctx, g.window + T - 1) if g.window > 0 else ctx.copy()
    tensors = 1 if g.k_eq_v else 2
    kv = int(span.astype("int64").sum()) * g.num_kv_heads * g.head_dim * 2 * tensors
    q = B * T * g.num_q_heads * g.head_dim * 2
    out = B * T * g.num_q_heads * g.head_dim * 4
    ints = 2 * B * 4
    append = 2 * B * T * g.num_kv_heads * g.head_dim * 2 * tensors + B * 4
    return {"kv": kv, "decode": kv + q + out + ints, "append": append}


def bench_multi_token(args, w):
    """T tokens per row: gemma_kv_append_multi then gemma_attn_decode_multi per step,
    rotating over enough cache copies (>= 1 GiB) to keep the Infinity Cache out of it."""
    import numpy as np
    import torch
    from decode_attention_split_amd import api, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = w.layers[0]
    B, T = w.batch, w.tokens
    gen_cpu = synth.generator(w.seed)
    ctx = synth.uniform_int(gen_cpu, B, w.ctx_lo, w.ctx_hi).numpy().astype(np.int32)
    gdev = synth.generator(w.seed, device=dev)
    cache_shape = (B, g.num_kv_heads, g.capacity, g.head_dim)
    cache_bytes = int(np.prod(cache_shape)) * 2 * (1 if g.k_eq_v else 2)
    copies = int(min(128, max(2, math.ceil((1 << 30) / cache_bytes))))
    sets = []
    for _ in range(copies):
        q = synth.normal_bf16(gdev, (B, T, g.num_q_heads, g.head_dim), device=dev)
        k = synth.normal_bf16(gdev, cache_shape, device=dev)
        v = None if g.k_eq_v else synth.normal_bf16(gdev, cache_shape, device=dev)
        sets.append((q, k, v))
    k_new = synth.normal_bf16(gdev, (B, T, g.num_kv_heads, g.head_dim), device=dev)
    v_new = None if g.k_eq_v else synth.normal_bf16(gdev, k_new.shape, device=dev)
    out = torch.empty((B, T, g.num_q_heads, g.head_dim), dtype=torch.float32, device=dev)
    ctx_t = torch.from_numpy(ctx).to(dev)
    q0_t = ctx_t - T
    max_ctx = w.ctx_hi if g.kind == api.RING else g.capacity
    shape = api.make_shape(B, g.num_q_heads, g.num_kv_heads, g.head_dim, g.capacity, g.kind,
                           max_ctx)
    ws = torch.empty((max(1, api.workspace_bytes_multi(shape, T, g.window)),), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        q, k, v = sets[i % copies]
        api.kv_append_multi(k, v, k_new, v_new, q0_t, g.kind)
        api.decode_multi(q, k, v, ctx_t, q0_t, g.window, g.softcap, g.q_scale, g.kind, out=out,
                         workspace=ws, max_ctx=max_ctx)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)  # (the rotation goes on: the timed launches find cold copies)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    lb = multi_token_bytes(g, B, T, ctx)
    nbytes = lb["decode"] + lb["append"]
    gbps = nbytes / (ms * 1e-3) / 1e9
    log(f"{w.name}: {ms * 1e3:.2f} us per step (append + decode), {gbps:.1f} GB/s")
    result = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name + " (one layer: T-token append + multi-token decode)",
                   "batch": B, "tokens": T, "layers": 1, "ctx_mean": float(ctx.mean()),
                   "accumulate": "fp32", "algorithmic_bytes_per_step": int(nbytes),
                   "cache_copies": copies},
        "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "layer_tokens_per_s": round(B * T / (ms * 1e-3), 1),
        "roofline": {"kernel": "T-token append + multi-token decode, per step", "bound": "hbm",
                     "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "bytes_per_launch": int(nbytes), "avg_launch_us": round(ms * 1e3, 3)},
    }
    if not args.no_cpu_baseline:
        import oracle
        q, k, v = sets[0]
        qb, kb, vb = synth.bits(q), synth.bits(k), None if v is None else synth.bits(v)
        threads = oracle.num_threads_default()
        rows, spent, done = 0, 0.0, 0
        while rows < B and spent < args.cpu_seconds:
            sl = slice(rows, min(B, rows + 2))
            t0 = time.perf_counter()
            oracle.decode_multi(qb[sl], kb[sl], None if vb is None else vb[sl], ctx[sl],
                                ctx[sl] - T, g.window, g.softcap, g.q_scale, g.kind,
                                nthreads=threads)
            spent += time.perf_counter() - t0
            done += multi_token_bytes(g, sl.stop - sl.start, T, ctx[sl])["decode"]
            rows = sl.stop
        result["cpu_baseline"] = {"value": round(done / spent / 1e9, 4), "unit": "GB/s",
                                  "cores": int(min(threads, rows * T * g.num_q_heads)),
                                  "kind": "oracle", "host": host_cpu(),
                                  "sample": f"rows 0-{rows - 1} of the layer, all {T} tokens "
                                            f"(decode only), {spent:.1f}s of oracle time"}
    print(json.dumps(result), flush=True)


def fp8_layer_bytes(g, B, ctx, T=1):
    """Algorithmic bytes of one fp8 layer step with T tokens per row (at ctx - T ..
    ctx - 1): every key any token attends to (the union of the T windows) read once, D
    codes plus a float32 scale per key (K, and V unless K = V), q, out, the int inputs,
    and the quantizing append of T rows (read the bf16 row, write its codes and scale)."""
    import numpy as np
    if T == 1:
        n = valid_keys(g, ctx).astype("int64")
    else:
        n = (np.minimum(ctx, g.window + T - 1) if g.window > 0 else ctx.copy()).astype("int64")
    tensors = 1 if g.k_eq_v else 2
    kv = int(n.sum()) * g.num_kv_heads * (g.head_dim + 4) * tensors
    q = B * T * g.num_q_heads * g.head_dim * 2
    out = B * T * g.num_q_heads * g.head_dim * 4
    ints = 2 * B * 4
    append = B * T * g.num_kv_heads * (g.head_dim * 2 + g.head_dim + 4) * tensors + B * 4
    return {"kv": kv, "decode": kv + q + out + ints, "append": append}


def bench_fp8(args, w):
    """One layer over fp8 caches: quantizing append of the T current tokens (T = 1, or the
    tokens verified by speculative decoding), then decode, rotating over enough cache
    copies (>= 1 GiB) to keep the Infinity Cache out of it."""
    import numpy as np
    import torch
    from decode_attention_split_amd import api, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = w.layers[0]
    B, T = w.batch, w.tokens
    ctx = synth.uniform_int(synth.generator(w.seed), B, w.ctx_lo, w.ctx_hi).numpy() \
        .astype(np.int32)
    gdev = synth.generator(w.seed, device=dev)
    W = g.capacity
    tensors = 1 if g.k_eq_v else 2
    cache_bytes = B * g.num_kv_heads * W * (g.head_dim + 4) * tensors
    copies = int(min(128, max(2, math.ceil((1 << 30) / cache_bytes))))
    ctx_t = torch.from_numpy(ctx).to(dev)
    sets = []
    for _ in range(copies):
        # fill each cache by quantizing W random bf16 tokens per row (positions ctx-W..ctx-1)
        kc = torch.empty((B, g.num_kv_heads, W, g.head_dim), dtype=torch.uint8, device=dev)
        ks = torch.empty((B, g.num_kv_heads, W), dtype=torch.float32, device=dev)
        vc = None if g.k_eq_v else torch.empty_like(kc)
        vs = None if g.k_eq_v else torch.empty_like(ks)
        for part in range(0, W, 256):
            n = min(256, W - part)
            kn = synth.normal_bf16(gdev, (B, n, g.num_kv_heads, g.head_dim), device=dev)
            vn = None if g.k_eq_v else synth.normal_bf16(gdev, kn.shape, device=dev)
            api.kv_append_fp8(kc, ks, vc, vs, kn, vn, ctx_t - W + part, g.kind)
        qshape = (B, g.num_q_heads, g.head_dim) if T == 1 else (B, T, g.num_q_heads, g.head_dim)
        q = synth.normal_bf16(gdev, qshape, device=dev)
        sets.append((q, kc, ks, vc, vs))
    nshape = (B, g.num_kv_heads, g.head_dim) if T == 1 else (B, T, g.num_kv_heads, g.head_dim)
    k_new = synth.normal_bf16(gdev, nshape, device=dev)
    v_new = None if g.k_eq_v else synth.normal_bf16(gdev, k_new.shape, device=dev)
    out = torch.empty(qshape, dtype=torch.float32, device=dev)
    pos_t = ctx_t - T
    max_ctx = w.ctx_hi if g.kind == api.RING else g.capacity
    shape = api.make_shape(B, g.num_q_heads, g.num_kv_heads, g.head_dim, W, g.kind, max_ctx)
    ws = torch.empty((max(1, api.workspace_bytes_fp8(shape, T, g.window)),), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        q, kc, ks, vc, vs = sets[i % copies]
        if T == 1:  # quantizing append + decode in one call (one launch on the vector kernel)
            api.decode_append_fp8(q, kc, ks, vc, vs, k_new, v_new, pos_t, ctx_t, pos_t,
                                  g.window, g.softcap, g.q_scale, g.kind, out=out, workspace=ws,
                                  max_ctx=max_ctx)
            return
        api.kv_append_fp8(kc, ks, vc, vs, k_new, v_new, pos_t, g.kind)
        api.decode_fp8(q, kc, ks, vc, vs, ctx_t, pos_t, g.window, g.softcap, g.q_scale, g.kind,
                       out=out, workspace=ws, max_ctx=max_ctx)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)  # (the rotation goes on: the timed launches find cold copies)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    lb = fp8_layer_bytes(g, B, ctx, T)
    nbytes = lb["decode"] + lb["append"]
    gbps = nbytes / (ms * 1e-3) / 1e9
    log(f"{w.name}: {ms * 1e3:.2f} us per step (append + decode), {gbps:.1f} GB/s")
    result = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 cache, bf16 q, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": w.name + " (one layer: quantizing append + decode)",
                   "batch": B, "tokens": T, "layers": 1, "ctx_mean": float(ctx.mean()),
                   "accumulate": "fp32", "algorithmic_bytes_per_step": int(nbytes),
                   "cache_copies": copies},
        "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "layer_tokens_per_s": round(B * T / (ms * 1e-3), 1),
        "roofline": {"kernel": "fp8 quantizing append + decode, per step", "bound": "hbm",
                     "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "bytes_per_launch": int(nbytes), "avg_launch_us": round(ms * 1e3, 3)},
    }
    if not args.no_cpu_baseline:
        import oracle
        q, kc, ks, vc, vs = sets[0]
        qb = synth.bits(q)
        kcn, ksn = kc.cpu().numpy(), ks.cpu().numpy()
        vcn = None if vc is None else vc.cpu().numpy()
        vsn = None if vs is None else vs.cpu().numpy()
        threads = oracle.num_threads_default()
        rows, spent, done = 0, 0.0, 0
        while rows < B and spent < args.cpu_seconds:
            sl = slice(rows, min(B, rows + 4))
            t0 = time.perf_counter()
            oracle.decode_fp8_multi(qb[sl], kcn[sl], ksn[sl], None if vcn is None else vcn[sl],
                                    None if vsn is None else vsn[sl], ctx[sl], ctx[sl] - T,
                                    g.window, g.softcap, g.q_scale, g.kind, nthreads=threads)
            spent += time.perf_counter() - t0
            done += fp8_layer_bytes(g, sl.stop - sl.start, ctx[sl], T)["decode"]
            rows = sl.stop
        result["cpu_baseline"] = {"value": round(done / spent / 1e9, 4), "unit": "GB/s",
                                  "cores": int(min(threads, rows * g.num_q_heads)),
                                  "kind": "oracle", "host": host_cpu(),
                                  "sample": f"rows 0-{rows - 1} of the layer (decode only), "
                                            f"{spent:.1f}s of oracle time"}
    print(json.dumps(result), flush=True)


def cpu_baseline(cache, qs, outs, ctx, w, per_layer, target_s):
    """The fp64 oracle, as it stands, on whole layers of the same step (all 32 rows),
    taken in schedule order until about target_s seconds of oracle time.  Each layer's
    oracle output is also compared with the layer's GPU output from the timed run (the
    caches hold the appended token, the outputs the last step's decode): max-abs and
    relative L2 per layer against the parity bar (1e-2, 2e-3)."""
    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    import oracle
    from decode_attention_split_amd import synth

    ctx = np.asarray(ctx, np.int32)
    qpos = ctx - 1
    done_bytes, spent, layers, errs = 0, 0.0, [], []
    threads = oracle.num_threads_default()
    for li, g in enumerate(w.layers):
        k = synth.bits(cache.k[li])
        v = None if cache.v[li] is None else synth.bits(cache.v[li])
        q = synth.bits(qs[li])
        t0 = time.perf_counter()
        ref, _, _, _ = oracle.decode(q, k, v, ctx, qpos, g.window, g.softcap, g.q_scale, g.kind,
                                     nthreads=threads)
        spent += time.perf_counter() - t0
        done_bytes += per_layer[li]["decode"]
        layers.append(li)
        got = outs[li].double().cpu().numpy()
        d = got - ref
        errs.append((li, float(np.abs(d).max()), float(np.linalg.norm(d) / np.linalg.norm(ref)),
                     bool(np.isfinite(got).all())))
        del k, v
        log(f"oracle layer {li}: {spent:.1f}s cumulative")
        if spent >= target_s and li % 6 == 5:
            break
    units = max(g.num_q_heads for g in w.layers) * len(ctx)
    worst_abs = max(errs, key=lambda e: e[1])
    worst_rel = max(errs, key=lambda e: e[2])
    check = {
        "layers_checked": len(errs),
        "max_abs": worst_abs[1], "max_abs_layer": worst_abs[0],
        "rel_l2": worst_rel[2], "rel_l2_layer": worst_rel[0],
        "all_finite": all(e[3] for e in errs),
        "tolerance": {"max_abs": 1e-2, "rel_l2": 2e-3},
        "pass": all(e[3] and e[1] <= 1e-2 and e[2] <= 2e-3 for e in errs),
        "per_layer": [[e[0], float(f"{e[1]:.3e}"), float(f"{e[2]:.3e}")] for e in errs],
    }
    log(f"oracle check: {len(errs)} layers, worst max_abs {worst_abs[1]:.2e} (layer "
        f"{worst_abs[0]}), worst rel_l2 {worst_rel[2]:.2e} (layer {worst_rel[0]})")
    return {
        "value": round(done_bytes / spent / 1e9, 4),
        "unit": "GB/s",
        "cores": int(min(threads, units)),
        "kind": "oracle",
        "sample": f"layers {layers[0]}-{layers[-1]} of the 48-layer step (whole layers, all "
                  f"{len(ctx)} rows, decode only), {spent:.1f}s of oracle time",
        "host": host_cpu(),
    }, check


def host_cpu():
    """Model name and logical CPU count of the host, for the CPU baseline."""
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return f"{model} ({os.cpu_count()} logical CPUs visible)"


if __name__ == "__main__":
    main()
