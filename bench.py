#!/usr/bin/env python3
"""Benchmark of the quantized MoE layer on one MI355X.

A step is one pass of the whole layer over one decode batch: router logits and
top-k gating, bucketing, the NVFP4 dequant-fused SwiGLU experts, the
gate-weighted combine and the usage-histogram update.  Workload: 128 experts,
top-8, hidden 2048, intermediate 768, NVFP4 gate/up/down, decode batches of
1, 2, 4 and 8 tokens (one per request slot) and 16 and 32 (verification-sized
batches: a few slots with draft tokens); the headline line is the 8-token
batch.  Eight distinct seeded layers (2.7 GB of packed weights) are cycled and
every step gets fresh activations, so expert weights come from HBM and not
from the 256 MB Infinity Cache.  Each batch size's steps are captured in a HIP
graph and replayed.

Printed: one JSON line with the throughput (tokens/s), the FFN kernels'
roofline (expert-weight bytes of the active experts / FFN time from HIP events
on the launch stream, against 8 TB/s), and the CPU oracle timed on a bounded
sample beside it.
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
MFMA_BF16_PEAK_TFLOPS = 2500.0
N_LAYERS = 8          # distinct layers cycled per step
X_POOL = 64           # distinct activation batches per batch size


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=512)
    p.add_argument("--warmup", type=int, default=64)
    p.add_argument("--batches", type=str, default="1,2,4,8,16,32",
                   help="decode batch sizes; 16 and 32 are verification-sized batches "
                        "(a few slots with draft tokens)")
    p.add_argument("--keep-y", action="store_true",
                   help="decode steps write the expert outputs y and combine them in a "
                        "separate launch (default: moe_layer_forward, which fuses the down "
                        "projection with the combine for batches of 2 to 8)")
    p.add_argument("--head-batch", type=int, default=8,
                   help="the batch the headline value is reported for (largest if absent)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-mixed", action="store_true")
    p.add_argument("--no-q8", action="store_true")
    p.add_argument("--no-iq3", action="store_true")
    p.add_argument("--no-iq1", action="store_true")
    p.add_argument("--prefill-steps", type=int, default=10)
    p.add_argument("--tiered-steps", type=int, default=2048,
                   help="steps of the 48-layer tiered stack (0: skip)")
    p.add_argument("--tiered-prepare", choices=("async", "sync"), default="async",
                   help="tier prepare: on the device (moe_tier_prepare_async) or with a host "
                        "round trip per layer (moe_tier_prepare)")
    p.add_argument("--tiered-sets", type=int, default=4,
                   help="generated expert-weight sets used round-robin by the 48 layers")
    p.add_argument("--tiered-shared-sets", action="store_true",
                   help="layers share their set's pinned copy (default: one copy per layer, "
                        "experts reordered per layer)")
    p.add_argument("--tiered-graph-steps", type=int, default=512,
                   help="steps of the graph-captured tiered run (0: skip)")
    p.add_argument("--no-tiered-check", action="store_true",
                   help="skip the all-resident run the tiered outputs are compared with")
    p.add_argument("--cpu-sample-steps", type=int, default=192,
                   help="decode steps of the oracle on all host cores (about 10 s; "
                        "single-threaded: a sixteenth)")
    p.add_argument("--cpu-prefill-tokens", type=int, default=1024,
                   help="tokens of the prefill slice the oracle runs (extrapolated to 16384)")
    p.add_argument("--profile-steps", type=int, default=0,
                   help="only run this many eager steps per batch (for profilers)")
    p.add_argument("--profile-prefill", type=int, default=0,
                   help="only run this many prefill steps (for profilers)")
    p.add_argument("--profile-format", choices=("mixed", "q8", "iq3", "iq1"), default=None,
                   help="with --profile-prefill: run that many 4096-token prefill FFN calls "
                        "of this layer instead")
    p.add_argument("--copy-calibration", type=int, default=0,
                   help="only copy this many MiB device to device 8 times (counter calibration)")
    return p.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.md")
_T0 = time.time()


def progress(msg):
    """A progress line on stderr (stdout carries only the result line)."""
    print(f"[bench {time.time() - _T0:7.1f} s] {msg}", file=sys.stderr, flush=True)


def sources_digest():
    """sha256 over the library's kernel sources with comments and blank space
    removed: counter readings are only used while the code they were taken on
    is unchanged (a comment edit keeps them)."""
    import hashlib
    import re
    d = os.path.join(ROOT, "quantized_expert_ffn_router_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h")):
            with open(os.path.join(d, f), encoding="utf-8") as fh:
                code = fh.read()
            code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)
            code = re.sub(r"//[^\n]*", " ", code)
            code = " ".join(code.split())
            h.update(f.encode() + b"\0" + code.encode())
    return h.hexdigest()


def measured_traffic(kind):
    """HBM bytes per FFN call from the committed FETCH_SIZE / WRITE_SIZE
    summary, each scaled by its copy-kernel calibration factor; None when the
    summary is missing or was taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
        blob = text.split("```json", 1)[1].split("```", 1)[0]
        rec = json.loads(blob)
    except (OSError, IndexError, ValueError):
        return None
    if rec.get("sources_sha256") != sources_digest() or kind not in rec:
        return None
    r = rec[kind]
    return (r["fetch_kib_per_call"] * rec["fetch_factor"] +
            r["write_kib_per_call"] * rec["write_factor"]) * 1024.0


MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_counters.md")


def measured_mfma(kind):
    """MFMA activity of one prefill FFN call from the committed counter
    summary (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x SIMDs, summed over
    the call's kernels, and the flops the MFMA instructions issued); None when
    the summary is missing or was taken on other kernel sources."""
    try:
        with open(MFMA_FILE) as f:
            text = f.read()
        rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, IndexError, ValueError):
        return None
    if rec.get("sources_sha256") != sources_digest() or kind not in rec:
        return None
    r = rec[kind]
    return {"mfma_busy_frac": r["mfma_busy_frac"],
            "mfma_flops_issued_per_call": r["mfma_flops_issued_per_call"],
            "issued_over_useful": r["issued_over_useful"],
            "source": "profiles/mfma_counters.md"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this layer has no multi-GPU path "
              "(expert-parallel sharding is described in the design notes, not built).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import moegen
    import quantized_expert_ffn_router_amd as q

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        # A plain elementwise kernel that reads n bytes and writes n bytes.
        n = args.copy_calibration << 20
        a = torch.ones(n // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(8):
            torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "copies": 8}))
        return
    if args.profile_prefill and args.profile_format:
        print(json.dumps({"profile_run": True,
                          args.profile_format: measure_format(args, q, moegen, torch, dev,
                                                              args.profile_format)}))
        return
    if args.profile_prefill:
        args.prefill_steps = args.profile_prefill
        print(json.dumps({"profile_run": True, "prefill": measure_prefill(args, q, moegen, torch, dev)}))
        return
    W = moegen.WORKLOADS["decode"]
    batches = [int(b) for b in args.batches.split(",")]
    Bmax = max(batches)

    t0 = time.time()
    host_layers = [moegen.make_layer(W, layer=l) for l in range(N_LAYERS)]
    layers = [q.DeviceLayer(L) for L in host_layers]
    gen_s = time.time() - t0
    expert_bytes = layers[0].blob_bytes + 12  # packed codes + scales, 3 fp32 tensor scales
    buf = q.StepBuffers(layers[0], Bmax)
    stream = torch.cuda.Stream()

    # n_active of each step, copied on the device (no host sync inside steps)
    bk = buf.buckets
    na_off = bk.n_active - buf.bucket_buf.data_ptr()
    n_active_view = buf.bucket_buf[na_off:na_off + 4].view(torch.int32)

    results = {}
    for B in batches:
        xs = [torch.from_numpy(moegen.make_tokens(W, B, step=s, layer=B).view(np.int16).copy()).to(dev)
              for s in range(X_POOL)]

        def step(i):
            return q.layer_forward(layers[i % N_LAYERS], buf, xs[i % X_POOL], B, stream=stream,
                                   keep_y=args.keep_y)

        # cold: the first step of this batch size, before any warm-up (eager
        # launches; the first batch's also pays the library's first launches)
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            c0.record(stream)
            step(0)
            c1.record(stream)
        torch.cuda.synchronize()
        cold_us = c0.elapsed_time(c1) * 1e3

        with torch.cuda.stream(stream):
            for i in range(args.warmup):
                step(i)
        torch.cuda.synchronize()

        if args.profile_steps:
            with torch.cuda.stream(stream):
                for i in range(args.profile_steps):
                    step(i)
            torch.cuda.synchronize()
            continue

        # (1) FFN kernel time: HIP events on the launch stream around each
        #     moe_expert_ffn call (eager launches), expert bytes from the
        #     realised active-expert count of each step.
        n_ev = min(args.steps, 256)
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
        nact = torch.zeros(n_ev, dtype=torch.int32, device=dev)
        with torch.cuda.stream(stream):
            for i in range(n_ev):
                L = layers[i % N_LAYERS]
                d = L.desc
                x = xs[i % X_POOL]
                q.moe_route(d, x, B, buf.logits, buf.idx, buf.w, stream)
                q.moe_bucket(d, buf.idx, B, buf.buckets, buf.ws, buf.ws_bytes, stream)
                starts[i].record(stream)
                q.moe_expert_ffn(d, x, B, buf.buckets, buf.y, buf.y_dtype, buf.ws, buf.ws_bytes,
                                 stream)
                ends[i].record(stream)
                nact[i:i + 1].copy_(n_active_view)
                q.moe_combine(d, buf.y, buf.y_dtype, buf.buckets, buf.w, B, None, buf.out, stream)
                q.moe_expert_hist(d, buf.buckets, buf.hist, 5, 10, stream)
        torch.cuda.synchronize()
        ffn_ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
        na = nact.cpu().numpy().astype(np.float64)
        ffn_bytes = na * expert_bytes
        ffn_gbs = float(ffn_bytes.sum() / (ffn_ms.sum() * 1e-3) / 1e9)

        # (1b) the same FFN calls back to back from a HIP graph
        ffn_graph_us, ffn_graph_gbs = ffn_graph_rate(q, torch, layers, xs, B, buf, stream,
                                                     expert_bytes)

        # (2) whole-step throughput: exactly args.steps steps, replayed from
        # HIP graphs (one of X_POOL steps, replayed steps // X_POOL times, and
        # one of the remaining steps % X_POOL)
        full, rest = divmod(args.steps, X_POOL)
        graphs = []
        for n_in in ([X_POOL] if full else []) + ([rest] if rest else []):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(n_in):
                    step(i)
            graphs.append((g, n_in))
        torch.cuda.synchronize()
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):  # replay() launches on the current stream
            for g, _ in graphs:
                g.replay()
            torch.cuda.synchronize()
            t_start.record(stream)
            for g, n_in in graphs:
                for _ in range(full if n_in == X_POOL else 1):
                    g.replay()
            t_end.record(stream)
        torch.cuda.synchronize()
        total_ms = t_start.elapsed_time(t_end)
        steps_done = args.steps
        ms_step = total_ms / steps_done
        progress(f"decode batch {B}: {ms_step * 1e3:.2f} us/step")
        results[B] = dict(
            batch=B, steps=steps_done, ms_per_step=ms_step, tok_per_s=B / (ms_step * 1e-3),
            ffn_us=float(ffn_ms.mean() * 1e3), active_experts=float(na.mean()),
            expert_bytes_per_step=float(ffn_bytes.mean()), ffn_GBps=ffn_gbs,
            ffn_hbm_frac=ffn_gbs / HBM_PEAK_GBS, ffn_graph_us=ffn_graph_us,
            ffn_graph_GBps=ffn_graph_gbs, ffn_graph_hbm_frac=ffn_graph_gbs / HBM_PEAK_GBS,
            cold_first_step_us=cold_us)
        del graphs

    if args.profile_steps:
        print(json.dumps({"profile_run": True, "batches": batches}))
        return

    prefill = None if args.no_prefill else measure_prefill(args, q, moegen, torch, dev)
    progress("prefill done")
    del layers, buf
    torch.cuda.empty_cache()
    mixed = None if args.no_mixed else measure_format(args, q, moegen, torch, dev, "mixed")
    q8 = None if args.no_q8 else measure_format(args, q, moegen, torch, dev, "q8")
    iq3 = None if args.no_iq3 else measure_format(args, q, moegen, torch, dev, "iq3")
    iq1 = None if args.no_iq1 else measure_format(args, q, moegen, torch, dev, "iq1")
    progress("format layers done")
    torch.cuda.empty_cache()
    tiered = None if args.tiered_steps <= 0 else measure_tiered(args, q, moegen, torch)
    progress("tiered stack done")

    Bh = args.head_batch if args.head_batch in results else Bmax
    head = results[Bh]
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(W, host_layers[0], Bh, args.cpu_sample_steps, args.cpu_prefill_tokens)

    line = {
        "metric": "MoE-layer decode tok/s + expert-weight HBM GB/s (% peak); prefill TFLOP/s",
        "value": round(head["tok_per_s"], 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "accumulate_dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"decode step, batch {Bh}: 128 experts, top-8, hidden 2048, "
                        "intermediate 768, NVFP4 gate/up/down, bf16 activations",
            "batch": Bh, "experts": 128, "top_k": 8, "hidden": 2048, "intermediate": 768,
            "weights": "nvfp4", "layers_cycled": N_LAYERS, "hip_graph": True,
        },
        "roofline": {
            "kernel": "expert FFN (k_gemv_gateup32_nvfp4<8, 32> + k_gemv_down<1, 2, 2, false>, NVFP4)",
            "bound": "hbm",
            "achieved": round(head["ffn_graph_GBps"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(head["ffn_graph_hbm_frac"], 4),
            "traffic": measured_traffic("decode_ffn_b8") if Bh == 8 else None,
            "timing": "HIP events around replays of a graph of 128 moe_expert_ffn calls "
                      "(16 bucket sets, 8 layers); eager calls bracketed one by one include "
                      "the host's launch gaps: eager_achieved / eager_frac",
            "eager_achieved": round(head["ffn_GBps"], 1),
            "eager_frac": round(head["ffn_hbm_frac"], 4),
        },
        "per_batch": [
            {k: (round(v, 4) if isinstance(v, float) else v) for k, v in results[b].items()}
            for b in batches
        ],
        "prefill": prefill,
        "mixed": mixed,
        "q8_0": q8,
        "iq3g": iq3,
        "iq1g": iq1,
        "tiered": tiered,
        "cpu_baseline": cpu,
        "setup_s": round(gen_s, 1),
    }
    print(json.dumps(line))


def measure_prefill(args, q, moegen, torch, dev):
    """16384-token prefill of the same layer shape with the Zipf(1.1)-biased
    router: whole-layer time and the grouped-GEMM FFN's TFLOP/s
    (6 * T * k * H * I useful flops, HIP events on the launch stream)."""
    W = moegen.WORKLOADS["prefill"]
    L = moegen.make_layer(W, layer=100)
    dl = q.DeviceLayer(L)
    T = W.T
    buf = q.StepBuffers(dl, T, q.MOE_DTYPE_BF16)
    xs = [torch.from_numpy(moegen.make_tokens(W, T, step=s).view(np.int16).copy()).to(dev)
          for s in range(2)]
    stream = torch.cuda.Stream()
    d = dl.desc
    n = args.prefill_steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
    with torch.cuda.stream(stream):
        for i in range(2):
            q.layer_forward(dl, buf, xs[i % 2], T, stream=stream)
        torch.cuda.synchronize()
        for i in range(n):
            x = xs[i % 2]
            ev[i][0].record(stream)
            q.moe_route(d, x, T, buf.logits, buf.idx, buf.w, stream)
            q.moe_bucket(d, buf.idx, T, buf.buckets, buf.ws, buf.ws_bytes, stream)
            ev[i][1].record(stream)
            q.moe_expert_ffn(d, x, T, buf.buckets, buf.y, buf.y_dtype, buf.ws, buf.ws_bytes, stream)
            ev[i][2].record(stream)
            q.moe_combine(d, buf.y, buf.y_dtype, buf.buckets, buf.w, T, None, buf.out, stream)
            q.moe_expert_hist(d, buf.buckets, buf.hist, 5, 10, stream)
            ev[i][3].record(stream)
    torch.cuda.synchronize()
    route_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    ffn_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    layer_ms = float(np.mean([e[0].elapsed_time(e[3]) for e in ev]))
    flops = 6.0 * T * W.k * W.H * W.I
    tflops = flops / (ffn_ms * 1e-3) / 1e12
    counts = buf.bucket_view(W.E, T, W.k)["counts"]
    return {
        "workload": "prefill: 16384 tokens, 128 experts, top-8, hidden 2048, intermediate 768, "
                    "NVFP4, Zipf(1.1)-biased router, bf16 expert outputs",
        "steps": n, "layer_ms": round(layer_ms, 4), "tok_per_s": round(T / (layer_ms * 1e-3), 1),
        "route_bucket_ms": round(route_ms, 4), "ffn_ms": round(ffn_ms, 4),
        "ffn_tflops": round(tflops, 2),
        "roofline": {"kernel": "grouped GEMM (k_gemm_gateup_nvfp4<true, false> + k_gemm_down<1, true, true, 1>, NVFP4)", "bound": "mfma",
                     "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic("prefill_ffn"),
                     "mfma_counters": measured_mfma("prefill_ffn")},
        "expert_load": {"max": int(counts.max()), "min": int(counts.min()),
                        "mean": float(counts.mean())},
        "padding": mfma_rows(counts),
    }


FORMAT_LAYERS = {
    "mixed": "mixed layer: 256 experts, top-8, hidden 2048, intermediate 512, "
             "NVFP4 gate/up, Q6_K-style down",
    "q8": "Q8_0-down layer: 128 experts, top-8, hidden 2048, intermediate 768, "
          "NVFP4 gate/up, Q8_0 down",
    "iq3": "IQ3G-down layer: 128 experts, top-8, hidden 2048, intermediate 768, "
           "NVFP4 gate/up, IQ3-style grid down (own grid, 3.19 bits per weight)",
    "iq1": "IQ1G-down layer: 128 experts, top-8, hidden 2048, intermediate 768, "
           "NVFP4 gate/up, IQ1-style ternary grid down (own grid, 1.44 bits per weight)",
}


def ffn_graph_rate(q, torch, layers, xs, B, buf, stream, expert_bytes, combos=16, reps=4):
    """moe_expert_ffn calls back to back, replayed from a HIP graph: the
    buckets of the `combos` (layer, input) pairs that i % len(layers),
    i % len(xs) walk through are made beforehand, the graph holds 8 rounds of
    them, and HIP events bracket `reps` replays after a warm one.  Returns
    (us per call, GB/s over the active experts' bytes): the FFN's time as a
    graph-replayed step runs it, without the host's launch gaps between
    eager calls."""
    nl, nx = len(layers), len(xs)
    L0 = layers[0]
    gbufs = [q.StepBuffers(L0, B) for _ in range(combos)]
    with torch.cuda.stream(stream):
        for c, gb in enumerate(gbufs):
            d = layers[c % nl].desc
            q.moe_route(d, xs[c % nx], B, gb.logits, gb.idx, gb.w, stream)
            q.moe_bucket(d, gb.idx, B, gb.buckets, gb.ws, gb.ws_bytes, stream)
    torch.cuda.synchronize()
    na = np.array([gb.bucket_view(L0.E, B, L0.k)["n_active"] for gb in gbufs], np.float64)
    calls = 8 * combos
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for r in range(calls):
            c = r % combos
            q.moe_expert_ffn(layers[c % nl].desc, xs[c % nx], B, gbufs[c].buckets, buf.y,
                             buf.y_dtype, buf.ws, buf.ws_bytes, stream)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        graph.replay()
        e0.record(stream)
        for _ in range(reps):
            graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * calls)
    del graph, gbufs
    return us, float(na.mean() * expert_bytes / (us * 1e-6) / 1e9)


def measure_format(args, q, moegen, torch, dev, name):
    """A layer with another down-projection format (the mixed layer: 256
    experts, top-8, hidden 2048, intermediate 512, Q6_K-style down; the Q8_0,
    IQ3G and IQ1G layers: the decode layer's shape with that down format): decode
    batch 8 expert FFN (GB/s over the active experts' bytes, four layer copies
    cycled so the Infinity Cache cannot hold them; eager calls and graph
    replays, see ffn_graph_rate) and the 4096-token prefill FFN (TFLOP/s), HIP
    events on the launch stream around moe_expert_ffn."""
    W = moegen.WORKLOADS[name]
    n_layers = 4
    layers = [q.DeviceLayer(moegen.make_layer(W, layer=200 + l)) for l in range(n_layers)]
    expert_bytes = layers[0].blob_bytes + 8
    stream = torch.cuda.Stream()
    out = {"workload": FORMAT_LAYERS[name]}
    if args.profile_format:
        return measure_format_prefill(args, q, moegen, torch, dev, W, layers[0], stream, out,
                                      args.profile_prefill)
    # decode, batch 8
    B = 8
    buf = q.StepBuffers(layers[0], B)
    bk = buf.buckets
    na_off = bk.n_active - buf.bucket_buf.data_ptr()
    n_active_view = buf.bucket_buf[na_off:na_off + 4].view(torch.int32)
    xs = [torch.from_numpy(moegen.make_tokens(W, B, step=s, layer=300).view(np.int16).copy()).to(dev)
          for s in range(X_POOL)]
    n = 256
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    nact = torch.zeros(n, dtype=torch.int32, device=dev)
    with torch.cuda.stream(stream):
        for i in range(16 + n):
            L = layers[i % n_layers]
            x = xs[i % X_POOL]
            q.moe_route_bucket(L.desc, x, B, buf.logits, buf.idx, buf.w, buf.buckets, buf.ws,
                               buf.ws_bytes, None, 0, 0, stream)
            if i >= 16:
                ev[i - 16][0].record(stream)
            q.moe_expert_ffn(L.desc, x, B, buf.buckets, buf.y, buf.y_dtype, buf.ws, buf.ws_bytes,
                             stream)
            if i >= 16:
                ev[i - 16][1].record(stream)
                nact[i - 16:i - 15].copy_(n_active_view)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    na = nact.cpu().numpy().astype(np.float64)
    gbs = float((na * expert_bytes).sum() / (ms.sum() * 1e-3) / 1e9)
    g_us, g_gbs = ffn_graph_rate(q, torch, layers, xs, B, buf, stream, expert_bytes)
    out["decode_b8"] = {"ffn_us": round(float(ms.mean() * 1e3), 3),
                        "active_experts": round(float(na.mean()), 2),
                        "ffn_GBps": round(gbs, 1), "ffn_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                        "ffn_graph_us": round(g_us, 3), "ffn_graph_GBps": round(g_gbs, 1),
                        "ffn_graph_hbm_frac": round(g_gbs / HBM_PEAK_GBS, 4)}
    del buf
    return measure_format_prefill(args, q, moegen, torch, dev, W, layers[0], stream, out, 10)


def mfma_rows(counts, bm=128):
    """Rows the grouped GEMM multiplies (each expert's rows rounded up to whole
    128-row blocks) against the useful rows."""
    c = np.asarray(counts, dtype=np.int64)
    computed = int((-(-c // bm) * bm).sum())
    return {"rows_computed": computed, "rows_useful": int(c.sum()),
            "computed_over_useful": round(computed / max(1, int(c.sum())), 4)}


def measure_format_prefill(args, q, moegen, torch, dev, W, L, stream, out, n):
    """The 4096-token prefill FFN of a format layer: n timed calls after 2
    untimed ones (HIP events on the launch stream)."""
    T = W.extra["prefill_T"]
    buf = q.StepBuffers(L, T, q.MOE_DTYPE_BF16)
    x = torch.from_numpy(moegen.make_tokens(W, T, step=1).view(np.int16).copy()).to(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    with torch.cuda.stream(stream):
        q.moe_route_bucket(L.desc, x, T, buf.logits, buf.idx, buf.w, buf.buckets, buf.ws,
                           buf.ws_bytes, None, 0, 0, stream)
        for i in range(2 + n):
            if i >= 2:
                ev[i - 2][0].record(stream)
            q.moe_expert_ffn(L.desc, x, T, buf.buckets, buf.y, buf.y_dtype, buf.ws, buf.ws_bytes,
                             stream)
            if i >= 2:
                ev[i - 2][1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    flops = 6.0 * T * W.k * W.H * W.I
    tf = flops / (ms * 1e-3) / 1e12
    out["prefill_4096"] = {"ffn_ms": round(ms, 4), "ffn_tflops": round(tf, 2),
                           "frac_of_2500": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                           "padding": mfma_rows(buf.bucket_view(W.E, T, W.k)["counts"]),
                           "mfma_counters": measured_mfma(W.name + "_prefill")}
    return out


PCIE_GEN5_X16_GBPS = 63.0  # 32 GT/s x 16 lanes, 128b/130b encoding, one direction


def tier_copy_ceiling(q, moegen, torch, W, wset):
    """Host-to-HBM rate of the tier's own copy path: one layer of the given
    expert set in pinned host memory, no resident slots and staging for all
    experts, 64 tokens routed (so about 220 of the 256 experts active, every
    one a miss); moe_tier_prepare_async (planning kernel, then the copy kernel
    reading the pinned blobs) repeated on the same buckets, timed with HIP
    events on its stream.  Bytes: active experts x packed expert bytes."""
    from quantized_expert_ffn_router_amd.stack import LayerStack
    router = moegen.normal_f32(moegen.key(0, moegen.TAG_ROUTER, 777), W.E * W.H, W.w_std) \
        .reshape(W.E, W.H)
    stack = LayerStack([wset], [router], lambda l, e: None, L=1, k=W.k,
                       tiered={"resident": 0, "staging": W.E, "async": True})
    T = 64
    x = torch.from_numpy(moegen.make_tokens(W, T, step=5, layer=777).view(np.int16).copy()).cuda()
    stream = torch.cuda.current_stream()
    stack.step(x, T)
    torch.cuda.synchronize()
    buf = stack.buf
    bk = buf.bucket_view(W.E, T, W.k)
    n_act = bk["n_active"]
    reps = 8
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    q.moe_tier_prepare_async(stack.tier, 0, buf.buckets, stack.tables[0], stream)
    a.record(stream)
    for _ in range(reps):
        q.moe_tier_prepare_async(stack.tier, 0, buf.buckets, stack.tables[0], stream)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    gbs = reps * n_act * stack.eb / (ms * 1e-3) / 1e9
    stack.close()
    del stack
    torch.cuda.empty_cache()
    return {"GBps": round(gbs, 2), "experts_per_copy": n_act,
            "bytes_per_copy": n_act * stack_eb_bytes(W),
            "method": "moe_tier_prepare_async with every active expert a miss, 8 repeats"}


def stack_eb_bytes(W):
    import quantized_expert_ffn_router_amd as q
    return q.moe_expert_blob_bytes(W.H, W.I, q.MOE_FMT_NVFP4, W.fmt_down)


def measure_tiered(args, q, moegen, torch):
    """48 stacked mixed-format layers (256 experts, top-8, hidden 2048,
    intermediate 512, NVFP4 gate/up, Q6_K down), 96 experts resident per layer
    in HBM, the rest in pinned host RAM copied on demand; 8 tokens per step;
    router bias Zipf(1.2) with the ranking redrawn every 256 steps (drift);
    resident sets rebalanced from the usage histograms every 8 steps.

    Every layer holds its own pinned copy of its experts (4 generated weight
    sets, experts reordered per layer), so the host footprint is that of 48
    distinct layers.  The eager run's outputs of every step are compared bit
    for bit with an all-resident stack's; then the whole 48-layer step is
    captured as one HIP graph and replayed, also compared."""
    import resource
    from quantized_expert_ffn_router_amd.stack import LayerStack
    W = moegen.WORKLOADS["tiered"]
    Lyr, R, S, T = W.extra["layers"], W.extra["resident"], 64, W.T
    drift, rb_every = W.extra["drift"], 8
    n_steps, n_graph = args.tiered_steps, min(args.tiered_graph_steps, args.tiered_steps)
    sets = [moegen.make_layer(W, layer=200 + i) for i in range(args.tiered_sets)]
    routers = [moegen.normal_f32(moegen.key(0, moegen.TAG_ROUTER, 300 + l), W.E * W.H, W.w_std)
               .reshape(W.E, W.H) for l in range(Lyr)]
    perms = None if args.tiered_shared_sets else \
        [moegen.permutation(moegen.key(0, moegen.TAG_PERM, 300 + l), W.E) for l in range(Lyr)]

    def bias(l, epoch):
        b, _ = moegen.zipf_bias(moegen.key(0, moegen.TAG_BIAS, 300 + l, epoch), W.E, W.zipf_s,
                                W.zipf_alpha)
        return b

    progress("tiered: weight sets generated")
    h2d_ceiling = tier_copy_ceiling(q, moegen, torch, W, sets[0])
    memlock = resource.getrlimit(resource.RLIMIT_MEMLOCK)
    tiered_cfg = {"resident": R, "staging": S, "async": args.tiered_prepare == "async"}
    footprint_note = None
    try:
        stack = LayerStack(sets, routers, bias, L=Lyr, k=W.k, tiered=tiered_cfg, layer_perms=perms)
    except (RuntimeError, q.MoeError) as e:  # pinned host memory refused
        if perms is None:
            raise
        footprint_note = f"per-layer pinned copies refused ({e}); expert sets shared by layers"
        perms = None
        torch.cuda.empty_cache()
        stack = LayerStack(sets, routers, bias, L=Lyr, k=W.k, tiered=tiered_cfg)
    ref = None if args.no_tiered_check else \
        LayerStack(sets, routers, bias, L=Lyr, k=W.k, layer_perms=perms)
    del sets
    progress("tiered: stacks built")
    # fresh tokens for every step (a recycled pool would make the routing periodic)
    xs = torch.from_numpy(np.stack([moegen.make_tokens(W, T, step=s, layer=999)
                                    for s in range(n_steps)]).view(np.int16)).cuda()
    x = torch.empty_like(xs[0])
    out_t = torch.empty((n_steps, T, W.H), dtype=torch.int16, device="cuda")
    for st in range(4):  # warm: first fill of the resident sets
        x.copy_(xs[st])
        stack.step(x, T, epoch=0)
    stack.rebalance()
    torch.cuda.synchronize()
    s0, _ = q.moe_tier_stats_get(stack.tier)
    t = time.time()
    per_epoch = []
    prev = s0
    for st in range(n_steps):
        x.copy_(xs[st])
        stack.step(x, T, epoch=st // drift)
        out_t[st].copy_(x)
        if (st + 1) % rb_every == 0:
            stack.rebalance()
        if (st + 1) % drift == 0:
            cur, _ = q.moe_tier_stats_get(stack.tier)
            per_epoch.append(round((cur["misses"] - prev["misses"]) /
                                   max(1, (cur["misses"] - prev["misses"]) + (cur["hits"] - prev["hits"])), 4))
            prev = cur
    torch.cuda.synchronize()
    wall = time.time() - t
    s1, _ = q.moe_tier_stats_get(stack.tier)
    d = {k: s1[k] - s0[k] for k in s1}
    h2d_gbs = d["h2d_bytes"] / wall / 1e9

    progress(f"tiered: {n_steps} eager steps in {wall:.1f} s")
    # the same steps, captured: one graph of the 48-layer step, replayed on the
    # step's input, biases refilled at epoch changes, rebalanced every 8 steps
    graph = None
    if n_graph > 0 and args.tiered_prepare == "async":
        stack.use_bias_buffers(epoch=0)
        out_g = torch.empty((n_graph, T, W.H), dtype=torch.int16, device="cuda")
        g = stack.capture(x, T)
        torch.cuda.synchronize()
        g0, _ = q.moe_tier_stats_get(stack.tier)
        t = time.time()
        for st in range(n_graph):
            if st % drift == 0:
                stack.set_epoch(st // drift)
            x.copy_(xs[st])
            g.replay()
            out_g[st].copy_(x)
            if (st + 1) % rb_every == 0:
                stack.rebalance()
        torch.cuda.synchronize()
        gwall = time.time() - t
        g1, _ = q.moe_tier_stats_get(stack.tier)
        gd = {k: g1[k] - g0[k] for k in ("hits", "misses", "h2d_bytes")}
        graph = {"steps": n_graph, "wall_s": round(gwall, 3),
                 "ms_per_step": round(gwall / n_graph * 1e3, 3),
                 "tok_per_s": round(T * n_graph / gwall, 2),
                 "miss_rate": round(gd["misses"] / max(1, gd["misses"] + gd["hits"]), 4),
                 "h2d_GBps": round(gd["h2d_bytes"] / gwall / 1e9, 2)}
        del g
    host_gb = stack.host_bytes / 1e9
    stack.close()
    del stack
    torch.cuda.empty_cache()

    progress("tiered: graph-captured run done")
    check, ideal_per_epoch = None, None
    if ref is not None:
        # The all-resident run routes exactly as the tiered one (its outputs
        # are compared bit for bit), so it also counts, per layer, the steps
        # in which each expert is active: at an epoch's end the best static
        # resident set in hindsight (the R most often active experts of each
        # layer) gives the miss rate no placement policy could beat.
        out_r = torch.empty_like(out_t)
        active = torch.zeros((Lyr, W.E), dtype=torch.int32, device="cuda")
        ideal_per_epoch = []
        for st in range(n_steps):
            x.copy_(xs[st])
            ref.step(x, T, epoch=st // drift, active_acc=active)
            out_r[st].copy_(x)
            if (st + 1) % drift == 0:
                a = np.sort(active.cpu().numpy().astype(np.int64), axis=1)[:, ::-1]
                ideal_per_epoch.append(round(1.0 - a[:, :R].sum() / max(1, a.sum()), 4))
                active.zero_()
        torch.cuda.synchronize()
        same = (out_t == out_r).reshape(n_steps, -1).all(dim=1).cpu().numpy()
        check = {"steps": n_steps, "equal": bool(same.all()),
                 "first_differing_step": None if same.all() else int(np.argmin(same))}
        if graph is not None:
            gsame = (out_g == out_r[:n_graph]).reshape(n_graph, -1).all(dim=1).cpu().numpy()
            graph["equal_all_resident"] = bool(gsame.all())
        ref.close()
        del ref, out_r
    return {
        "workload": "tiered decode: 48 layers x (256 experts, top-8, hidden 2048, intermediate "
                    "512, NVFP4 gate/up, Q6_K down), 96 resident per layer, 8 tokens/step, "
                    "Zipf(1.2) routing drifting every 256 steps",
        "prepare": args.tiered_prepare,
        "steps": n_steps, "wall_s": round(wall, 3),
        "tok_per_s": round(T * n_steps / wall, 2),
        "ms_per_step": round(wall / n_steps * 1e3, 3),
        "miss_rate": round(d["misses"] / max(1, d["misses"] + d["hits"]), 4),
        "miss_rate_per_epoch": per_epoch,
        "ideal_miss_rate_per_epoch": ideal_per_epoch,
        "ideal_note": "best static resident set per epoch in hindsight: the 96 most often "
                      "active experts of each layer over the epoch's steps",
        "inputs": "fresh seeded tokens for every step",
        "h2d_GBps": round(h2d_gbs, 2),
        "copy_path_ceiling": h2d_ceiling,
        "pcie_gen5_x16_spec_GBps": PCIE_GEN5_X16_GBPS,
        "h2d_frac_of_ceiling": round(h2d_gbs / h2d_ceiling["GBps"], 4),
        "h2d_frac_of_spec": round(h2d_gbs / PCIE_GEN5_X16_GBPS, 4),
        "frac_above_1_flag": (h2d_gbs > h2d_ceiling["GBps"]) or (h2d_gbs > PCIE_GEN5_X16_GBPS),
        "host_footprint_GB": round(host_gb, 2),
        "per_layer_host_copies": perms is not None,
        "expert_sets": args.tiered_sets,
        "footprint_note": footprint_note,
        "rlimit_memlock": [int(v) for v in memlock],
        "bit_exact_vs_all_resident": check,
        "graph_captured": graph,
        "counters": d,
    }


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(W, L, B, n_steps, prefill_tokens):
    """The oracle as it stands, on bounded samples of the same workloads:
    decode steps of batch B on one layer, on all host cores (its OpenMP build:
    the same loops, the listed assignments in parallel, same results) and
    single-threaded; and a slice of the 16384-token prefill on all cores,
    extrapolated per token.  Reported in the metric's units."""
    import ctypes
    import moegen
    import oracle
    threads = int(ctypes.CDLL(oracle._LIB_OMP).omp_get_max_threads()) \
        if os.path.exists(oracle._LIB_OMP) else 1
    oracle.lib(True)  # load before timing
    t = time.time()
    for s in range(n_steps):
        oracle.layer(moegen.make_tokens(W, B, step=10_000 + s), L, parallel=True)
    dt_all = time.time() - t
    progress(f"cpu baseline: {n_steps} decode steps on all cores in {dt_all:.1f} s")
    n_single = max(1, n_steps // 16)
    t = time.time()
    for s in range(n_single):
        oracle.layer(moegen.make_tokens(W, B, step=20_000 + s), L)
    dt_one = time.time() - t
    progress(f"cpu baseline: {n_single} decode steps on one core in {dt_one:.1f} s")
    WP = moegen.WORKLOADS["prefill"]
    LP = moegen.make_layer(WP, layer=100)
    xp = moegen.make_tokens(WP, prefill_tokens, step=0)
    t = time.time()
    oracle.layer(xp, LP, parallel=True)
    dt_pre = time.time() - t
    pre_tok_s = prefill_tokens / dt_pre
    flops = 6.0 * WP.k * WP.H * WP.I  # per token, as the GPU figure counts them
    return {
        "value": round(B * n_steps / dt_all, 3), "unit": "tok/s", "cores": threads,
        "kind": "oracle",
        "sample": f"{n_steps} decode steps of batch {B} on one layer, plain C in double "
                  f"precision, OpenMP build on {threads} threads ({dt_all:.1f} s)",
        "cpu_model": cpu_model(), "nproc": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "single_thread": {"value": round(B * n_single / dt_one, 3), "unit": "tok/s", "cores": 1,
                          "sample": f"{n_single} decode steps of batch {B} ({dt_one:.1f} s)"},
        "prefill": {"value": round(pre_tok_s, 3), "unit": "tok/s", "cores": threads,
                    "gflops_equiv": round(pre_tok_s * flops / 1e9, 3),
                    "sample": f"{prefill_tokens}-token slice of the 16384-token prefill layer "
                              f"(Zipf(1.1) router bias) on {threads} threads ({dt_pre:.1f} s); "
                              f"16384 tokens extrapolated at this per-token rate: "
                              f"{16384 / pre_tok_s:.0f} s"},
    }


if __name__ == "__main__":
    main()
