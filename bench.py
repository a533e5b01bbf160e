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
    p.add_argument("--head-batch", type=int, default=8,
                   help="the batch the headline value is reported for (largest if absent)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-mixed", action="store_true")
    p.add_argument("--no-q8", action="store_true")
    p.add_argument("--prefill-steps", type=int, default=10)
    p.add_argument("--tiered-steps", type=int, default=2048,
                   help="steps of the 48-layer tiered stack (0: skip)")
    p.add_argument("--tiered-prepare", choices=("async", "sync"), default="async",
                   help="tier prepare: on the device (moe_tier_prepare_async) or with a host "
                        "round trip per layer (moe_tier_prepare)")
    p.add_argument("--tiered-sets", type=int, default=4,
                   help="distinct expert-weight sets shared round-robin by the 48 layers")
    p.add_argument("--cpu-sample-steps", type=int, default=12)
    p.add_argument("--profile-steps", type=int, default=0,
                   help="only run this many eager steps per batch (for profilers)")
    p.add_argument("--profile-prefill", type=int, default=0,
                   help="only run this many prefill steps (for profilers)")
    p.add_argument("--copy-calibration", type=int, default=0,
                   help="only copy this many MiB device to device 8 times (counter calibration)")
    return p.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.md")


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
            return q.layer_forward(layers[i % N_LAYERS], buf, xs[i % X_POOL], B, stream=stream)

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

        # (2) whole-step throughput: the steps captured in a HIP graph
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(X_POOL):
                step(i)
        torch.cuda.synchronize()
        reps = max(1, args.steps // X_POOL)
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):  # replay() launches on the current stream
            g.replay()
            torch.cuda.synchronize()
            t_start.record(stream)
            for _ in range(reps):
                g.replay()
            t_end.record(stream)
        torch.cuda.synchronize()
        total_ms = t_start.elapsed_time(t_end)
        steps_done = reps * X_POOL
        ms_step = total_ms / steps_done
        results[B] = dict(
            batch=B, steps=steps_done, ms_per_step=ms_step, tok_per_s=B / (ms_step * 1e-3),
            ffn_us=float(ffn_ms.mean() * 1e3), active_experts=float(na.mean()),
            expert_bytes_per_step=float(ffn_bytes.mean()), ffn_GBps=ffn_gbs,
            ffn_hbm_frac=ffn_gbs / HBM_PEAK_GBS)
        del g

    if args.profile_steps:
        print(json.dumps({"profile_run": True, "batches": batches}))
        return

    prefill = None if args.no_prefill else measure_prefill(args, q, moegen, torch, dev)
    del layers, buf
    torch.cuda.empty_cache()
    mixed = None if args.no_mixed else measure_format(args, q, moegen, torch, dev, "mixed")
    q8 = None if args.no_q8 else measure_format(args, q, moegen, torch, dev, "q8")
    torch.cuda.empty_cache()
    tiered = None if args.tiered_steps <= 0 else measure_tiered(args, q, moegen, torch)

    Bh = args.head_batch if args.head_batch in results else Bmax
    head = results[Bh]
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(W, host_layers[0], Bh, args.cpu_sample_steps)

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
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"decode step, batch {Bh}: 128 experts, top-8, hidden 2048, "
                        "intermediate 768, NVFP4 gate/up/down, bf16 activations",
            "batch": Bh, "experts": 128, "top_k": 8, "hidden": 2048, "intermediate": 768,
            "weights": "nvfp4", "layers_cycled": N_LAYERS, "hip_graph": True,
        },
        "roofline": {
            "kernel": "expert FFN (k_gemv_gateup_nvfp4<4, 2> + k_gemv_down<1, 2, 2, false>, NVFP4)",
            "bound": "hbm",
            "achieved": round(head["ffn_GBps"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(head["ffn_hbm_frac"], 4),
            "traffic": measured_traffic("decode_ffn_b8") if Bh == 8 else None,
        },
        "per_batch": [
            {k: (round(v, 4) if isinstance(v, float) else v) for k, v in results[b].items()}
            for b in batches
        ],
        "prefill": prefill,
        "mixed": mixed,
        "q8_0": q8,
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
                     "traffic": measured_traffic("prefill_ffn")},
        "expert_load": {"max": int(counts.max()), "min": int(counts.min()),
                        "mean": float(counts.mean())},
    }


FORMAT_LAYERS = {
    "mixed": "mixed layer: 256 experts, top-8, hidden 2048, intermediate 512, "
             "NVFP4 gate/up, Q6_K-style down",
    "q8": "Q8_0-down layer: 128 experts, top-8, hidden 2048, intermediate 768, "
          "NVFP4 gate/up, Q8_0 down",
}


def measure_format(args, q, moegen, torch, dev, name):
    """A layer with another down-projection format (the mixed layer: 256
    experts, top-8, hidden 2048, intermediate 512, Q6_K-style down; the Q8_0
    layer: the decode layer's shape with Q8_0 down): decode batch 8 expert FFN
    (GB/s over the active experts' bytes, four layer copies cycled so the
    Infinity Cache cannot hold them) and the 4096-token prefill FFN (TFLOP/s),
    HIP events on the launch stream around moe_expert_ffn."""
    W = moegen.WORKLOADS[name]
    n_layers = 4
    layers = [q.DeviceLayer(moegen.make_layer(W, layer=200 + l)) for l in range(n_layers)]
    expert_bytes = layers[0].blob_bytes + 8
    stream = torch.cuda.Stream()
    out = {"workload": FORMAT_LAYERS[name]}
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
    out["decode_b8"] = {"ffn_us": round(float(ms.mean() * 1e3), 3),
                        "active_experts": round(float(na.mean()), 2),
                        "ffn_GBps": round(gbs, 1), "ffn_hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    del buf
    # prefill, 4096 tokens
    T = W.extra["prefill_T"]
    L = layers[0]
    buf = q.StepBuffers(L, T, q.MOE_DTYPE_BF16)
    x = torch.from_numpy(moegen.make_tokens(W, T, step=1).view(np.int16).copy()).to(dev)
    n = 10
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
                           "frac_of_2500": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
    return out


def measure_tiered(args, q, moegen, torch):
    """48 stacked mixed-format layers (256 experts, top-8, hidden 2048,
    intermediate 512, NVFP4 gate/up, Q6_K down), 96 experts resident per layer
    in HBM, the rest in pinned host RAM copied on demand; 8 tokens per step;
    router bias Zipf(1.2) with the ranking redrawn every 256 steps (drift);
    resident sets rebalanced from the usage histograms every 8 steps."""
    from quantized_expert_ffn_router_amd.stack import LayerStack
    W = moegen.WORKLOADS["tiered"]
    Lyr, R, S, T = W.extra["layers"], W.extra["resident"], 64, W.T
    drift, rb_every = W.extra["drift"], 8
    sets = [moegen.make_layer(W, layer=200 + i) for i in range(args.tiered_sets)]
    routers = [moegen.normal_f32(moegen.key(0, moegen.TAG_ROUTER, 300 + l), W.E * W.H, W.w_std)
               .reshape(W.E, W.H) for l in range(Lyr)]

    def bias(l, epoch):
        b, _ = moegen.zipf_bias(moegen.key(0, moegen.TAG_BIAS, 300 + l, epoch), W.E, W.zipf_s,
                                W.zipf_alpha)
        return b

    stack = LayerStack(sets, routers, bias, L=Lyr, k=W.k,
                       tiered={"resident": R, "staging": S,
                               "async": args.tiered_prepare == "async"})
    del sets
    # pinned host -> HBM copy ceiling on this machine (one expert-sized copy stream)
    hb = torch.empty(256 << 20, dtype=torch.uint8, pin_memory=True)
    db = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    db.copy_(hb, non_blocking=True)
    torch.cuda.synchronize()
    t = time.time()
    for _ in range(4):
        db.copy_(hb, non_blocking=True)
    torch.cuda.synchronize()
    h2d_ceiling = 4 * (256 << 20) / (time.time() - t) / 1e9
    del hb, db
    xs = [torch.from_numpy(moegen.make_tokens(W, T, step=s, layer=999).view(np.int16).copy()).cuda()
          for s in range(16)]
    x = torch.empty_like(xs[0])
    stream = torch.cuda.current_stream()
    for st in range(4):  # warm: first fill of the resident sets
        x.copy_(xs[st % 16])
        stack.step(x, T, epoch=0)
    stack.rebalance()
    torch.cuda.synchronize()
    s0, _ = q.moe_tier_stats_get(stack.tier)
    t = time.time()
    per_epoch = []
    prev = s0
    for st in range(args.tiered_steps):
        x.copy_(xs[st % 16])
        stack.step(x, T, epoch=st // drift)
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
    stack.close()
    d = {k: s1[k] - s0[k] for k in s1}
    h2d_gbs = d["h2d_bytes"] / wall / 1e9
    return {
        "workload": "tiered decode: 48 layers x (256 experts, top-8, hidden 2048, intermediate "
                    "512, NVFP4 gate/up, Q6_K down), 96 resident per layer, 8 tokens/step, "
                    "Zipf(1.2) routing drifting every 256 steps",
        "prepare": args.tiered_prepare,
        "steps": args.tiered_steps, "wall_s": round(wall, 3),
        "tok_per_s": round(T * args.tiered_steps / wall, 2),
        "ms_per_step": round(wall / args.tiered_steps * 1e3, 3),
        "miss_rate": round(d["misses"] / max(1, d["misses"] + d["hits"]), 4),
        "miss_rate_per_epoch": per_epoch,
        "h2d_GBps": round(h2d_gbs, 2), "pinned_h2d_ceiling_GBps": round(h2d_ceiling, 2),
        "h2d_frac_of_ceiling": round(h2d_gbs / h2d_ceiling, 4),
        "expert_sets": args.tiered_sets,
        "counters": d,
    }


def cpu_baseline(W, L, B, n_steps):
    """The oracle as it stands, single-threaded, on a bounded sample: n_steps
    decode steps of batch B on one layer.  Reported in the same unit."""
    import moegen
    import oracle
    t = time.time()
    for s in range(n_steps):
        x = moegen.make_tokens(W, B, step=10_000 + s)
        oracle.layer(x, L)
    dt = time.time() - t
    return {"value": round(B * n_steps / dt, 3), "unit": "tok/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_steps} decode steps of batch {B} on one layer, single-threaded "
                      f"plain C in double precision ({dt:.1f} s)"}


if __name__ == "__main__":
    main()
