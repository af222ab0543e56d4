#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE layer on one MI355X.

Workload (the headline): decode through 48 MoE layers of 512 experts each,
hidden 2048, expert intermediate 512, top-10, 3-bit group-64 experts, batch 1,
a 2048-slot pool per layer with a random expert -> slot table, router logits
N(0,1) plus a per-expert Zipf(1.1) bias.  One step = one decode token through
all 48 layers: per layer route (softmax, top-k, renormalise) and the experts
forward (sort by expert, slot resolve, gate/up, SwiGLU, down, weighted
combine); each layer's output is the next layer's input.  The step is captured
once in a HIP graph and replayed.

Each layer reads the output of a pre-norm residual chain,
x_{l+1} = x_l + moe_l(rmsnorm(x_l)); the residual add and the norm are model glue
(one small launch per layer from libmoebench.so), and the layer kernel is also
timed alone (48 launches in a graph of their own) for the roofline.

Also reported: 4K-token prefill (4 chunks of 1024 tokens through the same 48
layers, every expert resident, MFMA path), the mixed two-class workload at batch 1
and 8, the 8-bit batch-32 layer with cache-aware substitution, prefill through a
cache smaller than a layer (passes of 64 experts installed one by one), bf16
experts, measured ceilings (streamed reads, latency, MFMA peak, launch floor) and
the CPU oracle on the host cores.

Prints ONE JSON line.  Only one GPU is supported (--gpus 1).
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--prefill-reps", type=int, default=3)
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-bf16", action="store_true", help="skip the unquantized bf16 expert lines")
    p.add_argument("--cpu-layers", type=int, default=12, help="oracle sample: decode layers")
    p.add_argument("--eager", action="store_true", help="no HIP graph (launch-bound)")
    p.add_argument("--replay", action="store_true",
                   help="only the cache replay: mixed 48-layer decode through the miss pipeline")
    p.add_argument("--replay-tokens", type=int, default=48, help="timed decode steps per replay")
    p.add_argument("--replay-warmup", type=int, default=32, help="untimed steps (cache warm-up)")
    p.add_argument("--replay-share", type=float, default=0.5, help="device share of each layer's experts")
    p.add_argument("--io-threads", type=int, default=8)
    p.add_argument("--copy-streams", type=int, default=2, help="install copy streams (1 to 4)")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the mixed, 8-bit substitution, bounded prefill and ceiling lines")
    p.add_argument("--ceilings", action="store_true",
                   help="only the ceiling microbenchmarks (full read curve, latency, MFMA peak, launch floor)")
    p.add_argument("--bounded-only", action="store_true",
                   help="run only the bounded-cache prefill line (for a copy/kernel timeline)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 1 GiB device copy (to scale the FETCH_SIZE / WRITE_SIZE "
                        "counters of a profiling run)")
    return p.parse_args()


# Sources of the fused decode kernel; the measured HBM traffic recorded in the
# profile summary below holds only while their hash matches.
DECODE_SOURCES = ["quantized_routed_expert_softmax_amd/csrc/decode1.hip",
                  "quantized_routed_expert_softmax_amd/csrc/decode_dev.h",
                  "quantized_routed_expert_softmax_amd/csrc/route_dev.h",
                  "quantized_routed_expert_softmax_amd/csrc/moe_dev.h",
                  "include/moe.h"]
TRAFFIC_SUMMARY = "profiles/decode1_kernel_3_3_16_1_10_2_2_4-decode48.md"


def decode_sources_sha256():
    """sha256 of the decode kernel's sources with comments and blank lines
    removed (an edit of the documentation does not change the kernel)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
        h.update(code.encode())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the fused decode kernel from the committed
    rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or
    None when the summary is missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, TRAFFIC_SUMMARY)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel sources sha256 (comments and blank lines removed)") != decode_sources_sha256():
        return None
    try:
        return int(fields["HBM bytes per launch"])
    except (KeyError, ValueError):
        return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class DecodeModel:
    """48 layers of device state for the decode / prefill workloads."""

    def __init__(self, torch, B, synth, wl):
        self.torch, self.B, self.synth, self.wl = torch, B, synth, wl
        dev = torch.device("cuda")
        self.lay = synth.Layout(wl.H, wl.I, wl.bits_gu, wl.bits_d)
        self.desc = B.moe_size_class_init(wl.H, wl.I, wl.bits_gu, wl.bits_d, wl.slots_per_layer)
        self.tables_np, self.pools, self.tables = [], [], []
        for l in range(wl.layers):
            t = synth.slot_table(synth.rng_for(wl.seed, 4, l), wl.E, wl.slots_per_layer)
            pool = torch.empty((wl.slots_per_layer, self.lay.slot_bytes), dtype=torch.uint8, device=dev)
            synth.fill_pool_device(pool, self.lay, t, wl.seed, l)
            self.tables_np.append(t)
            self.tables.append(torch.from_numpy(t).to(dev))
            self.pools.append(pool.view(-1))
        torch.cuda.synchronize()


def decode_inputs(torch, synth, wl):
    lg = np.stack([synth.gen_logits(synth.rng_for(wl.seed, 3, l), 1, wl.E,
                                    synth.zipf_bias(synth.rng_for(wl.seed, 2, l), wl.E, wl.zipf_s))
                   for l in range(wl.layers)])
    x0 = synth.gen_x(synth.rng_for(wl.seed, 1), 1, wl.H)
    return lg, x0


def replay_main(args, torch, B, synth):
    """Decode steps of the mixed workload (48 layers, 128 experts, top-8, two size
    classes) through a device cache that holds a share of each layer's experts,
    filled by the miss pipeline from an expert store in host memory.  Per layer:
    route on the GPU, bring the routing to the host once, prepare (hits touched,
    misses installed on the copy stream), forward, release."""
    wl = synth.WORKLOADS["mixed"]
    dev = torch.device("cuda")
    L, E, k, H, I = wl.layers, wl.E, wl.k, wl.H, wl.I
    kinds = sorted({synth.layer_bits(wl, l) for l in range(L)})
    layer_class = [kinds.index(synth.layer_bits(wl, l)) for l in range(L)]
    n_layers_c = [layer_class.count(c) for c in range(len(kinds))]
    lays = [synth.Layout(H, I, bg, bd) for bg, bd in kinds]

    # expert store: every expert of every layer, generated on the device, kept in
    # host memory (stands in for the file the one-time conversion writes)
    t_setup = time.time()
    total = sum(E * lays[c].slot_bytes for c in layer_class)
    store_np = np.empty(total, np.uint8)
    tmp = torch.empty(E * max(l.slot_bytes for l in lays), dtype=torch.uint8, device=dev)
    off = 0
    for l in range(L):
        sb = lays[layer_class[l]].slot_bytes
        pool = tmp[:E * sb].view(E, sb)
        synth.fill_pool_device(pool, lays[layer_class[l]], np.arange(E), wl.seed, l)
        torch.from_numpy(store_np[off:off + E * sb]).copy_(pool.view(-1))
        off += E * sb
    del tmp
    torch.cuda.synchronize()
    log(f"replay store {total / 1e9:.2f} GB in {time.time() - t_setup:.1f}s")

    # router-driven stack for the lookahead runs, shaped like a pre-norm MoE block:
    # n_l = rmsnorm(x_l), layer l routes with its router on n_l and
    # x_{l+1} = x_l + moe_l(n_l); routers N(0, 1/H), so logits are ~N(0, 1).  The
    # norm and the residual add are model glue around the layer (torch ops).
    gr = torch.Generator(device=dev)
    gr.manual_seed(wl.seed * 104729 + 1)
    routers = (torch.randn((L, E, H), generator=gr, device=dev) / float(np.sqrt(H))).to(torch.bfloat16)

    def run(T, share, host_mode, resident_first=False, n_copy=args.copy_streams, ahead=None,
            policy=B.MOE_EVICT_LRU, per_layer=False):
        slots = [max(int(round(share * E)) * n, T * k) for n in n_layers_c]
        classes = [B.moe_size_class_init(H, I, bg, bd, s) for (bg, bd), s in zip(kinds, slots)]
        pools = [torch.empty(d.n_slots * d.slot_bytes, dtype=torch.uint8, device=dev) for d in classes]
        cache = B.moe_cache_create(classes, layer_class, E, policy=policy, per_layer=per_layer)
        store = B.moe_store_open_memory(store_np, classes, layer_class, E)
        copies = [torch.cuda.Stream() for _ in range(n_copy)]
        host_bytes = {"all": total, "none": 0}[host_mode]
        t0 = time.time()
        p = B.moe_pipeline_create(cache, store, pools, host_tier_bytes=host_bytes,
                                  host_preload=host_bytes > 0, io_threads=args.io_threads,
                                  staging_rows=2 * args.io_threads, copy_streams=copies)
        t_create = time.time() - t0
        try:
            if resident_first:  # every expert installed before the run
                for l in range(L):
                    B.moe_pipeline_prefetch(p, l, np.arange(E, dtype=np.int32))
                B.moe_pipeline_drain(p)
            g = torch.Generator(device=dev)
            g.manual_seed(wl.seed * 7919 + T)
            n_tok = args.replay_warmup + args.replay_tokens
            logits = torch.randn((n_tok, L, T, E), generator=g, device=dev, dtype=torch.float32)
            x0 = torch.randn((T, H), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
            xbuf = [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(2)]
            n_r = 1 + (ahead or 0)
            x0s = torch.randn((n_tok, T, H), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
            lbuf = torch.empty((n_r, T, E), dtype=torch.float32, device=dev)
            ids_all = torch.empty((n_r * T, k), dtype=torch.int32, device=dev)
            w_all = torch.empty((n_r * T, k), dtype=torch.float32, device=dev)
            ids_host_all = torch.empty((n_r * T, k), dtype=torch.int32, pin_memory=True)
            ids, w, ids_host = ids_all[:T], w_all[:T], ids_host_all[:T]
            ybuf = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
            table = torch.full((E,), -1, dtype=torch.int32, device=dev)
            ws = torch.zeros(B.moe_forward_workspace_size(T, k, E, classes[0]) + 4096, dtype=torch.uint8,
                             device=dev)
            err = torch.zeros(1, dtype=torch.int32, device=dev)
            ev = torch.cuda.Event()

            def token_router(t):
                x = x0s[t]
                for l in range(L):
                    c = layer_class[l]
                    n = min(n_r, L - l)
                    xf = x.float()
                    xn = (xf * torch.rsqrt(xf.pow(2).mean(dim=-1, keepdim=True) + 1e-6)).to(torch.bfloat16)
                    B.moe_router_logits(xn, routers[l:l + n], logits=lbuf[:n])
                    B.moe_route_topk(lbuf[:n].view(n * T, E), k, topk_ids=ids_all[:n * T],
                                     topk_w=w_all[:n * T], err_word=err)
                    ids_host_all[:n * T].copy_(ids_all[:n * T], non_blocking=True)
                    ev.record()
                    ev.synchronize()
                    hn = ids_host_all.numpy()
                    B.moe_pipeline_prepare(p, l, hn[:T], table)
                    for a in range(1, n):  # guesses of the next layers from x_l
                        B.moe_pipeline_prefetch(p, l + a, hn[a * T:(a + 1) * T])
                    B.moe_experts_forward(xn, ids, w, E, table, pools[c], classes[c], out=ybuf, ws=ws,
                                          err_word=err)
                    B.moe_pipeline_release(p, l)
                    x = torch.add(x, ybuf, out=xbuf[l & 1])

            def token(t):
                if ahead is not None:
                    return token_router(t)
                x = x0
                for l in range(L):
                    c = layer_class[l]
                    B.moe_route_topk(logits[t, l], k, topk_ids=ids, topk_w=w, err_word=err)
                    ids_host.copy_(ids, non_blocking=True)  # the layer's routing, to the host once
                    ev.record()
                    ev.synchronize()
                    B.moe_pipeline_prepare(p, l, ids_host.numpy(), table)
                    y = xbuf[l & 1]
                    B.moe_experts_forward(x, ids, w, E, table, pools[c], classes[c], out=y, ws=ws,
                                          err_word=err)
                    B.moe_pipeline_release(p, l)
                    x = y

            for t in range(args.replay_warmup):
                token(t)
            B.moe_pipeline_drain(p)
            torch.cuda.synchronize()
            before = [B.moe_pipeline_stats_get(p, c) for c in range(len(classes))]
            t0 = time.perf_counter()
            for t in range(args.replay_warmup, n_tok):
                token(t)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
            after = [B.moe_pipeline_stats_get(p, c) for c in range(len(classes))]
            assert int(err.item()) == 0, f"device error word {int(err.item()):#x}"
            assert bool(torch.isfinite(xbuf[(L - 1) & 1].float()).all())
            per_class = []
            copied = 0
            for c in range(len(classes)):
                d = {key: after[c][key] - before[c][key] for key in after[c]}
                copied += d["bytes_copied"]
                hits = d["hits"] + d["inflight_hits"]
                per_class.append({
                    "class": c, "bits_gate_up": kinds[c][0], "bits_down": kinds[c][1],
                    "guesses_started": d["prefetches"], "guesses_skipped": d["prefetch_skipped"],
                    "layers": n_layers_c[c], "slot_bytes": classes[c].slot_bytes,
                    "slots": classes[c].n_slots, "requests": d["requests"],
                    "hit_rate": round(hits / max(d["requests"], 1), 4),
                    "misses_per_token": round((d["requests"] - hits) / args.replay_tokens, 2),
                    "host_hits": d["host_hits"], "store_reads": d["store_reads"]})
            return {"batch": T, "share": share, "host_tier": host_mode, "copy_streams": n_copy,
                    "routing": "logits N(0,1)" if ahead is None else f"routers on x_l, {ahead} layers guessed",
                    "eviction": ("LFU" if policy == B.MOE_EVICT_LFU else "LRU") + (" per layer" if per_layer else " per class"),
                    "tok_s": round(T * args.replay_tokens / wall, 2),
                    "ms_per_step": round(1000 * wall / args.replay_tokens, 3),
                    "install_GBps": round(copied / wall / 1e9, 2),
                    "install_bytes_per_token": int(copied / (T * args.replay_tokens)),
                    "pipeline_create_s": round(t_create, 2),
                    "classes": per_class}
        finally:
            B.moe_pipeline_destroy(p)
            B.moe_cache_destroy(cache)
            B.moe_store_close(store)
            del pools
            torch.cuda.empty_cache()

    # host-to-device ceiling the installs run against: pinned host -> device copies,
    # one large copy and expert-row-sized copies on one and two streams
    h2d = {}
    row = lays[0].slot_bytes
    n_rows = 256
    src = torch.empty(n_rows * row, dtype=torch.uint8, pin_memory=True)
    src.fill_(1)
    dst = torch.empty(n_rows * row, dtype=torch.uint8, device=dev)
    best = 0.0
    for _ in range(3):  # best of three
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        dst.copy_(src, non_blocking=True)
        torch.cuda.synchronize()
        best = max(best, n_rows * row / (time.perf_counter() - t0) / 1e9)
    h2d["one_copy_GBps"] = round(best, 2)
    for ns in (1, 2):
        sts = [torch.cuda.Stream() for _ in range(ns)]
        best = 0.0
        for _ in range(3):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(n_rows):
                with torch.cuda.stream(sts[i % ns]):
                    dst[i * row:(i + 1) * row].copy_(src[i * row:(i + 1) * row], non_blocking=True)
            torch.cuda.synchronize()
            best = max(best, n_rows * row / (time.perf_counter() - t0) / 1e9)
        h2d[f"row_copies_{ns}_streams_GBps"] = round(best, 2)
    del src, dst
    log(json.dumps({"h2d": h2d, "row_bytes": row}))

    runs = []
    for T in (1, 8):
        runs.append(run(T, 1.0, "none", resident_first=True))
        log(json.dumps(runs[-1]))
        for mode in ("all", "none"):
            runs.append(run(T, args.replay_share, mode))
            log(json.dumps(runs[-1]))
        for ahead in (0, 2):  # router-driven stack, without and with the lookahead guesses
            runs.append(run(T, args.replay_share, "all", ahead=ahead))
            log(json.dumps(runs[-1]))
        if T == 1:  # eviction variants on the router-driven stack with guesses
            for policy, per_layer in ((B.MOE_EVICT_LFU, False), (B.MOE_EVICT_LRU, True)):
                runs.append(run(T, args.replay_share, "all", ahead=2, policy=policy, per_layer=per_layer))
                log(json.dumps(runs[-1]))
        runs.append(run(T, 1.0, "none", resident_first=True, ahead=0))
        log(json.dumps(runs[-1]))
    main_run = next(r for r in runs if r["batch"] == 1 and r["host_tier"] == "all" and r["share"] < 1
                    and r["routing"].startswith("logits") and r["eviction"] == "LRU per class")
    result = {
        "metric": "mixed decode replay tok/s through the bounded cache (per-class hit rates)",
        "value": main_run["tok_s"], "unit": "tok/s", "n_gpus": 1,
        "steps": args.replay_tokens, "warmup": args.replay_warmup,
        "ms_per_step": main_run["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "mixed: 48 layers x (hidden 2048, 128 experts, intermediate 768, top-8), "
                               "4-bit experts with 6-bit down on every 4th layer (two size classes), "
                               f"device share {args.replay_share} of each layer's experts, "
                               "router logits N(0,1), store in host memory",
                   "io_threads": args.io_threads, "copy_streams": args.copy_streams,
                   "store_GB": round(total / 1e9, 3)},
        "h2d_reference": dict(h2d, row_bytes=row),
        "runs": runs,
    }
    print(json.dumps(result), flush=True)


def bf16_lines(torch, B, synth, wl, dev, err):
    """The decode layer shape with unquantized bf16 experts (6.29 MB each): decode
    steps through 8 layer pools (25 GB, more than the 256 MB Infinity Cache can
    hold, so experts stream from HBM), and one 1024-token prefill chunk."""
    H, E, I, k = wl.H, wl.E, wl.I, wl.k
    lay = synth.Layout(H, I, 16, 16)
    n_pools = 8
    desc = B.moe_size_class_init(H, I, 16, 16, E)
    pools = []
    for l in range(n_pools):
        pool = torch.empty((E, lay.slot_bytes), dtype=torch.uint8, device=dev)
        synth.fill_pool_device(pool, lay, np.arange(E), 7, l)
        pools.append(pool.view(-1))
    table = torch.arange(E, dtype=torch.int32, device=dev)
    steps = 48
    lg = torch.stack([torch.from_numpy(synth.gen_logits(
        synth.rng_for(7, 3, s), 1, E, synth.zipf_bias(synth.rng_for(7, 2, s), E, wl.zipf_s))) for s in range(steps)]).to(dev)
    x = torch.from_numpy(synth.gen_x(synth.rng_for(7, 1), 1, H).view(np.int16)).to(dev).view(torch.bfloat16)
    ids = torch.empty((steps, 1, k), dtype=torch.int32, device=dev)
    w = torch.empty((steps, 1, k), dtype=torch.float32, device=dev)
    out = torch.empty((1, H), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(B.moe_forward_workspace_size(1, k, E, desc), dtype=torch.uint8, device=dev)

    def dec():
        for s_ in range(steps):
            B.moe_layer_forward(lg[s_], x, table, pools[s_ % n_pools], desc, k, topk_ids=ids[s_], topk_w=w[s_],
                                out=out, ws=ws, err_word=err)

    dec()
    torch.cuda.synchronize()
    # the 48 layer-steps captured in one HIP graph, as the headline decode step is
    graph = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(graph, stream=st):
            dec()
    torch.cuda.current_stream().wait_stream(st)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / (5 * steps)
    ids_np = ids.cpu().numpy()
    distinct = float(np.mean([len(set(ids_np[s_].reshape(-1).tolist())) for s_ in range(steps)]))
    dec_bytes = distinct * lay.slot_bytes
    # prefill chunk
    pw = synth.WORKLOADS["prefill"]
    T = pw.T
    plg = torch.from_numpy(synth.gen_logits(synth.rng_for(7, 5), T, E)).to(dev)
    px = torch.from_numpy(synth.gen_x(synth.rng_for(7, 6), T, H).view(np.int16)).to(dev).view(torch.bfloat16)
    pids = torch.empty((T, k), dtype=torch.int32, device=dev)
    pwt = torch.empty((T, k), dtype=torch.float32, device=dev)
    pout = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    pws = torch.zeros(B.moe_forward_workspace_size(T, k, E, desc), dtype=torch.uint8, device=dev)
    run = lambda: B.moe_layer_forward(plg, px, table, pools[0], desc, k, topk_ids=pids, topk_w=pwt, out=pout,
                                      ws=pws, err_word=err)
    run()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        run()
    e1.record()
    torch.cuda.synchronize()
    p_us = e0.elapsed_time(e1) * 1000.0 / 5
    assert int(err.item()) == 0, f"device error word {int(err.item()):#x}"
    flops = 2.0 * T * k * 3 * H * I
    p_bytes = E * lay.slot_bytes
    del pools
    torch.cuda.empty_cache()
    return {
        "workload": "decode layer shape (H 2048, E 512, I 512, top-10) with bf16 experts, 6291456 B each",
        "decode_us_per_layer": round(us, 2),
        "decode_hbm_gbs": round(dec_bytes / (us * 1e-6) / 1e9, 1),
        "decode_hbm_frac": round(dec_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "decode_path": "one-token kernel decode1_kernel<16,16,16,1,10,1,1,2>: routing, gate/up + SwiGLU, down and combine in one launch per layer, 48 layer-steps in one HIP graph",
        "prefill_chunk_us": round(p_us, 2),
        "prefill_hbm_gbs": round(p_bytes / (p_us * 1e-6) / 1e9, 1),
        "prefill_hbm_frac": round(p_bytes / (p_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "prefill_useful_tflops": round(flops / (p_us * 1e-6) / 1e12, 1),
    }


def graph_of(torch, fn):
    """Capture fn() once into a HIP graph (after one eager warm-up call)."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def time_replays(torch, graph, reps):
    """ms per replay of a graph, HIP events on the replay stream."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    graph.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class Chain:
    """A pre-norm residual decode chain over L layers: n_l = rmsnorm(x_l),
    y_l = moe_l(n_l), x_{l+1} = x_l + y_l.  The norm and the residual add are
    model glue (one libmoebench launch per layer), outside the layer kernel."""

    def __init__(self, torch, mb, T, H, L, x0):
        dev = x0.device
        self.torch, self.mb, self.L = torch, mb, L
        self.xs = [x0] + [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(L)]
        self.ns = [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(L + 1)]
        self.ys = [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(L)]

    def glue(self, l):
        if l == 0:
            self.mb.residual_rmsnorm(self.xs[0], None, None, self.ns[0])
        else:
            self.mb.residual_rmsnorm(self.xs[l - 1], self.ys[l - 1], self.xs[l], self.ns[l])

    def step(self, layer):
        """layer(l, n_l, y_l) enqueues layer l."""
        for l in range(self.L):
            self.glue(l)
            layer(l, self.ns[l], self.ys[l])
        self.glue(self.L)

    def layers_only(self, layer):
        for l in range(self.L):
            layer(l, self.ns[l], self.ys[l])

    def final(self):
        return self.xs[self.L]


def check_layer_vs_oracle(torch, B, oracle, synth, lg_l, n_l, y_l, ids_l, w_l, table_l, pool_l, n_slots,
                          lay, E, k, threads, tokens=None):
    """Routing bit-exact and the layer output within max-abs 2e-2 / rel-L2 1e-2
    of the oracle, fed the layer's own input (the oracle gets only the routed
    experts' rows, copied from the device)."""
    ids_o, w_o = oracle.route(lg_l, k)
    ids_g = ids_l.cpu().numpy()
    assert np.array_equal(ids_g, ids_o), "routing ids differ from the oracle"
    assert np.array_equal(w_l.cpu().numpy().view(np.uint32), w_o.view(np.uint32))
    used = sorted(set(ids_o.reshape(-1).tolist()))
    idx = torch.as_tensor([int(table_l[e]) for e in used], device=pool_l.device)
    rows = pool_l.view(n_slots, -1).index_select(0, idx).cpu().numpy()
    t2 = np.full(E, -1, np.int32)
    t2[used] = np.arange(len(used), dtype=np.int32)
    x_bits = n_l.view(torch.int16).cpu().numpy().view(np.uint16)
    tk = None if tokens is None else np.asarray(tokens, np.int32)
    ref = oracle.layer(x_bits, ids_o, w_o, t2, rows, lay.H, lay.I, lay.bits_gu, lay.bits_d, E, tokens=tk,
                       threads=threads)
    got = y_l.float().cpu().numpy().astype(np.float64)
    if tokens is not None:
        got = got[tokens]
    d = float(np.abs(got - ref).max())
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    assert d <= 2e-2 and rel <= 1e-2, f"layer output vs oracle: max-abs {d:.3e} rel-L2 {rel:.3e}"
    return {"max_abs": round(d, 6), "rel_l2": round(rel, 6)}


# ------------------------------ ceilings ------------------------------------ #
def ceilings(torch, mb, dev, quick=False):
    """Measured ceilings of this GPU for the kernel shapes here: streamed reads of
    given bytes per launch (48 launches back to back in a HIP graph, each on
    bytes no earlier launch of the graph touched), idle memory latency, the bf16
    MFMA peak and the launch floor."""
    out = {}
    pool_bytes = 4 << 30
    buf = torch.empty(pool_bytes, dtype=torch.uint8, device=dev)
    buf.fill_(3)
    sink = torch.zeros(16, dtype=torch.int32, device=dev)
    base = buf.data_ptr()
    rng = np.random.default_rng(12345)
    row = 1376256  # one 3-bit expert row of the decode layer shape

    def curve_point(n_rows, row_bytes, launches, shapes, scattered):
        """Best GB/s over launch shapes (total workgroups) for n_rows rows per launch."""
        per_launch = n_rows * row_bytes
        if scattered:  # rows at random row-aligned offsets, distinct across the graph
            slots = pool_bytes // row_bytes
            pick = rng.permutation(slots)[:n_rows * launches]
            addr = base + pick.astype(np.int64) * row_bytes
        else:  # one contiguous region per launch, consecutive launches disjoint
            span = max(per_launch, 1)
            n_reg = max(1, pool_bytes // span)
            addr = np.array([base + ((i // n_rows) % n_reg) * span + (i % n_rows) * row_bytes
                             for i in range(n_rows * launches)], dtype=np.int64)
        rows_t = torch.from_numpy(addr).to(dev)
        best = None
        for wg in shapes:
            wpr = max(1, wg // n_rows)

            def fn():
                for i in range(launches):
                    mb.read_rows(rows_t[i * n_rows:(i + 1) * n_rows], n_rows, row_bytes, sink, wpr)
            g = graph_of(torch, fn)
            ms = time_replays(torch, g, 5)
            us = ms * 1000.0 / launches
            gbs = per_launch / (us * 1e-6) / 1e9
            if best is None or gbs > best["GBps"]:
                best = {"bytes_per_launch": per_launch, "rows": n_rows, "row_bytes": row_bytes,
                        "us_per_launch": round(us, 3), "GBps": round(gbs, 1), "workgroups": wpr * n_rows}
            del g
        return best

    shapes = (256, 512, 1024, 2048, 4096)
    curve = []
    for mbytes in ((1, 4, 16, 64, 256, 1024) if not quick else (16, 256)):
        nb = mbytes << 20
        launches = 48 if nb <= (64 << 20) else max(2, min(48, pool_bytes // nb))
        curve.append(curve_point(1, nb, launches, shapes, scattered=False))
        log(json.dumps({"ceiling_read": curve[-1]}))
    out["read_contiguous"] = curve
    out["read_decode_rows"] = curve_point(10, row, 48, shapes, scattered=True)
    log(json.dumps({"ceiling_decode_rows": out["read_decode_rows"]}))
    out["read_prefill_rows"] = curve_point(512, row, 4, shapes + (8192, 16384), scattered=True)
    log(json.dumps({"ceiling_prefill_rows": out["read_prefill_rows"]}))

    # idle latency per level: one lane chasing a random cycle of 64-byte nodes,
    # timed in-kernel.  L2 (1 MiB) and MALL (32 MiB) chains are warmed by a full
    # lap in the same launch first; the HBM chain (4 GiB) is timed on nodes no
    # earlier hop touched.
    lat = {}
    hops = 20000
    for name, nbytes, warm_lap in (("l2_1MiB", 1 << 20, True), ("mall_32MiB", 32 << 20, True),
                                   ("hbm_4GiB", 4 << 30, False)):
        n = nbytes // 64
        g = torch.Generator(device=dev)
        g.manual_seed(99)
        perm = torch.randperm(n, generator=g, device=dev, dtype=torch.int64)
        nxt = torch.zeros((n, 16), dtype=torch.int32, device=dev)
        nxt[perm, 0] = torch.roll(perm, -1).to(torch.int32)
        o = torch.zeros(2, dtype=torch.int32, device=dev)
        start = int(perm[n // 2].item())
        mb.chase(nxt, start, n + hops if warm_lap else 0, hops, o)
        torch.cuda.synchronize()
        lat[name + "_ns"] = round(int(o[1].item()) * 10.0 / hops, 1)   # per dependent load
        del nxt, perm
    out["latency"] = lat
    log(json.dumps({"latency": lat}))

    # bf16 MFMA peak: 8 independent 16x16x32 chains per wave
    fs = torch.zeros(1 << 16, dtype=torch.float32, device=dev)
    best = 0.0
    for grid in (1024, 2048, 4096):
        iters = 500
        mb.mfma_loop(grid, iters, fs)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        mb.mfma_loop(grid, iters, fs)
        e1.record()
        torch.cuda.synchronize()
        flops = grid * 4.0 * iters * 8 * (16 * 16 * 32 * 2)
        best = max(best, flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    out["mfma_bf16_tflops"] = round(best, 1)

    # launch floor: empty kernels of the decode kernel's launch shape, 48 in a graph
    def fn():
        for _ in range(48):
            mb.empty(256, 640)
    g = graph_of(torch, fn)
    out["empty_launch_us_in_graph"] = round(time_replays(torch, g, 10) * 1000.0 / 48, 3)
    del buf, g
    torch.cuda.empty_cache()
    return out


# ------------------------------- mixed (two classes) ------------------------ #
def mixed_lines(torch, B, mb, synth, dev, err, steps):
    """The mixed workload, every expert resident: 48 layers (hidden 2048, 128
    experts, intermediate 768, top-8), 4-bit experts with 6-bit down on layers
    l % 4 == 3 (two size classes, own pools); the pre-norm residual chain at
    batch 1 and batch 8, captured in one HIP graph per batch."""
    wl = synth.WORKLOADS["mixed"]
    L, E, k, H, I = wl.layers, wl.E, wl.k, wl.H, wl.I
    lays, descs, pools, tables = [], [], [], []
    for l in range(L):
        bg, bd = synth.layer_bits(wl, l)
        lay = synth.Layout(H, I, bg, bd)
        t = synth.slot_table(synth.rng_for(wl.seed, 4, l), E, E)
        pool = torch.empty((E, lay.slot_bytes), dtype=torch.uint8, device=dev)
        synth.fill_pool_device(pool, lay, t, wl.seed, l)
        lays.append(lay)
        descs.append(B.moe_size_class_init(H, I, bg, bd, E))
        pools.append(pool.view(-1))
        tables.append(torch.from_numpy(t).to(dev))
    res = {}
    for T in (1, 8):
        logits = torch.from_numpy(np.stack([synth.gen_logits(synth.rng_for(wl.seed, 3, l, T), T, E)
                                            for l in range(L)])).to(dev)
        x0 = torch.from_numpy(synth.gen_x(synth.rng_for(wl.seed, 1, T), T, H).view(np.int16)).to(dev).view(torch.bfloat16)
        ch = Chain(torch, mb, T, H, L, x0)
        ids = torch.empty((L, T, k), dtype=torch.int32, device=dev)
        w = torch.empty((L, T, k), dtype=torch.float32, device=dev)
        ws = torch.zeros(max(B.moe_forward_workspace_size(T, k, E, d) for d in descs[:4]), dtype=torch.uint8,
                         device=dev)

        def layer(l, n, y):
            B.moe_layer_forward(logits[l], n, tables[l], pools[l], descs[l], k, topk_ids=ids[l], topk_w=w[l],
                                out=y, ws=ws, err_word=err)

        g_step = graph_of(torch, lambda: ch.step(layer))
        ms_step = time_replays(torch, g_step, steps)
        g_lay = graph_of(torch, lambda: ch.layers_only(layer))
        ms_lay = time_replays(torch, g_lay, steps)
        assert int(err.item()) == 0, f"device error word {int(err.item()):#x}"
        ids_np = ids.cpu().numpy()
        step_bytes = sum(len(set(ids_np[l].reshape(-1).tolist())) * lays[l].slot_bytes for l in range(L))
        res[f"batch{T}"] = {
            "tok_s": round(T * 1000.0 / ms_step, 1),
            "ms_per_step": round(ms_step, 4),
            "layer_us": round(ms_lay * 1000.0 / L, 3),
            "expert_bytes_per_step": int(step_bytes),
            "hbm_gbs": round(step_bytes / (ms_lay * 1e-3) / 1e9, 1),
            "hbm_frac": round(step_bytes / (ms_lay * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "final_x_std": round(float(ch.final().float().std()), 4),
        }
        del g_step, g_lay
    del pools
    torch.cuda.empty_cache()
    res["workload"] = ("mixed: 48 layers x (hidden 2048, 128 experts, intermediate 768, top-8), 4-bit "
                       "experts, 6-bit down on layers l % 4 == 3 (two size classes: 2654208 and 3047424 B), "
                       "every expert resident, pre-norm residual chain, one HIP graph per step")
    res["kernel"] = ("moe_layer_forward, one launch per layer at batch 1: decode1_kernel<4,4,8,3,8,2,2,4> on the "
                     "4-bit layers, decode1_kernel<4,6,8,3,8,2,2,4> on the 6-bit-down layers; batch 8: routing, "
                     "sort (with the permute of x), mfma_lds_kernel gate/up and down, combine")
    res["frac_basis"] = "distinct routed experts' bytes per step / the 48 layer launches' time (graph of layer launches only)"
    return res


# ------------------------ 8-bit experts with substitution ------------------- #
def int8_subst_line(torch, B, synth, dev, err, reps):
    """One layer of 8-bit experts (hidden 4096, 256 experts, intermediate 1024,
    top-8), batch 32, cache-aware substitution at L = 0.15 against a 25%-resident
    set: routing on the resident mask, the misses installed from pinned host
    rows (timed on their own), then the timed route + experts forward."""
    wl = synth.WORKLOADS["int8sub"]
    E, k, T, H, I = wl.E, wl.k, wl.T, wl.H, wl.I
    lay = synth.Layout(H, I, wl.bits_gu, wl.bits_d)
    n_slots = 192
    src = torch.empty((E, lay.slot_bytes), dtype=torch.uint8, device=dev)
    synth.fill_pool_device(src, lay, np.arange(E), wl.seed, 0)
    host = torch.empty((E, lay.slot_bytes), dtype=torch.uint8, pin_memory=True)
    host.copy_(src)
    del src
    desc = B.moe_size_class_init(H, I, wl.bits_gu, wl.bits_d, n_slots)
    cache = B.moe_cache_create([desc], [0], E)
    pool = torch.zeros((n_slots, lay.slot_bytes), dtype=torch.uint8, device=dev)
    try:
        resident = synth.rng_for(wl.seed, 6).choice(E, wl.resident, replace=False)
        for e in resident:
            _, slot, _ = B.moe_cache_acquire(cache, 0, int(e))
            B.moe_cache_install(pool.view(-1), desc, slot, host[int(e)])
            B.moe_cache_fill_done(cache, 0, int(e), None)
        torch.cuda.synchronize()
        table0 = torch.from_numpy(B.moe_cache_table(cache, 0, E)).to(dev)
        lg = torch.from_numpy(synth.gen_logits(synth.rng_for(wl.seed, 3), T, E)).to(dev)
        x = torch.from_numpy(synth.gen_x(synth.rng_for(wl.seed, 1), T, H).view(np.int16)).to(dev).view(torch.bfloat16)
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        B.moe_route_topk(lg, k, mode=B.MOE_ROUTE_SUBST, L=wl.subst_L, slot_table=table0, topk_ids=ids,
                         topk_w=w, err_word=err)
        ids_np = ids.cpu().numpy()
        # the misses, installed on a copy stream (timed: the PCIe-bound part)
        copy = torch.cuda.Stream()
        need = sorted(set(ids_np.reshape(-1).tolist()))
        misses = []
        for e in need:
            rc, slot, nf = B.moe_cache_acquire(cache, 0, e)
            if nf:
                misses.append((e, slot))
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(copy)
        for e, slot in misses:
            B.moe_cache_install(pool.view(-1), desc, slot, host[e], stream=copy)
        e1.record(copy)
        torch.cuda.synchronize()
        inst_ms = e0.elapsed_time(e1)
        for e, _ in misses:
            B.moe_cache_fill_done(cache, 0, e, None)
        table1 = torch.from_numpy(B.moe_cache_table(cache, 0, E)).to(dev)
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        ws = torch.zeros(B.moe_forward_workspace_size(T, k, E, desc), dtype=torch.uint8, device=dev)
        res = {}
        for name, path in (("auto", B.MOE_PATH_AUTO), ("gemv", B.MOE_PATH_GEMV)):
            def fn():
                B.moe_route_topk(lg, k, mode=B.MOE_ROUTE_SUBST, L=wl.subst_L, slot_table=table0, topk_ids=ids,
                                 topk_w=w, err_word=err)
                B.moe_experts_forward(x, ids, w, E, table1, pool.view(-1), desc, out=out, ws=ws, err_word=err,
                                      path=path)
            g = graph_of(torch, fn)
            res[name] = time_replays(torch, g, reps)
            del g
        assert int(err.item()) == 0, f"device error word {int(err.item()):#x}"
        best = min(res, key=res.get)
        ms = res[best]
        step_bytes = len(need) * lay.slot_bytes + T * E * 4 + 2 * T * H * 2
        pids = torch.empty((T, k), dtype=torch.int32, device=dev)
        pwt = torch.empty((T, k), dtype=torch.float32, device=dev)
        B.moe_route_topk(lg, k, topk_ids=pids, topk_w=pwt, err_word=err)
        plain_ids = pids.cpu().numpy()
        return {
            "workload": "8-bit experts (hidden 4096, 256 experts, intermediate 1024, top-8), batch 32, "
                        "substitution L = 0.15 on a 64-of-256 resident set, one layer",
            "tok_s": round(T * 1000.0 / ms, 1),
            "us_per_step": round(ms * 1000.0, 2),
            "path": best,
            "us_per_path": {kk: round(v * 1000.0, 2) for kk, v in res.items()},
            "distinct_experts": len(need),
            "distinct_experts_plain_routing": len(set(plain_ids.reshape(-1).tolist())),
            "algorithmic_bytes": int(step_bytes),
            "hbm_gbs": round(step_bytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "installs": {"count": len(misses), "bytes": len(misses) * lay.slot_bytes,
                         "ms": round(inst_ms, 3),
                         "GBps": round(len(misses) * lay.slot_bytes / (inst_ms * 1e-3) / 1e9, 2),
                         "source": "pinned host rows, one copy stream (not in the timed step)"},
        }
    finally:
        B.moe_cache_destroy(cache)
        del pool, host
        torch.cuda.empty_cache()


# --------------------------- prefill through the cache ---------------------- #
def prefill_bounded_line(torch, B, synth, dev, err, n_layers=4, slots=128, n_copy=4, pool=None):
    """1024-token chunks of the decode layer shape through a cache of `slots`
    slots for `n_layers` layers (one size class, fewer slots than one layer's 512
    hit experts): every layer runs in 8 passes of 64 experts, each pass
    installed from the pinned host tier before it runs (moe_pipeline_prefill)."""
    wl = synth.WORKLOADS["prefill"]
    E, k, T, H, I = wl.E, wl.k, wl.T, wl.H, wl.I
    lay = synth.Layout(H, I, wl.bits_gu, wl.bits_d)
    store = np.empty(n_layers * E * lay.slot_bytes, np.uint8)
    tmp = torch.empty((E, lay.slot_bytes), dtype=torch.uint8, device=dev)
    for l in range(n_layers):
        synth.fill_pool_device(tmp, lay, np.arange(E), wl.seed, l)
        torch.from_numpy(store[l * E * lay.slot_bytes:(l + 1) * E * lay.slot_bytes]).copy_(tmp.view(-1))
    del tmp
    desc = B.moe_size_class_init(H, I, wl.bits_gu, wl.bits_d, slots)
    if pool is None:
        pool = torch.zeros(slots * lay.slot_bytes, dtype=torch.uint8, device=dev)
    cache = B.moe_cache_create([desc], [0] * n_layers, E)
    st = B.moe_store_open_memory(store, [desc], [0] * n_layers, E)
    # four copy streams: with one copy per row they gave 26.8 GB/s of installs per
    # layer-chunk against 18.6 GB/s with two (each stream waits for the release
    # of the pass before the last before its copies, so more streams keep more
    # copies in flight); a pass is now one coalesced copy
    copies = [torch.cuda.Stream() for _ in range(n_copy)]
    p = B.moe_pipeline_create(cache, st, [pool], host_tier_bytes=store.nbytes, host_preload=True, io_threads=4,
                              staging_rows=8, copy_streams=copies)
    try:
        table = torch.full((E,), -1, dtype=torch.int32, device=dev)
        ws = torch.zeros(B.moe_forward_workspace_size(T, k, E, desc), dtype=torch.uint8, device=dev)
        chunks = []
        for c in range(2):
            lg = [torch.from_numpy(synth.gen_logits(synth.rng_for(wl.seed, 3, c, l), T, E)).to(dev)
                  for l in range(n_layers)]
            x = torch.from_numpy(synth.gen_x(synth.rng_for(wl.seed, 1, c), T, H).view(np.int16)).to(dev).view(torch.bfloat16)
            chunks.append((lg, x))
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        ids_h = torch.empty((T, k), dtype=torch.int32, pin_memory=True)
        outs = [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(2)]
        ev = torch.cuda.Event()

        def run_chunk(c):
            lg, x = chunks[c]
            npass = 0
            for l in range(n_layers):
                B.moe_route_topk(lg[l], k, topk_ids=ids, topk_w=w, err_word=err)
                ids_h.copy_(ids, non_blocking=True)   # the layer's routing, to the host once
                ev.record()
                ev.synchronize()
                y = outs[l & 1]
                _, n = B.moe_pipeline_prefill(p, l, ids_h.numpy(), x, ids, w, table, desc, out=y, ws=ws,
                                              err_word=err)
                npass += n
                x = y
            return npass

        run_chunk(0)   # warm-up (fills the cache with the last layer's passes)
        B.moe_pipeline_drain(p)
        torch.cuda.synchronize()
        s0 = B.moe_pipeline_stats_get(p, 0)
        t0 = time.perf_counter()
        npass = run_chunk(1)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        s1 = B.moe_pipeline_stats_get(p, 0)
        assert int(err.item()) == 0, f"device error word {int(err.item()):#x}"
        copied = s1["bytes_copied"] - s0["bytes_copied"]
        lc_ms = wall * 1000.0 / n_layers
        return {
            "workload": f"1024-token chunk of the decode layer shape (H 2048, E 512, I 512, top-10, 3-bit) "
                        f"through a {slots}-slot cache for {n_layers} layers; host tier holds every row",
            "passes_per_layer": npass / n_layers,
            "layer_chunk_ms": round(lc_ms, 3),
            "tok_s_4k_prompt_48_layers": round(T / (48 * lc_ms * 1e-3), 1),
            "install_GBps": round(copied / wall / 1e9, 2),
            "installs_per_layer": (s1["requests"] - s0["requests"] - (s1["hits"] - s0["hits"])) / n_layers,
            "hits_per_layer": (s1["hits"] - s0["hits"]) / n_layers,
            "copy_streams": n_copy,
            "bound": "host-to-device copies (every pass installs 64 rows of 1.38 MB)",
        }
    finally:
        B.moe_pipeline_destroy(p)
        B.moe_store_close(st)
        B.moe_cache_destroy(cache)
        del pool
        torch.cuda.empty_cache()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the routed-expert layer runs on a single "
              f"device); --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    import torch

    import quantized_routed_expert_softmax_amd as moe  # noqa: F401
    from quantized_routed_expert_softmax_amd import benchlib as mb
    from quantized_routed_expert_softmax_amd import binding as B
    from quantized_routed_expert_softmax_amd import synth

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    B.lib()  # fail loudly if the HIP library is missing
    mb.lib()
    dev = torch.device("cuda")
    if args.replay:
        replay_main(args, torch, B, synth)
        return
    if args.calibrate_copy:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_per_copy": n, "copies": 3}), flush=True)
        return
    if args.ceilings:
        print(json.dumps({"ceilings": ceilings(torch, mb, dev)}), flush=True)
        return
    if args.bounded_only:
        r = prefill_bounded_line(torch, B, synth, dev, torch.zeros(1, dtype=torch.int32, device=dev))
        print(json.dumps({"prefill_bounded": r}), flush=True)
        return
    # the bounded-cache prefill first, before the decode pools exist: its pinned
    # host tier mapped after a 135 GB device allocate/free cycle made a share of
    # its 88 MB installs up to 2x slower (54 -> 42 GB/s per layer-chunk); a
    # serving process sets up its host tier and pools at load time
    bounded = None
    if not args.no_extra and not args.no_prefill:
        bounded = prefill_bounded_line(torch, B, synth, dev, torch.zeros(1, dtype=torch.int32, device=dev))
        log(json.dumps({"prefill_bounded": bounded}))
        torch.cuda.empty_cache()
    wl = synth.WORKLOADS["decode"]
    t_setup = time.time()
    model = DecodeModel(torch, B, synth, wl)
    lg_np, x0_np = decode_inputs(torch, synth, wl)
    logits = torch.from_numpy(lg_np).to(dev)                      # [L, 1, E]
    x0 = torch.from_numpy(x0_np.view(np.int16)).to(dev).view(torch.bfloat16)
    ids = torch.empty((wl.layers, 1, wl.k), dtype=torch.int32, device=dev)
    w = torch.empty((wl.layers, 1, wl.k), dtype=torch.float32, device=dev)
    ws = torch.zeros(B.moe_forward_workspace_size(1, wl.k, wl.E, model.desc), dtype=torch.uint8, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    chain = Chain(torch, mb, 1, wl.H, wl.layers, x0)
    log(f"setup {time.time() - t_setup:.1f}s")

    def layer(l, n, y):
        # router + experts of layer l (one fused launch at decode batch sizes)
        B.moe_layer_forward(logits[l], n, model.tables[l], model.pools[l], model.desc, wl.k,
                            topk_ids=ids[l], topk_w=w[l], out=y, ws=ws, err_word=err)

    def step():
        chain.step(layer)

    for _ in range(2):   # eager warm-up (also required before graph capture)
        step()
    torch.cuda.synchronize()
    assert int(err.item()) == 0, f"device error word {int(err.item()):#x}"

    graph = None if args.eager else graph_of(torch, step)

    def run_step():
        if graph is not None:
            graph.replay()
        else:
            step()

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        run_step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    assert int(err.item()) == 0, f"device error word {int(err.item()):#x}"
    final = chain.final().float()
    assert bool(torch.isfinite(final).all())
    final_std = float(final.std())
    log(f"decode chain: final x std {final_std:.4f}")

    # --- the layer kernel alone: the same 48 launches on the chain's layer
    # inputs, in a graph of their own; one launch averages ms / 48 ---
    g_layers = graph_of(torch, lambda: chain.layers_only(layer))
    for _ in range(args.warmup):
        g_layers.replay()
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        g_layers.replay()
    ev1.record()
    torch.cuda.synchronize()
    fwd_ms_avg = ev0.elapsed_time(ev1) / args.steps / wl.layers
    del g_layers
    glue_us = (ms_per_step / wl.layers - fwd_ms_avg) * 1000.0
    ids_np = ids.cpu().numpy()
    distinct = [len(set(ids_np[l].reshape(-1).tolist())) for l in range(wl.layers)]
    # algorithmic bytes of one launch: the distinct routed experts' rows, the
    # router logits, x and out
    bytes_per_launch = float(np.mean(distinct)) * model.lay.slot_bytes + wl.E * 4 + 2 * wl.H * 2
    achieved_gbs = bytes_per_launch / (fwd_ms_avg * 1e-3) / 1e9
    step_bytes = sum(distinct) * model.lay.slot_bytes
    decode_gbs_step = step_bytes / (ms_per_step * 1e-3) / 1e9

    result = {
        "metric": "decode tok/s + HBM GB/s on quant expert bytes; 4K-prefill tok/s (MFMA util)",
        "value": round(1000.0 / ms_per_step, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode: 48 layers x (hidden 2048, 512 experts, intermediate 512, "
                               "top-10), 3-bit g64 experts, batch 1, 2048-slot pool per layer, "
                               "Zipf(1.1)-biased router logits; pre-norm residual chain "
                               "x_{l+1} = x_l + moe_l(rmsnorm(x_l))",
                   "global_batch": 1, "layers": wl.layers, "graph": graph is not None,
                   "wall_s_timed": round(wall, 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "decode1_kernel<3,3,16,1,10,2,2,4> (moe_layer_forward: route + hit list + "
                               "gate/up + SwiGLU + down + combine, one launch per layer)",
                     "avg_launch_us": round(fwd_ms_avg * 1000.0, 3),
                     "bytes_per_launch": int(bytes_per_launch)},
        "decode_expert_bytes_per_token": int(step_bytes),
        "decode_gbs_whole_step": round(decode_gbs_step, 1),
        "decode_chain": {"glue_us_per_layer": round(glue_us, 3), "final_x_std": round(final_std, 4),
                         "glue": "residual add + RMSNorm between layers, one libmoebench launch per layer"},
    }

    # ------------------------------- prefill ------------------------------- #
    if not args.no_prefill:
        pw = synth.WORKLOADS["prefill"]
        T, chunks = pw.T, pw.chunks
        plg = torch.empty((chunks, wl.layers, T, wl.E), dtype=torch.float32, device=dev)
        for c in range(chunks):
            for l in range(wl.layers):
                plg[c, l] = torch.from_numpy(synth.gen_logits(synth.rng_for(pw.seed, 3, c, l), T, wl.E)).to(dev)
        px = [torch.from_numpy(synth.gen_x(synth.rng_for(pw.seed, 1, c), T, wl.H).view(np.int16)).to(dev)
              .view(torch.bfloat16) for c in range(chunks)]
        pbuf = [torch.empty((T, wl.H), dtype=torch.bfloat16, device=dev) for _ in range(2)]
        pids = torch.empty((T, wl.k), dtype=torch.int32, device=dev)
        pw_ = torch.empty((T, wl.k), dtype=torch.float32, device=dev)
        pws = torch.zeros(B.moe_forward_workspace_size(T, wl.k, wl.E, model.desc), dtype=torch.uint8,
                          device=dev)
        pstart = [torch.cuda.Event(enable_timing=True) for _ in range(wl.layers)]
        pend = [torch.cuda.Event(enable_timing=True) for _ in range(wl.layers)]

        def prefill(timing=False):
            for c in range(chunks):
                x = px[c]
                for l in range(wl.layers):
                    y = pbuf[l & 1]
                    if timing and c == 0:
                        pstart[l].record()
                    B.moe_layer_forward(plg[c, l], x, model.tables[l], model.pools[l], model.desc, wl.k,
                                        topk_ids=pids, topk_w=pw_, out=y, ws=pws, err_word=err)
                    if timing and c == 0:
                        pend[l].record()
                    x = y

        prefill()
        torch.cuda.synchronize()
        pe0, pe1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        pe0.record()
        for _ in range(args.prefill_reps):
            prefill()
        pe1.record()
        torch.cuda.synchronize()
        p_ms = pe0.elapsed_time(pe1) / args.prefill_reps
        torch.cuda._sleep(20_000_000)
        prefill(timing=True)
        torch.cuda.synchronize()
        lc_ms = float(np.mean([a.elapsed_time(b) for a, b in zip(pstart, pend)]))
        assert int(err.item()) == 0, f"device error word {int(err.item()):#x}"
        pairs = T * wl.k
        flops = 2.0 * pairs * 3 * wl.H * wl.I
        lc_bytes = wl.E * model.lay.slot_bytes
        result["prefill"] = {
            "workload": "4K prompt = 4 chunks x 1024 tokens, 48 layers, all 512 experts resident",
            "tok_s": round(T * chunks / (p_ms * 1e-3), 1),
            "ms_per_prompt": round(p_ms, 3),
            "layer_chunk_us": round(lc_ms * 1000.0, 2),
            "useful_tflops": round(flops / (lc_ms * 1e-3) / 1e12, 2),
            "mfma_frac_of_bf16_peak": round(flops / (lc_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "hbm_gbs": round(lc_bytes / (lc_ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(lc_bytes / (lc_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        }

    # ----------------------------- CPU oracle ------------------------------ #
    if not args.no_cpu:
        import oracle
        # the first and last layer of the last timed step against the oracle, each
        # fed that layer's own input (not timed)
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
        checks = {}
        for l in (0, wl.layers - 1):
            checks[f"layer{l}"] = check_layer_vs_oracle(
                torch, B, oracle, synth, lg_np[l], chain.ns[l], chain.ys[l], ids[l], w[l], model.tables_np[l],
                model.pools[l], wl.slots_per_layer, model.lay, wl.E, wl.k, threads)
        result["decode_chain"]["oracle_check"] = checks
        nl = min(args.cpu_layers, wl.layers)
        x = x0_np.copy()
        t_cpu = 0.0
        for l in range(nl):
            # the routed experts' rows, copied once from the device (not timed)
            ids_l, w_l = oracle.route(lg_np[l], wl.k)
            used = sorted(set(ids_l.reshape(-1).tolist()))
            idx = torch.as_tensor([int(model.tables_np[l][e]) for e in used], device=dev)
            rows = model.pools[l].view(wl.slots_per_layer, -1).index_select(0, idx).cpu().numpy()
            table = np.full(wl.E, -1, np.int32)
            table[used] = np.arange(len(used), dtype=np.int32)
            t0 = time.perf_counter()
            ids_l, w_l = oracle.route(lg_np[l], wl.k)
            out = oracle.layer(x, ids_l, w_l, table, rows, wl.H, wl.I, wl.bits_gu, wl.bits_d, wl.E,
                               threads=1)
            t_cpu += time.perf_counter() - t0
            x = synth.f32_to_bf16_bits(out.astype(np.float32))
        per_layer = t_cpu / nl
        cores = len(os.sched_getaffinity(0))
        result["cpu_baseline"] = {
            "value": round(1.0 / (per_layer * wl.layers), 5),
            "unit": "tok/s",
            "cores": 1,
            "kind": "oracle",
            "sample": f"{nl} of 48 decode layers of one token (route + fp64 layer), scaled to 48 "
                      f"layers; the oracle parallelises over tokens only, so batch 1 uses one core",
            "seconds": round(t_cpu, 2),
            "host_cores_available": cores,
            "cpu_model": cpu_model(),
        }
        if not args.no_prefill:
            # one layer of one 1024-token chunk (all 512 experts) on every host core,
            # scaled to 48 layers x 4 chunks (extrapolated)
            pw = synth.WORKLOADS["prefill"]
            rows = model.pools[0].view(wl.slots_per_layer, -1).index_select(
                0, torch.as_tensor(model.tables_np[0].astype(np.int64), device=dev)).cpu().numpy()
            plg0 = synth.gen_logits(synth.rng_for(pw.seed, 3, 0, 0), pw.T, wl.E)
            px0 = synth.gen_x(synth.rng_for(pw.seed, 1, 0), pw.T, wl.H)
            t0 = time.perf_counter()
            ids_l, w_l = oracle.route(plg0, wl.k)
            oracle.layer(px0, ids_l, w_l, np.arange(wl.E, dtype=np.int32), rows, wl.H, wl.I, wl.bits_gu,
                         wl.bits_d, wl.E, threads=cores)
            t_pf = time.perf_counter() - t0
            result["cpu_baseline_prefill"] = {
                "value": round(pw.T / (t_pf * wl.layers), 3),
                "unit": "tok/s (4K prompt, 48 layers)",
                "cores": cores,
                "kind": "oracle",
                "sample": "one layer of one 1024-token chunk (route + fp64 layer, every expert hit), "
                          "scaled to 48 layers x 4 chunks: extrapolated",
                "seconds": round(t_pf, 2),
                "cpu_model": cpu_model(),
            }
    del model
    torch.cuda.empty_cache()

    if not args.no_extra:
        result["mixed"] = mixed_lines(torch, B, mb, synth, dev, err, max(5, args.steps // 4))
        log(json.dumps({"mixed": result["mixed"]}))
        result["int8_subst"] = int8_subst_line(torch, B, synth, dev, err, 20)
        log(json.dumps({"int8_subst": result["int8_subst"]}))
        if bounded is not None:
            result["prefill_bounded"] = bounded

    # ------------------------ unquantized bf16 experts ---------------------- #
    if not args.no_bf16:
        result["bf16_experts"] = bf16_lines(torch, B, synth, wl, dev, err)

    # ------------------------------ ceilings -------------------------------- #
    if not args.no_extra:
        ce = ceilings(torch, mb, dev, quick=True)
        result["ceilings"] = ce
        dr = ce["read_decode_rows"]["GBps"]
        result["roofline"]["measured_ceiling"] = {
            "GBps": dr, "frac": round(achieved_gbs / dr, 4),
            "what": "best streamed read of ten scattered 1376256-byte rows per launch, 48 launches in a "
                    "HIP graph (the decode layer's bytes per launch)"}
        if "prefill" in result:
            pr_ = ce["read_prefill_rows"]["GBps"]
            result["prefill"]["measured_ceiling"] = {
                "GBps": pr_, "frac": round(result["prefill"]["hbm_gbs"] / pr_, 4),
                "what": "best streamed read of 512 scattered 1376256-byte rows per launch"}

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
