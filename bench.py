#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE layer on one MI355X.

Workload (the headline): decode of a 48-layer MoE with 512 experts per layer,
hidden 2048, expert intermediate 512, top-10, 3-bit group-64 experts, batch 1,
a 2048-slot pool per layer with a random expert -> slot table, router logits
N(0,1) plus a per-expert Zipf(1.1) bias.  One step = one decode token through
all 48 layers: per layer route (softmax, top-k, renormalise) and the experts
forward (sort by expert, slot resolve, gate/up, SwiGLU, down, weighted
combine); each layer's output is the next layer's input.  The step is captured
once in a HIP graph and replayed.

Also reported: 4K-token prefill (4 chunks of 1024 tokens through the same 48
layers, every expert resident, MFMA path) and the CPU oracle on the host cores.

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
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 1 GiB device copy (to scale the FETCH_SIZE / WRITE_SIZE "
                        "counters of a profiling run)")
    return p.parse_args()


# Sources of the fused decode kernel; the measured HBM traffic recorded in the
# profile summary below holds only while their hash matches.
DECODE_SOURCES = ["quantized_routed_expert_softmax_amd/csrc/decode.hip",
                  "quantized_routed_expert_softmax_amd/csrc/route_dev.h",
                  "quantized_routed_expert_softmax_amd/csrc/moe_dev.h",
                  "include/moe.h"]
TRAFFIC_SUMMARY = "profiles/decode_layer_kernel_3_3_1_1-decode48.md"


def decode_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
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
    if fields.get("kernel sources sha256") != decode_sources_sha256():
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
        "decode_path": "fused decode kernel decode_layer_kernel<16,16,1,1,8>: routing, sort, gate/up + SwiGLU, down and combine in one launch per layer, 48 layer-steps in one HIP graph",
        "prefill_chunk_us": round(p_us, 2),
        "prefill_hbm_gbs": round(p_bytes / (p_us * 1e-6) / 1e9, 1),
        "prefill_hbm_frac": round(p_bytes / (p_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "prefill_useful_tflops": round(flops / (p_us * 1e-6) / 1e12, 1),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the routed-expert layer runs on a single "
              f"device); --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    import torch

    import quantized_routed_expert_softmax_amd as moe
    from quantized_routed_expert_softmax_amd import binding as B
    from quantized_routed_expert_softmax_amd import synth

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    B.lib()  # fail loudly if the HIP library is missing
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
    wl = synth.WORKLOADS["decode"]
    t_setup = time.time()
    model = DecodeModel(torch, B, synth, wl)
    lg_np, x0_np = decode_inputs(torch, synth, wl)
    logits = torch.from_numpy(lg_np).to(dev)                      # [L, 1, E]
    x0 = torch.from_numpy(x0_np.view(np.int16)).to(dev).view(torch.bfloat16)
    xbuf = [torch.empty((1, wl.H), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    ids = torch.empty((wl.layers, 1, wl.k), dtype=torch.int32, device=dev)
    w = torch.empty((wl.layers, 1, wl.k), dtype=torch.float32, device=dev)
    ws = torch.zeros(B.moe_forward_workspace_size(1, wl.k, wl.E, model.desc), dtype=torch.uint8, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    log(f"setup {time.time() - t_setup:.1f}s")

    def step(timing=None):
        # per layer: router + experts (one fused launch at decode batch sizes)
        x = x0
        for l in range(wl.layers):
            y = xbuf[l & 1]
            if timing is not None:
                timing[0][l].record()
            B.moe_layer_forward(logits[l], x, model.tables[l], model.pools[l], model.desc, wl.k,
                                topk_ids=ids[l], topk_w=w[l], out=y, ws=ws, err_word=err)
            if timing is not None:
                timing[1][l].record()
            x = y
        return x

    # warm up eagerly (also required before graph capture)
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    assert int(err.item()) == 0, f"device error word {int(err.item()):#x}"

    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()

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
    out_final = xbuf[(wl.layers - 1) & 1].float()
    assert bool(torch.isfinite(out_final).all())

    # --- per-launch duration: the timed region above is `steps` replays of a
    # graph of 48 back-to-back launches (one per layer), bracketed by HIP events
    # on the replay stream, so one launch averages ms_per_step / 48 ---
    fwd_ms_avg = ms_per_step / wl.layers
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
                               "Zipf(1.1)-biased router logits",
                   "global_batch": 1, "layers": wl.layers, "graph": graph is not None,
                   "wall_s_timed": round(wall, 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "decode_layer_kernel<3,3,1,1> (moe_layer_forward: route + sort + "
                               "gate/up + SwiGLU + down + combine, one launch per layer)",
                     "avg_launch_us": round(fwd_ms_avg * 1000.0, 3),
                     "bytes_per_launch": int(bytes_per_launch)},
        "decode_expert_bytes_per_token": int(step_bytes),
        "decode_gbs_whole_step": round(decode_gbs_step, 1),
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

    # ------------------------ unquantized bf16 experts ---------------------- #
    if not args.no_bf16:
        result["bf16_experts"] = bf16_lines(torch, B, synth, wl, dev, err)

    # ----------------------------- CPU oracle ------------------------------ #
    if not args.no_cpu:
        import oracle
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
        result["cpu_baseline"] = {
            "value": round(1.0 / (per_layer * wl.layers), 5),
            "unit": "tok/s",
            "cores": 1,
            "kind": "oracle",
            "sample": f"{nl} of 48 decode layers of one token (route + fp64 layer), scaled to 48 "
                      f"layers; the oracle parallelises over tokens only, so batch 1 uses one core",
            "seconds": round(t_cpu, 2),
            "host_cores_available": len(os.sched_getaffinity(0)),
        }

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
