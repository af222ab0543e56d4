"""Miss pipeline on the GPU: expert store -> (pinned host tier) -> device slot
pools of two size classes, installs on a copy stream, reservations by events.

A replay of decode steps through a cache that holds half of each layer's experts
must give, layer by layer, bit-identical outputs to the same kernels run on
pools that hold every expert (the kernels read only the bytes of the slot the
table names, so where an expert sits cannot change a bit).  The cache's
per-class hits and misses must equal the plain LRU model in tests/lru_model.py
when every install has completed between layers, and the device pools must hold
exactly the store's rows.

Sources: "RFC: stream MoE experts from disk in from_pretrained", How the
prototype works (Cache, Reads and Host tier bullets); "POC: Experts offload",
commit messages (reused pinned staging buffers, one small table copy per layer,
host rows kept until their copy has finished, predicted reads still in flight
bypassed); "moe: expert slots in size classes", PR description (a separate slot
pool and LRU for every class, an equal fraction for every layer).
"""
import numpy as np
import pytest

from lru_model import CacheModel
from quantized_routed_expert_softmax_amd import binding as B
from quantized_routed_expert_softmax_amd import synth

pytestmark = pytest.mark.gpu

H, I, E, K = 256, 128, 16, 4
LAYER_BITS = [(4, 4), (4, 4), (4, 6), (4, 4), (4, 4), (4, 6)]   # two size classes


def _torch():
    import torch
    return torch


class Replay:
    """Store rows, routing and inputs of a small mixed-class decode run."""

    def __init__(self, seed=0, tokens=6, T=1, share=0.5, bits=LAYER_BITS):
        self.T, self.tokens = T, tokens
        kinds = sorted(set(bits))
        self.layer_class = [kinds.index(b) for b in bits]
        self.L = len(bits)
        per_class_layers = [self.layer_class.count(c) for c in range(len(kinds))]
        self.class_slots = [max(int(share * E) * n, T * K) for n in per_class_layers]
        self.classes = [B.moe_size_class_init(H, I, bg, bd, n)
                        for (bg, bd), n in zip(kinds, self.class_slots)]
        self.full = [B.moe_size_class_init(H, I, bg, bd, E) for (bg, bd) in kinds]
        rng = synth.rng_for(seed, 1)
        rows = []
        for l, (bg, bd) in enumerate(bits):
            lay = synth.Layout(H, I, bg, bd)
            for e in range(E):
                rows.append(synth.expert_row(lay, synth.random_code_expert(rng, H, I, bg, bd)))
        self.store_bytes = np.ascontiguousarray(np.concatenate(rows))
        rl = synth.rng_for(seed, 2)
        self.logits = [synth.gen_logits(rl, T, E) for _ in range(tokens * self.L)]
        self.x0 = [synth.gen_x(synth.rng_for(seed, 3, t), T, H) for t in range(tokens)]

    def row(self, layer, e):
        sb = [self.classes[c].slot_bytes for c in self.layer_class]
        off = sum(E * s for s in sb[:layer]) + e * sb[layer]
        return self.store_bytes[off:off + sb[layer]]

    def route_all(self):
        """Routing of every (token, layer) on the GPU, brought to the host once."""
        torch = _torch()
        ids, ws = [], []
        for lg in self.logits:
            i, w = B.moe_route_topk(torch.from_numpy(lg).cuda(), K)
            ids.append(i)
            ws.append(w)
        host = [i.cpu().numpy() for i in ids]
        return ids, ws, host

    def reference(self, ids, ws):
        """Every expert resident (identity tables): outputs of every (token, layer)."""
        torch = _torch()
        pools = []
        for l in range(self.L):
            c = self.layer_class[l]
            p = torch.from_numpy(np.ascontiguousarray(
                np.stack([self.row(l, e) for e in range(E)]))).cuda()
            pools.append((p, self.full[c]))
        table = torch.arange(E, dtype=torch.int32, device="cuda")
        ws_buf = torch.zeros(B.moe_forward_workspace_size(self.T, K, E, self.full[0]) + 4096,
                             dtype=torch.uint8, device="cuda")
        outs = []
        for t in range(self.tokens):
            x = torch.from_numpy(self.x0[t].view(np.int16)).cuda().view(torch.bfloat16)
            for l in range(self.L):
                p, d = pools[l]
                j = t * self.L + l
                x = B.moe_experts_forward(x, ids[j], ws[j], E, table, p.view(-1), d, ws=ws_buf)
                outs.append(x)
        torch.cuda.synchronize()
        return [o.cpu() for o in outs]


def run_pipeline(rp: Replay, ids, ws, ids_host, store, host_tier_bytes=0, preload=False,
                 io_threads=2, staging_rows=4, drain_each=False, prefetch=False, model=None,
                 n_copy=1, policy=B.MOE_EVICT_LRU, per_layer=False):
    """Decode steps through the pipeline; no host synchronisation between layers
    unless drain_each.  Returns (outputs, per-class stats, pools, cache tables)."""
    torch = _torch()
    pools = [torch.zeros(d.n_slots * d.slot_bytes, dtype=torch.uint8, device="cuda")
             for d in rp.classes]
    cache = B.moe_cache_create(rp.classes, rp.layer_class, E, policy=policy, per_layer=per_layer)
    copies = [torch.cuda.Stream() for _ in range(n_copy)]
    p = B.moe_pipeline_create(cache, store, pools, host_tier_bytes=host_tier_bytes,
                              host_preload=preload, io_threads=io_threads,
                              staging_rows=staging_rows, copy_streams=copies)
    try:
        table = torch.full((E,), -1, dtype=torch.int32, device="cuda")
        ws_buf = torch.zeros(B.moe_forward_workspace_size(rp.T, K, E, rp.classes[0]) + 4096,
                             dtype=torch.uint8, device="cuda")
        outs = []
        for t in range(rp.tokens):
            x = torch.from_numpy(rp.x0[t].view(np.int16)).cuda().view(torch.bfloat16)
            for l in range(rp.L):
                j = t * rp.L + l
                c = rp.layer_class[l]
                B.moe_pipeline_prepare(p, l, ids_host[j], table)
                if model is not None:
                    model.prepare(l, ids_host[j], last_first=True)
                if prefetch and j + 1 < len(ids_host):   # a perfect guess of the next layer
                    B.moe_pipeline_prefetch(p, (l + 1) % rp.L, ids_host[j + 1])
                x = B.moe_experts_forward(x, ids[j], ws[j], E, table, pools[c], rp.classes[c], ws=ws_buf)
                outs.append(x)
                B.moe_pipeline_release(p, l)
                if drain_each:
                    B.moe_pipeline_drain(p)
        B.moe_pipeline_drain(p)
        torch.cuda.synchronize()
        stats = [B.moe_pipeline_stats_get(p, c) for c in range(len(rp.classes))]
        cstats = [B.moe_cache_class_stats(cache, c) for c in range(len(rp.classes))]
        tables = [B.moe_cache_table(cache, l, E) for l in range(rp.L)]
        host_rows = [B.moe_pipeline_host_rows(p, c) for c in range(len(rp.classes))]
        return [o.cpu() for o in outs], stats, cstats, pools, tables, host_rows
    finally:
        B.moe_pipeline_destroy(p)
        B.moe_cache_destroy(cache)


def check_outputs(got, ref):
    assert len(got) == len(ref)
    for i, (a, b) in enumerate(zip(got, ref)):
        assert a.view(_torch().int16).equal(b.view(_torch().int16)), f"output {i} differs"


def check_pools(rp, pools, tables):
    for l in range(rp.L):
        c = rp.layer_class[l]
        sb = rp.classes[c].slot_bytes
        pool = pools[c].cpu().numpy()
        for e in range(E):
            s = int(tables[l][e])
            if s >= 0:
                assert np.array_equal(pool[s * sb:(s + 1) * sb], rp.row(l, e)), (l, e)


@pytest.fixture(scope="module")
def replay():
    rp = Replay(seed=0, tokens=6, T=1)
    ids, ws, host = rp.route_all()
    ref = rp.reference(ids, ws)
    return rp, ids, ws, host, ref


@pytest.mark.parametrize("kind", ["file", "memory"])
def test_replay_from_store_matches_resident_run_and_lru_model(replay, kind, tmp_path):
    """No host tier: every device miss is a store read into a reused pinned
    buffer, then one copy.  Installs complete between layers (drain), so the cache
    follows the LRU model exactly."""
    rp, ids, ws, host, ref = replay
    if kind == "file":
        path = tmp_path / "experts.bin"
        rp.store_bytes.tofile(path)
        store = B.moe_store_open_file(str(path), rp.classes, rp.layer_class, E)
    else:
        store = B.moe_store_open_memory(rp.store_bytes, rp.classes, rp.layer_class, E)
    try:
        model = CacheModel(rp.class_slots, rp.layer_class, E)
        outs, stats, cstats, pools, tables, _ = run_pipeline(rp, ids, ws, host, store,
                                                             drain_each=True, model=model)
    finally:
        B.moe_store_close(store)
    check_outputs(outs, ref)
    check_pools(rp, pools, tables)
    for c in range(len(rp.classes)):
        mh, mm, mev = model.class_stats(c)
        assert cstats[c] == (mh, mm, mev)
        st = stats[c]
        assert st["requests"] == mh + mm and st["hits"] == mh and st["inflight_hits"] == 0
        assert st["store_reads"] == mm and st["host_hits"] == 0
        assert st["bytes_copied"] == mm * rp.classes[c].slot_bytes == st["bytes_read"]
        assert mev > 0                       # the half-size cache really evicts
    for l in range(rp.L):
        assert tables[l].tolist() == model.table(l)


@pytest.mark.parametrize("policy,per_layer", [(B.MOE_EVICT_LFU, False), (B.MOE_EVICT_LRU, True),
                                              (B.MOE_EVICT_LFU, True)])
def test_replay_eviction_variants_match_model(replay, policy, per_layer):
    """LFU and per-layer LRU caches behind the pipeline: same outputs, and the
    per-class counters and tables of the plain model."""
    rp, ids, ws, host, ref = replay
    store = B.moe_store_open_memory(rp.store_bytes, rp.classes, rp.layer_class, E)
    try:
        model = CacheModel(rp.class_slots, rp.layer_class, E, lfu=policy == B.MOE_EVICT_LFU,
                           per_layer=per_layer)
        outs, stats, cstats, pools, tables, _ = run_pipeline(rp, ids, ws, host, store, drain_each=True,
                                                             model=model, policy=policy,
                                                             per_layer=per_layer, n_copy=2)
    finally:
        B.moe_store_close(store)
    check_outputs(outs, ref)
    check_pools(rp, pools, tables)
    for c in range(len(rp.classes)):
        assert cstats[c] == model.class_stats(c)
    for l in range(rp.L):
        assert tables[l].tolist() == model.table(l)


def test_replay_overlapped_installs_without_host_waits(replay):
    """No drains: each prepare only enqueues, the copy stream waits on the use
    event of a slot's previous forward, the compute stream on the install events.
    Smallest legal cache (one layer's experts per class), so nearly every install
    overwrites a slot whose previous forward is still queued."""
    rp0, ids, ws, host, ref = replay
    rp = Replay(seed=0, tokens=6, T=1, share=0.0)   # class slots = T*K
    assert rp.class_slots == [K, K]
    store = B.moe_store_open_memory(rp.store_bytes, rp.classes, rp.layer_class, E)
    try:
        outs, stats, cstats, pools, tables, _ = run_pipeline(rp, ids, ws, host, store, io_threads=4,
                                                             staging_rows=4, n_copy=2)
    finally:
        B.moe_store_close(store)
    check_outputs(outs, ref)
    check_pools(rp, pools, tables)
    for c, st in enumerate(stats):
        assert st["requests"] == st["hits"] + st["inflight_hits"] + st["host_hits"] + st["store_reads"]
        assert cstats[c][1] == st["host_hits"] + st["store_reads"]


def test_replay_host_tier_preloaded(replay):
    """Host tier big enough for every expert and preloaded: device misses are
    copies from pinned host rows, the store is read once at creation."""
    rp, ids, ws, host, ref = replay
    store = B.moe_store_open_memory(rp.store_bytes, rp.classes, rp.layer_class, E)
    try:
        model = CacheModel(rp.class_slots, rp.layer_class, E)
        outs, stats, cstats, pools, tables, host_rows = run_pipeline(
            rp, ids, ws, host, store, host_tier_bytes=rp.store_bytes.size, preload=True,
            drain_each=True, model=model, n_copy=2)
    finally:
        B.moe_store_close(store)
    check_outputs(outs, ref)
    check_pools(rp, pools, tables)
    for c in range(len(rp.classes)):
        n_layers = rp.layer_class.count(c)
        assert host_rows[c] == n_layers * E
        st = stats[c]
        mh, mm, _ = model.class_stats(c)
        assert st["store_reads"] == 0 and st["host_hits"] == mm and st["hits"] == mh
        assert st["bytes_read"] == n_layers * E * rp.classes[c].slot_bytes


def test_replay_partial_host_tier_and_perfect_guesses(replay):
    """A host tier of about a third of the experts (rows recycled by their own
    LRU) and a guess of the next layer's experts issued before each forward: the
    guessed experts are resident or on their way when their layer asks."""
    rp, ids, ws, host, ref = replay
    store = B.moe_store_open_memory(rp.store_bytes, rp.classes, rp.layer_class, E)
    try:
        outs, stats, cstats, pools, tables, host_rows = run_pipeline(
            rp, ids, ws, host, store, host_tier_bytes=rp.store_bytes.size // 3, io_threads=3,
            staging_rows=3, prefetch=True, n_copy=3)
    finally:
        B.moe_store_close(store)
    check_outputs(outs, ref)
    check_pools(rp, pools, tables)
    assert all(0 < r < rp.layer_class.count(c) * E for c, r in enumerate(host_rows))
    demand_misses = 0
    for c, st in enumerate(stats):
        misses = st["requests"] - st["hits"] - st["inflight_hits"]
        demand_misses += misses
        assert st["host_hits"] + st["store_reads"] == misses + st["prefetches"]
        assert st["prefetches"] > 0
    # only the first layer of the run is not guessed
    assert demand_misses <= K


def test_replay_batch_of_tokens_with_duplicate_experts():
    """Two tokens per step: a layer asks for up to 2k experts, some shared."""
    rp = Replay(seed=5, tokens=4, T=2)
    ids, ws, host = rp.route_all()
    ref = rp.reference(ids, ws)
    store = B.moe_store_open_memory(rp.store_bytes, rp.classes, rp.layer_class, E)
    try:
        model = CacheModel(rp.class_slots, rp.layer_class, E)
        outs, stats, cstats, pools, tables, _ = run_pipeline(rp, ids, ws, host, store, drain_each=True,
                                                             model=model)
    finally:
        B.moe_store_close(store)
    check_outputs(outs, ref)
    for c in range(len(rp.classes)):
        assert cstats[c] == model.class_stats(c)


def test_prepare_twice_without_release_is_rejected(replay):
    torch = _torch()
    rp, ids, ws, host, ref = replay
    store = B.moe_store_open_memory(rp.store_bytes, rp.classes, rp.layer_class, E)
    pools = [torch.zeros(d.n_slots * d.slot_bytes, dtype=torch.uint8, device="cuda")
             for d in rp.classes]
    cache = B.moe_cache_create(rp.classes, rp.layer_class, E)
    p = B.moe_pipeline_create(cache, store, pools, io_threads=1, staging_rows=1,
                              copy_streams=[torch.cuda.Stream()])
    try:
        table = torch.full((E,), -1, dtype=torch.int32, device="cuda")
        B.moe_pipeline_prepare(p, 0, host[0], table)
        with pytest.raises(B.MoeError) as ei:
            B.moe_pipeline_prepare(p, 0, host[0], table)
        assert ei.value.code == B.MOE_E_BUSY
        with pytest.raises(B.MoeError):
            B.moe_pipeline_release(p, 1)          # layer 1 was never prepared
        with pytest.raises(B.MoeError):
            B.moe_pipeline_prepare(p, 1, np.array([E], np.int32), table)   # id out of range
        with pytest.raises(B.MoeError):                                    # another compute stream
            B.moe_pipeline_prepare(p, 1, host[1], table, stream=torch.cuda.Stream())
        B.moe_pipeline_release(p, 0)
        B.moe_pipeline_drain(p)
        torch.cuda.synchronize()
        assert (table.cpu().numpy() >= 0).sum() == len(set(host[0].reshape(-1).tolist()))
    finally:
        B.moe_pipeline_destroy(p)
        B.moe_cache_destroy(cache)
        B.moe_store_close(store)


class RouterModel:
    """A residual decode stack driven by routers: layer l routes with its router
    on x_l, and x_{l+1} = x_l + moe_l(x_l).  The lookahead runs the routers of
    layers l+1 and l+2 on x_l too, to guess their experts ("RFC ...", How the
    prototype works, Reads bullet)."""

    def __init__(self, rp: Replay, seed=7):
        torch = _torch()
        rng = synth.rng_for(seed, 9)
        w = (rng.standard_normal((rp.L, E, H)) / np.sqrt(H)).astype(np.float32)
        self.routers = torch.from_numpy(synth.f32_to_bf16_bits(w).view(np.int16)).cuda().view(torch.bfloat16)
        self.rp = rp

    def run(self, forward, prepare=None, prefetch=None, release=None, ahead=2):
        """Decode every token; forward(l, x, ids, w) returns moe_l(x).  Returns the
        per-layer outputs and the routed ids of every (token, layer)."""
        torch = _torch()
        rp = self.rp
        outs, routed = [], []
        for t in range(rp.tokens):
            x = torch.from_numpy(rp.x0[t].view(np.int16)).cuda().view(torch.bfloat16)
            for l in range(rp.L):
                n = min(1 + ahead, rp.L - l)
                logits = B.moe_router_logits(x, self.routers[l:l + n])
                ids, w = B.moe_route_topk(logits.view(n * rp.T, E), K)
                ids_h = ids.cpu().numpy()          # this layer's routing + the guesses
                routed.append(ids_h[:rp.T].copy())
                if prepare is not None:
                    prepare(l, ids_h[:rp.T])
                if prefetch is not None:
                    for a in range(1, n):
                        prefetch(l + a, ids_h[a * rp.T:(a + 1) * rp.T])
                y = forward(l, x, ids[:rp.T], w[:rp.T])
                if release is not None:
                    release(l)
                x = x + y
                outs.append(y)
        torch.cuda.synchronize()
        return [o.cpu() for o in outs], routed


def test_lookahead_guesses_match_resident_run_and_cut_misses():
    """Guesses of the next two layers' experts, issued from the current hidden
    state, start installs before those layers route; outputs stay bit-identical
    to an all-resident run of the same router-driven stack (the guesses change
    where experts sit, never what a layer computes), and they cut the demand
    misses of the same routing sequence."""
    torch = _torch()
    rp = Replay(seed=3, tokens=5, T=1)
    model = RouterModel(rp)
    full_pools = []
    for l in range(rp.L):
        full_pools.append(torch.from_numpy(np.ascontiguousarray(
            np.stack([rp.row(l, e) for e in range(E)]))).cuda().view(-1))
    ident = torch.arange(E, dtype=torch.int32, device="cuda")
    ws_ref = torch.zeros(B.moe_forward_workspace_size(rp.T, K, E, rp.full[0]) + 4096,
                         dtype=torch.uint8, device="cuda")

    def fwd_ref(l, x, ids, w):
        return B.moe_experts_forward(x, ids, w, E, ident, full_pools[l], rp.full[rp.layer_class[l]], ws=ws_ref)

    ref, ref_ids = model.run(fwd_ref)
    misses = {}
    for ahead in (0, 2):
        store = B.moe_store_open_memory(rp.store_bytes, rp.classes, rp.layer_class, E)
        pools = [torch.zeros(d.n_slots * d.slot_bytes, dtype=torch.uint8, device="cuda") for d in rp.classes]
        cache = B.moe_cache_create(rp.classes, rp.layer_class, E)
        p = B.moe_pipeline_create(cache, store, pools, host_tier_bytes=rp.store_bytes.size,
                                  host_preload=True, io_threads=2, staging_rows=2,
                                  copy_streams=[torch.cuda.Stream(), torch.cuda.Stream()])
        table = torch.full((E,), -1, dtype=torch.int32, device="cuda")
        ws_buf = torch.zeros(B.moe_forward_workspace_size(rp.T, K, E, rp.classes[0]) + 4096,
                             dtype=torch.uint8, device="cuda")
        try:
            def fwd(l, x, ids, w):
                c = rp.layer_class[l]
                return B.moe_experts_forward(x, ids, w, E, table, pools[c], rp.classes[c], ws=ws_buf)

            got, got_ids = model.run(
                fwd, prepare=lambda l, ids: B.moe_pipeline_prepare(p, l, ids, table),
                prefetch=lambda l, ids: B.moe_pipeline_prefetch(p, l, ids),
                release=lambda l: B.moe_pipeline_release(p, l), ahead=ahead)
            B.moe_pipeline_drain(p)
            stats = [B.moe_pipeline_stats_get(p, c) for c in range(len(rp.classes))]
        finally:
            B.moe_pipeline_destroy(p)
            B.moe_cache_destroy(cache)
            B.moe_store_close(store)
        assert all(np.array_equal(a, b) for a, b in zip(got_ids, ref_ids))
        check_outputs(got, ref)
        m = sum(st["requests"] - st["hits"] - st["inflight_hits"] for st in stats)
        prefetches = sum(st["prefetches"] for st in stats)
        assert sum(st["host_hits"] for st in stats) == m + prefetches
        assert (prefetches > 0) == (ahead > 0)
        misses[ahead] = m
    assert misses[2] < misses[0]
