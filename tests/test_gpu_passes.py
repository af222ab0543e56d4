"""Prefill in passes of at most 64 hit experts, on the GPU.

Almost every expert of a layer is hit by a long prompt; the hit experts run in
ascending id, 64 per pass, so that only one pass's experts must be resident at a
time ("RFC: stream MoE experts from disk in from_pretrained", How the prototype
works, Prefill bullet; "POC: Experts offload", commit messages: the sorted
prefill's batches of 64 experts).

Checked here:
  * sort once, passes one by one (or in groups), combine once: bit-identical to
    the one-launch MFMA forward, and within max-abs 2e-2 / rel-L2 1e-2 of the
    oracle;
  * a pass reads only its own experts' slots: a table holding nothing but the
    pass's experts (placed elsewhere in a fresh pool) gives the same bits;
  * the pipeline driver runs a layer through a size class with fewer slots than
    the layer hits experts (64 slots for 128 hit experts; 128 slots for the
    1024-token chunk of the decode layer shape that hits all 512), installing
    every pass before it runs: pass count, per-class install counts and the
    oracle on every / sampled tokens.
"""
import os

import numpy as np
import pytest

import oracle
from quantized_routed_expert_softmax_amd import binding as B
from quantized_routed_expert_softmax_amd import synth

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
REL_L2 = 1e-2
THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def _torch():
    import torch
    return torch


def to_dev(a):
    return _torch().from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(x_bits):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda().view(torch.bfloat16)


def bits16(t):
    return t.view(_torch().int16).cpu().numpy()


def check_close(got_bf16, ref, what=""):
    got = got_bf16.float().cpu().numpy().astype(np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), what
    d = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert d.max() <= MAX_ABS and rel <= REL_L2, f"{what}: max-abs {d.max():.3e} rel-L2 {rel:.3e}"


def err_word():
    return _torch().zeros(1, dtype=_torch().int32, device="cuda")


def run_in_passes(x, ids, w, E, table, pool, desc, groups):
    """Sort, then the pass ranges in `groups` one call each, then combine."""
    torch = _torch()
    ew = err_word()
    ws = B.moe_prefill_sort(x, ids, E, desc, err_word=ew)
    for (p0, p1) in groups:
        B.moe_prefill_pass(x.shape[0], ids.shape[1], E, p0, p1, table, pool, desc, ws, err_word=ew)
    out = B.moe_prefill_combine(w, E, desc, ws)
    torch.cuda.synchronize()
    return out, int(ew.item())


# (T, H, E, I, k, bits_gu, bits_d, seed): several passes with a ragged last one,
# exactly one full pass, fewer hit experts than one pass, each code width
PASS_CASES = [
    (256, 256, 128, 128, 8, 4, 4, 700),
    (300, 256, 200, 128, 6, 3, 3, 701),     # 4 passes, the last of 8 experts
    (96, 256, 64, 192, 4, 8, 6, 702),       # one pass
    (5, 128, 300, 64, 3, 4, 8, 703),        # 15 hit experts of 300
    (130, 192, 150, 128, 8, 16, 16, 704),   # bf16 experts
    (64, 128, 1024, 64, 32, 6, 4, 705),     # maximum E and k: 16 passes
]


@pytest.mark.parametrize("case", PASS_CASES)
def test_passes_match_one_launch_and_oracle(case):
    T, H, E, I, k, bg, bd, seed = case
    pr = synth.make_problem(seed, T, H, E, I, k, bg, bd, n_slots=E + 3)
    ids_o, w_o = oracle.route(pr.logits, k)
    ids, w = to_dev(ids_o), to_dev(w_o)
    desc = B.moe_size_class_init(H, I, bg, bd, pr.pool.shape[0])
    x, table, pool = dev_bf16(pr.x), to_dev(pr.table), to_dev(pr.pool.reshape(-1))
    pt = B.moe_pass_table_host(ids_o, E)
    _, _, pt_o = oracle.sort(ids_o, E, 64)
    assert np.array_equal(pt, pt_o)
    n_pass, n_max = int(pt[1]), (E + 63) // 64
    ew = err_word()
    ref_gpu = B.moe_experts_forward(x, ids, w, E, table, pool, desc, err_word=ew, path=B.MOE_PATH_MFMA)
    _torch().cuda.synchronize()
    assert int(ew.item()) == 0
    # one pass per call, every pass (past the hit count too: empty no-ops)
    one_by_one = [(q, q + 1) for q in range(n_max)]
    halves = [(0, n_max // 2), (n_max // 2, n_max)]
    for groups in (one_by_one, halves, [(0, n_max)]):
        out, ew_ = run_in_passes(x, ids, w, E, table, pool, desc, groups)
        assert ew_ == 0
        assert np.array_equal(bits16(out), bits16(ref_gpu)), groups
    ref = oracle.layer(pr.x, ids_o, w_o, pr.table, pr.pool, H, I, bg, bd, E, threads=THREADS)
    check_close(out, ref, f"passes {case}")
    assert n_pass == (int(pt[0]) + 63) // 64


@pytest.mark.parametrize("case", PASS_CASES[:2] + PASS_CASES[3:4])
def test_pass_reads_only_its_experts(case):
    """Each pass runs against a table that holds only that pass's experts, in a
    pool where they sit at other slots than before: the result does not change."""
    torch = _torch()
    T, H, E, I, k, bg, bd, seed = case
    pr = synth.make_problem(seed, T, H, E, I, k, bg, bd, n_slots=E + 3)
    ids_o, w_o = oracle.route(pr.logits, k)
    ids, w = to_dev(ids_o), to_dev(w_o)
    desc = B.moe_size_class_init(H, I, bg, bd, 64)
    lay = pr.lay
    pt = B.moe_pass_table_host(ids_o, E)
    n_hit, n_pass = int(pt[0]), int(pt[1])
    starts = pt[2 + E:]
    x = dev_bf16(pr.x)
    full_desc = B.moe_size_class_init(H, I, bg, bd, pr.pool.shape[0])
    ref_gpu = B.moe_experts_forward(x, ids, w, E, to_dev(pr.table), to_dev(pr.pool.reshape(-1)), full_desc,
                                    path=B.MOE_PATH_MFMA)
    ew = err_word()
    ws = B.moe_prefill_sort(x, ids, E, desc, err_word=ew)
    rng = synth.rng_for(seed, 77)
    keep = []  # the pools must stay alive until the kernels ran
    for q in range(n_pass):
        hits = pt[2 + starts[q]:2 + starts[q + 1]]
        slots = rng.permutation(64)[:len(hits)]
        table = np.full(E, -1, np.int32)
        pool = np.zeros((64, lay.slot_bytes), np.uint8)
        for e, s in zip(hits, slots):
            table[e] = s
            pool[s] = pr.pool[pr.table[e]]
        tq, pq = to_dev(table), to_dev(pool.reshape(-1))
        keep.append((tq, pq))
        B.moe_prefill_pass(T, k, E, q, q + 1, tq, pq, desc, ws, err_word=ew)
    out = B.moe_prefill_combine(w, E, desc, ws)
    torch.cuda.synchronize()
    assert int(ew.item()) == 0
    assert n_hit > 0
    assert np.array_equal(bits16(out), bits16(ref_gpu))


def test_pass_of_absent_expert_sets_error_word():
    """Running a pass whose experts are not in the table flags NOT_RESIDENT."""
    T, H, E, I, k = 64, 128, 128, 64, 4
    pr = synth.make_problem(706, T, H, E, I, k, 4, 4, n_slots=E)
    ids_o, w_o = oracle.route(pr.logits, k)
    desc = B.moe_size_class_init(H, I, 4, 4, E)
    table = pr.table.copy()
    pt = B.moe_pass_table_host(ids_o, E)
    table[pt[2 + pt[2 + E + 1]]] = -1   # first expert of pass 1 absent
    ew = err_word()
    x = dev_bf16(pr.x)
    ws = B.moe_prefill_sort(x, to_dev(ids_o), E, desc, err_word=ew)
    B.moe_prefill_pass(T, k, E, 0, 1, to_dev(table), to_dev(pr.pool.reshape(-1)), desc, ws, err_word=ew)
    _torch().cuda.synchronize()
    assert int(ew.item()) == 0   # pass 0 does not read the absent expert
    B.moe_prefill_pass(T, k, E, 1, 2, to_dev(table), to_dev(pr.pool.reshape(-1)), desc, ws, err_word=ew)
    _torch().cuda.synchronize()
    assert int(ew.item()) == B.MOE_ERRW_NOT_RESIDENT


def test_prefill_argument_checks():
    torch = _torch()
    desc = B.moe_size_class_init(128, 64, 4, 4, 8)
    ws = torch.zeros(B.moe_forward_workspace_size(4, 2, 100, desc), dtype=torch.uint8, device="cuda")
    table = torch.zeros(100, dtype=torch.int32, device="cuda")
    pool = torch.zeros(8 * desc.slot_bytes, dtype=torch.uint8, device="cuda")
    for (p0, p1) in ((-1, 1), (0, 3), (2, 1)):   # passes are 0..1 for E = 100
        with pytest.raises(B.MoeError) as ei:
            B.moe_prefill_pass(4, 2, 100, p0, p1, table, pool, desc, ws)
        assert ei.value.code == B.MOE_E_INVALID
    small = torch.zeros(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.MoeError) as ei:
        B.moe_prefill_pass(4, 2, 100, 0, 1, table, pool, desc, small)
    assert ei.value.code == B.MOE_E_WORKSPACE
    B.moe_prefill_pass(4, 2, 100, 1, 1, table, pool, desc, ws)   # empty range: no-op


# --------------------------------------------------------------------------- #
# through the cache: fewer slots than hit experts                              #
# --------------------------------------------------------------------------- #
def _pipeline_layer(rows, lay, E, n_slots, x_bits, ids_o, w_o, host_tier):
    """One layer run by moe_pipeline_prefill through a one-layer cache of
    `n_slots` slots, the store holding `rows` (uint8 [E, slot_bytes] host)."""
    torch = _torch()
    desc = B.moe_size_class_init(lay.H, lay.I, lay.bits_gu, lay.bits_d, n_slots)
    pool = torch.zeros(n_slots * lay.slot_bytes, dtype=torch.uint8, device="cuda")
    cache = B.moe_cache_create([desc], [0], E)
    store = B.moe_store_open_memory(rows.reshape(-1), [desc], [0], E)
    copy = [torch.cuda.Stream(), torch.cuda.Stream()]
    p = B.moe_pipeline_create(cache, store, [pool], host_tier_bytes=rows.nbytes if host_tier else 0,
                              host_preload=host_tier, io_threads=4, staging_rows=8, copy_streams=copy)
    try:
        T, k = ids_o.shape
        table = torch.full((E,), -1, dtype=torch.int32, device="cuda")
        ew = err_word()
        out, n_pass = B.moe_pipeline_prefill(p, 0, ids_o, dev_bf16(x_bits), to_dev(ids_o), to_dev(w_o),
                                             table, desc, err_word=ew)
        B.moe_pipeline_drain(p)
        torch.cuda.synchronize()
        stats = B.moe_pipeline_stats_get(p, 0)
        cstats = B.moe_cache_class_stats(cache, 0)
        assert int(ew.item()) == 0
        return out, n_pass, stats, cstats
    finally:
        B.moe_pipeline_destroy(p)
        B.moe_store_close(store)
        B.moe_cache_destroy(cache)


@pytest.mark.parametrize("host_tier", [False, True])
def test_pipeline_prefill_fewer_slots_than_hit_experts(host_tier):
    """T 256, E 128, top-8 through a 64-slot class: two passes, each installed
    before it runs (the second evicts the first)."""
    T, H, E, I, k = 256, 512, 128, 256, 8
    pr = synth.make_problem(710, T, H, E, I, k, 4, 4, n_slots=E, gaussian=False)
    ids_o, w_o = oracle.route(pr.logits, k)
    rows = np.ascontiguousarray(np.stack([pr.pool[pr.table[e]] for e in range(E)]))
    canon = np.arange(E, dtype=np.int32)
    pt = B.moe_pass_table_host(ids_o, E)
    assert pt[0] == E and pt[1] == 2
    out, n_pass, st, cst = _pipeline_layer(rows, pr.lay, E, 64, pr.x, ids_o, w_o, host_tier)
    assert n_pass == 2
    assert st["requests"] == E and st["hits"] == 0
    assert cst == (0, E, E - 64)   # every hit expert installed once; pass 1 evicted pass 0
    if host_tier:
        assert st["host_hits"] == E and st["store_reads"] == 0
    else:
        assert st["store_reads"] == E
    ref = oracle.layer(pr.x, ids_o, w_o, canon, rows, H, I, 4, 4, E, threads=THREADS)
    check_close(out, ref, "pipeline prefill 64 slots")
    # the same bits as the all-resident one-launch forward
    desc = B.moe_size_class_init(H, I, 4, 4, E)
    full = B.moe_experts_forward(dev_bf16(pr.x), to_dev(ids_o), to_dev(w_o), E, to_dev(canon),
                                 to_dev(rows.reshape(-1)), desc, path=B.MOE_PATH_MFMA)
    assert np.array_equal(bits16(out), bits16(full))


def test_pipeline_prefill_chunk_full_size_128_slots():
    """The 1024-token chunk of the decode layer shape (H2048, E512, I512, top-10,
    3-bit) hits all 512 experts: 8 passes through a 128-slot class, every expert
    installed from the host tier just before its pass.  64 sampled tokens against
    the oracle; all tokens bit-identical to the all-resident forward."""
    torch = _torch()
    wl = synth.WORKLOADS["prefill"]
    lay = synth.Layout(wl.H, wl.I, wl.bits_gu, wl.bits_d)
    E, k, T = wl.E, wl.k, wl.T
    src = torch.zeros((E, lay.slot_bytes), dtype=torch.uint8, device="cuda")
    synth.fill_pool_device(src, lay, np.arange(E), wl.seed, 5)
    rows = src.cpu().numpy()
    lg = synth.gen_logits(synth.rng_for(wl.seed, 3, 5), T, E)
    x = synth.gen_x(synth.rng_for(wl.seed, 1, 5), T, wl.H)
    ids_o, w_o = oracle.route(lg, k)
    pt = B.moe_pass_table_host(ids_o, E)
    assert pt[0] == 512 and pt[1] == 8
    out, n_pass, st, cst = _pipeline_layer(rows, lay, E, 128, x, ids_o, w_o, True)
    assert n_pass == 8
    assert cst == (0, E, E - 128) and st["host_hits"] == E
    assert st["bytes_copied"] == E * lay.slot_bytes
    desc = B.moe_size_class_init(lay.H, lay.I, lay.bits_gu, lay.bits_d, E)
    full = B.moe_experts_forward(dev_bf16(x), to_dev(ids_o), to_dev(w_o), E,
                                 torch.arange(E, dtype=torch.int32, device="cuda"), src.view(-1), desc,
                                 path=B.MOE_PATH_MFMA)
    torch.cuda.synchronize()
    assert np.array_equal(bits16(out), bits16(full))
    tokens = sorted(synth.rng_for(wl.seed, 10).choice(T, 62, replace=False).tolist()) + [0, T - 1]
    tokens = sorted(set(tokens))
    ref = oracle.layer(x, ids_o, w_o, np.arange(E, dtype=np.int32), rows, lay.H, lay.I, lay.bits_gu,
                       lay.bits_d, E, tokens=np.asarray(tokens, np.int32), threads=THREADS)
    check_close(out[tokens], ref, "pipeline prefill chunk, 128 slots")
