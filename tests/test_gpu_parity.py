"""GPU parity: every C-ABI entry point against the CPU oracle on the same seeded
inputs.  Indices (routing ids, sort outputs) and routing weights must be
bit-exact; layer outputs must be within max-abs 2e-2 and rel-L2 1e-2 of the
oracle's fp64 result (bf16 output).

Shapes: small cases that span several tiles with ragged tails, and the full
workload shapes (one layer each), checked on all outputs or on sampled tokens
the oracle computes one by one.
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


def dev_bf16(x_bits):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda().view(torch.bfloat16)


def to_dev(a):
    return _torch().from_numpy(np.ascontiguousarray(a)).cuda()


def check_close(got_bf16, ref, what=""):
    got = got_bf16.float().cpu().numpy().astype(np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), what
    d = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert d.max() <= MAX_ABS and rel <= REL_L2, f"{what}: max-abs {d.max():.3e} rel-L2 {rel:.3e}"
    return d.max(), rel


def err_word():
    torch = _torch()
    return torch.zeros(1, dtype=torch.int32, device="cuda")


# --------------------------------------------------------------------------- #
# routing                                                                      #
# --------------------------------------------------------------------------- #
ROUTE_CASES = [
    # (T, E, k, zipf_s, seed)
    (16, 8, 2, 0.0, 0),          # tiny
    (1, 512, 10, 1.1, 2),        # decode step (Zipf-biased)
    (64, 512, 10, 1.1, 21),
    (1024, 512, 10, 0.0, 3),     # prefill chunk
    (1, 128, 8, 0.0, 4),         # mixed, batch 1
    (8, 128, 8, 0.0, 41),        # mixed, batch 8
    (32, 256, 8, 0.0, 5),        # int8 batch
    (37, 100, 7, 0.0, 6),        # E not a multiple of 64, ragged T
    (9, 1024, 32, 0.0, 7),       # maximum E and k
    (5, 1000, 1, 0.0, 8),        # k = 1
    (3, 3, 3, 0.0, 9),           # k = E
    (2, 1, 1, 0.0, 10),          # E = 1
]


@pytest.mark.parametrize("T,E,k,zipf,seed", ROUTE_CASES)
def test_route_plain_bit_exact(T, E, k, zipf, seed):
    rng = synth.rng_for(seed, 100)
    bias = synth.zipf_bias(synth.rng_for(seed, 101), E, zipf) if zipf else None
    lg = synth.gen_logits(rng, T, E, bias)
    ids, w = B.moe_route_topk(to_dev(lg), k)
    ids_o, w_o = oracle.route(lg, k)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), w_o.view(np.uint32))


@pytest.mark.parametrize("T,E,k,resident,L,seed", [
    (32, 256, 8, 64, 0.15, 5),    # int8 workload: 25% resident, L = 0.15
    (1, 512, 10, 128, 0.15, 2),
    (64, 128, 8, 32, 0.5, 11),
    (16, 8, 2, 3, 0.15, 12),
    (20, 256, 8, 0, 0.15, 13),    # nothing resident: same as plain
    (20, 256, 8, 256, 0.15, 14),  # everything resident: same as plain
    (20, 256, 8, 64, 0.0, 15),    # L = 0: same as plain
    (20, 256, 8, 64, 3.0, 16),    # large L: resident experts win
])
def test_route_substitution_bit_exact(T, E, k, resident, L, seed):
    lg = synth.gen_logits(synth.rng_for(seed, 102), T, E)
    table = synth.slot_table(synth.rng_for(seed, 103), E, E, resident=resident)
    ids, w = B.moe_route_topk(to_dev(lg), k, mode=B.MOE_ROUTE_SUBST, L=L, slot_table=to_dev(table))
    ids_o, w_o = oracle.route(lg, k, mode=1, L=L, slot_table=table)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), w_o.view(np.uint32))


def test_route_ties_and_underflow():
    # many equal logits and logits far below the max (exp underflows to 0)
    lg = np.zeros((6, 200), dtype=np.float32)
    lg[1, ::3] = 1.0
    lg[2, :] = -100.0
    lg[2, 17] = 0.0
    lg[3, :] = np.repeat(np.arange(50, dtype=np.float32), 4)
    lg[4, 150:] = -90.0
    lg[5] = synth.gen_logits(synth.rng_for(17), 1, 200)[0].round(1)
    for k in (1, 5, 32):
        ids, w = B.moe_route_topk(to_dev(lg), k)
        ids_o, w_o = oracle.route(lg, k)
        assert np.array_equal(ids.cpu().numpy(), ids_o)
        assert np.array_equal(w.cpu().numpy().view(np.uint32), w_o.view(np.uint32))


def test_route_nonfinite_sets_error_word():
    torch = _torch()
    lg = synth.gen_logits(synth.rng_for(18), 8, 64)
    lg[3, 5] = np.inf
    lg[6, 0] = np.nan
    ew = err_word()
    B.moe_route_topk(to_dev(lg), 4, err_word=ew)
    torch.cuda.synchronize()
    assert int(ew.item()) & B.MOE_ERRW_NONFINITE
    ew2 = err_word()
    B.moe_route_topk(to_dev(synth.gen_logits(synth.rng_for(19), 8, 64)), 4, err_word=ew2)
    torch.cuda.synchronize()
    assert int(ew2.item()) == 0


# --------------------------------------------------------------------------- #
# sort                                                                         #
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("T,E,k,P,kind", [
    (1, 512, 10, 64, "route"),       # decode
    (16, 8, 2, 64, "route"),         # tiny
    (8, 128, 8, 64, "route"),        # batch 8
    (32, 256, 8, 64, "route"),       # 256 pairs
    (128, 64, 8, 64, "route"),       # exactly 1024 pairs (single-block path)
    (129, 64, 8, 64, "route"),       # 1032 pairs (tile path, ragged last tile)
    (1024, 512, 10, 64, "route"),    # prefill chunk, 40 tiles
    (300, 1000, 7, 16, "route"),     # odd E, small passes
    (2048, 16, 2, 4, "skew"),        # every pair on 2 experts
    (1, 1, 1, 64, "route"),
])
def test_sort_bit_exact(T, E, k, P, kind):
    if kind == "route":
        lg = synth.gen_logits(synth.rng_for(T, E, 104), T, E)
        ids, _ = oracle.route(lg, k)
    else:
        ids = np.tile(np.array([[3, 11]], dtype=np.int32), (T, 1))
    off, sp, pt = B.moe_sort_by_expert(to_dev(ids), E, pass_experts=P)
    off_o, sp_o, pt_o = oracle.sort(ids, E, P)
    assert np.array_equal(off.cpu().numpy(), off_o)
    assert np.array_equal(sp.cpu().numpy(), sp_o)
    assert np.array_equal(pt.cpu().numpy(), pt_o)


def test_sort_flags_bad_ids():
    torch = _torch()
    ids = np.array([[0, 1], [2, 9], [-1, 3]], dtype=np.int32)
    ew = err_word()
    off, sp, pt = B.moe_sort_by_expert(to_dev(ids), 8, err_word=ew)
    torch.cuda.synchronize()
    assert int(ew.item()) & B.MOE_ERRW_BAD_ID
    # valid pairs are still sorted, the bad ones dropped
    o = off.cpu().numpy()
    assert o[-1] == 4 and sp.cpu().numpy()[:4].tolist() == [0, 1, 2, 5]


# --------------------------------------------------------------------------- #
# forward: small shapes, both kernel paths                                     #
# --------------------------------------------------------------------------- #
def run_forward(pr, ids, w, path, table=None, pool=None, n_slots=None):
    torch = _torch()
    lay = pr.lay
    pool_np = pr.pool if pool is None else pool
    table_np = pr.table if table is None else table
    desc = B.moe_size_class_init(lay.H, lay.I, lay.bits_gu, lay.bits_d,
                                 pool_np.shape[0] if n_slots is None else n_slots)
    ew = err_word()
    out = B.moe_experts_forward(dev_bf16(pr.x), to_dev(ids), to_dev(w), pr.E, to_dev(table_np),
                                to_dev(pool_np.reshape(-1)), desc, err_word=ew, path=path)
    torch.cuda.synchronize()
    return out, int(ew.item())


SMALL = [
    # (T, H, E, I, k, bits_gu, bits_d)
    (16, 256, 8, 128, 2, 4, 4),     # tiny workload
    (5, 128, 6, 64, 3, 3, 3),
    (7, 192, 5, 64, 2, 6, 3),
    (4, 64, 4, 128, 4, 8, 8),
    (3, 128, 3, 192, 1, 4, 6),
    (33, 256, 12, 128, 3, 3, 4),    # 2+ M-tiles for some experts, ragged
    (64, 128, 8, 64, 2, 8, 6),
    (1, 512, 16, 256, 4, 3, 3),
    (16, 256, 8, 128, 2, 16, 16),   # unquantized bf16 experts
    (5, 128, 6, 64, 3, 16, 4),      # bf16 gate/up, 4-bit down
    (33, 256, 12, 128, 3, 4, 16),   # 4-bit gate/up, bf16 down, 2+ M-tiles
]


@pytest.mark.parametrize("path", [B.MOE_PATH_GEMV, B.MOE_PATH_GEMV3, B.MOE_PATH_MFMA])
@pytest.mark.parametrize("shape", SMALL)
def test_forward_small(shape, path):
    T, H, E, I, k, bg, bd = shape
    pr = synth.make_problem(200 + T + H, T, H, E, I, k, bg, bd, n_slots=E + 5)
    ids, w = oracle.route(pr.logits, k)
    out, ew = run_forward(pr, ids, w, path)
    assert ew == 0
    ref = oracle.layer(pr.x, ids, w, pr.table, pr.pool, H, I, bg, bd, E, threads=THREADS)
    check_close(out, ref, f"{shape} path {path}")


@pytest.mark.parametrize("bits", [4, 3])
def test_forward_many_rows_per_expert_mfma(bits):
    """One expert takes 150 rows: several K sweeps of 4 M-tiles plus a ragged tile
    (width 3 runs the kernel that loads its stages straight into LDS)."""
    T, H, E, I, k = 150, 128, 4, 64, 2
    pr = synth.make_problem(301, T, H, E, I, k, bits, bits)
    ids = np.stack([np.array([1, (t % 3) + (t % 3 >= 1)], dtype=np.int32) for t in range(T)])
    w = np.full((T, k), 0.5, dtype=np.float32)
    out, ew = run_forward(pr, ids, w, B.MOE_PATH_MFMA)
    assert ew == 0
    ref = oracle.layer(pr.x, ids, w, pr.table, pr.pool, H, I, bits, bits, E, threads=THREADS)
    check_close(out, ref, f"skewed {bits}-bit")


@pytest.mark.parametrize("shape", [
    # (T, H, E, I, k): K = 320 and 448 end in a half stage of 64 inputs after an
    # odd / even number of full stages; the two LDS buffers alternate through it
    (9, 320, 6, 448, 2),
    (5, 192, 4, 320, 3),
    (40, 448, 3, 64, 2),
])
def test_forward_mfma_width3_k_tails(shape):
    T, H, E, I, k = shape
    pr = synth.make_problem(900 + T + H, T, H, E, I, k, 3, 3, n_slots=E + 1)
    ids, w = oracle.route(pr.logits, k)
    out, ew = run_forward(pr, ids, w, B.MOE_PATH_MFMA)
    assert ew == 0
    ref = oracle.layer(pr.x, ids, w, pr.table, pr.pool, H, I, 3, 3, E, threads=THREADS)
    check_close(out, ref, f"{shape} width 3")


@pytest.mark.parametrize("bits", [(3, 3), (4, 6), (8, 8)])
def test_forward_mfma_one_tile_sweeps(bits):
    """Small batches over many experts (at most two pairs per expert on average)
    run the MFMA kernels in sweeps of 16 rows: one expert given 40 of the 96
    pairs takes three sweeps (16, 16, 8), the others one each."""
    T, H, E, I, k = 48, 256, 96, 128, 2
    bg, bd = bits
    pr = synth.make_problem(950 + bg + bd, T, H, E, I, k, bg, bd, n_slots=E + 3)
    ids = np.empty((T, k), np.int32)
    ids[:, 0] = np.where(np.arange(T) < 40, 0, 1 + np.arange(T) % (E - 1))
    ids[:, 1] = 1 + (np.arange(T) * 7) % (E - 1)
    ids[:, 1] = np.where(ids[:, 1] == ids[:, 0], 1 + (ids[:, 1] % (E - 1)), ids[:, 1])
    assert all(len(set(r)) == k for r in ids.tolist())
    w = np.tile(np.array([0.625, 0.375], np.float32), (T, 1))
    out, ew = run_forward(pr, ids, w, B.MOE_PATH_MFMA)
    assert ew == 0
    ref = oracle.layer(pr.x, ids, w, pr.table, pr.pool, H, I, bg, bd, E, threads=THREADS)
    check_close(out, ref, f"one-tile sweeps {bits}")


@pytest.mark.parametrize("path", [B.MOE_PATH_GEMV, B.MOE_PATH_GEMV3, B.MOE_PATH_MFMA])
def test_forward_deterministic_and_placement_free(path):
    pr = synth.tiny_problem()
    ids, w = oracle.route(pr.logits, pr.k)
    a, _ = run_forward(pr, ids, w, path)
    b, _ = run_forward(pr, ids, w, path)
    assert np.array_equal(a.view(_torch().int16).cpu().numpy(), b.view(_torch().int16).cpu().numpy())
    # a permuted slot table with the rows moved gives bit-identical output
    perm = synth.rng_for(51).permutation(pr.pool.shape[0] + 5)
    pool2 = np.zeros((pr.pool.shape[0] + 5, pr.pool.shape[1]), np.uint8)
    table2 = np.empty_like(pr.table)
    for e in range(pr.E):
        table2[e] = perm[pr.table[e]]
        pool2[table2[e]] = pr.pool[pr.table[e]]
    c, _ = run_forward(pr, ids, w, path, table=table2, pool=pool2)
    assert np.array_equal(a.view(_torch().int16).cpu().numpy(), c.view(_torch().int16).cpu().numpy())


def test_forward_paths_agree():
    pr = synth.make_problem(7, 8, 256, 16, 128, 4, 3, 3)
    ids, w = oracle.route(pr.logits, 4)
    a, _ = run_forward(pr, ids, w, B.MOE_PATH_GEMV)
    b, _ = run_forward(pr, ids, w, B.MOE_PATH_MFMA)
    d = np.abs(a.float().cpu().numpy() - b.float().cpu().numpy())
    assert d.max() < 1e-2


def test_forward_error_words():
    pr = synth.tiny_problem()
    ids, w = oracle.route(pr.logits, pr.k)
    for path in (B.MOE_PATH_GEMV, B.MOE_PATH_GEMV3, B.MOE_PATH_MFMA):
        table = pr.table.copy()
        table[ids[0, 0]] = -1
        _, ew = run_forward(pr, ids, w, path, table=table)
        assert ew & B.MOE_ERRW_NOT_RESIDENT
        table = pr.table.copy()
        table[ids[0, 0]] = 8  # == n_slots
        _, ew = run_forward(pr, ids, w, path, table=table)
        assert ew & B.MOE_ERRW_BAD_SLOT
        bad = ids.copy()
        bad[2, 1] = 99
        _, ew = run_forward(pr, bad, w, path)
        assert ew & B.MOE_ERRW_BAD_ID


# --------------------------------------------------------------------------- #
# forward: full workload shapes (one layer each)                               #
# --------------------------------------------------------------------------- #
def device_pool(lay, n_slots, slots, seed, layer):
    torch = _torch()
    pool = torch.zeros((n_slots, lay.slot_bytes), dtype=torch.uint8, device="cuda")
    synth.fill_pool_device(pool, lay, slots, seed, layer)
    return pool


def host_rows(pool, slots):
    torch = _torch()
    idx = torch.as_tensor(np.asarray(slots, dtype=np.int64), device=pool.device)
    return pool.index_select(0, idx).cpu().numpy()


def forward_dev(x, ids, w, E, table, pool, lay, path=B.MOE_PATH_AUTO):
    torch = _torch()
    desc = B.moe_size_class_init(lay.H, lay.I, lay.bits_gu, lay.bits_d, pool.shape[0])
    ew = err_word()
    out = B.moe_experts_forward(x, ids, w, E, table, pool.view(-1), desc, err_word=ew, path=path)
    torch.cuda.synchronize()
    return out, int(ew.item())


def oracle_on_rows(x_bits, ids, w, table, pool, lay, E, tokens):
    """Oracle with only the routed experts' rows copied to the host."""
    used = sorted(set(ids[tokens].reshape(-1).tolist()))
    rows = host_rows(pool, [int(table[e]) for e in used])
    t2 = np.full(E, -1, np.int32)
    for i, e in enumerate(used):
        t2[e] = i
    return oracle.layer(x_bits, ids, w, t2, rows, lay.H, lay.I, lay.bits_gu, lay.bits_d, E,
                        tokens=np.asarray(tokens, np.int32), threads=THREADS)


@pytest.mark.parametrize("layer", [0, 31])
def test_forward_decode_layer_full_size(layer):
    """48 x (H2048, E512, I512, top-10), 3-bit, batch 1, 2048-slot pool with a
    random slot table; one layer checked on every output."""
    wl = synth.WORKLOADS["decode"]
    lay = synth.Layout(wl.H, wl.I, wl.bits_gu, wl.bits_d)
    table = synth.slot_table(synth.rng_for(wl.seed, 4, layer), wl.E, wl.slots_per_layer)
    pool = device_pool(lay, wl.slots_per_layer, table, wl.seed, layer)
    bias = synth.zipf_bias(synth.rng_for(wl.seed, 2, layer), wl.E, wl.zipf_s)
    lg = synth.gen_logits(synth.rng_for(wl.seed, 3, layer), 1, wl.E, bias)
    x = synth.gen_x(synth.rng_for(wl.seed, 1, layer), 1, wl.H)
    ids, w = B.moe_route_topk(to_dev(lg), wl.k)
    ids_o, w_o = oracle.route(lg, wl.k)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    ref = oracle_on_rows(x, ids_o, w_o, table, pool, lay, wl.E, [0])
    for path in (B.MOE_PATH_AUTO, B.MOE_PATH_GEMV3, B.MOE_PATH_MFMA):
        out, ew = forward_dev(dev_bf16(x), ids, w, wl.E, to_dev(table), pool, lay, path)
        assert ew == 0
        check_close(out, ref, f"decode layer {layer} path {path}")
    # router + experts in one launch
    desc = B.moe_size_class_init(lay.H, lay.I, lay.bits_gu, lay.bits_d, pool.shape[0])
    ew = err_word()
    out, ids2, w2 = B.moe_layer_forward(to_dev(lg), dev_bf16(x), to_dev(table), pool.view(-1), desc,
                                        wl.k, err_word=ew)
    _torch().cuda.synchronize()
    assert int(ew.item()) == 0
    assert np.array_equal(ids2.cpu().numpy(), ids_o)
    assert np.array_equal(w2.cpu().numpy().view(np.uint32), w_o.view(np.uint32))
    check_close(out, ref, f"decode layer {layer} moe_layer_forward")


def test_forward_prefill_chunk_full_size():
    """1024-token chunk, same layer shape, all 512 experts resident; every output
    checked for 64 sampled tokens (the first and last among them), plus
    properties of all rows."""
    torch = _torch()
    wl = synth.WORKLOADS["prefill"]
    lay = synth.Layout(wl.H, wl.I, wl.bits_gu, wl.bits_d)
    table = synth.slot_table(synth.rng_for(wl.seed, 4), wl.E, wl.E)
    pool = device_pool(lay, wl.E, np.arange(wl.E), wl.seed, 0)
    lg = synth.gen_logits(synth.rng_for(wl.seed, 3), wl.T, wl.E)
    x = synth.gen_x(synth.rng_for(wl.seed, 1), wl.T, wl.H)
    ids, w = B.moe_route_topk(to_dev(lg), wl.k)
    ids_o, w_o = oracle.route(lg, wl.k)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    off, sp, pt = B.moe_sort_by_expert(ids, wl.E)
    off_o, sp_o, pt_o = oracle.sort(ids_o, wl.E, 64)
    assert np.array_equal(sp.cpu().numpy(), sp_o) and np.array_equal(pt.cpu().numpy(), pt_o)
    assert pt_o[0] == 512 and pt_o[1] == 8
    out, ew = forward_dev(dev_bf16(x), ids, w, wl.E, to_dev(table), pool, lay)
    assert ew == 0
    o = out.float()
    assert bool(torch.isfinite(o).all())
    mid = synth.rng_for(wl.seed, 9).choice(np.arange(1, wl.T - 1), 62, replace=False)
    tokens = [0] + sorted(mid.tolist()) + [wl.T - 1]
    ref = oracle_on_rows(x, ids_o, w_o, table, pool, lay, wl.E, tokens)
    check_close(out[tokens], ref, "prefill sampled tokens")


@pytest.mark.parametrize("T", [1, 1024])
def test_forward_bf16_experts_full_size(T):
    """Unquantized bf16 experts of the decode shape (H2048, E512, I512, top-10):
    the fused decode kernel at batch 1 (AUTO), the three-launch GEMV and the MFMA
    paths too; the MFMA path for a 1024-token chunk (sampled tokens)."""
    torch = _torch()
    H, E, I, k = 2048, 512, 512, 10
    lay = synth.Layout(H, I, 16, 16)
    assert lay.slot_bytes == 6291456
    table = synth.slot_table(synth.rng_for(6, 4, T), E, E)
    pool = device_pool(lay, E, table, 6, T)
    lg = synth.gen_logits(synth.rng_for(6, 3, T), T, E)
    x = synth.gen_x(synth.rng_for(6, 1, T), T, H)
    ids, w = B.moe_route_topk(to_dev(lg), k)
    ids_o, w_o = oracle.route(lg, k)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    tokens = [0] if T == 1 else sorted(synth.rng_for(6, 9).choice(T, 10, replace=False).tolist()) + [T - 1]
    ref = oracle_on_rows(x, ids_o, w_o, table, pool, lay, E, tokens)
    paths = (B.MOE_PATH_AUTO, B.MOE_PATH_GEMV3, B.MOE_PATH_MFMA) if T == 1 else (B.MOE_PATH_AUTO,)
    for path in paths:
        out, ew = forward_dev(dev_bf16(x), ids, w, E, to_dev(table), pool, lay, path)
        assert ew == 0
        assert bool(torch.isfinite(out.float()).all())
        check_close(out[tokens], ref, f"bf16 experts T {T} path {path}")
    if T == 1:  # router + experts entry point: the fused decode kernel routes too
        desc = B.moe_size_class_init(H, I, 16, 16, pool.shape[0])
        ew = err_word()
        out, _, _ = B.moe_layer_forward(to_dev(lg), dev_bf16(x), to_dev(table), pool.view(-1), desc, k,
                                        err_word=ew)
        torch.cuda.synchronize()
        assert int(ew.item()) == 0
        check_close(out, ref, "bf16 experts moe_layer_forward")


@pytest.mark.parametrize("T", [1, 8])
@pytest.mark.parametrize("layer", [2, 3])   # layer 3 is a 6-bit-down (class B) layer
def test_forward_mixed_classes_full_size(T, layer):
    wl = synth.WORKLOADS["mixed"]
    bg, bd = synth.layer_bits(wl, layer)
    lay = synth.Layout(wl.H, wl.I, bg, bd)
    assert lay.slot_bytes == (3047424 if layer == 3 else 2654208)
    table = synth.slot_table(synth.rng_for(wl.seed, 4, layer), wl.E, wl.slots_per_layer)
    pool = device_pool(lay, wl.slots_per_layer, table, wl.seed, layer)
    lg = synth.gen_logits(synth.rng_for(wl.seed, 3, layer, T), T, wl.E)
    x = synth.gen_x(synth.rng_for(wl.seed, 1, layer, T), T, wl.H)
    ids, w = B.moe_route_topk(to_dev(lg), wl.k)
    ids_o, w_o = oracle.route(lg, wl.k)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    tokens = list(range(T))
    ref = oracle_on_rows(x, ids_o, w_o, table, pool, lay, wl.E, tokens)
    for path in (B.MOE_PATH_AUTO, B.MOE_PATH_GEMV3, B.MOE_PATH_MFMA):
        out, ew = forward_dev(dev_bf16(x), ids, w, wl.E, to_dev(table), pool, lay, path)
        assert ew == 0
        check_close(out, ref, f"mixed layer {layer} T {T} path {path}")
    # router + experts in one launch (one token: the one-token kernel routes itself)
    desc = B.moe_size_class_init(lay.H, lay.I, bg, bd, wl.slots_per_layer)
    ew = err_word()
    out, ids_l, w_l = B.moe_layer_forward(to_dev(lg), dev_bf16(x), to_dev(table), pool.view(-1), desc, wl.k,
                                          err_word=ew)
    _torch().cuda.synchronize()
    assert int(ew.item()) == 0
    assert np.array_equal(ids_l.cpu().numpy(), ids_o)
    assert np.array_equal(w_l.cpu().numpy().view(np.uint32), w_o.view(np.uint32))
    check_close(out, ref, f"mixed layer {layer} T {T} moe_layer_forward")


def test_int8_substitution_with_installs_full_size():
    """8-bit experts (H4096, E256, I1024, top-8), batch 32, 64 of 256 experts
    resident, cache-aware substitution at L = 0.15; misses are installed from
    pinned host rows through the host cache before the forward."""
    torch = _torch()
    wl = synth.WORKLOADS["int8sub"]
    lay = synth.Layout(wl.H, wl.I, wl.bits_gu, wl.bits_d)
    E, k, T = wl.E, wl.k, wl.T
    n_slots = 192
    # host tier: every expert's row in pinned memory (random codes, recipe of
    # random_code_expert), generated on the device and copied once
    src_pool = device_pool(lay, E, np.arange(E), wl.seed, 0)
    host = torch.empty((E, lay.slot_bytes), dtype=torch.uint8, pin_memory=True)
    host.copy_(src_pool)
    del src_pool
    desc = B.moe_size_class_init(lay.H, lay.I, lay.bits_gu, lay.bits_d, n_slots)
    cache = B.moe_cache_create([desc], [0], E)
    pool = torch.zeros((n_slots, lay.slot_bytes), dtype=torch.uint8, device="cuda")
    try:
        resident = synth.rng_for(wl.seed, 6).choice(E, wl.resident, replace=False)
        for e in resident:
            _, slot, nf = B.moe_cache_acquire(cache, 0, int(e))
            assert nf == 1
            B.moe_cache_install(pool.view(-1), desc, slot, host[int(e)])
            B.moe_cache_fill_done(cache, 0, int(e), None)
        torch.cuda.synchronize()
        table0 = B.moe_cache_table(cache, 0, E)
        assert (table0 >= 0).sum() == wl.resident
        lg = synth.gen_logits(synth.rng_for(wl.seed, 3), T, E)
        ids, w = B.moe_route_topk(to_dev(lg), k, mode=B.MOE_ROUTE_SUBST, L=wl.subst_L,
                                  slot_table=to_dev(table0))
        ids_o, w_o = oracle.route(lg, k, mode=1, L=wl.subst_L, slot_table=table0)
        assert np.array_equal(ids.cpu().numpy(), ids_o)
        assert np.array_equal(w.cpu().numpy().view(np.uint32), w_o.view(np.uint32))
        plain_ids, _ = oracle.route(lg, k)
        # substitution lands more picks on resident experts than plain routing
        assert np.isin(ids_o, resident).sum() > np.isin(plain_ids, resident).sum()
        # miss path: install every routed expert that is not resident
        copy = torch.cuda.Stream()
        events = []
        for e in sorted(set(ids_o.reshape(-1).tolist())):
            rc, slot, nf = B.moe_cache_acquire(cache, 0, e)
            assert rc == B.MOE_OK
            if nf:
                ev = torch.cuda.Event()
                B.moe_cache_install(pool.view(-1), desc, slot, host[e], stream=copy, event=ev)
                B.moe_cache_fill_done(cache, 0, e, ev)
                events.append(ev)
        for ev in events:
            torch.cuda.current_stream().wait_event(ev)
        table1 = B.moe_cache_table(cache, 0, E)
        assert np.all(table1[ids_o.reshape(-1)] >= 0)
        x = synth.gen_x(synth.rng_for(wl.seed, 1), T, wl.H)
        # oracle: canonical placement (expert e in row e of the host tier)
        tokens = list(range(T))  # every token of the batch
        ref = oracle.layer(x, ids_o, w_o, np.arange(E, dtype=np.int32), host.numpy(), lay.H,
                           lay.I, 8, 8, E, tokens=np.asarray(tokens, np.int32), threads=THREADS)
        for path in (B.MOE_PATH_AUTO, B.MOE_PATH_GEMV):
            ew = err_word()
            out = B.moe_experts_forward(dev_bf16(x), ids, w, E, to_dev(table1), pool.view(-1), desc,
                                        err_word=ew, path=path)
            torch.cuda.synchronize()
            assert int(ew.item()) == 0
            assert B.moe_cache_poll(cache) == 0
            check_close(out[tokens], ref, f"int8 subst path {path}")
    finally:
        B.moe_cache_destroy(cache)


# --------------------------------------------------------------------------- #
# router + experts in one launch                                               #
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("shape", [
    (1, 256, 8, 128, 2, 4, 4, 0),
    (8, 128, 16, 64, 8, 4, 6, 1),     # 64 pairs: the largest fused batch
    (3, 512, 16, 256, 4, 3, 3, 1),
    (2, 256, 10, 64, 5, 8, 8, 0),
    (9, 128, 16, 64, 8, 3, 3, 0),     # 72 pairs: falls back to two calls
    (2, 128, 640, 64, 6, 4, 4, 1),    # E > 512: router kernel, then the fused experts
    (1, 128, 1024, 64, 32, 3, 3, 0),  # maximum E and k
])
def test_layer_forward_matches_route_plus_forward(shape):
    torch = _torch()
    T, H, E, I, k, bg, bd, subst = shape
    pr = synth.make_problem(400 + T + H, T, H, E, I, k, bg, bd, n_slots=E + 2,
                            resident=None)
    mode = B.MOE_ROUTE_SUBST if subst else B.MOE_ROUTE_PLAIN
    ids_o, w_o = oracle.route(pr.logits, k, mode=mode, L=0.15, slot_table=pr.table)
    desc = B.moe_size_class_init(H, I, bg, bd, pr.pool.shape[0])
    ew = err_word()
    out, ids, w = B.moe_layer_forward(to_dev(pr.logits), dev_bf16(pr.x), to_dev(pr.table),
                                      to_dev(pr.pool.reshape(-1)), desc, k, mode=mode, L=0.15,
                                      err_word=ew)
    torch.cuda.synchronize()
    assert int(ew.item()) == 0
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), w_o.view(np.uint32))
    ref = oracle.layer(pr.x, ids_o, w_o, pr.table, pr.pool, H, I, bg, bd, E, threads=THREADS)
    check_close(out, ref, f"layer_forward {shape}")
    # identical to the two-call form (route, then the experts on the AUTO path)
    out2, _ = run_forward(pr, ids_o, w_o, B.MOE_PATH_AUTO)
    assert np.array_equal(out.view(torch.int16).cpu().numpy(), out2.view(torch.int16).cpu().numpy())


@pytest.mark.parametrize("T,E,k,mode,kind,seed", [
    (1, 512, 10, 0, "normal", 601),
    (1, 512, 10, 1, "zipf", 602),
    (2, 512, 32, 0, "normal", 603),
    (3, 512, 1, 1, "normal", 604),
    (1, 100, 8, 0, "normal", 605),    # last wave partly filled
    (2, 64, 5, 1, "normal", 606),     # a single full wave
    (1, 128, 8, 0, "ties", 607),      # coarse logits: many equal keys
    (1, 512, 10, 0, "ties", 608),     # ... more than 64 candidates
    (3, 300, 16, 1, "ties", 609),
])
def test_layer_forward_workgroup_routing(T, E, k, mode, kind, seed):
    """For T <= 3 and E >= 64 the fused kernel routes each token with all of a
    workgroup's waves; ids and weights must equal the oracle's bit for bit,
    including ties (lower id first) and the more-than-64-candidates case."""
    torch = _torch()
    H, I = 128, 64
    pr = synth.make_problem(seed, T, H, E, I, k, 4, 4, n_slots=E + 3,
                            resident=(E // 2 if mode else None), gaussian=False,
                            zipf_s=(1.1 if kind == "zipf" else 0.0))
    lg = pr.logits
    if kind == "ties":
        lg = (np.round(lg * 2.0) / 2.0).astype(np.float32)
    desc = B.moe_size_class_init(H, I, 4, 4, pr.pool.shape[0])
    ew = err_word()
    out, ids, w = B.moe_layer_forward(to_dev(lg), dev_bf16(pr.x), to_dev(pr.table),
                                      to_dev(pr.pool.reshape(-1)), desc, k, mode=mode, L=0.15,
                                      err_word=ew)
    torch.cuda.synchronize()
    ids_o, w_o = oracle.route(lg, k, mode=mode, L=0.15, slot_table=pr.table)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), w_o.view(np.uint32))
    hit_missing = bool((pr.table[ids_o.reshape(-1)] < 0).any())
    assert int(ew.item()) == (B.MOE_ERRW_NOT_RESIDENT if hit_missing else 0)
    if not hit_missing:
        ref = oracle.layer(pr.x, ids_o, w_o, pr.table, pr.pool, H, I, 4, 4, E, threads=THREADS)
        check_close(out, ref, f"wg routing {T} {E} {k}")


def _boundary_rows(E, k, seed):
    """Logit rows that drive the plain-mode routing by logit order through each of
    its branches: a clear gap after the k-th largest logit (taken by logit order),
    the (k+1)-th one ulp below or equal to the k-th (near-tie: routed by key
    instead), chosen logits one ulp apart with the larger one on the larger id (p
    may round equal, then the smaller id goes first), the k-th far below the max
    (p underflows: routed by key), large magnitudes, and coarse values (ties)."""
    rng = synth.rng_for(seed, 700)
    rows = []
    base = synth.gen_logits(rng, 1, E)[0]
    rows.append(base.copy())
    order = np.argsort(-base, kind="stable")
    kk = min(k, E - 1)
    r = base.copy()
    r[order[kk]] = np.nextafter(r[order[kk - 1]], np.float32(-np.inf))
    rows.append(r)
    r = base.copy()
    r[order[kk]] = r[order[kk - 1]]
    rows.append(r)
    r = base.copy()
    hi = np.sort(rng.choice(E, size=min(2 * kk, E), replace=False))
    for a, b in zip(hi[0::2], hi[1::2]):  # b > a: the larger logit on the larger id
        r[a] = np.float32(3.0)
        r[b] = np.nextafter(np.float32(3.0), np.float32(np.inf))
    rows.append(r)
    r = np.full(E, -80.0, np.float32) + rng.standard_normal(E).astype(np.float32)
    r[rng.integers(E)] = 0.0
    rows.append(r)
    rows.append((base * 3000.0).astype(np.float32))
    rows.append((np.round(base * 2.0) / 2.0).astype(np.float32))
    r = base.copy()
    r[order[:kk]] += np.float32(1.0)
    r[order[kk]] = r[order[kk - 1]] - np.float32(2.0 ** -9)  # just at the gap bound
    rows.append(r.astype(np.float32))
    return np.stack(rows).astype(np.float32)


@pytest.mark.parametrize("E,k", [(512, 10), (512, 15), (512, 16), (512, 1), (320, 8), (100, 7), (64, 15)])
def test_layer_forward_logit_order_routing(E, k):
    """Plain-mode routing inside the fused kernel (T <= 3, 64 <= E <= 512, k <= 15
    by logit order; k = 16 by key): ids and weights equal the oracle's bit for bit
    on rows built to reach every branch, one, two and three tokens per call."""
    torch = _torch()
    H, I = 128, 64
    rows = _boundary_rows(E, k, 710 + E + k)
    pr = synth.make_problem(711, 3, H, E, I, k, 4, 4, n_slots=E, gaussian=False)
    desc = B.moe_size_class_init(H, I, 4, 4, E)
    x, table, pool = dev_bf16(pr.x), to_dev(pr.table), to_dev(pr.pool.reshape(-1))
    for T in (1, 2, 3):
        for i in range(0, rows.shape[0], T):
            lg = rows[i:i + T]
            if lg.shape[0] < T:
                lg = np.concatenate([lg, rows[:T - lg.shape[0]]])
            ew = err_word()
            _, ids, w = B.moe_layer_forward(to_dev(lg), x[:T], table, pool, desc, k, err_word=ew)
            torch.cuda.synchronize()
            ids_o, w_o = oracle.route(lg, k)
            assert np.array_equal(ids.cpu().numpy(), ids_o), (T, i)
            assert np.array_equal(w.cpu().numpy().view(np.uint32), w_o.view(np.uint32)), (T, i)
            assert int(ew.item()) == 0


def test_layer_forward_routing_nonfinite():
    """A non-finite logit in the fused kernel's routing: error bit set, that
    token's ids 0..k-1 with weight 0 (as the router kernel), the other tokens
    routed as usual."""
    torch = _torch()
    H, I, E, k = 128, 64, 512, 10
    pr = synth.make_problem(712, 3, H, E, I, k, 4, 4, n_slots=E, gaussian=False)
    desc = B.moe_size_class_init(H, I, 4, 4, E)
    for bad in (np.nan, np.inf, -np.inf):
        lg = pr.logits.copy()
        lg[1, 333] = bad
        ew = err_word()
        _, ids, w = B.moe_layer_forward(to_dev(lg), dev_bf16(pr.x), to_dev(pr.table),
                                        to_dev(pr.pool.reshape(-1)), desc, k, err_word=ew)
        torch.cuda.synchronize()
        assert int(ew.item()) & B.MOE_ERRW_NONFINITE
        ids, w = ids.cpu().numpy(), w.cpu().numpy()
        assert np.array_equal(ids[1], np.arange(k)) and not w[1].any()
        ids_o, w_o = oracle.route(lg[[0, 2]], k)
        assert np.array_equal(ids[[0, 2]], ids_o)
        assert np.array_equal(w[[0, 2]].view(np.uint32), w_o.view(np.uint32))


def test_fused_decode_repeated_calls_and_graph_replay():
    """The fused kernel's h exchange lives in the workspace's reserved prefix:
    1024 call-tag counters (dwords 64..1087, all equal to the number of fused
    calls made on the workspace) and the tagged h words after them.  Many calls
    on one workspace, eager and replayed from a HIP graph, give the same bits,
    never time out, and keep every counter equal."""
    torch = _torch()
    pr = synth.make_problem(77, 4, 256, 16, 128, 4, 3, 3)
    desc = B.moe_size_class_init(256, 128, 3, 3, pr.pool.shape[0])
    lg, x = to_dev(pr.logits), dev_bf16(pr.x)
    table, pool = to_dev(pr.table), to_dev(pr.pool.reshape(-1))
    ws = torch.zeros(B.moe_forward_workspace_size(4, 4, 16, desc), dtype=torch.uint8, device="cuda")
    ew = err_word()
    outs = []
    for _ in range(30):
        out, _, _ = B.moe_layer_forward(lg, x, table, pool, desc, 4, ws=ws, err_word=ew)
        outs.append(out.view(torch.int16).clone())
    torch.cuda.synchronize()
    assert int(ew.item()) == 0
    assert all(torch.equal(outs[0], o) for o in outs)
    gen = ws[:8192].view(torch.int32)
    assert int(gen[:64].count_nonzero().item()) == 0
    assert bool((gen[64:64 + 1024] == 30).all())
    assert int(gen[64 + 1024:].count_nonzero().item()) == 0
    # every tagged word written carries a tag of one of the calls (1..30)
    xw = ws[8192:8192 + 8 * 32768].view(torch.int64).cpu().numpy()
    tags = (xw >> 32) & 0xFFFFFFFF
    assert tags.max() <= 30 and int((tags == 30).sum()) > 0
    out_g = torch.empty_like(out)
    ids_g = torch.empty((4, 4), dtype=torch.int32, device="cuda")
    w_g = torch.empty((4, 4), dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(3):
                B.moe_layer_forward(lg, x, table, pool, desc, 4, topk_ids=ids_g, topk_w=w_g, out=out_g,
                                    ws=ws, err_word=ew)
    torch.cuda.current_stream().wait_stream(s)
    for r in range(5):
        out_g.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), outs[0]), f"replay {r}"
        # eager work between replays
        B.moe_layer_forward(lg, x, table, pool, desc, 4, ws=ws, err_word=ew)
        torch.cuda.synchronize()
    assert int(ew.item()) == 0
    gen = ws[:8192].view(torch.int32)
    assert bool((gen[64:64 + 1024] == 30 + 5 * 3 + 5).all())
