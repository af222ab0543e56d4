"""moe_layer_forward_static: the layer forward on the library's own scratch (no
workspace argument, nothing allocated), called through the C-ABI and checked
bit for bit against moe_layer_forward with a caller workspace, on consecutive
calls that shrink, and against the oracle within the layer tolerance."""
import os

import numpy as np
import pytest

import oracle
from quantized_routed_expert_softmax_amd import binding as B
from quantized_routed_expert_softmax_amd import synth

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def _torch():
    import torch
    return torch


def to_dev(a):
    return _torch().from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(x_bits):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda().view(torch.bfloat16)


def _layer(T, H, E, I, k, bg, bd, seed, n_slots):
    torch = _torch()
    lay = synth.Layout(H, I, bg, bd)
    table = synth.slot_table(synth.rng_for(seed, 4), E, n_slots)
    pool = torch.zeros((n_slots, lay.slot_bytes), dtype=torch.uint8, device="cuda")
    synth.fill_pool_device(pool, lay, table, seed, 0)
    desc = B.moe_size_class_init(H, I, bg, bd, n_slots)
    return lay, table, pool, desc


def _both(lg, x, table, pool, desc, k, mode=B.MOE_ROUTE_PLAIN, L=0.0):
    """(static result, workspace result), each (out, ids, w, err)."""
    torch = _torch()
    res = []
    for fn in (B.moe_layer_forward_static, B.moe_layer_forward):
        ew = torch.zeros(1, dtype=torch.int32, device="cuda")
        out, ids, w = fn(to_dev(lg), dev_bf16(x), to_dev(table), pool.view(-1), desc, k, mode=mode, L=L,
                         err_word=ew)
        torch.cuda.synchronize()
        res.append((out.view(torch.int16).cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy(), int(ew.item())))
    return res


def _same(a, b):
    for u, v in zip(a, b):
        assert np.array_equal(np.asarray(u), np.asarray(v))


def test_static_matches_workspace_entry_point_two_calls_shrinking():
    """Decode layer shape (H2048, E512, I512, top-10, 3-bit, 2048-slot pool):
    four tokens, then one token, then four again, on the same scratch."""
    H, E, I, k = 2048, 512, 512, 10
    lay, table, pool, desc = _layer(4, H, E, I, k, 3, 3, 31, 2048)
    for T, seed in ((4, 1), (1, 2), (4, 3)):
        bias = synth.zipf_bias(synth.rng_for(seed, 2), E, 1.1)
        lg = synth.gen_logits(synth.rng_for(seed, 3), T, E, bias)
        x = synth.gen_x(synth.rng_for(seed, 1), T, H)
        st, ref = _both(lg, x, table, pool, desc, k)
        assert st[3] == 0 and ref[3] == 0
        _same(st, ref)
        ids_o, w_o = oracle.route(lg, k)
        assert np.array_equal(st[1], ids_o)
        assert np.array_equal(st[2].view(np.uint32), w_o.view(np.uint32))
        if T == 1:   # the layer output against the oracle on the routed rows
            used = sorted(set(ids_o.reshape(-1).tolist()))
            rows = pool.index_select(0, to_dev(np.asarray([table[e] for e in used], np.int64))).cpu().numpy()
            t2 = np.full(E, -1, np.int32)
            t2[used] = np.arange(len(used), dtype=np.int32)
            ref_o = oracle.layer(x, ids_o, w_o, t2, rows, H, I, 3, 3, E, threads=THREADS)
            got = st[0].view(np.uint16).astype(np.uint32) << 16
            got = got.view(np.float32).astype(np.float64)
            d = np.abs(got - ref_o)
            rel = np.linalg.norm(got - ref_o) / np.linalg.norm(ref_o)
            assert d.max() <= 2e-2 and rel <= 1e-2


def test_static_larger_batches_then_smaller():
    """Batch 32 of the 8-bit layer (256 pairs: router kernel, then the experts on
    the scratch), substitution mode; then batch 8 of the mixed layer (the fused
    one-launch path)."""
    lay, table, pool, desc = _layer(32, 4096, 256, 1024, 8, 8, 8, 5, 256)
    lg = synth.gen_logits(synth.rng_for(5, 3), 32, 256)
    x = synth.gen_x(synth.rng_for(5, 1), 32, 4096)
    st, ref = _both(lg, x, table, pool, desc, 8, mode=B.MOE_ROUTE_SUBST, L=0.15)
    assert st[3] == 0
    _same(st, ref)
    lay, table, pool, desc = _layer(8, 2048, 128, 768, 8, 4, 6, 4, 128)
    lg = synth.gen_logits(synth.rng_for(4, 3), 8, 128)
    x = synth.gen_x(synth.rng_for(4, 1), 8, 2048)
    st, ref = _both(lg, x, table, pool, desc, 8)
    assert st[3] == 0
    _same(st, ref)


def test_static_refuses_layers_beyond_its_scratch():
    torch = _torch()
    H, E, I, k, T = 2048, 512, 512, 10, 1024
    desc = B.moe_size_class_init(H, I, 3, 3, 1)
    assert B.moe_forward_workspace_size(T, k, E, desc) > B.MOE_STATIC_SCRATCH_BYTES
    lg = torch.zeros((T, E), dtype=torch.float32, device="cuda")
    x = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    table = torch.zeros(E, dtype=torch.int32, device="cuda")
    pool = torch.zeros(desc.slot_bytes, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.MoeError) as ei:
        B.moe_layer_forward_static(lg, x, table, pool, desc, k)
    assert ei.value.code == B.MOE_E_WORKSPACE
