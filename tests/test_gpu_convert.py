"""GPU parity of the one-time conversion (moe_quantize_experts): the rows the
HIP converter writes must equal the oracle's rows byte for byte (codes, scale,
bias and zero padding are all integer results), for every code width, fp32 and
bf16 weights, ragged group counts, the edge cases of the quantization rule, and
the full workload shapes; converted rows then serve a store file and a layer
forward checked against the oracle's layer.

Source: "RFC: stream MoE experts from disk in from_pretrained", How the
prototype works, Quantized experts bullet.
"""
import ctypes
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


def _weights(rng, n, H, I, scale=1.0):
    w_gu = (rng.standard_normal((n, 2 * I, H)) * scale / np.sqrt(H)).astype(np.float32)
    w_d = (rng.standard_normal((n, H, I)) * scale / np.sqrt(I)).astype(np.float32)
    return w_gu, w_d


def _bf16_round(a):
    """fp32 array -> the fp32 values of its nearest bf16 (via torch, CPU)."""
    torch = _torch()
    return torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()


def _convert_gpu(w_gu, w_d, desc, bf16=False):
    torch = _torch()
    a = torch.from_numpy(w_gu).cuda()
    b = torch.from_numpy(w_d).cuda()
    if bf16:
        a, b = a.to(torch.bfloat16), b.to(torch.bfloat16)
    rows = B.moe_quantize_experts(a, b, desc)
    torch.cuda.synchronize()
    return rows.cpu().numpy()


def _check_rows(rows, w_gu, w_d, H, I, bg, bd):
    for e in range(w_gu.shape[0]):
        want = oracle.convert_expert(w_gu[e], w_d[e], H, I, bg, bd)
        got = rows[e]
        if not np.array_equal(got, want):
            bad = np.nonzero(got != want)[0]
            raise AssertionError(f"expert {e}: {bad.size} bytes differ, first at {bad[:8].tolist()} "
                                 f"(layout {oracle.layout(H, I, bg, bd).tolist()})")


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("H,I,bg,bd", [
    (192, 128, 3, 3), (256, 64, 4, 6), (128, 192, 8, 8), (192, 64, 16, 16), (320, 128, 3, 16),
    (64, 64, 6, 4), (448, 320, 3, 4),
])
def test_convert_matches_oracle(H, I, bg, bd, bf16):
    rng = synth.rng_for(500 + H + I + bg * 7 + bd, int(bf16))
    w_gu, w_d = _weights(rng, 3, H, I)
    desc = B.moe_size_class_init(H, I, bg, bd, 1)
    rows = _convert_gpu(w_gu, w_d, desc, bf16)
    if bf16:  # the converter sees the bf16 values
        w_gu, w_d = _bf16_round(w_gu), _bf16_round(w_d)
    _check_rows(rows, w_gu, w_d, H, I, bg, bd)


@pytest.mark.parametrize("bits", [3, 4, 6, 8])
def test_convert_edge_groups(bits):
    """Constant groups (scale 0), signed zeros, exact grids with ties at half
    codes, a huge spread next to a tiny one, subnormal fp16 scales, and minima
    that round to fp16 zero."""
    H, I = 128, 64
    rng = synth.rng_for(600, bits)
    w_gu, w_d = _weights(rng, 2, H, I)
    g = w_gu.reshape(2, 2 * I, H // 64, 64)
    g[0, 0, 0, :] = 0.3                                   # constant
    g[0, 1, 0, :] = 0.0
    g[0, 1, 0, ::2] = -0.0                                # signed zeros
    qmax = (1 << bits) - 1
    s0 = 2.0 ** -6                                        # exact ties: (k + 1/2) s0 above a zero minimum
    g[0, 2, 0, :] = (np.arange(64) % qmax + 0.5) * s0
    g[0, 2, 0, 0], g[0, 2, 0, 1] = 0.0, qmax * s0
    g[0, 3, 0, :] = rng.standard_normal(64) * 1e3         # large spread
    g[0, 3, 1, :] = rng.standard_normal(64) * 1e-6        # subnormal scale
    g[0, 4, 0, :] = rng.uniform(1e-9, 2e-9, 64)           # minimum rounds to fp16 zero
    g[0, 5, 1, :] = -rng.uniform(1e-9, 2e-9, 64)          # ... to fp16 -0
    g[1, 6, 0, :] = 65000.0
    g[1, 6, 0, 5] = -65000.0                              # scale near the fp16 top
    desc = B.moe_size_class_init(H, I, bits, bits, 1)
    rows = _convert_gpu(w_gu, w_d, desc)
    _check_rows(rows, w_gu, w_d, H, I, bits, bits)


def test_convert_full_workload_shapes():
    """The decode / prefill layer (H 2048, I 512, 3-bit) and the 8-bit batch
    layer (H 4096, I 1024), two experts each, byte for byte."""
    for (H, I, b), seed in [((2048, 512, 3), 700), ((4096, 1024, 8), 701), ((2048, 768, 4), 702)]:
        rng = synth.rng_for(seed, 0)
        w_gu, w_d = _weights(rng, 2, H, I)
        desc = B.moe_size_class_init(H, I, b, b, 1)
        rows = _convert_gpu(w_gu, w_d, desc)
        _check_rows(rows, w_gu, w_d, H, I, b, b)


def test_convert_store_and_forward(tmp_path):
    """Converted rows written as a store file come back through the store and,
    installed in a pool, give the oracle's layer output on those rows."""
    torch = _torch()
    T, H, E, I, k, bits = 24, 256, 8, 128, 2, 4
    rng = synth.rng_for(800, 0)
    w_gu, w_d = _weights(rng, E, H, I)
    desc = B.moe_size_class_init(H, I, bits, bits, E)
    rows = _convert_gpu(w_gu, w_d, desc)
    path = str(tmp_path / "experts.bin")
    rows.tofile(path)
    st = B.moe_store_open_file(path, [desc], [0], E)
    try:
        buf = np.empty(desc.slot_bytes, dtype=np.uint8)
        for e in (0, E - 1):
            B.moe_store_read(st, 0, e, buf)
            assert np.array_equal(buf, rows[e])
    finally:
        B.moe_store_close(st)
    perm = synth.rng_for(800, 1).permutation(E).astype(np.int32)   # expert e in slot perm[e]
    pool = np.zeros((E, desc.slot_bytes), dtype=np.uint8)
    pool[perm] = rows
    pool_d = torch.from_numpy(pool).cuda().view(-1)
    x = synth.gen_x(synth.rng_for(800, 2), T, H)
    lg = synth.gen_logits(synth.rng_for(800, 3), T, E)
    ids, w = oracle.route(lg, k)
    xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = B.moe_experts_forward(xd, torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(), E,
                                torch.from_numpy(perm).cuda(), pool_d, desc, err_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref = oracle.layer(x, ids, w, perm, pool, H, I, bits, bits, E, threads=THREADS)
    got = out.float().cpu().numpy().astype(np.float64)
    d = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert d.max() <= 2e-2 and rel <= 1e-2, (d.max(), rel)


def test_convert_zero_experts_and_bad_arguments():
    torch = _torch()
    desc = B.moe_size_class_init(128, 64, 3, 3, 1)
    empty_gu = torch.empty((0, 128, 128), dtype=torch.float32, device="cuda")
    empty_d = torch.empty((0, 128, 64), dtype=torch.float32, device="cuda")
    out = B.moe_quantize_experts(empty_gu, empty_d, desc)
    assert out.shape == (0, desc.slot_bytes)
    a = torch.zeros((1, 128, 128), dtype=torch.float32, device="cuda")
    b = torch.zeros((1, 128, 64), dtype=torch.float32, device="cuda")
    rows = torch.empty((2 * desc.slot_bytes,), dtype=torch.uint8, device="cuda")
    f = B.lib().moe_quantize_experts
    pa, pb = ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr())
    # rows not 256-byte aligned; unknown dtype; NULL weights
    assert f(pa, pb, B.MOE_DTYPE_F32, 1, ctypes.byref(desc), ctypes.c_void_p(rows.data_ptr() + 16), None) \
        == B.MOE_E_INVALID
    assert f(pa, pb, 7, 1, ctypes.byref(desc), ctypes.c_void_p(rows.data_ptr()), None) == B.MOE_E_INVALID
    assert f(None, pb, B.MOE_DTYPE_F32, 1, ctypes.byref(desc), ctypes.c_void_p(rows.data_ptr()), None) \
        == B.MOE_E_INVALID
