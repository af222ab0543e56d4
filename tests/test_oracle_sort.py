"""Pins of the oracle's sort by expert and pass table.

Brute force: an O(n^2) stable placement written from the definition (pair p
goes to offsets[e] + #{p' < p with the same expert}).  Source: "POC: Experts
offload", commit messages (the sorted prefill's batches of 64 experts); "RFC:
stream MoE experts from disk in from_pretrained", How the prototype works,
Prefill (sorted gather, 64 experts per batch).
"""
import numpy as np
import pytest

import oracle
from quantized_routed_expert_softmax_amd import synth


def brute(ids, E, P):
    flat = ids.reshape(-1).tolist()
    n = len(flat)
    counts = [sum(1 for v in flat if v == e) for e in range(E)]
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    out = [None] * n
    for p in range(n):
        e = flat[p]
        rank = sum(1 for q in range(p) if flat[q] == e)
        out[offsets[e] + rank] = p
    hit = [e for e in range(E) if counts[e] > 0]
    n_pass = (len(hit) + P - 1) // P
    pt = [len(hit), n_pass] + hit + [-1] * (E - len(hit))
    n_pass_max = (E + P - 1) // P
    pt += [min(q * P, len(hit)) for q in range(n_pass_max + 1)]
    return offsets, out, pt


@pytest.mark.parametrize("T,k,E,P", [(16, 2, 8, 64), (1, 10, 512, 64), (7, 3, 5, 2), (50, 8, 128, 64),
                                     (40, 4, 200, 16), (0, 4, 8, 64), (33, 1, 1, 64), (64, 8, 256, 64)])
def test_sort_brute_force(T, k, E, P):
    rng = synth.rng_for(30, T, k, E)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32) \
        if T else np.zeros((0, k), np.int32)
    off, sp, pt = oracle.sort(ids, E, P)
    b_off, b_sp, b_pt = brute(ids, E, P)
    assert off.tolist() == b_off
    assert sp.tolist() == b_sp
    assert pt.tolist() == b_pt


def test_sort_invariants_prefill_shape():
    lg = synth.gen_logits(synth.rng_for(31), 1024, 512)
    ids, _ = oracle.route(lg, 10)
    off, sp, pt = oracle.sort(ids, 512, 64)
    assert off[-1] == 1024 * 10 and off[0] == 0
    assert np.array_equal(np.diff(off), np.bincount(ids.ravel(), minlength=512))
    assert np.array_equal(np.sort(sp), np.arange(10240))
    flat = ids.ravel()
    for e in range(512):
        seg = sp[off[e]:off[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)
    # near-uniform routing: every expert hit, 8 passes of 64
    assert pt[0] == 512 and pt[1] == 8
    assert pt[2:2 + 512].tolist() == list(range(512))
    assert pt[2 + 512:].tolist() == [0, 64, 128, 192, 256, 320, 384, 448, 512]


def test_sort_rejects_bad_id():
    with pytest.raises(oracle.OracleError):
        oracle.sort(np.array([[0, 9]], dtype=np.int32), 8, 64)
