"""Pins of the oracle's routing (softmax, top-k, weights, substitution).

Each check ties the oracle to something other than itself: math.exp / fp64
softmax, a sort of the raw logits, exhaustive search, hand-derived cases in
tests/golden/route_subst.txt, and invariants.  Sources: "RFC: stream MoE experts
from disk in from_pretrained", Motivation (top-k of E experts per token);
BigMoeOnEdge commit message adding cache-aware substitution.
"""
import itertools
import math
import os

import numpy as np
import pytest

import oracle
from quantized_routed_expert_softmax_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def ulp_f32(x: float) -> float:
    return float(np.spacing(np.float32(abs(x))))


def test_exp_c_within_2ulp_of_libm():
    xs = np.concatenate([np.linspace(-86.0, 0.0, 20001, dtype=np.float32),
                         -np.logspace(-8, 1.9, 3001).astype(np.float32),
                         np.array([0.0, -0.5, -1.0, -2.0, -math.log(2)], dtype=np.float32)])
    got = oracle.exp_c(xs)
    for x, g in zip(xs.tolist(), got.tolist()):
        ref = math.exp(x)
        assert abs(g - ref) <= 2 * ulp_f32(ref), (x, g, ref)


def test_exp_c_special_values():
    assert oracle.exp_c(np.float32(0.0)) == 1.0
    assert oracle.exp_c(np.float32(-86.5)) == 0.0
    assert oracle.exp_c(np.float32(-1000.0)) == 0.0


def softmax64(lg):
    z = lg.astype(np.float64) - lg.max(axis=1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("E", [1, 2, 8, 63, 64, 65, 128, 256, 512, 1000, 1024])
def test_softmax_close_to_fp64(E):
    lg = synth.gen_logits(synth.rng_for(11, E), 7, E)
    p = oracle.softmax(lg)
    ref = softmax64(lg)
    # error budget in units of u = 2^-24: exp_c 2 ulp (<= 4u) on each term, the
    # same relative error carried into Z, (E/64 - 1) + 6 additions of positive
    # terms, one division.
    u = 2.0 ** -24
    bound = (4 + 4 + (-(-E // 64) + 5) + 1) * u
    assert np.all(np.abs(p - ref) <= bound * ref)
    assert np.all(np.abs(p.astype(np.float64).sum(axis=1) - 1.0) < 1e-5)


@pytest.mark.parametrize("E,k", [(8, 2), (64, 8), (128, 8), (256, 8), (512, 10), (1024, 32), (5, 5), (3, 1)])
def test_topk_matches_sorted_logits(E, k):
    """softmax is monotone, so the top-k of p is the top-k of the logits (ties in
    p aside, which the check detects and skips)."""
    lg = synth.gen_logits(synth.rng_for(12, E, k), 40, E)
    ids, w, p = oracle.route(lg, k, return_p=True)
    for t in range(lg.shape[0]):
        order = np.lexsort((np.arange(E), -lg[t].astype(np.float64)))
        if k < E and p[t][order[k - 1]] == p[t][order[k]]:
            continue
        assert list(ids[t]) == list(order[:k])
        # stable sort of (-p, id) over the oracle's own probabilities as well
        order_p = np.lexsort((np.arange(E), -p[t].astype(np.float64)))
        assert list(ids[t]) == list(order_p[:k])


def test_topk_exhaustive_small():
    rng = synth.rng_for(13)
    for _ in range(60):
        E = int(rng.integers(1, 9))
        k = int(rng.integers(1, E + 1))
        lg = rng.standard_normal((1, E)).astype(np.float32)
        ids, w = oracle.route(lg, k)
        best = max(itertools.combinations(range(E), k), key=lambda s: sum(lg[0, i] for i in s))
        assert sorted(ids[0].tolist()) == sorted(best)
        assert all(lg[0, ids[0, j]] >= lg[0, ids[0, j + 1]] for j in range(k - 1))


def test_ties_go_to_lower_id():
    lg = np.array([[0.5, 1.0, 1.0, 0.5, 1.0, -3.0]], dtype=np.float32)
    ids, _ = oracle.route(lg, 4)
    assert ids[0].tolist() == [1, 2, 4, 0]


@pytest.mark.parametrize("E,k", [(8, 2), (512, 10), (128, 8), (256, 8), (64, 1), (16, 16)])
def test_weights_against_fp64_closed_form(E, k):
    lg = synth.gen_logits(synth.rng_for(14, E, k), 30, E)
    ids, w = oracle.route(lg, k)
    ref_p = softmax64(lg)
    for t in range(lg.shape[0]):
        sel = ref_p[t, ids[t]]
        ref = sel / sel.sum()
        assert np.allclose(w[t], ref, rtol=2e-6, atol=1e-9)
        assert abs(float(w[t].astype(np.float64).sum()) - 1.0) <= k * 2 ** -23
    if k == 1:
        assert np.all(w == 1.0)


def test_k_equals_E_gives_softmax():
    lg = synth.gen_logits(synth.rng_for(15), 5, 16)
    ids, w = oracle.route(lg, 16)
    ref = softmax64(lg)
    for t in range(5):
        assert np.allclose(w[t], ref[t, ids[t]], rtol=3e-6)


def test_nonfinite_logit_raises():
    lg = np.zeros((2, 8), dtype=np.float32)
    lg[1, 3] = np.nan
    with pytest.raises(oracle.OracleError):
        oracle.route(lg, 2)


def _golden_subst():
    rows = []
    with open(os.path.join(GOLDEN, "route_subst.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, L, lg, mask, ids, w = [c.strip() for c in line.split("|")]
            rows.append((int(k), float(L), [float(v) for v in lg.split()],
                         [int(v) for v in mask.split()], [int(v) for v in ids.split()],
                         [float(v) for v in w.split()]))
    return rows


@pytest.mark.parametrize("case", _golden_subst())
def test_substitution_golden(case):
    k, L, lg, mask, ids_ref, w_ref = case
    table = np.where(np.array(mask) > 0, np.arange(len(mask)), -1).astype(np.int32)
    ids, w = oracle.route(np.array([lg], dtype=np.float32), k, mode=1, L=L, slot_table=table)
    assert ids[0].tolist() == ids_ref
    assert np.allclose(w[0], w_ref, atol=2e-6)


def test_substitution_reduces_to_plain():
    lg = synth.gen_logits(synth.rng_for(16), 64, 256)
    ids0, w0 = oracle.route(lg, 8)
    table = synth.slot_table(synth.rng_for(17), 256, 256, resident=64)
    ids1, w1 = oracle.route(lg, 8, mode=1, L=0.0, slot_table=table)
    assert np.array_equal(ids0, ids1) and np.array_equal(w0, w1)
    empty = np.full(256, -1, dtype=np.int32)
    ids2, w2 = oracle.route(lg, 8, mode=1, L=0.15, slot_table=empty)
    assert np.array_equal(ids0, ids2) and np.array_equal(w0, w2)


def test_substitution_large_L_picks_resident_top_k():
    """With L = 2 every resident key exceeds max p, so the k chosen are the top-k
    of p among resident experts (tokens whose resident keys collide within
    rounding are skipped: p + c rounds at the ulp of c)."""
    E, k = 256, 8
    lg = synth.gen_logits(synth.rng_for(18), 32, E)
    table = synth.slot_table(synth.rng_for(19), E, E, resident=64)
    res = np.flatnonzero(table >= 0)
    ids, w = oracle.route(lg, k, mode=1, L=2.0, slot_table=table)
    ref_p = softmax64(lg)
    checked = 0
    for t in range(32):
        order = res[np.lexsort((res, -lg[t, res].astype(np.float64)))]
        ps = ref_p[t, order[:k + 1]]
        if np.min(np.abs(np.diff(ps))) < 1e-6:
            continue
        checked += 1
        assert ids[t].tolist() == order[:k].tolist()
        sel = ref_p[t, ids[t]]
        assert np.allclose(w[t], sel / sel.sum(), rtol=2e-6)
    assert checked >= 16


def test_substitution_selection_is_top_k_of_biased_score():
    """fp64 check of the rule itself: the chosen set maximises p + c*[resident]
    (margins far above rounding; near-ties are skipped)."""
    E, k, L = 256, 8, 0.15
    lg = synth.gen_logits(synth.rng_for(20), 32, E)
    table = synth.slot_table(synth.rng_for(21), E, E, resident=64)
    ids, w = oracle.route(lg, k, mode=1, L=L, slot_table=table)
    p = softmax64(lg)
    moved = 0
    for t in range(32):
        c = L * (p[t].max() - p[t].min())
        key = p[t] + c * (table >= 0)
        order = np.argsort(-key, kind="stable")
        if abs(key[order[k - 1]] - key[order[k]]) < 1e-6:
            continue
        assert sorted(ids[t].tolist()) == sorted(order[:k].tolist())
        moved += len(set(ids[t].tolist()) - set(np.argsort(-p[t], kind="stable")[:k].tolist()))
    assert moved > 0  # the mode does change some choices at L = 0.15


# --------------------------------------------------------------------------- #
# The logit-order shortcut of the decode kernel's routing (plain mode):       #
# a model of its selection rule, checked against the oracle's top-k.          #
# --------------------------------------------------------------------------- #
def _order_bits(l):
    u = np.asarray(l, np.float32).view(np.uint32)
    return np.where(u & 0x80000000, ~u, u | 0x80000000).astype(np.uint32)


def _order_bits_logit(v):
    v = np.asarray(v, np.uint32)
    return np.where(v & 0x80000000, v & 0x7FFFFFFF, ~v).astype(np.uint32).view(np.float32)


def _logit_order_choice(row, k):
    """The 32-bit keys (order bits, low 9 bits = 511 - id), the k largest as the
    chosen set, and the gap test on the bucket bounds of the k-th and (k+1)-th
    keys; returns (test passed, chosen ids)."""
    E = row.shape[0]
    ids = np.arange(E, dtype=np.uint32)
    keys = (_order_bits(row) & np.uint32(0xFFFFFE00)) | (np.uint32(511) - ids)
    c = np.sort(keys)[::-1]
    chosen = (np.uint32(511) - (c[:k] & np.uint32(0x1FF))).astype(np.int64)
    lo_in = _order_bits_logit(c[k - 1] & np.uint32(0xFFFFFE00))
    hi_out = _order_bits_logit(c[k] | np.uint32(0x1FF))
    m = np.float32(row.max())
    ok = (np.float32(lo_in - m) >= np.float32(-64.0)) and (np.float32(lo_in - hi_out) >= np.float32(2.0 ** -9))
    return bool(ok), chosen


def _shortcut_rows(rng, E, k):
    rows = [synth.gen_logits(rng, 1, E)[0] for _ in range(40)]
    rows += [(synth.gen_logits(rng, 1, E)[0] * s).astype(np.float32) for s in (1e-3, 0.05, 30.0, 3000.0)]
    rows += [(np.round(synth.gen_logits(rng, 1, E)[0] * q) / q).astype(np.float32) for q in (2.0, 64.0, 4096.0)]
    base = synth.gen_logits(rng, 1, E)[0]
    order = np.argsort(-base, kind="stable")
    for d in (0.0, 1e-7, 2.0 ** -10, 2.0 ** -9, 2.0 ** -9 + 1e-6, 3e-3):
        r = base.copy()
        r[order[:k]] += np.float32(4.0)
        r[order[k]] = np.float32(r[order[:k]].min() - np.float32(d))
        rows.append(r.astype(np.float32))
    r = np.full(E, -70.0, np.float32) + rng.standard_normal(E).astype(np.float32)
    r[3] = 0.0
    rows.append(r)
    r = np.zeros(E, np.float32)
    rows.append(r)
    return rows


@pytest.mark.parametrize("E,k", [(512, 10), (512, 15), (512, 1), (300, 8), (64, 15)])
def test_logit_order_shortcut_matches_contract_top_k(E, k):
    """Where the gap test passes, the k largest logit keys are exactly the
    contract's top-k set (computed by the oracle from p); the test must pass on
    ordinary logits and fail on near-ties at the boundary and far underflow."""
    rng = synth.rng_for(4242, E, k)
    passed = 0
    for row in _shortcut_rows(rng, E, k):
        ok, chosen = _logit_order_choice(row, k)
        ids_o, _ = oracle.route(row[None, :], k)
        if ok:
            passed += 1
            assert set(chosen.tolist()) == set(ids_o[0].tolist())
    assert passed >= 30  # ordinary rows take the shortcut
    # boundary cases: an exact tie and a 1e-7 gap must fail the test
    base = synth.gen_logits(rng, 1, E)[0]
    order = np.argsort(-base, kind="stable")
    for d in (0.0, 1e-7):
        r = base.copy()
        r[order[k]] = np.float32(r[order[k - 1]] - np.float32(d))
        assert not _logit_order_choice(r, k)[0]


def test_logit_order_gap_bound_holds_for_exp_c():
    """The bound the shortcut rests on: logits 2^-10 apart (and at least m - 64)
    give strictly ordered p under the contract's arithmetic, near every exp_c
    range-reduction boundary (n ln 2 for integer n) and at random points."""
    rng = synth.rng_for(4243)
    m = np.float32(0.0)
    lb = np.concatenate([(-np.arange(0, 93) * np.log(2)).astype(np.float32),
                         -rng.uniform(0, 64, 4000).astype(np.float32)])
    lb = lb[lb >= -64.0]
    la = (lb - np.float32(2.0 ** -10)).astype(np.float32)
    eb = oracle.exp_c((lb - m).astype(np.float32))
    ea = oracle.exp_c((la - m).astype(np.float32))
    for Z in (np.float32(1.0), np.float32(3.7), np.float32(511.25)):
        pb = (eb / Z).astype(np.float32)
        pa = (ea / Z).astype(np.float32)
        assert np.all(pa < pb)
