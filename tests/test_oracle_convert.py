"""Pins of the oracle's one-time conversion of expert weights into slot rows
("RFC: stream MoE experts from disk in from_pretrained", How the prototype
works, Quantized experts bullet: experts converted once to the affine format,
one contiguous row each).

The rounding of scale and bias to fp16 and of width-16 weights to bf16 is
checked against numpy's and torch's own conversions; the quantization rule
against hand-derived groups (tests/golden/quantize_groups.txt), exact grids
that must come back unchanged, and the error bound of the dequantized weights;
the row against the oracle's pinned decoder (oracle.code, oracle.dequant) and
layout.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from quantized_routed_expert_softmax_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _expand(spec: str, n=64):
    if spec.strip() == "i":
        return [float(i) for i in range(n)]
    if spec.strip() == "i/4-4":
        return [i / 4 - 4 for i in range(n)]
    out = []
    for tok in spec.split():
        if "*" in tok:
            k, v = tok.split("*")
            out += [float(v)] * int(k)
        else:
            out.append(float(tok))
    assert len(out) == n, spec
    return out


def _groups():
    rows = []
    with open(os.path.join(GOLDEN, "quantize_groups.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            b, vals, sz, codes = [c.strip() for c in line.split("|")]
            s, z = [int(v, 16) for v in sz.split()]
            rows.append((int(b), _expand(vals), s, z, [int(c) for c in _expand(codes)]))
    return rows


@pytest.mark.parametrize("case", _groups())
def test_quantize_golden_groups(case):
    bits, vals, s, z, codes = case
    w = np.array([vals], dtype=np.float32)
    q, sc, bi = oracle.quantize(w, bits)
    assert int(sc[0, 0]) == s and int(bi[0, 0]) == z
    assert q[0].tolist() == codes


def _tie_points(rng, n, dec_bits_to_float, top):
    """Exact midpoints between neighbouring patterns (the tie cases) plus random
    values of every magnitude, as doubles."""
    pats = rng.integers(0, top, size=n)
    lo = dec_bits_to_float(pats.astype(np.uint16))
    hi = dec_bits_to_float((pats + 1).astype(np.uint16))
    mids = (lo + hi) / 2
    rand = np.exp(rng.uniform(np.log(1e-9), np.log(7e4), size=n)) * rng.choice([-1.0, 1.0], size=n)
    return np.concatenate([mids, -mids, rand, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf)])


def test_round_half_matches_numpy():
    rng = np.random.default_rng(7)
    xs = _tie_points(rng, 4000, lambda p: p.view(np.float16).astype(np.float64), 0x7BFF)
    xs = np.concatenate([xs, [0.0, -0.0, 65504.0, 65519.99, 65520.0, 65536.0, 2.0 ** -25, 2.0 ** -24,
                              3 * 2.0 ** -26, 2.0 ** -14, 1e-30]])
    with np.errstate(over="ignore"):
        want = xs.astype(np.float16).view(np.uint16)
    got = np.array([oracle.round_half(x) for x in xs], dtype=np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(xs[i], hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(8)
    def dec(p):
        return (p.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    xs = _tie_points(rng, 4000, dec, 0x7F7F).astype(np.float32)  # fp32 inputs, as the converter sees
    xs = np.concatenate([xs[np.isfinite(xs)], np.array([0.0, -0.0, 3.3895314e38, 1e-40], dtype=np.float32)])
    want = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.round_bf16(float(x)) for x in xs], dtype=np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(xs[i], hex(got[i]), hex(want[i])) for i in bad[:5]]


@pytest.mark.parametrize("bits", [3, 4, 6, 8])
def test_quantize_exact_grid_comes_back(bits):
    """Weights on an fp16 grid z0 + s0*q0 (q0 reaching 0 and 2^b - 1 in each
    group) quantize to exactly (q0, s0, z0)."""
    rng = np.random.default_rng(100 + bits)
    R, C = 6, 256
    qmax = (1 << bits) - 1
    q0 = rng.integers(0, qmax + 1, size=(R, C)).astype(np.uint8)
    q0.reshape(R, C // 64, 64)[:, :, 0] = 0
    q0.reshape(R, C // 64, 64)[:, :, 1] = qmax
    e = rng.integers(-10, -3, size=(R, C // 64))
    s0 = (1 + rng.integers(0, 1024, size=(R, C // 64)) / 1024.0) * 2.0 ** e
    z0 = rng.integers(-2047, 2048, size=(R, C // 64)) * 2.0 ** (e - 10)
    w = (z0[..., None] + s0[..., None] * q0.reshape(R, C // 64, 64).astype(np.float64)).reshape(R, C)
    assert np.array_equal(w.astype(np.float32).astype(np.float64), w)  # exact in fp32
    q, s, z = oracle.quantize(w.astype(np.float32), bits)
    assert np.array_equal(q, q0)
    assert np.array_equal(s.view(np.float16).astype(np.float64), s0)
    zz = z.view(np.float16).astype(np.float64)
    assert np.array_equal(zz, z0 + 0.0)


@pytest.mark.parametrize("bits", [3, 4, 6, 8])
def test_quantize_error_bound(bits):
    """|w - (s q + z)| <= s/2 where no clamp applies; at most s/2 + |min - z| +
    (max - min) 2^-10 anywhere (fp16 rounding of scale and bias)."""
    rng = np.random.default_rng(200 + bits)
    w = (rng.standard_normal((16, 512)) * np.exp(rng.uniform(-6, 3, size=(16, 1)))).astype(np.float32)
    q, s, z = oracle.quantize(w, bits)
    qmax = (1 << bits) - 1
    assert int(q.max()) <= qmax
    g = w.astype(np.float64).reshape(16, 8, 64)
    sd = s.view(np.float16).astype(np.float64)[..., None]
    zd = z.view(np.float16).astype(np.float64)[..., None]
    deq = sd * q.reshape(16, 8, 64) + zd
    err = np.abs(deq - g)
    inner = (q.reshape(16, 8, 64) > 0) & (q.reshape(16, 8, 64) < qmax)
    assert np.all(err[inner] <= sd.repeat(64, 2)[inner] / 2 * (1 + 1e-12))
    bound = sd / 2 + np.abs(g.min(axis=2, keepdims=True) - zd) + (g.max(axis=2, keepdims=True)
                                                                 - g.min(axis=2, keepdims=True)) * 2.0 ** -10
    assert np.all(err <= bound)
    # the extremes reach the end codes
    assert np.all(q.reshape(16, 8, 64).min(axis=2) == 0)
    assert np.all(q.reshape(16, 8, 64).max(axis=2) >= qmax - 1)


@pytest.mark.parametrize("bits_gu,bits_d", [(3, 3), (4, 6), (8, 8), (16, 16), (3, 16)])
def test_convert_expert_row_decodes(bits_gu, bits_d):
    """The converted row, read back with the pinned decoder, holds the quantizer's
    codes, scale and bias in the pinned layout, and zeros between blocks."""
    H, I = 192, 128
    rng = np.random.default_rng(300 + bits_gu * 17 + bits_d)
    w_gu = (rng.standard_normal((2 * I, H)) / np.sqrt(H)).astype(np.float32)
    w_d = (rng.standard_normal((H, I)) / np.sqrt(I)).astype(np.float32)
    row = oracle.convert_expert(w_gu, w_d, H, I, bits_gu, bits_d)
    offs = oracle.layout(H, I, bits_gu, bits_d)
    assert row.size == offs[4]
    for which, (w, R, C, b) in enumerate([(w_gu, 2 * I, H, bits_gu), (w_d, H, I, bits_d)]):
        codes_at, sb_at = int(offs[2 * which]), int(offs[2 * which + 1])
        rb = C * b // 8
        deq = oracle.dequant(row, H, I, bits_gu, bits_d, which)
        if b == 16:
            want = torch.from_numpy(w).to(torch.bfloat16).to(torch.float64).numpy()
            assert np.array_equal(deq, want)
            continue
        q, s, z = oracle.quantize(w, b)
        for r in (0, R // 2, R - 1):
            got = [oracle.code(row[codes_at + r * rb: codes_at + (r + 1) * rb], b, c) for c in range(C)]
            assert got == q[r].tolist()
        sb = row[sb_at: sb_at + R * (C // 64) * 4].view("<u2").reshape(R, C // 64, 2)
        assert np.array_equal(sb[:, :, 0], s) and np.array_equal(sb[:, :, 1], z)
        sd = s.view(np.float16).astype(np.float64).repeat(64, axis=1)
        zd = z.view(np.float16).astype(np.float64).repeat(64, axis=1)
        assert np.array_equal(deq, sd * q + zd)
    # padding between and after blocks is zero
    ends = [offs[0] + 2 * I * H * bits_gu // 8, offs[1] + (0 if bits_gu == 16 else 2 * I * (H // 64) * 4),
            offs[2] + H * I * bits_d // 8, offs[3] + (0 if bits_d == 16 else H * (I // 64) * 4)]
    starts = list(offs[1:5])
    for a, b in zip(ends, starts):
        assert not row[int(a):int(b)].any()


@pytest.mark.parametrize("bits", [3, 4, 8])
def test_convert_agrees_with_input_generator(bits):
    """A second, separately written quantizer (the input generator's, in numpy)
    gives the same codes, scale and bias on gaussian weights."""
    rng = np.random.default_rng(400 + bits)
    w = (rng.standard_normal((8, 256)) * 0.05).astype(np.float32)
    q, s, z = oracle.quantize(w, bits)
    q2, s2, z2 = synth.quantize(w, bits)
    assert np.array_equal(q, q2)
    assert np.array_equal(s, s2.view(np.uint16)) and np.array_equal(z, z2.view(np.uint16))
