"""Seeded synthetic inputs for the routed-expert MoE layer.

This module only *makes inputs*: router logits, hidden states, quantized expert
rows written in the slot byte format, slot tables.  It holds none of the layer's
arithmetic (no routing, no dequantization, no matmul) and imports neither the
GPU library nor the CPU oracle, so both can be fed from it.

Shapes and distributions follow the workloads on the pages:
  * "RFC: stream MoE experts from disk in from_pretrained", section "Motivation":
    48 MoE layers, each of 512 experts with 10 routed per token, experts
    quantized to 3 bits, prompts processed in 1K-token chunks.
  * "moe: expert slots in size classes", PR description: mixed-quant models whose
    layers need different bytes per expert (two size classes).
  * BigMoeOnEdge commit message on cache-aware substitution: L = 0.15.
There are no trained weights or datasets here: every value is drawn from a
seeded generator (numpy PCG64 on the host; torch's seeded device generator for
the multi-GB pools of the large workloads).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

GROUP = 64
ALIGN = 256
PACK = 32


def _align(n: int, a: int = ALIGN) -> int:
    return (n + a - 1) // a * a


@dataclass(frozen=True)
class Layout:
    """Byte layout of one expert row (the slot format described in include/moe.h)."""
    H: int
    I: int
    bits_gu: int
    bits_d: int

    @property
    def gu_codes_bytes(self) -> int:
        return 2 * self.I * self.H * self.bits_gu // 8

    @property
    def gu_sb_bytes(self) -> int:  # width 16 (bf16 weights) has no scale/bias
        return 0 if self.bits_gu == 16 else 2 * self.I * (self.H // GROUP) * 4

    @property
    def d_codes_bytes(self) -> int:
        return self.H * self.I * self.bits_d // 8

    @property
    def d_sb_bytes(self) -> int:
        return 0 if self.bits_d == 16 else self.H * (self.I // GROUP) * 4

    @property
    def off_gu_codes(self) -> int:
        return 0

    @property
    def off_gu_sb(self) -> int:
        return _align(self.gu_codes_bytes)

    @property
    def off_d_codes(self) -> int:
        return _align(self.off_gu_sb + self.gu_sb_bytes)

    @property
    def off_d_sb(self) -> int:
        return _align(self.off_d_codes + self.d_codes_bytes)

    @property
    def slot_bytes(self) -> int:
        return _align(self.off_d_sb + self.d_sb_bytes)


# --------------------------------------------------------------------------- #
# Workloads (sizes and structure; the recipe is also written out in the design doc) #
# --------------------------------------------------------------------------- #
@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    T: int
    H: int
    E: int
    I: int
    k: int
    bits_gu: int
    bits_d: int
    seed: int
    slots_per_layer: int          # pool slots per layer
    resident: int                 # experts resident per layer
    zipf_s: float = 0.0           # per-expert Zipf bias on the logits (0 = none)
    subst_L: float | None = None  # cache-aware substitution strength
    mixed_every: int = 0          # every n-th layer uses bits_d_alt for down
    bits_d_alt: int = 0
    chunks: int = 1               # prefill chunks per prompt


WORKLOADS = {
    "tiny": Workload("tiny", 1, 16, 256, 8, 128, 2, 4, 4, 0, 8, 8),
    "decode": Workload("decode", 48, 1, 2048, 512, 512, 10, 3, 3, 2, 2048, 512, zipf_s=1.1),
    "prefill": Workload("prefill", 48, 1024, 2048, 512, 512, 10, 3, 3, 3, 512, 512, chunks=4),
    "mixed": Workload("mixed", 48, 1, 2048, 128, 768, 8, 4, 4, 4, 128, 128,
                      mixed_every=4, bits_d_alt=6),
    "int8sub": Workload("int8sub", 1, 32, 4096, 256, 1024, 8, 8, 8, 5, 256, 64, subst_L=0.15),
}


def layer_bits(w: Workload, layer: int) -> tuple[int, int]:
    """Code widths (gate_up, down) of a layer: every `mixed_every`-th layer
    (layers l with l % n == n - 1) takes the wider down code."""
    if w.mixed_every and layer % w.mixed_every == w.mixed_every - 1:
        return w.bits_gu, w.bits_d_alt
    return w.bits_gu, w.bits_d


# --------------------------------------------------------------------------- #
# Small helpers                                                                #
# --------------------------------------------------------------------------- #
def rng_for(seed: int, *stream: int) -> np.random.Generator:
    """Independent PCG64 stream per (seed, purpose, layer, ...)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *stream])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def gen_x(rng: np.random.Generator, T: int, H: int) -> np.ndarray:
    """Hidden states: N(0,1) rounded to bf16; returned as uint16 bit patterns."""
    return f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))


def zipf_bias(rng: np.random.Generator, E: int, s: float) -> np.ndarray:
    """Per-expert log-Zipf bias: -s*ln(rank), rank a seeded permutation of 1..E."""
    rank = rng.permutation(E) + 1
    return (-s * np.log(rank)).astype(np.float32)


def gen_logits(rng: np.random.Generator, T: int, E: int, bias: np.ndarray | None = None) -> np.ndarray:
    lg = rng.standard_normal((T, E), dtype=np.float32)
    if bias is not None:
        lg = (lg + bias[None, :]).astype(np.float32)
    return lg


def slot_table(rng: np.random.Generator, E: int, n_slots: int, resident: int | None = None) -> np.ndarray:
    """Expert -> slot table: the first E entries of a seeded permutation of the
    pool's slots; with `resident` < E only that many experts (chosen at random)
    keep their slot and the rest are -1."""
    perm = rng.permutation(n_slots)[:E].astype(np.int32)
    if resident is not None and resident < E:
        keep = np.zeros(E, dtype=bool)
        keep[rng.choice(E, size=resident, replace=False)] = True
        perm = np.where(keep, perm, -1).astype(np.int32)
    return perm


# --------------------------------------------------------------------------- #
# Test quantizer and packer (they make data; nothing here runs the layer)     #
# --------------------------------------------------------------------------- #
def quantize(w: np.ndarray, bits: int):
    """Group-wise affine quantization of an [R, C] float matrix, group 64 along C.

    scale = (max - min) / (2^b - 1) and bias = min, each rounded to fp16; the code
    is round-to-nearest of (w - bias)/scale clamped to [0, 2^b - 1]; a group with
    zero (fp16) scale gets code 0.  Returns (codes uint8 [R, C], scale fp16
    [R, C/64], bias fp16 [R, C/64])."""
    R, C = w.shape
    assert C % GROUP == 0
    g = w.astype(np.float64).reshape(R, C // GROUP, GROUP)
    lo = g.min(axis=2)
    hi = g.max(axis=2)
    qmax = (1 << bits) - 1
    scale16 = ((hi - lo) / qmax).astype(np.float16)
    bias16 = lo.astype(np.float16)
    s = scale16.astype(np.float64)[..., None]
    z = bias16.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint((g - z) / np.where(s > 0, s, 1.0)), 0.0)
    q = np.clip(q, 0, qmax).astype(np.uint8).reshape(R, C)
    return q, scale16, bias16


def pack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    """Pack codes [R, C] (values < 2^bits) into the slot format's code block:
    per pack unit of 32 columns, `bits` little-endian uint32 words with column
    32u+i at bits [bits*i, bits*i+bits) of the unit's little-endian integer."""
    R, C = q.shape
    assert C % PACK == 0 and int(q.max(initial=0)) < (1 << bits)
    units = q.reshape(R, C // PACK, PACK).astype(np.uint64)
    out = np.zeros((R, C // PACK, bits), dtype=np.uint64)
    for i in range(PACK):
        bit = bits * i
        word, off = divmod(bit, 32)
        v = units[:, :, i] << np.uint64(off)
        out[:, :, word] |= v & np.uint64(0xFFFFFFFF)
        if off + bits > 32:
            out[:, :, word + 1] |= v >> np.uint64(32)
    return out.astype("<u4").view(np.uint8).reshape(R, C * bits // 8)


def pack_scale_bias(scale16: np.ndarray, bias16: np.ndarray) -> np.ndarray:
    """[R, G] fp16 scale and bias -> [R, G*4] bytes, (scale, bias) per group."""
    R, G = scale16.shape
    sb = np.empty((R, G, 2), dtype="<f2")
    sb[:, :, 0] = scale16
    sb[:, :, 1] = bias16
    return sb.view(np.uint8).reshape(R, G * 4)


@dataclass
class ExpertQ:
    """One expert: codes and fp16 scale/bias of gate_up [2I, H] and down [H, I]."""
    gu_q: np.ndarray
    gu_s: np.ndarray
    gu_z: np.ndarray
    d_q: np.ndarray
    d_s: np.ndarray
    d_z: np.ndarray


def expert_row(lay: Layout, e: ExpertQ) -> np.ndarray:
    """Serialise one expert into its slot row (uint8 [slot_bytes]).  A width-16
    block holds the bf16 bit patterns (uint16 "codes") in row order and has no
    scale/bias."""
    row = np.zeros(lay.slot_bytes, dtype=np.uint8)
    a = pack_codes(e.gu_q, lay.bits_gu).reshape(-1)
    row[lay.off_gu_codes:lay.off_gu_codes + a.size] = a
    if lay.bits_gu != 16:
        a = pack_scale_bias(e.gu_s, e.gu_z).reshape(-1)
        row[lay.off_gu_sb:lay.off_gu_sb + a.size] = a
    a = pack_codes(e.d_q, lay.bits_d).reshape(-1)
    row[lay.off_d_codes:lay.off_d_codes + a.size] = a
    if lay.bits_d != 16:
        a = pack_scale_bias(e.d_s, e.d_z).reshape(-1)
        row[lay.off_d_sb:lay.off_d_sb + a.size] = a
    return row


def _quantize_or_bf16(w: np.ndarray, bits: int):
    if bits == 16:  # unquantized: bf16 bit patterns as 16-bit codes, no scale/bias
        return f32_to_bf16_bits(w), None, None
    return quantize(w, bits)


def gaussian_expert(rng: np.random.Generator, H: int, I: int, bits_gu: int, bits_d: int):
    """fp32 weights N(0, 1/fan_in) quantized by the test quantizer (width 16:
    rounded to bf16).  Returns (ExpertQ, w_gu fp32 [2I, H], w_d fp32 [I -> H] as [H, I])."""
    w_gu = (rng.standard_normal((2 * I, H), dtype=np.float32) / np.float32(math.sqrt(H))).astype(np.float32)
    w_d = (rng.standard_normal((H, I), dtype=np.float32) / np.float32(math.sqrt(I))).astype(np.float32)
    gq, gs, gz = _quantize_or_bf16(w_gu, bits_gu)
    dq, ds, dz = _quantize_or_bf16(w_d, bits_d)
    return ExpertQ(gq, gs, gz, dq, ds, dz), w_gu, w_d


def random_code_expert(rng: np.random.Generator, H: int, I: int, bits_gu: int, bits_d: int) -> ExpertQ:
    """Uniform random codes; per-group scale chosen so the dequantized weights are
    zero-mean with standard deviation about 1/sqrt(fan_in):
    scale = sqrt(12/(4^b - 1))/sqrt(fan_in) * U(0.9, 1.1), bias = -scale*(2^b-1)/2."""
    def one(R, C, b):
        if b == 16:  # bf16 weights N(0, 1/fan_in)
            w = (rng.standard_normal((R, C), dtype=np.float32) / np.float32(math.sqrt(C))).astype(np.float32)
            return f32_to_bf16_bits(w), None, None
        q = rng.integers(0, 1 << b, size=(R, C), dtype=np.uint8)
        base = math.sqrt(12.0 / (4 ** b - 1)) / math.sqrt(C)
        s = (base * rng.uniform(0.9, 1.1, size=(R, C // GROUP))).astype(np.float16)
        z = (-s.astype(np.float64) * ((1 << b) - 1) / 2).astype(np.float16)
        return q, s, z
    gq, gs, gz = one(2 * I, H, bits_gu)
    dq, ds, dz = one(H, I, bits_d)
    return ExpertQ(gq, gs, gz, dq, ds, dz)


# --------------------------------------------------------------------------- #
# Whole small problems (host numpy arrays)                                     #
# --------------------------------------------------------------------------- #
@dataclass
class Problem:
    lay: Layout
    T: int
    E: int
    k: int
    x: np.ndarray            # uint16 [T, H] bf16 bits
    logits: np.ndarray       # float32 [T, E]
    table: np.ndarray        # int32 [E]
    pool: np.ndarray         # uint8 [n_slots, slot_bytes]
    experts: list            # ExpertQ per expert id
    w_gu: list | None = None  # unquantized fp32 weights per expert (gaussian only)
    w_d: list | None = None


def make_problem(seed: int, T: int, H: int, E: int, I: int, k: int, bits_gu: int, bits_d: int,
                 n_slots: int | None = None, resident: int | None = None, gaussian: bool = True,
                 zipf_s: float = 0.0) -> Problem:
    """A whole layer problem held on the host: x, logits, a pool whose occupied
    slots hold every resident expert, and the expert -> slot table."""
    lay = Layout(H, I, bits_gu, bits_d)
    n_slots = E if n_slots is None else n_slots
    r = rng_for(seed, 1)
    x = gen_x(r, T, H)
    bias = zipf_bias(rng_for(seed, 2), E, zipf_s) if zipf_s else None
    logits = gen_logits(rng_for(seed, 3), T, E, bias)
    table = slot_table(rng_for(seed, 4), E, n_slots, resident)
    pool = np.zeros((n_slots, lay.slot_bytes), dtype=np.uint8)
    experts, wg, wd = [], [], []
    re = rng_for(seed, 5)
    for e in range(E):
        if gaussian:
            eq, a, b = gaussian_expert(re, H, I, bits_gu, bits_d)
            wg.append(a)
            wd.append(b)
        else:
            eq = random_code_expert(re, H, I, bits_gu, bits_d)
        experts.append(eq)
        if table[e] >= 0:
            pool[table[e]] = expert_row(lay, eq)
    return Problem(lay, T, E, k, x, logits, table, pool, experts,
                   wg if gaussian else None, wd if gaussian else None)


def tiny_problem() -> Problem:
    w = WORKLOADS["tiny"]
    return make_problem(w.seed, w.T, w.H, w.E, w.I, w.k, w.bits_gu, w.bits_d, n_slots=w.slots_per_layer)


# --------------------------------------------------------------------------- #
# Large pools generated on the device (torch's seeded generator)              #
# --------------------------------------------------------------------------- #
def fill_pool_device(pool, lay: Layout, slots, seed: int, layer: int):
    """Fill the given slots of a device pool tensor (uint8 [n_slots, slot_bytes])
    with random codes and the scale/bias recipe of random_code_expert (width 16:
    bf16 weights N(0, 1/fan_in)).

    Codes are uniform random bytes (uniform codes for every width, since the
    code block is a plain bit stream).  Uses torch's seeded device generator; the
    oracle reads the same bytes back from the device, so nothing is regenerated."""
    import torch
    dev = pool.device
    g = torch.Generator(device=dev)
    g.manual_seed((seed * 1000003 + layer * 7919 + 12345) & 0x7FFFFFFFFFFFFFFF)
    slots_t = torch.as_tensor(np.asarray(slots, dtype=np.int64), device=dev)
    n = slots_t.numel()
    if n == 0:
        return
    sb = lay.slot_bytes
    for (off_c, nbytes_c, off_sb, R, C, b) in (
        (lay.off_gu_codes, lay.gu_codes_bytes, lay.off_gu_sb, 2 * lay.I, lay.H, lay.bits_gu),
        (lay.off_d_codes, lay.d_codes_bytes, lay.off_d_sb, lay.H, lay.I, lay.bits_d),
    ):
        if b == 16:  # unquantized: bf16 weights N(0, 1/fan_in), no scale/bias
            w = torch.randn((n, R * C), device=dev, generator=g, dtype=torch.float32) / math.sqrt(C)
            pool[slots_t, off_c:off_c + nbytes_c] = w.to(torch.bfloat16).view(torch.uint8)
            del w
            continue
        codes = torch.randint(0, 256, (n, nbytes_c), dtype=torch.uint8, device=dev, generator=g)
        pool[slots_t, off_c:off_c + nbytes_c] = codes
        del codes
        base = math.sqrt(12.0 / (4 ** b - 1)) / math.sqrt(C)
        u = torch.rand((n, R, C // GROUP), device=dev, generator=g, dtype=torch.float32)
        s = (base * (0.9 + 0.2 * u)).to(torch.float16)
        z = (-s.to(torch.float32) * ((1 << b) - 1) / 2).to(torch.float16)
        pair = torch.stack([s, z], dim=-1).contiguous().view(torch.uint8).reshape(n, -1)
        pool[slots_t, off_sb:off_sb + pair.shape[1]] = pair
        del u, s, z, pair
    assert sb == lay.slot_bytes
