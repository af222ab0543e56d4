"""CPU oracle of the routed-expert MoE layer (ctypes wrapper around moe_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path.  It shares no code with
the GPU library.  Every function says which page passage it follows; the C file
holds the arithmetic.

All arrays are numpy.  Routing and sorting return exactly what the GPU must
return (fp32 decision, integer indices); the layer returns fp64 outputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

RC_NAMES = {0: "ok", 1: "invalid argument", 2: "routed expert not resident",
            3: "slot out of range", 4: "non-finite logit", 5: "expert id out of range"}


class OracleError(RuntimeError):
    def __init__(self, rc: int):
        super().__init__(f"oracle: {RC_NAMES.get(rc, rc)}")
        self.rc = rc


def build(force: bool = False) -> str:
    """Compile moe_oracle.c with gcc (no contraction of fp32 mul+add)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp",
                               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            i32, i64, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_float
            lib.oracle_exp_c.argtypes = [f32]
            lib.oracle_exp_c.restype = f32
            lib.oracle_softmax.argtypes = [P, i32, i32, P]
            lib.oracle_route.argtypes = [P, i32, i32, i32, i32, f32, P, P, P, P]
            lib.oracle_sort.argtypes = [P, i32, i32, i32, i32, P, P, P]
            lib.oracle_layout.argtypes = [i32, i32, i32, i32, P]
            lib.oracle_code.argtypes = [P, i32, i32]
            lib.oracle_code.restype = ctypes.c_uint32
            lib.oracle_dequant.argtypes = [P, i32, i32, i32, i32, i32, P]
            lib.oracle_layer.argtypes = [P, i32, i32, i32, i32, i32, P, P, i32, i32, P, P, i64,
                                         P, i32, P, i32]
            lib.oracle_router_logits.argtypes = [P, i32, i32, P, i32, i32, P]
            lib.oracle_round_half.argtypes = [ctypes.c_double]
            lib.oracle_round_half.restype = ctypes.c_uint16
            lib.oracle_round_bf16.argtypes = [ctypes.c_double]
            lib.oracle_round_bf16.restype = ctypes.c_uint16
            lib.oracle_quantize.argtypes = [P, i32, i32, i32, P, P, P]
            lib.oracle_convert_expert.argtypes = [P, P, i32, i32, i32, i32, P]
            for f in ("oracle_softmax", "oracle_route", "oracle_sort", "oracle_layout",
                      "oracle_dequant", "oracle_layer", "oracle_router_logits", "oracle_quantize",
                      "oracle_convert_expert"):
                getattr(lib, f).restype = ctypes.c_int
            _lib = lib
    return _lib


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int):
    if rc != 0:
        raise OracleError(rc)


def exp_c(x) -> np.ndarray:
    """The routing contract's exp on fp32 inputs (Cody-Waite + degree-7 Taylor)."""
    lib = _load()
    xs = np.asarray(x, dtype=np.float32).ravel()
    return np.array([lib.oracle_exp_c(float(v)) for v in xs], dtype=np.float32).reshape(np.shape(x))


def softmax(logits: np.ndarray) -> np.ndarray:
    """fp32 softmax per token in the contract's summation order."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = lg.shape
    p = np.empty((T, E), dtype=np.float32)
    _check(_load().oracle_softmax(_p(lg), T, E, _p(p)))
    return p


def route(logits: np.ndarray, k: int, mode: int = 0, L: float = 0.0,
          slot_table: np.ndarray | None = None, return_p: bool = False):
    """Softmax top-k with renormalised weights ("RFC ...", Motivation);
    mode 1 = cache-aware substitution (BigMoeOnEdge substitution commit)."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = lg.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    p = np.empty((T, E), dtype=np.float32)
    st = None if slot_table is None else np.ascontiguousarray(slot_table, dtype=np.int32)
    _check(_load().oracle_route(_p(lg), T, E, k, mode, float(L), _p(st), _p(ids), _p(w), _p(p)))
    return (ids, w, p) if return_p else (ids, w)


def pass_table_size(E: int, P: int) -> int:
    return 2 + E + (E + P - 1) // P + 1


def sort(ids: np.ndarray, E: int, P: int = 64):
    """Stable sort of pair ids by expert and the pass table ("POC: Experts
    offload", commit messages: the sorted prefill's batches of 64 experts)."""
    a = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = a.shape
    off = np.empty(E + 1, dtype=np.int32)
    sp = np.empty(T * k, dtype=np.int32)
    pt = np.empty(pass_table_size(E, P), dtype=np.int32)
    _check(_load().oracle_sort(_p(a), T, k, E, P, _p(off), _p(sp), _p(pt)))
    return off, sp, pt


def layout(H: int, I: int, bits_gu: int, bits_d: int) -> np.ndarray:
    """[gate_up codes, gate_up scale/bias, down codes, down scale/bias, slot bytes]."""
    offs = np.empty(5, dtype=np.int64)
    _check(_load().oracle_layout(H, I, bits_gu, bits_d, _p(offs)))
    return offs


def code(row: np.ndarray, bits: int, c: int) -> int:
    r = np.ascontiguousarray(row, dtype=np.uint8)
    return int(_load().oracle_code(_p(r), bits, c))


def dequant(slot_row: np.ndarray, H: int, I: int, bits_gu: int, bits_d: int, which: int) -> np.ndarray:
    """Dequantized gate_up [2I, H] (which=0) or down [H, I] (which=1), fp64."""
    r = np.ascontiguousarray(slot_row, dtype=np.uint8)
    shape = (2 * I, H) if which == 0 else (H, I)
    out = np.empty(shape, dtype=np.float64)
    _check(_load().oracle_dequant(_p(r), H, I, bits_gu, bits_d, which, _p(out)))
    return out


def layer(x_bf16: np.ndarray, ids: np.ndarray, w: np.ndarray, slot_table: np.ndarray,
          pool: np.ndarray, H: int, I: int, bits_gu: int, bits_d: int, E: int,
          tokens: np.ndarray | None = None, threads: int = 1) -> np.ndarray:
    """The routed-expert layer in fp64 for all tokens (or the listed ones):
    out[t] = sum_j w[t,j] * down_e(silu(gate_e x_t) * up_e x_t) ("RFC ...",
    How the prototype works: gated, concatenated, untransposed experts, no bias)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    T = x.shape[0]
    a = np.ascontiguousarray(ids, dtype=np.int32)
    k = a.shape[1]
    ww = np.ascontiguousarray(w, dtype=np.float32)
    st = np.ascontiguousarray(slot_table, dtype=np.int32)
    pl = np.ascontiguousarray(pool, dtype=np.uint8)
    n_slots = pl.shape[0]
    tk = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    n_out = T if tk is None else tk.shape[0]
    out = np.empty((n_out, H), dtype=np.float64)
    _check(_load().oracle_layer(_p(x), T, H, I, bits_gu, bits_d, _p(a), _p(ww), k, E, _p(st),
                                _p(pl), n_slots, _p(tk), n_out, _p(out), threads))
    return out


def router_logits(x_bf16: np.ndarray, w_bf16: np.ndarray) -> np.ndarray:
    """Router logits of consecutive layers on one set of hidden states, fp64:
    logits[m, t, e] = sum_i x[t, i] * Wr_m[e, i] ("RFC ...", How the prototype
    works, Reads: applying the following layers' routers to the present hidden
    state predicts their experts).  x: bf16 bits [T, H]; w: bf16 bits [n, E, H]."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    T, H = x.shape
    n, E, H2 = w.shape
    if H2 != H:
        raise ValueError("router width differs from the hidden size")
    out = np.empty((n, T, E), dtype=np.float64)
    _check(_load().oracle_router_logits(_p(x), T, H, _p(w), n, E, _p(out)))
    return out


# --------------------------------------------------------------------------- #
# One-time conversion of expert weights ("RFC: stream MoE experts from disk in  #
# from_pretrained", How the prototype works, Quantized experts bullet)         #
# --------------------------------------------------------------------------- #
def round_half(x: float) -> int:
    """fp16 bit pattern nearest to x (ties to the even pattern)."""
    return int(_load().oracle_round_half(float(x)))


def round_bf16(x: float) -> int:
    """bf16 bit pattern nearest to x (ties to the even pattern)."""
    return int(_load().oracle_round_bf16(float(x)))


def quantize(w: np.ndarray, bits: int):
    """Min/max affine quantization of an fp32 [R, C] matrix in groups of 64 along C:
    (codes uint8 [R, C], scale fp16 bits uint16 [R, C/64], bias fp16 bits uint16 [R, C/64])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    R, C = w.shape
    q = np.empty((R, C), dtype=np.uint8)
    s = np.empty((R, C // 64), dtype=np.uint16)
    z = np.empty((R, C // 64), dtype=np.uint16)
    _check(_load().oracle_quantize(_p(w), R, C, bits, _p(q), _p(s), _p(z)))
    return q, s, z


def convert_expert(w_gu: np.ndarray, w_d: np.ndarray, H: int, I: int, bits_gu: int, bits_d: int) -> np.ndarray:
    """One expert's slot row (uint8 [slot_bytes]) from fp32 gate_up [2I, H] and down [H, I]."""
    a = np.ascontiguousarray(w_gu, dtype=np.float32)
    b = np.ascontiguousarray(w_d, dtype=np.float32)
    assert a.shape == (2 * I, H) and b.shape == (H, I)
    row = np.empty(int(layout(H, I, bits_gu, bits_d)[4]), dtype=np.uint8)
    _check(_load().oracle_convert_expert(_p(a), _p(b), H, I, bits_gu, bits_d, _p(row)))
    return row
