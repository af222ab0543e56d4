"""Thin ctypes binding of libmoe.so (include/moe.h).

Argument marshalling only: shapes, dtypes and devices of torch tensors are
checked, raw device pointers and the current HIP stream are passed on, and a
non-zero status becomes MoeError.  Every step of the layer runs in the HIP
kernels of libmoe.so; there is no fallback.  PyTorch only provides device
memory and streams.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "moe.h")

MOE_OK = 0
MOE_E_INVALID = -1
MOE_E_UNSUPPORTED = -2
MOE_E_NOT_RESIDENT = -3
MOE_E_NO_SLOT = -4
MOE_E_HIP = -5
MOE_E_BUSY = -6
MOE_E_WORKSPACE = -7
MOE_E_IO = -8

MOE_ERRW_NOT_RESIDENT = 0x1
MOE_ERRW_BAD_SLOT = 0x2
MOE_ERRW_NONFINITE = 0x4
MOE_ERRW_BAD_ID = 0x8
MOE_ERRW_TIMEOUT = 0x10

MOE_ROUTE_PLAIN = 0
MOE_ROUTE_SUBST = 1
MOE_PATH_AUTO = 0
MOE_PATH_GEMV = 1
MOE_PATH_MFMA = 2
MOE_PATH_GEMV3 = 3
MOE_SRC_HOST = 0
MOE_SRC_DEVICE = 1
MOE_DTYPE_F32 = 0
MOE_DTYPE_BF16 = 1
MOE_EVICT_LRU = 0
MOE_EVICT_LFU = 1

PASS_EXPERTS = 64

_lock = threading.Lock()
_lib = None


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"moe error {code}: {msg}")
        self.code = code


class SizeClassDesc(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("I", ctypes.c_int32), ("bits_gu", ctypes.c_int32),
                ("bits_d", ctypes.c_int32), ("group", ctypes.c_int32), ("align", ctypes.c_int32),
                ("n_slots", ctypes.c_int64), ("off_gu_codes", ctypes.c_int64),
                ("off_gu_sb", ctypes.c_int64), ("off_d_codes", ctypes.c_int64),
                ("off_d_sb", ctypes.c_int64), ("slot_bytes", ctypes.c_int64)]


class PipelineConfig(ctypes.Structure):
    _fields_ = [("host_tier_bytes", ctypes.c_int64), ("host_preload", ctypes.c_int32),
                ("io_threads", ctypes.c_int32), ("staging_rows", ctypes.c_int32),
                ("reserved0", ctypes.c_int32)]


class PipelineStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "requests", "hits", "inflight_hits", "host_hits", "store_reads", "prefetches",
        "prefetch_skipped", "bytes_copied", "bytes_read")]

    def as_dict(self) -> dict:
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


def lib() -> ctypes.CDLL:
    """Load libmoe.so; raises if it has not been built (no silent fallback)."""
    global _lib
    with _lock:
        if _lib is None:
            try:  # one HIP runtime per process: let torch load its own first
                import torch  # noqa: F401
            except ImportError:
                pass
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                                   "`python -m quantized_routed_expert_softmax_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            P, I32, I64, F32, SZ = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                                    ctypes.c_size_t)
            D = ctypes.POINTER(SizeClassDesc)
            sig = {
                "moe_size_class_init": (I32, [D, I32, I32, I32, I32, I32, I32, I64]),
                "moe_route_topk": (I32, [P, I32, I32, I32, I32, F32, P, P, P, P, P]),
                "moe_router_logits": (I32, [P, I32, I32, P, I32, I32, P, P]),
                "moe_sort_by_expert": (I32, [P, I32, I32, I32, I32, P, P, P, P, SZ, P, P]),
                "moe_sort_workspace_size": (SZ, [I32, I32, I32]),
                "moe_pass_table_size": (I32, [I32, I32]),
                "moe_experts_forward": (I32, [P, I32, P, P, I32, I32, P, P, D, P, P, SZ, P, P]),
                "moe_experts_forward_ex": (I32, [P, I32, P, P, I32, I32, P, P, D, P, P, SZ, P, I32, P]),
                "moe_forward_workspace_size": (SZ, [I32, I32, I32, D]),
                "moe_layer_forward": (I32, [P, I32, I32, I32, I32, F32, P, P, P, D, P, P, P, P, SZ, P, P]),
                "moe_layer_forward_static": (I32, [P, I32, I32, I32, I32, F32, P, P, P, D, P, P, P, P, P]),
                "moe_pass_table_host": (I32, [P, I32, I32, I32, I32, P]),
                "moe_prefill_sort": (I32, [P, I32, P, I32, I32, D, P, SZ, P, P]),
                "moe_prefill_pass": (I32, [I32, I32, I32, I32, I32, P, P, D, P, SZ, P, P]),
                "moe_prefill_combine": (I32, [I32, I32, I32, P, D, P, P, SZ, P]),
                "moe_cache_install": (I32, [P, D, I64, P, I32, P, P]),
                "moe_quantize_experts": (I32, [P, P, I32, I32, D, P, P]),
                "moe_cache_create": (P, [D, I32, P, I32, I32]),
                "moe_cache_create_ex": (P, [D, I32, P, I32, I32, I32, I32]),
                "moe_cache_destroy": (None, [P]),
                "moe_cache_acquire": (I32, [P, I32, I32, ctypes.POINTER(I64), ctypes.POINTER(I32)]),
                "moe_cache_fill_done": (I32, [P, I32, I32, P]),
                "moe_cache_poll": (I32, [P]),
                "moe_cache_pin": (I32, [P, I32, I32]),
                "moe_cache_unpin": (I32, [P, I32, I32]),
                "moe_cache_table": (I32, [P, I32, P]),
                "moe_cache_lookup": (I32, [P, I32, I32, ctypes.POINTER(I64)]),
                "moe_cache_stats": (I32, [P, ctypes.POINTER(I64), ctypes.POINTER(I64), ctypes.POINTER(I64)]),
                "moe_cache_class_of": (I32, [P, I32]),
                "moe_cache_shape": (I32, [P, ctypes.POINTER(I32), ctypes.POINTER(I32), ctypes.POINTER(I32)]),
                "moe_cache_class_desc": (I32, [P, I32, D]),
                "moe_cache_class_stats": (I32, [P, I32, ctypes.POINTER(I64), ctypes.POINTER(I64),
                                                ctypes.POINTER(I64)]),
                "moe_cache_abort_fill": (I32, [P, I32, I32]),
                "moe_store_open_file": (P, [ctypes.c_char_p, D, I32, P, I32, I32]),
                "moe_store_open_memory": (P, [P, I64, D, I32, P, I32, I32]),
                "moe_store_close": (None, [P]),
                "moe_store_bytes": (I64, [P]),
                "moe_store_row_offset": (I64, [P, I32, I32]),
                "moe_store_read": (I32, [P, I32, I32, P]),
                "moe_pipeline_create": (P, [P, P, P, ctypes.POINTER(PipelineConfig), P, I32]),
                "moe_pipeline_destroy": (None, [P]),
                "moe_pipeline_prepare": (I32, [P, I32, P, I32, P, P]),
                "moe_pipeline_release": (I32, [P, I32, P]),
                "moe_pipeline_prefetch": (I32, [P, I32, P, I32]),
                "moe_pipeline_prefill": (I32, [P, I32, P, P, I32, P, P, I32, P, P, P, SZ, P, P]),
                "moe_pipeline_drain": (I32, [P]),
                "moe_pipeline_stats_get": (I32, [P, I32, ctypes.POINTER(PipelineStats)]),
                "moe_pipeline_host_rows": (I64, [P, I32]),
                "moe_last_error": (ctypes.c_char_p, []),
            }
            for name, (res, args) in sig.items():
                f = getattr(L, name)
                f.restype = res
                f.argtypes = args
            _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/moe.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def _check(rc: int):
    if rc != MOE_OK:
        raise MoeError(rc, moe_last_error())


# --------------------------------------------------------------------------- #
# tensor marshalling                                                           #
# --------------------------------------------------------------------------- #
def _torch():
    import torch
    return torch


def _dev_ptr(t, dtype, name, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")
    return ctypes.c_void_p(t.data_ptr())


def _opt_ptr(t, dtype, name):
    return None if t is None else _dev_ptr(t, dtype, name)


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def moe_size_class_init(H: int, I: int, bits_gu: int, bits_d: int, n_slots: int,
                        group: int = 64, align: int = 256) -> SizeClassDesc:
    d = SizeClassDesc()
    _check(lib().moe_size_class_init(ctypes.byref(d), H, I, bits_gu, bits_d, group, align, n_slots))
    return d


def moe_route_topk(logits, k: int, mode: int = MOE_ROUTE_PLAIN, L: float = 0.0, slot_table=None,
                   topk_ids=None, topk_w=None, err_word=None, stream=None):
    """Softmax top-k routing (and cache-aware substitution in MOE_ROUTE_SUBST)."""
    torch = _torch()
    T, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check(lib().moe_route_topk(_dev_ptr(logits, torch.float32, "logits", 2), T, E, k, mode, L,
                                _opt_ptr(slot_table, torch.int32, "slot_table"),
                                _dev_ptr(topk_ids, torch.int32, "topk_ids"),
                                _dev_ptr(topk_w, torch.float32, "topk_w"),
                                _opt_ptr(err_word, torch.int32, "err_word"), _stream(stream)))
    return topk_ids, topk_w


def moe_router_logits(x, w, logits=None, stream=None):
    """Router logits of consecutive layers: x bf16 [T, H], w bf16 [n, E, H] -> fp32 [n, T, E]."""
    torch = _torch()
    T, H = x.shape
    n, E, H2 = w.shape
    if H2 != H:
        raise ValueError(f"router width {H2} differs from the hidden size {H}")
    if logits is None:
        logits = torch.empty((n, T, E), dtype=torch.float32, device=x.device)
    elif tuple(logits.shape) != (n, T, E):
        raise ValueError("logits must be [n, T, E]")
    _check(lib().moe_router_logits(_dev_ptr(x, torch.bfloat16, "x", 2), T, H,
                                   _dev_ptr(w, torch.bfloat16, "w", 3), n, E,
                                   _dev_ptr(logits, torch.float32, "logits", 3), _stream(stream)))
    return logits


def moe_pass_table_size(E: int, pass_experts: int = PASS_EXPERTS) -> int:
    return lib().moe_pass_table_size(E, pass_experts)


def moe_sort_workspace_size(T: int, k: int, E: int) -> int:
    return lib().moe_sort_workspace_size(T, k, E)


def moe_sort_by_expert(topk_ids, E: int, pass_experts: int = PASS_EXPERTS, err_word=None, ws=None,
                       stream=None):
    """Stable sort of (token, j) pairs by expert; returns (offsets, sorted_pairs, pass_table)."""
    torch = _torch()
    T, k = topk_ids.shape
    dev = topk_ids.device
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sorted_pairs = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    pass_table = torch.empty(moe_pass_table_size(E, pass_experts), dtype=torch.int32, device=dev)
    need = moe_sort_workspace_size(T, k, E)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check(lib().moe_sort_by_expert(_dev_ptr(topk_ids, torch.int32, "topk_ids", 2), T, k, E,
                                    pass_experts, _dev_ptr(offsets, None, "offsets"),
                                    _dev_ptr(sorted_pairs, None, "sorted_pairs"),
                                    _dev_ptr(pass_table, None, "pass_table"),
                                    _dev_ptr(ws, torch.uint8, "ws"), ws.numel(),
                                    _opt_ptr(err_word, torch.int32, "err_word"), _stream(stream)))
    return offsets, sorted_pairs[:T * k], pass_table


def moe_forward_workspace_size(T: int, k: int, E: int, desc: SizeClassDesc) -> int:
    return lib().moe_forward_workspace_size(T, k, E, ctypes.byref(desc))


def moe_experts_forward(x, topk_ids, topk_w, E: int, slot_table, slot_pool, desc: SizeClassDesc,
                        out=None, ws=None, err_word=None, path: int = MOE_PATH_AUTO, stream=None):
    """The routed experts of one layer: out = sum_j w_j * down(silu(gate x) * up x)."""
    torch = _torch()
    T, H = x.shape
    k = topk_ids.shape[1]
    if H != desc.H:
        raise ValueError(f"x has {H} columns, size class has H={desc.H}")
    if slot_pool.numel() < desc.n_slots * desc.slot_bytes:
        raise ValueError("slot_pool smaller than n_slots * slot_bytes")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if ws is None:  # zero-filled: the first MOE_WS_RESERVED_BYTES must start at zero
        ws = torch.zeros(max(moe_forward_workspace_size(T, k, E, desc), 256), dtype=torch.uint8,
                         device=x.device)
    _check(lib().moe_experts_forward_ex(
        _dev_ptr(x, torch.bfloat16, "x", 2), T, _dev_ptr(topk_ids, torch.int32, "topk_ids", 2),
        _dev_ptr(topk_w, torch.float32, "topk_w", 2), k, E,
        _dev_ptr(slot_table, torch.int32, "slot_table", 1), _dev_ptr(slot_pool, torch.uint8, "slot_pool"),
        ctypes.byref(desc), _dev_ptr(out, torch.bfloat16, "out", 2), _dev_ptr(ws, torch.uint8, "ws"),
        ws.numel(), _opt_ptr(err_word, torch.int32, "err_word"), path, _stream(stream)))
    return out


def moe_layer_forward(logits, x, slot_table, slot_pool, desc: SizeClassDesc, k: int,
                      mode: int = MOE_ROUTE_PLAIN, L: float = 0.0, topk_ids=None, topk_w=None, out=None,
                      ws=None, err_word=None, stream=None):
    """Router + routed experts of one layer (one launch for decode-sized batches).
    Returns (out, topk_ids, topk_w)."""
    torch = _torch()
    T, E = logits.shape
    H = x.shape[1]
    if H != desc.H:
        raise ValueError(f"x has {H} columns, size class has H={desc.H}")
    if slot_pool.numel() < desc.n_slots * desc.slot_bytes:
        raise ValueError("slot_pool smaller than n_slots * slot_bytes")
    dev = x.device
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if ws is None:
        ws = torch.zeros(max(moe_forward_workspace_size(T, k, E, desc), 256), dtype=torch.uint8, device=dev)
    _check(lib().moe_layer_forward(
        _dev_ptr(logits, torch.float32, "logits", 2), T, E, k, mode, L, _dev_ptr(x, torch.bfloat16, "x", 2),
        _dev_ptr(slot_table, torch.int32, "slot_table", 1), _dev_ptr(slot_pool, torch.uint8, "slot_pool"),
        ctypes.byref(desc), _dev_ptr(topk_ids, torch.int32, "topk_ids", 2),
        _dev_ptr(topk_w, torch.float32, "topk_w", 2), _dev_ptr(out, torch.bfloat16, "out", 2),
        _dev_ptr(ws, torch.uint8, "ws"), ws.numel(), _opt_ptr(err_word, torch.int32, "err_word"),
        _stream(stream)))
    return out, topk_ids, topk_w


def moe_pass_table_host(topk_ids, E: int, pass_experts: int = PASS_EXPERTS):
    """Pass table of host ids (int32 [T, k] numpy) computed on the host."""
    import numpy as np
    a = np.ascontiguousarray(topk_ids, dtype=np.int32)
    T, k = a.shape
    pt = np.empty(moe_pass_table_size(E, pass_experts), dtype=np.int32)
    _check(lib().moe_pass_table_host(ctypes.c_void_p(a.ctypes.data), T, k, E, pass_experts,
                                     ctypes.c_void_p(pt.ctypes.data)))
    return pt


def _fwd_ws(T, k, E, desc, ws, dev):
    torch = _torch()
    if ws is None:
        ws = torch.zeros(max(moe_forward_workspace_size(T, k, E, desc), 256), dtype=torch.uint8, device=dev)
    return ws


def moe_prefill_sort(x, topk_ids, E: int, desc: SizeClassDesc, ws=None, err_word=None, stream=None):
    """Sort the pairs by expert and permute x into the forward workspace; returns ws."""
    torch = _torch()
    T, H = x.shape
    k = topk_ids.shape[1]
    if H != desc.H:
        raise ValueError(f"x has {H} columns, size class has H={desc.H}")
    ws = _fwd_ws(T, k, E, desc, ws, x.device)
    _check(lib().moe_prefill_sort(_dev_ptr(x, torch.bfloat16, "x", 2), T,
                                  _dev_ptr(topk_ids, torch.int32, "topk_ids", 2), k, E, ctypes.byref(desc),
                                  _dev_ptr(ws, torch.uint8, "ws"), ws.numel(),
                                  _opt_ptr(err_word, torch.int32, "err_word"), _stream(stream)))
    return ws


def moe_prefill_pass(T: int, k: int, E: int, pass_begin: int, pass_end: int, slot_table, slot_pool,
                     desc: SizeClassDesc, ws, err_word=None, stream=None):
    """gate/up, SwiGLU and down of the hit experts of passes [pass_begin, pass_end)."""
    torch = _torch()
    if slot_pool.numel() < desc.n_slots * desc.slot_bytes:
        raise ValueError("slot_pool smaller than n_slots * slot_bytes")
    _check(lib().moe_prefill_pass(T, k, E, pass_begin, pass_end,
                                  _dev_ptr(slot_table, torch.int32, "slot_table", 1),
                                  _dev_ptr(slot_pool, torch.uint8, "slot_pool"), ctypes.byref(desc),
                                  _dev_ptr(ws, torch.uint8, "ws"), ws.numel(),
                                  _opt_ptr(err_word, torch.int32, "err_word"), _stream(stream)))


def moe_prefill_combine(topk_w, E: int, desc: SizeClassDesc, ws, out=None, stream=None):
    """out[t] = sum_j w[t, j] * y[t, j] after the last pass."""
    torch = _torch()
    T, k = topk_w.shape
    if out is None:
        out = torch.empty((T, desc.H), dtype=torch.bfloat16, device=topk_w.device)
    _check(lib().moe_prefill_combine(T, k, E, _dev_ptr(topk_w, torch.float32, "topk_w", 2),
                                     ctypes.byref(desc), _dev_ptr(out, torch.bfloat16, "out", 2),
                                     _dev_ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)))
    return out


MOE_STATIC_SCRATCH_BYTES = 8 << 20


def moe_layer_forward_static(logits, x, slot_table, slot_pool, desc: SizeClassDesc, k: int,
                             mode: int = MOE_ROUTE_PLAIN, L: float = 0.0, topk_ids=None, topk_w=None,
                             out=None, err_word=None, stream=None):
    """moe_layer_forward on the library's own scratch (no workspace argument; the
    library allocates nothing).  Returns (out, topk_ids, topk_w)."""
    torch = _torch()
    T, E = logits.shape
    H = x.shape[1]
    if H != desc.H:
        raise ValueError(f"x has {H} columns, size class has H={desc.H}")
    if slot_pool.numel() < desc.n_slots * desc.slot_bytes:
        raise ValueError("slot_pool smaller than n_slots * slot_bytes")
    dev = x.device
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _check(lib().moe_layer_forward_static(
        _dev_ptr(logits, torch.float32, "logits", 2), T, E, k, mode, L, _dev_ptr(x, torch.bfloat16, "x", 2),
        _dev_ptr(slot_table, torch.int32, "slot_table", 1), _dev_ptr(slot_pool, torch.uint8, "slot_pool"),
        ctypes.byref(desc), _dev_ptr(topk_ids, torch.int32, "topk_ids", 2),
        _dev_ptr(topk_w, torch.float32, "topk_w", 2), _dev_ptr(out, torch.bfloat16, "out", 2),
        _opt_ptr(err_word, torch.int32, "err_word"), _stream(stream)))
    return out, topk_ids, topk_w


def moe_quantize_experts(w_gu, w_d, desc: SizeClassDesc, out=None, stream=None):
    """Slot rows (uint8 [n, slot_bytes], device) of n experts from gate_up
    [n, 2I, H] and down [n, H, I] weights (float32 or bfloat16, device)."""
    torch = _torch()
    if w_gu.dtype != w_d.dtype or w_gu.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("weights must both be float32 or both bfloat16")
    n = w_gu.shape[0]
    if tuple(w_gu.shape) != (n, 2 * desc.I, desc.H) or tuple(w_d.shape) != (n, desc.H, desc.I):
        raise ValueError("weights must be [n, 2I, H] and [n, H, I]")
    if out is None:
        out = torch.empty((n, desc.slot_bytes), dtype=torch.uint8, device=w_gu.device)
    elif tuple(out.shape) != (n, desc.slot_bytes):
        raise ValueError("out must be [n, slot_bytes]")
    dt = MOE_DTYPE_F32 if w_gu.dtype == torch.float32 else MOE_DTYPE_BF16
    _check(lib().moe_quantize_experts(_dev_ptr(w_gu, None, "w_gu"), _dev_ptr(w_d, None, "w_d"), dt, n,
                                      ctypes.byref(desc), _dev_ptr(out, torch.uint8, "out"), _stream(stream)))
    return out


def moe_cache_install(slot_pool, desc: SizeClassDesc, slot: int, src, stream=None, event=None):
    """Async copy of one expert row into `slot`; src is a pinned host or device uint8 tensor."""
    torch = _torch()
    if src.numel() < desc.slot_bytes or src.dtype != torch.uint8 or not src.is_contiguous():
        raise ValueError("src must be a contiguous uint8 tensor of at least slot_bytes")
    if src.device.type == "cuda":
        kind = MOE_SRC_DEVICE
    else:
        if not src.is_pinned():
            raise ValueError("host source must be pinned memory")
        kind = MOE_SRC_HOST
    ev = None if event is None else ctypes.c_void_p(event.cuda_event)
    _check(lib().moe_cache_install(_dev_ptr(slot_pool, torch.uint8, "slot_pool"), ctypes.byref(desc),
                                   slot, ctypes.c_void_p(src.data_ptr()), kind, _stream(stream), ev))


# --------------------------------------------------------------------------- #
# host cache                                                                   #
# --------------------------------------------------------------------------- #
def moe_cache_create(classes: list[SizeClassDesc], layer_class: list[int], E: int,
                     policy: int = MOE_EVICT_LRU, per_layer: bool = False) -> int:
    arr = (SizeClassDesc * len(classes))(*classes)
    lc = (ctypes.c_int32 * len(layer_class))(*layer_class)
    if policy == MOE_EVICT_LRU and not per_layer:
        h = lib().moe_cache_create(arr, len(classes), lc, len(layer_class), E)
    else:
        h = lib().moe_cache_create_ex(arr, len(classes), lc, len(layer_class), E, policy, int(per_layer))
    if not h:
        raise MoeError(MOE_E_INVALID, moe_last_error())
    return h


def moe_cache_destroy(c: int):
    lib().moe_cache_destroy(c)


def moe_cache_acquire(c: int, layer: int, expert: int) -> tuple[int, int, int]:
    """Returns (status, slot, needs_fill); status is MOE_OK or MOE_E_BUSY, other
    codes raise."""
    slot = ctypes.c_int64(-1)
    nf = ctypes.c_int32(0)
    rc = lib().moe_cache_acquire(c, layer, expert, ctypes.byref(slot), ctypes.byref(nf))
    if rc not in (MOE_OK, MOE_E_BUSY):
        _check(rc)
    return rc, slot.value, nf.value


def moe_cache_fill_done(c: int, layer: int, expert: int, event=None):
    ev = None if event is None else ctypes.c_void_p(event.cuda_event)
    _check(lib().moe_cache_fill_done(c, layer, expert, ev))


def moe_cache_poll(c: int) -> int:
    rc = lib().moe_cache_poll(c)
    if rc < 0:
        _check(rc)
    return rc


def moe_cache_pin(c: int, layer: int, expert: int):
    _check(lib().moe_cache_pin(c, layer, expert))


def moe_cache_unpin(c: int, layer: int, expert: int):
    _check(lib().moe_cache_unpin(c, layer, expert))


def moe_cache_table(c: int, layer: int, E: int):
    import numpy as np
    t = np.empty(E, dtype=np.int32)
    _check(lib().moe_cache_table(c, layer, t.ctypes.data_as(ctypes.c_void_p)))
    return t


def moe_cache_lookup(c: int, layer: int, expert: int) -> int:
    s = ctypes.c_int64(-1)
    _check(lib().moe_cache_lookup(c, layer, expert, ctypes.byref(s)))
    return s.value


def moe_cache_stats(c: int) -> tuple[int, int, int]:
    h, m, e = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib().moe_cache_stats(c, ctypes.byref(h), ctypes.byref(m), ctypes.byref(e)))
    return h.value, m.value, e.value


def moe_cache_class_of(c: int, layer: int) -> int:
    return lib().moe_cache_class_of(c, layer)


def moe_cache_shape(c: int) -> tuple[int, int, int]:
    a, b, e = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(lib().moe_cache_shape(c, ctypes.byref(a), ctypes.byref(b), ctypes.byref(e)))
    return a.value, b.value, e.value


def moe_cache_class_desc(c: int, cls: int) -> SizeClassDesc:
    d = SizeClassDesc()
    _check(lib().moe_cache_class_desc(c, cls, ctypes.byref(d)))
    return d


def moe_cache_class_stats(c: int, cls: int) -> tuple[int, int, int]:
    h, m, e = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib().moe_cache_class_stats(c, cls, ctypes.byref(h), ctypes.byref(m), ctypes.byref(e)))
    return h.value, m.value, e.value


def moe_cache_abort_fill(c: int, layer: int, expert: int):
    _check(lib().moe_cache_abort_fill(c, layer, expert))


# --------------------------------------------------------------------------- #
# expert store and miss pipeline                                               #
# --------------------------------------------------------------------------- #
_store_refs: dict = {}  # memory stores: keep the caller's bytes alive until close


def _classes_arg(classes, layer_class):
    arr = (SizeClassDesc * len(classes))(*classes)
    lc = (ctypes.c_int32 * len(layer_class))(*layer_class)
    return arr, lc


def moe_store_open_file(path: str, classes: list[SizeClassDesc], layer_class: list[int], E: int) -> int:
    arr, lc = _classes_arg(classes, layer_class)
    h = lib().moe_store_open_file(os.fsencode(path), arr, len(classes), lc, len(layer_class), E)
    if not h:
        raise MoeError(MOE_E_IO, moe_last_error())
    return h


def moe_store_open_memory(mem, classes: list[SizeClassDesc], layer_class: list[int], E: int) -> int:
    """`mem`: a C-contiguous uint8 numpy array or CPU torch tensor (kept alive here)."""
    import numpy as np
    if isinstance(mem, np.ndarray):
        if mem.dtype != np.uint8 or not mem.flags["C_CONTIGUOUS"]:
            raise ValueError("store memory must be a contiguous uint8 array")
        ptr, nbytes = mem.ctypes.data, mem.nbytes
    else:
        torch = _torch()
        if mem.device.type != "cpu" or mem.dtype != torch.uint8 or not mem.is_contiguous():
            raise ValueError("store memory must be a contiguous uint8 CPU tensor")
        ptr, nbytes = mem.data_ptr(), mem.numel()
    arr, lc = _classes_arg(classes, layer_class)
    h = lib().moe_store_open_memory(ctypes.c_void_p(ptr), nbytes, arr, len(classes), lc,
                                    len(layer_class), E)
    if not h:
        raise MoeError(MOE_E_INVALID, moe_last_error())
    _store_refs[h] = mem
    return h


def moe_store_close(s: int):
    lib().moe_store_close(s)
    _store_refs.pop(s, None)


def moe_store_bytes(s: int) -> int:
    return lib().moe_store_bytes(s)


def moe_store_row_offset(s: int, layer: int, expert: int) -> int:
    o = lib().moe_store_row_offset(s, layer, expert)
    if o < 0:
        raise MoeError(MOE_E_INVALID, moe_last_error())
    return o


def moe_store_read(s: int, layer: int, expert: int, dst):
    """Read one row into the contiguous uint8 numpy array `dst`."""
    if dst.dtype.itemsize != 1 or not dst.flags["C_CONTIGUOUS"]:
        raise ValueError("dst must be a contiguous byte array")
    _check(lib().moe_store_read(s, layer, expert, ctypes.c_void_p(dst.ctypes.data)))


def moe_pipeline_create(cache: int, store: int, pools: list, host_tier_bytes: int = 0,
                        host_preload: bool = False, io_threads: int = 4, staging_rows: int = 8,
                        copy_streams=None) -> int:
    """pools[c]: class c's device pool (uint8 tensor); copy_streams: torch streams (1 to 4)."""
    torch = _torch()
    ptrs = (ctypes.c_void_p * len(pools))(*[_dev_ptr(p, torch.uint8, f"pools[{i}]").value
                                           for i, p in enumerate(pools)])
    cfg = PipelineConfig(host_tier_bytes, int(bool(host_preload)), io_threads, staging_rows, 0)
    if not copy_streams:
        raise ValueError("copy_streams is required")
    if not isinstance(copy_streams, (list, tuple)):
        copy_streams = [copy_streams]
    arr = (ctypes.c_void_p * len(copy_streams))(*[_stream(st).value for st in copy_streams])
    h = lib().moe_pipeline_create(cache, store, ptrs, ctypes.byref(cfg), arr, len(copy_streams))
    if not h:
        raise MoeError(MOE_E_INVALID, moe_last_error())
    return h


def moe_pipeline_destroy(p: int):
    lib().moe_pipeline_destroy(p)


def _ids_arg(ids):
    import numpy as np
    a = np.ascontiguousarray(np.asarray(ids, dtype=np.int32).reshape(-1))
    return a, ctypes.c_void_p(a.ctypes.data), a.size


def moe_pipeline_prepare(p: int, layer: int, ids, table_dev, stream=None):
    """ids: host int32 array of the layer's routed experts (any shape)."""
    torch = _torch()
    a, ptr, n = _ids_arg(ids)
    _check(lib().moe_pipeline_prepare(p, layer, ptr, n, _dev_ptr(table_dev, torch.int32, "table_dev", 1),
                                      _stream(stream)))


def moe_pipeline_release(p: int, layer: int, stream=None):
    _check(lib().moe_pipeline_release(p, layer, _stream(stream)))


def moe_pipeline_prefetch(p: int, layer: int, ids) -> int:
    a, ptr, n = _ids_arg(ids)
    rc = lib().moe_pipeline_prefetch(p, layer, ptr, n)
    if rc < 0:
        raise MoeError(rc, moe_last_error())
    return rc


def moe_pipeline_prefill(p: int, layer: int, ids_host, x, topk_ids, topk_w, table_dev, desc: SizeClassDesc,
                         out=None, ws=None, err_word=None, stream=None) -> tuple:
    """One prefill layer pass by pass through the cache; returns (out, passes run).
    `desc` is the layer's size class (it sizes the workspace)."""
    torch = _torch()
    import numpy as np
    T, H = x.shape
    k = topk_ids.shape[1]
    E = table_dev.shape[0]
    a = np.ascontiguousarray(ids_host, dtype=np.int32)
    if a.shape != (T, k):
        raise ValueError("ids_host must be [T, k]")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    ws = _fwd_ws(T, k, E, desc, ws, x.device)
    rc = lib().moe_pipeline_prefill(p, layer, ctypes.c_void_p(a.ctypes.data),
                                    _dev_ptr(x, torch.bfloat16, "x", 2), T,
                                    _dev_ptr(topk_ids, torch.int32, "topk_ids", 2),
                                    _dev_ptr(topk_w, torch.float32, "topk_w", 2), k,
                                    _dev_ptr(table_dev, torch.int32, "table_dev", 1),
                                    _dev_ptr(out, torch.bfloat16, "out", 2), _dev_ptr(ws, torch.uint8, "ws"),
                                    ws.numel(), _opt_ptr(err_word, torch.int32, "err_word"), _stream(stream))
    if rc < 0:
        raise MoeError(rc, moe_last_error())
    return out, rc


def moe_pipeline_drain(p: int):
    _check(lib().moe_pipeline_drain(p))


def moe_pipeline_stats_get(p: int, cls: int) -> dict:
    st = PipelineStats()
    _check(lib().moe_pipeline_stats_get(p, cls, ctypes.byref(st)))
    return st.as_dict()


def moe_pipeline_host_rows(p: int, cls: int) -> int:
    return lib().moe_pipeline_host_rows(p, cls)
