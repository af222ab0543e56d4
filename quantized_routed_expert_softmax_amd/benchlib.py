"""ctypes binding of libmoebench.so: the model glue of the benchmark's decode
chain and the ceiling microbenchmarks (not part of the routed-expert layer).

Argument marshalling only; raises if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoebench.so")

_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            import torch  # noqa: F401  (one HIP runtime per process: torch's first)
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                                   "`python -m quantized_routed_expert_softmax_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            P, I32, I64, F32, U32 = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                                     ctypes.c_uint32)
            for name, args in {
                "mb_residual_rmsnorm": [P, P, I32, I32, F32, P, P, P],
                "mb_read_rows": [P, I32, I64, P, I32, P],
                "mb_chase": [P, U32, I32, I32, P, P],
                "mb_mfma_loop": [I32, I32, P, P],
                "mb_empty": [I32, I32, P],
            }.items():
                f = getattr(L, name)
                f.restype = I32
                f.argtypes = args
            _lib = L
    return _lib


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what} failed ({rc})")


def residual_rmsnorm(x, y, x_out, n_out, eps: float = 1e-6, stream=None):
    """x_out = x + y (bf16), n_out = rmsnorm(x_out) (no gain); y None: n_out = rmsnorm(x)."""
    import torch
    T, H = x.shape
    for t in (x, y, x_out, n_out):
        if t is not None and (t.dtype != torch.bfloat16 or not t.is_contiguous() or tuple(t.shape) != (T, H)):
            raise ValueError("residual_rmsnorm needs contiguous bf16 [T, H] tensors")
    _check(lib().mb_residual_rmsnorm(ctypes.c_void_p(x.data_ptr()),
                                     None if y is None else ctypes.c_void_p(y.data_ptr()), T, H, eps,
                                     None if x_out is None else ctypes.c_void_p(x_out.data_ptr()),
                                     ctypes.c_void_p(n_out.data_ptr()), _stream(stream)), "residual_rmsnorm")


def read_rows(rows_dev, n_rows: int, row_bytes: int, sink, wgs_per_row: int, stream=None):
    """Stream n_rows rows (device addresses in the int64 tensor rows_dev)."""
    _check(lib().mb_read_rows(ctypes.c_void_p(rows_dev.data_ptr()), n_rows, row_bytes,
                              ctypes.c_void_p(sink.data_ptr()), wgs_per_row, _stream(stream)), "read_rows")


def chase(next_buf, start: int, warm: int, hops: int, out, stream=None):
    """Follow the chain for `warm` untimed then `hops` timed loads; out (int32
    [2]) gets the node reached and the timed part's 100 MHz ticks."""
    _check(lib().mb_chase(ctypes.c_void_p(next_buf.data_ptr()), start, warm, hops,
                          ctypes.c_void_p(out.data_ptr()), _stream(stream)), "chase")


def mfma_loop(grid: int, iters: int, sink, stream=None):
    _check(lib().mb_mfma_loop(grid, iters, ctypes.c_void_p(sink.data_ptr()), _stream(stream)), "mfma_loop")


def empty(grid: int, block: int, stream=None):
    _check(lib().mb_empty(grid, block, _stream(stream)), "empty")
