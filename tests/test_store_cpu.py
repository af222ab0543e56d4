"""Expert store (host side of the miss pipeline): layer-major rows, each
expert a single unbroken row, file- or memory-backed.  No GPU call is made here.

Sources: "RFC: stream MoE experts from disk in from_pretrained", How the
prototype works, Quantized experts and Reads bullets (each expert a single
unbroken row, fetched by a single read); "POC: Experts offload", commit
message (one open file per shard serves every read).
"""
import ctypes

import numpy as np
import pytest

from quantized_routed_expert_softmax_amd import binding as B


def classes_two():
    a = B.moe_size_class_init(256, 128, 4, 4, 3)
    b = B.moe_size_class_init(256, 128, 4, 6, 2)
    return [a, b]


def rows_bytes(classes, layer_class, E, seed=0):
    rng = np.random.default_rng(seed)
    total = sum(E * classes[c].slot_bytes for c in layer_class)
    return rng.integers(0, 256, size=total, dtype=np.uint8)


@pytest.mark.parametrize("kind", ["file", "memory"])
def test_rows_read_back_from_their_offsets(kind, tmp_path):
    classes, layer_class, E = classes_two(), [0, 1, 0], 5
    data = rows_bytes(classes, layer_class, E)
    if kind == "file":
        path = tmp_path / "experts.bin"
        data.tofile(path)
        s = B.moe_store_open_file(str(path), classes, layer_class, E)
    else:
        s = B.moe_store_open_memory(data, classes, layer_class, E)
    try:
        assert B.moe_store_bytes(s) == data.size
        # offsets are running sums of E rows of each layer's class size
        base = 0
        for l, c in enumerate(layer_class):
            sb = classes[c].slot_bytes
            for e in range(E):
                off = B.moe_store_row_offset(s, l, e)
                assert off == base + e * sb
                dst = np.zeros(sb, dtype=np.uint8)
                B.moe_store_read(s, l, e, dst)
                assert np.array_equal(dst, data[off:off + sb])
            base += E * sb
        with pytest.raises(B.MoeError):
            B.moe_store_row_offset(s, 3, 0)
        with pytest.raises(B.MoeError):
            B.moe_store_read(s, 0, E, np.zeros(8, np.uint8))
    finally:
        B.moe_store_close(s)


def test_short_file_and_missing_file_are_io_errors(tmp_path):
    classes, layer_class, E = classes_two(), [0, 1], 4
    data = rows_bytes(classes, layer_class, E)
    path = tmp_path / "short.bin"
    data[:-1].tofile(path)
    with pytest.raises(B.MoeError) as ei:
        B.moe_store_open_file(str(path), classes, layer_class, E)
    assert ei.value.code == B.MOE_E_IO
    with pytest.raises(B.MoeError) as ei:
        B.moe_store_open_file(str(tmp_path / "absent.bin"), classes, layer_class, E)
    assert ei.value.code == B.MOE_E_IO
    with pytest.raises(B.MoeError):
        B.moe_store_open_memory(data[:-1], classes, layer_class, E)
    with pytest.raises(B.MoeError):
        B.moe_store_open_file(str(path), classes, [0, 2], E)   # class out of range


def test_pipeline_create_rejects_bad_configs_before_any_gpu_call():
    L = B.lib()
    classes, layer_class, E = classes_two(), [0, 1], 4
    data = rows_bytes(classes, layer_class, E)
    c = B.moe_cache_create(classes, layer_class, E)
    s = B.moe_store_open_memory(data, classes, layer_class, E)
    try:
        pools = (ctypes.c_void_p * 2)(0x10000, 0x20000)  # never dereferenced
        streams = (ctypes.c_void_p * 5)(*([0x1000] * 5))
        for threads, staging, host in ((0, 4, 0), (65, 80, 0), (4, 2, 0), (2, 4, -1)):
            cfg = B.PipelineConfig(host, 0, threads, staging, 0)
            assert not L.moe_pipeline_create(c, s, pools, ctypes.byref(cfg), streams, 1)
            assert B.moe_last_error()
        cfg = B.PipelineConfig(0, 0, 2, 4, 0)
        assert not L.moe_pipeline_create(None, s, pools, ctypes.byref(cfg), streams, 1)
        assert not L.moe_pipeline_create(c, None, pools, ctypes.byref(cfg), streams, 1)
        for n in (0, 5):                                   # 1 to 4 copy streams
            assert not L.moe_pipeline_create(c, s, pools, ctypes.byref(cfg), streams, n)
        nulls = (ctypes.c_void_p * 2)(0x1000, None)
        assert not L.moe_pipeline_create(c, s, pools, ctypes.byref(cfg), nulls, 2)
        s3 = B.moe_store_open_memory(rows_bytes(classes, [0, 1, 0], E), classes, [0, 1, 0], E)
        try:   # layer count differs from the cache's
            assert not L.moe_pipeline_create(c, s3, pools, ctypes.byref(cfg), streams, 1)
        finally:
            B.moe_store_close(s3)
    finally:
        B.moe_store_close(s)
        B.moe_cache_destroy(c)
