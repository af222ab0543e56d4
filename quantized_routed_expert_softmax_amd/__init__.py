"""Routed-expert MoE layer through a bounded, quantized expert cache, on AMD
Instinct MI355X (gfx950).

The layer runs in hand-written HIP kernels behind the C-ABI of include/moe.h
(libmoe.so, built by `build.py`); `binding` is its thin Python front end and
`synth` makes seeded synthetic inputs.
"""
from .binding import (  # noqa: F401
    MOE_ERRW_BAD_ID, MOE_ERRW_BAD_SLOT, MOE_ERRW_NONFINITE, MOE_ERRW_NOT_RESIDENT,
    MOE_ERRW_TIMEOUT, MOE_PATH_AUTO, MOE_PATH_GEMV, MOE_PATH_GEMV3, MOE_PATH_MFMA, MOE_ROUTE_PLAIN, MOE_ROUTE_SUBST,
    MoeError, SizeClassDesc, moe_cache_acquire, moe_cache_class_of, moe_cache_create,
    moe_cache_destroy, moe_cache_fill_done, moe_cache_install, moe_cache_lookup, moe_cache_pin,
    moe_cache_poll, moe_cache_stats, moe_cache_table, moe_cache_unpin, moe_experts_forward,
    moe_forward_workspace_size, moe_last_error, moe_layer_forward, moe_pass_table_size, moe_route_topk,
    moe_size_class_init, moe_sort_by_expert, moe_sort_workspace_size,
)
