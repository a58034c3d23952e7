"""Routed-expert MoE execution on one MI355X (gfx950).

The hot path lives in libmoert.so (HIP kernels + host C++), declared in
include/moert.h; ``binding`` exposes its C-ABI calls under the same names.
"""
from .binding import (  # noqa: F401
    MOE_BF16, MOE_CPU, MOE_F32, MOE_HYBRID, MOE_MXFP4, MOE_OFFLOAD, MoeConfig, MoertError,
    PlanView, PrefillView, Stats, config, lib, moe_cache_plan, moe_cache_resize, moe_create, moe_ctx_stats,
    moe_ctx_timing, moe_destroy, moe_expert_bytes, moe_expert_ffn, moe_host_pool_alloc, moe_host_pool_free,
    moe_last_error, moe_measure_bandwidth, moe_merge, moe_plan_view_get, moe_prefill_layer, moe_prefill_layer_noalloc, moe_prefill_view_get,
    moe_prefill_set_buffers, moe_recommend_mode, moe_route_topk, moe_set_cpu_layers, moe_set_split,
    moe_strerror)
