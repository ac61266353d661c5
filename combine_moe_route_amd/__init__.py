"""MoE token routing, dispatch and combine for one MI355X (gfx950).

The path runs in hand-written HIP kernels behind the C ABI of
``include/moe_route.h`` (libmoeroute.so, built by
``python -m combine_moe_route_amd.build``). This package is its thin ctypes
binding; torch provides device memory and the current stream only.

The binding is imported on first use of any API name, so building the
library never needs an existing one; using the API without the library
raises ImportError.
"""
_API = (
    "DispatchBuffers",
    "MoeRouteError",
    "alloc_dispatch",
    "moe_combine",
    "moe_combine_recv",
    "moe_combine_send",
    "moe_dispatch",
    "moe_dispatch_max_rows",
    "moe_dispatch_no_alloc",
    "moe_dispatch_workspace_bytes",
    "moe_grouped_gemm_fp8",
    "moe_grouped_gemm_workspace_bytes",
    "moe_harness_expert_scale",
    "moe_route_dispatch",
    "moe_route_replicas",
    "moe_route_topk",
    "moe_route_topk_shared",
    "status_string",
)

__all__ = list(_API)


def __getattr__(name):
    if name in _API:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")
