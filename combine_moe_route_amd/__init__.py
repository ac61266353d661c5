"""MoE token routing, dispatch and combine for one MI355X (gfx950).

The path runs in hand-written HIP kernels behind the C ABI of
``include/moe_route.h`` (libmoeroute.so, built by
``python -m combine_moe_route_amd.build``). This package is its thin ctypes
binding; torch provides device memory and the current stream only.
"""
from .binding import (  # noqa: F401
    DispatchBuffers,
    MoeRouteError,
    alloc_dispatch,
    moe_combine,
    moe_dispatch,
    moe_dispatch_max_rows,
    moe_dispatch_workspace_bytes,
    moe_harness_expert_scale,
    moe_route_topk,
    status_string,
)
