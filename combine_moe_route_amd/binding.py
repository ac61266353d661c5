"""ctypes binding of libmoeroute (include/moe_route.h).

Argument marshalling only: tensors are checked for dtype, device, shape and
contiguity, their device pointers and torch's current HIP stream are handed
to the C ABI, and a non-zero status becomes a MoeRouteError. Every step of
the path runs in the library's HIP kernels; torch only owns the memory and
the stream. If the library is missing this module raises at import: there
is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MOE_ROUTE_LIB", os.path.join(_HERE, "libmoeroute.so"))

MOE_OK, MOE_EINVAL, MOE_ENOSPC, MOE_EALIGN, MOE_EHIP, MOE_ENULL = 0, -1, -2, -3, -4, -5
MOE_OUT_BF16, MOE_OUT_FP8_E4M3 = 0, 1
MOE_MAX_EXPERTS = 1024
MOE_NO_ALLOC_SCRATCH_BYTES = 16 << 20

# every symbol include/moe_route.h declares
EXPORTS = (
    "moe_route_topk",
    "moe_route_topk_shared",
    "moe_route_replicas",
    "moe_dispatch_max_rows",
    "moe_dispatch_workspace_bytes",
    "moe_dispatch",
    "moe_dispatch_no_alloc",
    "moe_route_dispatch",
    "moe_combine",
    "moe_combine_send",
    "moe_combine_recv",
    "moe_grouped_gemm_workspace_bytes",
    "moe_grouped_gemm_fp8",
    "moe_harness_expert_scale",
    "moe_status_string",
)


class MoeRouteError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libmoeroute.so not found at {LIB_PATH}; build it with "
            "`python -m combine_moe_route_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.moe_route_topk.argtypes = [P, i64, i32, i32, P, P, P]
    lib.moe_route_topk.restype = i32
    lib.moe_route_topk_shared.argtypes = [P, i64, i32, i32, i32, ctypes.c_float, P, P, P]
    lib.moe_route_topk_shared.restype = i32
    lib.moe_route_replicas.argtypes = [P, i64, i32, i32, P, P]
    lib.moe_route_replicas.restype = i32
    lib.moe_dispatch_max_rows.argtypes = [i64, i32, i32, i32]
    lib.moe_dispatch_max_rows.restype = i64
    lib.moe_dispatch_workspace_bytes.argtypes = [i64, i32, i32, i32]
    lib.moe_dispatch_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_dispatch.argtypes = [P, P, i64, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P,
                                 P, ctypes.c_size_t, P]
    lib.moe_dispatch.restype = i32
    lib.moe_dispatch_no_alloc.argtypes = [P, P, i64, i32, i32, i32, i32, i32, i32, P, P, P, P, P,
                                          P, P, P]
    lib.moe_dispatch_no_alloc.restype = i32
    lib.moe_route_dispatch.argtypes = [P, P, i64, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P,
                                       P, P, P, P, ctypes.c_size_t, P]
    lib.moe_route_dispatch.restype = i32
    lib.moe_combine.argtypes = [P, P, P, i64, i32, i32, P, P]
    lib.moe_combine.restype = i32
    lib.moe_combine_send.argtypes = [P, P, P, P, i64, i32, i32, i32, i32, P, P, P]
    lib.moe_combine_send.restype = i32
    lib.moe_combine_recv.argtypes = [P, P, i64, i32, i32, P, P]
    lib.moe_combine_recv.restype = i32
    lib.moe_grouped_gemm_workspace_bytes.argtypes = [i64, i32]
    lib.moe_grouped_gemm_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_grouped_gemm_fp8.argtypes = [P, P, P, P, P, i32, i32, i32, i64, P, P,
                                         ctypes.c_size_t, P]
    lib.moe_grouped_gemm_fp8.restype = i32
    lib.moe_harness_expert_scale.argtypes = [P, P, P, P, P, i64, i32, i32, i32, i32, P, P]
    lib.moe_harness_expert_scale.restype = i32
    lib.moe_status_string.argtypes = [i32]
    lib.moe_status_string.restype = ctypes.c_char_p
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.moe_status_string(status).decode()


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeRouteError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, shape=None, device=None):
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name}: must be a GPU tensor")
    if device is not None and t.device != device:
        raise TypeError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


# ----------------------------------------------------------------- routing

def moe_route_topk(logits: torch.Tensor, k: int, topk_idx: Optional[torch.Tensor] = None,
                   topk_w: Optional[torch.Tensor] = None):
    """(topk_idx int32 [T,k], topk_w float32 [T,k]) from fp32 logits [T,E]."""
    _need(logits, "logits", torch.float32)
    T, E = logits.shape
    dev = logits.device
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _need(topk_idx, "topk_idx", torch.int32, (T, k), dev)
    _need(topk_w, "topk_w", torch.float32, (T, k), dev)
    _check("moe_route_topk", lib.moe_route_topk(_ptr(logits), T, E, k, _ptr(topk_idx),
                                                _ptr(topk_w), _stream(dev)))
    return topk_idx, topk_w


def moe_route_topk_shared(logits: torch.Tensor, k: int, n_shared: int, shared_w: float = 1.0,
                          topk_idx: Optional[torch.Tensor] = None,
                          topk_w: Optional[torch.Tensor] = None):
    """Routed top-k plus n_shared always-chosen experts E..E+n_shared-1:
    (topk_idx int32 [T,k+n_shared], topk_w float32 [T,k+n_shared])."""
    _need(logits, "logits", torch.float32)
    T, E = logits.shape
    dev = logits.device
    ks = k + n_shared
    if topk_idx is None:
        topk_idx = torch.empty((T, ks), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, ks), dtype=torch.float32, device=dev)
    _need(topk_idx, "topk_idx", torch.int32, (T, ks), dev)
    _need(topk_w, "topk_w", torch.float32, (T, ks), dev)
    _check("moe_route_topk_shared", lib.moe_route_topk_shared(
        _ptr(logits), T, E, k, n_shared, float(shared_w), _ptr(topk_idx), _ptr(topk_w),
        _stream(dev)))
    return topk_idx, topk_w


def moe_route_replicas(topk_idx: torch.Tensor, E: int, replica_base: torch.Tensor) -> torch.Tensor:
    """In place: logical expert ids -> physical replica ids (copy t mod count)."""
    _need(topk_idx, "topk_idx", torch.int32)
    dev = topk_idx.device
    T, k = topk_idx.shape
    _need(replica_base, "replica_base", torch.int32, (E + 1,), dev)
    _check("moe_route_replicas", lib.moe_route_replicas(_ptr(topk_idx), T, k, E,
                                                        _ptr(replica_base), _stream(dev)))
    return topk_idx


# ----------------------------------------------------------------- dispatch

def moe_dispatch_max_rows(T: int, E: int, k: int, row_align: int = 1) -> int:
    n = lib.moe_dispatch_max_rows(T, E, k, row_align)
    if n < 0:
        raise MoeRouteError("moe_dispatch_max_rows", MOE_EINVAL)
    return n


def moe_dispatch_workspace_bytes(T: int, E: int, k: int, groups: int = 1) -> int:
    return lib.moe_dispatch_workspace_bytes(T, E, k, groups)


class DispatchBuffers(NamedTuple):
    out: torch.Tensor             # [max_rows, H] bfloat16 or uint8 (E4M3 codes)
    out_scales: Optional[torch.Tensor]  # [max_rows, H/128] float32 (FP8 only)
    expert_counts: torch.Tensor   # [E] int32
    expert_offsets: torch.Tensor  # [E+1] int32; [E] = rows used
    group_offsets: torch.Tensor   # [groups+1] int32
    row_src: torch.Tensor         # [max_rows] int32
    dst_row: torch.Tensor         # [T, k] int32
    workspace: torch.Tensor       # uint8 workspace


def alloc_dispatch(T: int, H: int, E: int, k: int, groups: int = 1, row_align: int = 1,
                   fp8: bool = False, device="cuda", workspace: bool = True) -> DispatchBuffers:
    """Capacity-sized output buffers and workspace for moe_dispatch and
    moe_route_dispatch (a 16-byte placeholder workspace when `workspace` is
    false, for moe_dispatch_no_alloc)."""
    dev = torch.device(device)
    R = moe_dispatch_max_rows(T, E, k, row_align)
    ws = max(moe_dispatch_workspace_bytes(T, E, k, groups), 16) if workspace else 16
    return DispatchBuffers(
        out=torch.empty((R, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev),
        out_scales=torch.empty((R, H // 128), dtype=torch.float32, device=dev) if fp8 else None,
        expert_counts=torch.empty(E, dtype=torch.int32, device=dev),
        expert_offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
        group_offsets=torch.empty(groups + 1, dtype=torch.int32, device=dev),
        row_src=torch.empty(R, dtype=torch.int32, device=dev),
        dst_row=torch.empty((T, k), dtype=torch.int32, device=dev),
        workspace=torch.empty(ws, dtype=torch.uint8, device=dev),
    )


def moe_dispatch(x: torch.Tensor, topk_idx: torch.Tensor, E: int, groups: int = 1,
                 row_align: int = 1, fp8: bool = False,
                 bufs: Optional[DispatchBuffers] = None) -> DispatchBuffers:
    """Stable per-expert scatter of bf16 x [T,H] (see include/moe_route.h)."""
    _need(x, "x", torch.bfloat16)
    T, H = x.shape
    dev = x.device
    _need(topk_idx, "topk_idx", torch.int32, None, dev)
    if topk_idx.dim() != 2 or topk_idx.shape[0] != T:
        raise ValueError(f"topk_idx: shape {tuple(topk_idx.shape)}, expected ({T}, k)")
    k = topk_idx.shape[1]
    if bufs is None:
        bufs = alloc_dispatch(T, H, E, k, groups, row_align, fp8, dev)
    R = moe_dispatch_max_rows(T, E, k, row_align)
    _need(bufs.out, "out", torch.uint8 if fp8 else torch.bfloat16, (R, H), dev)
    if fp8:
        _need(bufs.out_scales, "out_scales", torch.float32, (R, H // 128), dev)
    _need(bufs.expert_counts, "expert_counts", torch.int32, (E,), dev)
    _need(bufs.expert_offsets, "expert_offsets", torch.int32, (E + 1,), dev)
    _need(bufs.group_offsets, "group_offsets", torch.int32, (groups + 1,), dev)
    _need(bufs.row_src, "row_src", torch.int32, (R,), dev)
    _need(bufs.dst_row, "dst_row", torch.int32, (T, k), dev)
    _need(bufs.workspace, "workspace", torch.uint8, None, dev)
    _check("moe_dispatch", lib.moe_dispatch(
        _ptr(x), _ptr(topk_idx), T, H, E, k, groups, row_align,
        MOE_OUT_FP8_E4M3 if fp8 else MOE_OUT_BF16, _ptr(bufs.out),
        _ptr(bufs.out_scales) if fp8 else None, _ptr(bufs.expert_counts),
        _ptr(bufs.expert_offsets), _ptr(bufs.group_offsets), _ptr(bufs.row_src),
        _ptr(bufs.dst_row), _ptr(bufs.workspace), bufs.workspace.numel(), _stream(dev)))
    return bufs


def moe_route_dispatch(logits: torch.Tensor, x: torch.Tensor, k: int, groups: int = 1,
                       row_align: int = 1, fp8: bool = False,
                       bufs: Optional[DispatchBuffers] = None,
                       topk_idx: Optional[torch.Tensor] = None,
                       topk_w: Optional[torch.Tensor] = None):
    """Routing and dispatch in one call: (topk_idx int32 [T,k], topk_w float32
    [T,k], DispatchBuffers), the same results as moe_route_topk followed by
    moe_dispatch."""
    _need(logits, "logits", torch.float32)
    T, E = logits.shape
    dev = logits.device
    _need(x, "x", torch.bfloat16, None, dev)
    if x.dim() != 2 or x.shape[0] != T:
        raise ValueError(f"x: shape {tuple(x.shape)}, expected ({T}, H)")
    H = x.shape[1]
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _need(topk_idx, "topk_idx", torch.int32, (T, k), dev)
    _need(topk_w, "topk_w", torch.float32, (T, k), dev)
    if bufs is None:
        bufs = alloc_dispatch(T, H, E, k, groups, row_align, fp8, dev)
    R = moe_dispatch_max_rows(T, E, k, row_align)
    _need(bufs.out, "out", torch.uint8 if fp8 else torch.bfloat16, (R, H), dev)
    if fp8:
        _need(bufs.out_scales, "out_scales", torch.float32, (R, H // 128), dev)
    _need(bufs.expert_counts, "expert_counts", torch.int32, (E,), dev)
    _need(bufs.expert_offsets, "expert_offsets", torch.int32, (E + 1,), dev)
    _need(bufs.group_offsets, "group_offsets", torch.int32, (groups + 1,), dev)
    _need(bufs.row_src, "row_src", torch.int32, (R,), dev)
    _need(bufs.dst_row, "dst_row", torch.int32, (T, k), dev)
    _need(bufs.workspace, "workspace", torch.uint8, None, dev)
    _check("moe_route_dispatch", lib.moe_route_dispatch(
        _ptr(logits), _ptr(x), T, H, E, k, groups, row_align,
        MOE_OUT_FP8_E4M3 if fp8 else MOE_OUT_BF16, _ptr(topk_idx), _ptr(topk_w), _ptr(bufs.out),
        _ptr(bufs.out_scales) if fp8 else None, _ptr(bufs.expert_counts),
        _ptr(bufs.expert_offsets), _ptr(bufs.group_offsets), _ptr(bufs.row_src),
        _ptr(bufs.dst_row), _ptr(bufs.workspace), bufs.workspace.numel(), _stream(dev)))
    return topk_idx, topk_w, bufs


def moe_dispatch_no_alloc(x: torch.Tensor, topk_idx: torch.Tensor, E: int, groups: int = 1,
                          row_align: int = 1, fp8: bool = False,
                          bufs: Optional[DispatchBuffers] = None) -> DispatchBuffers:
    """moe_dispatch on the library's own scratch (no workspace argument); the
    returned buffers' workspace field is an unused placeholder."""
    _need(x, "x", torch.bfloat16)
    T, H = x.shape
    dev = x.device
    _need(topk_idx, "topk_idx", torch.int32, None, dev)
    if topk_idx.dim() != 2 or topk_idx.shape[0] != T:
        raise ValueError(f"topk_idx: shape {tuple(topk_idx.shape)}, expected ({T}, k)")
    k = topk_idx.shape[1]
    if bufs is None:
        bufs = alloc_dispatch(T, H, E, k, groups, row_align, fp8, dev, workspace=False)
    R = moe_dispatch_max_rows(T, E, k, row_align)
    _need(bufs.out, "out", torch.uint8 if fp8 else torch.bfloat16, (R, H), dev)
    if fp8:
        _need(bufs.out_scales, "out_scales", torch.float32, (R, H // 128), dev)
    _need(bufs.expert_counts, "expert_counts", torch.int32, (E,), dev)
    _need(bufs.expert_offsets, "expert_offsets", torch.int32, (E + 1,), dev)
    _need(bufs.group_offsets, "group_offsets", torch.int32, (groups + 1,), dev)
    _need(bufs.row_src, "row_src", torch.int32, (R,), dev)
    _need(bufs.dst_row, "dst_row", torch.int32, (T, k), dev)
    with torch.cuda.device(dev):   # the library's scratch is per current device
        _check("moe_dispatch_no_alloc", lib.moe_dispatch_no_alloc(
            _ptr(x), _ptr(topk_idx), T, H, E, k, groups, row_align,
            MOE_OUT_FP8_E4M3 if fp8 else MOE_OUT_BF16, _ptr(bufs.out),
            _ptr(bufs.out_scales) if fp8 else None, _ptr(bufs.expert_counts),
            _ptr(bufs.expert_offsets), _ptr(bufs.group_offsets), _ptr(bufs.row_src),
            _ptr(bufs.dst_row), _stream(dev)))
    return bufs


# ----------------------------------------------------------------- combine

def moe_combine(expert_out: torch.Tensor, dst_row: torch.Tensor, topk_w: torch.Tensor,
                y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y bf16 [T,H] = sum_j topk_w[t,j] * expert_out[dst_row[t,j]] (fp32 accumulation)."""
    _need(expert_out, "expert_out", torch.bfloat16)
    dev = expert_out.device
    H = expert_out.shape[1]
    _need(dst_row, "dst_row", torch.int32, None, dev)
    T, k = dst_row.shape
    _need(topk_w, "topk_w", torch.float32, (T, k), dev)
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _need(y, "y", torch.bfloat16, (T, H), dev)
    _check("moe_combine", lib.moe_combine(_ptr(expert_out), _ptr(dst_row), _ptr(topk_w), T, H, k,
                                          _ptr(y), _stream(dev)))
    return y


def moe_combine_send(expert_out: torch.Tensor, dst_row: torch.Tensor, topk_w: torch.Tensor,
                     topk_idx: torch.Tensor, E: int, groups: int,
                     partial: Optional[torch.Tensor] = None,
                     partial_count: Optional[torch.Tensor] = None):
    """Sending half of the sender-side partial-reduction combine:
    (partial bf16 [T,k,H], partial_count int32 [T])."""
    _need(expert_out, "expert_out", torch.bfloat16)
    dev = expert_out.device
    H = expert_out.shape[1]
    _need(dst_row, "dst_row", torch.int32, None, dev)
    T, k = dst_row.shape
    _need(topk_w, "topk_w", torch.float32, (T, k), dev)
    _need(topk_idx, "topk_idx", torch.int32, (T, k), dev)
    if partial is None:
        partial = torch.empty((T, k, H), dtype=torch.bfloat16, device=dev)
    if partial_count is None:
        partial_count = torch.empty(T, dtype=torch.int32, device=dev)
    _need(partial, "partial", torch.bfloat16, (T, k, H), dev)
    _need(partial_count, "partial_count", torch.int32, (T,), dev)
    _check("moe_combine_send", lib.moe_combine_send(
        _ptr(expert_out), _ptr(dst_row), _ptr(topk_w), _ptr(topk_idx), T, H, E, k, groups,
        _ptr(partial), _ptr(partial_count), _stream(dev)))
    return partial, partial_count


def moe_combine_recv(partial: torch.Tensor, partial_count: torch.Tensor,
                     y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Receiving half: y bf16 [T,H] = sum of the token's partial rows (fp32)."""
    _need(partial, "partial", torch.bfloat16)
    dev = partial.device
    T, k, H = partial.shape
    _need(partial_count, "partial_count", torch.int32, (T,), dev)
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _need(y, "y", torch.bfloat16, (T, H), dev)
    _check("moe_combine_recv", lib.moe_combine_recv(_ptr(partial), _ptr(partial_count), T, H, k,
                                                    _ptr(y), _stream(dev)))
    return y


# ----------------------------------------------------------------- stand-in experts

def moe_harness_expert_scale(bufs: DispatchBuffers, topk_idx: torch.Tensor, E: int,
                             fp8: bool = False, identity: bool = False,
                             expert_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Stand-in experts (not part of the path): bf16 [max_rows, H]."""
    R, H = bufs.out.shape
    dev = bufs.out.device
    if expert_out is None:
        expert_out = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
    _need(expert_out, "expert_out", torch.bfloat16, (R, H), dev)
    if topk_idx.numel() == 0:
        # no tokens: the dispatch used no rows, so there is nothing to fill
        # (and torch hands out no address for the empty routing table)
        return expert_out
    _check("moe_harness_expert_scale", lib.moe_harness_expert_scale(
        _ptr(bufs.out), _ptr(bufs.out_scales) if fp8 else None, _ptr(bufs.row_src),
        _ptr(topk_idx), _ptr(bufs.expert_offsets), R, H, E,
        MOE_OUT_FP8_E4M3 if fp8 else MOE_OUT_BF16, int(identity), _ptr(expert_out),
        _stream(dev)))
    return expert_out


# ----------------------------------------------------------------- grouped GEMM

def moe_grouped_gemm_workspace_bytes(max_rows: int, E: int) -> int:
    return int(lib.moe_grouped_gemm_workspace_bytes(max_rows, E))


def moe_grouped_gemm_fp8(a: torch.Tensor, a_scales: torch.Tensor, expert_offsets: torch.Tensor,
                         w: torch.Tensor, w_scales: torch.Tensor,
                         y: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Block-scaled FP8 grouped GEMM over the dispatch segments: y bf16
    [max_rows, N]; rows at or past expert_offsets[E] are left as they were.
    a: uint8 E4M3 codes [max_rows, K], a_scales fp32 [max_rows, K/128],
    w: uint8 E4M3 codes [E, N, K], w_scales fp32 [E, N/128, K/128]."""
    _need(a, "a", torch.uint8)
    dev = a.device
    R, K = a.shape
    _need(a_scales, "a_scales", torch.float32, (R, K // 128), dev)
    _need(w, "w", torch.uint8, None, dev)
    E, N, Kw = w.shape
    if Kw != K:
        raise ValueError(f"w: inner size {Kw}, expected {K}")
    _need(w_scales, "w_scales", torch.float32, (E, N // 128, K // 128), dev)
    _need(expert_offsets, "expert_offsets", torch.int32, (E + 1,), dev)
    if y is None:
        y = torch.empty((R, N), dtype=torch.bfloat16, device=dev)
    _need(y, "y", torch.bfloat16, (R, N), dev)
    ws_bytes = moe_grouped_gemm_workspace_bytes(R, E)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    _check("moe_grouped_gemm_fp8", lib.moe_grouped_gemm_fp8(
        _ptr(a), _ptr(a_scales), _ptr(expert_offsets), _ptr(w), _ptr(w_scales), E, N, K, R,
        _ptr(y), _ptr(workspace), workspace.numel(), _stream(dev)))
    return y
