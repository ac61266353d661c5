"""CPU oracle for the MoE dispatch/combine path (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package. The HIP library and its binding never do.

The arithmetic lives in ``moe_oracle.c`` (plain C, fp64 where the method
leaves the precision open). ``build()`` compiles it with gcc three times:
``plain`` (single-threaded, the default), ``omp`` (the same source with
-fopenmp: its pragmas spread independent per-token and per-block iterations
over the host cores) and ``san`` (single-threaded, with AddressSanitizer and
UndefinedBehaviorSanitizer; load it in a process started with libasan
preloaded). Loading never compiles: a missing or stale library raises, so a
benchmark never builds anything on the machine it measures. bf16 arrays are
uint16 bit patterns, E4M3 arrays are uint8 codes.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
from typing import NamedTuple, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")

_COMMON = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra"]
VARIANTS = {
    "plain": (os.path.join(_HERE, "libmoeoracle.so"), ["-Wno-unknown-pragmas"]),
    "omp": (os.path.join(_HERE, "libmoeoracle_omp.so"), ["-fopenmp"]),
    "san": (os.path.join(_HERE, "libmoeoracle_san.so"),
            ["-Wno-unknown-pragmas", "-g", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]),
}


def gcc_command(variant: str):
    path, extra = VARIANTS[variant]
    return _COMMON + extra + ["-o", path, _SRC, "-lm"]


def build(variants=tuple(VARIANTS)) -> None:
    """Compile the oracle library variants with gcc."""
    for v in variants:
        subprocess.run(gcc_command(v), check=True)


def stale(variant: str) -> bool:
    path = VARIANTS[variant][0]
    return not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC)


_variant = os.environ.get("MOE_ORACLE_VARIANT", "plain")
_libs = {}


def set_variant(variant: str) -> None:
    """Library variant used by the calls that follow (plain, omp or san)."""
    global _variant
    if variant not in VARIANTS:
        raise ValueError(f"unknown oracle variant {variant!r}")
    _variant = variant


def variant() -> str:
    return _variant


@contextlib.contextmanager
def using(variant: str):
    """Run the enclosed calls on another library variant."""
    prev = _variant
    set_variant(variant)
    try:
        yield
    finally:
        set_variant(prev)


def _load():
    if _variant in _libs:
        return _libs[_variant]
    path = VARIANTS[_variant][0]
    if stale(_variant):
        raise RuntimeError(f"oracle library {path} is missing or older than {_SRC}; "
                           "build it first (python -c 'import oracle; oracle.build()')")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i64, i32 = ctypes.c_int64, ctypes.c_int
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = i32
    lib.oracle_route_topk.argtypes = [P, i64, i32, i32, P, P]
    lib.oracle_route_topk.restype = None
    lib.oracle_dispatch.argtypes = [P, P, i64, i32, i32, i32, i32, i32, i32,
                                    P, P, P, P, P, P, P]
    lib.oracle_dispatch.restype = i64
    lib.oracle_expert_scale.argtypes = [P, P, P, P, i64, i32, i32, i32, i32, P]
    lib.oracle_expert_scale.restype = None
    lib.oracle_combine.argtypes = [P, P, P, i64, i32, i32, P]
    lib.oracle_combine.restype = None
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_value.restype = ctypes.c_float
    lib.oracle_bf16_from_double.argtypes = [ctypes.c_double]
    lib.oracle_bf16_from_double.restype = ctypes.c_uint16
    lib.oracle_quantize_block.argtypes = [P, P, P]
    lib.oracle_quantize_block.restype = None
    lib.oracle_quantize_blocks.argtypes = [P, i64, P, P]
    lib.oracle_quantize_blocks.restype = None
    lib.oracle_combine_sender.argtypes = [P, P, P, P, i64, i32, i32, i32, i32, P, P, P]
    lib.oracle_combine_sender.restype = None
    lib.oracle_route_topk_shared.argtypes = [P, i64, i32, i32, i32, ctypes.c_float, P, P]
    lib.oracle_route_topk_shared.restype = None
    lib.oracle_route_replicas.argtypes = [P, i64, i32, i32, P]
    lib.oracle_route_replicas.restype = None
    lib.oracle_e4m3_encode_array.argtypes = [P, P, i64]
    lib.oracle_e4m3_encode_array.restype = None
    lib.oracle_e4m3_encode_bits.argtypes = [ctypes.c_uint32, i64, P]
    lib.oracle_e4m3_encode_bits.restype = None
    lib.oracle_quantize_weights.argtypes = [P, i64, i64, P, P]
    lib.oracle_quantize_weights.restype = None
    lib.oracle_grouped_gemm_fp8.argtypes = [P, P, P, i32, P, P, i32, i32, P, P, P]
    lib.oracle_grouped_gemm_fp8.restype = None
    lib.oracle_grouped_gemm_fp8_at.argtypes = [P, P, P, i32, P, P, i32, i32, P, P, i64, P, P, P]
    lib.oracle_grouped_gemm_fp8_at.restype = None
    _libs[_variant] = lib
    return lib


def threads() -> int:
    """Host threads the current variant's parallel loops use."""
    return int(_load().oracle_threads())


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def route_topk(logits: np.ndarray, k: int):
    """(topk_idx int32 [T,k], topk_w float32 [T,k])."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _load().oracle_route_topk(_p(logits), T, E, k, _p(idx), _p(w))
    return idx, w


def route_topk_shared(logits: np.ndarray, k: int, n_shared: int, shared_w: float = 1.0):
    """Routed top-k plus n_shared always-chosen experts E..E+n_shared-1."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    idx = np.empty((T, k + n_shared), np.int32)
    w = np.empty((T, k + n_shared), np.float32)
    _load().oracle_route_topk_shared(_p(logits), T, E, k, n_shared, shared_w, _p(idx), _p(w))
    return idx, w


def route_replicas(topk_idx: np.ndarray, E: int, replica_base: np.ndarray) -> np.ndarray:
    """Logical expert ids -> physical replica ids (copy t mod count)."""
    idx = np.array(topk_idx, dtype=np.int32, copy=True, order="C")
    T, k = idx.shape
    base = _c(replica_base, np.int32)
    assert base.shape == (E + 1,)
    _load().oracle_route_replicas(_p(idx), T, k, E, _p(base))
    return idx


class Dispatch(NamedTuple):
    out: np.ndarray            # [num_rows, H] uint16 (bf16) or uint8 (E4M3)
    scales: Optional[np.ndarray]  # [num_rows, H/128] float32, FP8 only
    expert_counts: np.ndarray  # [E]
    expert_offsets: np.ndarray  # [E+1]
    group_offsets: np.ndarray  # [G+1]
    row_src: np.ndarray        # [num_rows]
    dst_row: np.ndarray        # [T,k]
    num_rows: int


def max_rows(T: int, E: int, k: int, row_align: int) -> int:
    return T * k + E * (row_align - 1)


def dispatch(x: np.ndarray, topk_idx: np.ndarray, E: int, groups: int = 1,
             row_align: int = 1, fp8: bool = False) -> Dispatch:
    x = _c(x, np.uint16)
    topk_idx = _c(topk_idx, np.int32)
    T, H = x.shape
    k = topk_idx.shape[1]
    cap = max_rows(T, E, k, row_align)
    out = np.zeros((cap, H), np.uint8 if fp8 else np.uint16)
    scales = np.zeros((cap, H // 128), np.float32) if fp8 else None
    counts = np.empty(E, np.int32)
    offs = np.empty(E + 1, np.int32)
    goff = np.empty(groups + 1, np.int32)
    row_src = np.full(cap, -2, np.int32)
    dst_row = np.empty((T, k), np.int32)
    R = _load().oracle_dispatch(_p(x), _p(topk_idx), T, H, E, k, groups, row_align,
                                int(fp8), _p(out), _p(scales), _p(counts), _p(offs),
                                _p(goff), _p(row_src), _p(dst_row))
    R = int(R)
    return Dispatch(out[:R], None if scales is None else scales[:R], counts, offs,
                    goff, row_src[:R], dst_row, R)


def expert_scale(d: Dispatch, topk_idx: np.ndarray, E: int, fp8: bool,
                 identity: bool = False) -> np.ndarray:
    """Stand-in experts: bf16 [num_rows, H]."""
    H = d.out.shape[1]
    topk_idx = _c(topk_idx, np.int32)
    y = np.empty((d.num_rows, H), np.uint16)
    disp = _c(d.out, np.uint8 if fp8 else np.uint16)
    sc = _c(d.scales, np.float32) if fp8 else None
    _load().oracle_expert_scale(_p(disp), _p(sc), _p(_c(d.row_src, np.int32)),
                                _p(topk_idx), d.num_rows, H, E, int(fp8),
                                int(identity), _p(y))
    return y


def combine(expert_out: np.ndarray, dst_row: np.ndarray, topk_w: np.ndarray) -> np.ndarray:
    """y bf16 [T,H] (uint16)."""
    expert_out = _c(expert_out, np.uint16)
    dst_row = _c(dst_row, np.int32)
    topk_w = _c(topk_w, np.float32)
    T, k = dst_row.shape
    H = expert_out.shape[1]
    y = np.empty((T, H), np.uint16)
    _load().oracle_combine(_p(expert_out), _p(dst_row), _p(topk_w), T, H, k, _p(y))
    return y


def combine_sender(expert_out: np.ndarray, dst_row: np.ndarray, topk_w: np.ndarray,
                   topk_idx: np.ndarray, E: int, groups: int):
    """Sender-side partial reduction: (partial uint16 [T,k,H], count int32 [T],
    y uint16 [T,H]); rows of partial past count[t] are zero."""
    expert_out = _c(expert_out, np.uint16)
    dst_row = _c(dst_row, np.int32)
    topk_w = _c(topk_w, np.float32)
    topk_idx = _c(topk_idx, np.int32)
    T, k = dst_row.shape
    H = expert_out.shape[1]
    partial = np.zeros((T, k, H), np.uint16)
    count = np.empty(T, np.int32)
    y = np.empty((T, H), np.uint16)
    _load().oracle_combine_sender(_p(expert_out), _p(dst_row), _p(topk_w), _p(topk_idx), T, H,
                                  E, k, groups, _p(partial), _p(count), _p(y))
    return partial, count, y


def e4m3_encode(v: float) -> int:
    return int(_load().oracle_e4m3_encode(float(v)))


def e4m3_value(code: int) -> float:
    return float(_load().oracle_e4m3_value(int(code)))


def e4m3_encode_array(v: np.ndarray) -> np.ndarray:
    """Elementwise E4M3 codes of a float32 array."""
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    _load().oracle_e4m3_encode_array(_p(v), _p(out), v.size)
    return out


def e4m3_encode_bits(start: int, count: int) -> np.ndarray:
    """E4M3 codes of the float32 bit patterns start .. start+count-1."""
    out = np.empty(count, np.uint8)
    _load().oracle_e4m3_encode_bits(start, count, _p(out))
    return out


def bf16_from_double(d: float) -> int:
    return int(_load().oracle_bf16_from_double(float(d)))


def quantize_block(xblock: np.ndarray):
    """(codes uint8 [128], scale float32) for one 128-element bf16 block."""
    xb = _c(xblock, np.uint16)
    assert xb.shape == (128,)
    q = np.empty(128, np.uint8)
    s = np.empty(1, np.float32)
    _load().oracle_quantize_block(_p(xb), _p(q), _p(s))
    return q, s[0]


def quantize_blocks(x: np.ndarray):
    """(codes uint8 [n, 128], scales float32 [n]) for n 1x128 bf16 blocks
    [n, 128] (uint16)."""
    xb = _c(x, np.uint16)
    assert xb.ndim == 2 and xb.shape[1] == 128
    n = xb.shape[0]
    q = np.empty((n, 128), np.uint8)
    s = np.empty(n, np.float32)
    _load().oracle_quantize_blocks(_p(xb), n, _p(q), _p(s))
    return q, s


def quantize_weights(w: np.ndarray):
    """128x128-block E4M3 quantisation of fp32 weights [..., N, K]:
    (codes uint8 [..., N, K], scales float32 [..., N/128, K/128])."""
    w = _c(w, np.float32)
    N, K = w.shape[-2:]
    assert N % 128 == 0 and K % 128 == 0
    lead = w.shape[:-2]
    wf = w.reshape(-1, N, K)
    q = np.empty(wf.shape, np.uint8)
    s = np.empty((wf.shape[0], N // 128, K // 128), np.float32)
    for i in range(wf.shape[0]):
        _load().oracle_quantize_weights(_p(wf[i]), N, K, _p(q[i]), _p(s[i]))
    return q.reshape(w.shape), s.reshape(lead + (N // 128, K // 128))


class Gemm(NamedTuple):
    y: np.ndarray        # uint16 bf16 bits
    y64: np.ndarray      # float64 exact-order sum
    mag: np.ndarray      # float64 sum of absolute terms


def grouped_gemm_fp8(a: np.ndarray, a_scales: np.ndarray, expert_offsets: np.ndarray,
                     w: np.ndarray, w_scales: np.ndarray) -> Gemm:
    """Block-scaled FP8 grouped GEMM over the padded segments. Rows at or
    past expert_offsets[E] are returned as zero."""
    a = _c(a, np.uint8)
    a_scales = _c(a_scales, np.float32)
    off = _c(expert_offsets, np.int32)
    w = _c(w, np.uint8)
    w_scales = _c(w_scales, np.float32)
    E, N, K = w.shape
    assert off.shape == (E + 1,) and a.shape[1] == K and a_scales.shape == (a.shape[0], K // 128)
    assert w_scales.shape == (E, N // 128, K // 128) and int(off[E]) <= a.shape[0]
    rows = a.shape[0]
    y = np.zeros((rows, N), np.uint16)
    y64 = np.zeros((rows, N), np.float64)
    mag = np.zeros((rows, N), np.float64)
    _load().oracle_grouped_gemm_fp8(_p(a), _p(a_scales), _p(off), E, _p(w), _p(w_scales), N, K,
                                    _p(y), _p(y64), _p(mag))
    return Gemm(y, y64, mag)


def grouped_gemm_fp8_at(a: np.ndarray, a_scales: np.ndarray, expert_offsets: np.ndarray,
                        w: np.ndarray, w_scales: np.ndarray, rows: np.ndarray,
                        cols: np.ndarray) -> Gemm:
    """The grouped GEMM at chosen (row, column) positions only; every row
    must lie below expert_offsets[E]."""
    a = _c(a, np.uint8)
    a_scales = _c(a_scales, np.float32)
    off = _c(expert_offsets, np.int32)
    w = _c(w, np.uint8)
    w_scales = _c(w_scales, np.float32)
    E, N, K = w.shape
    rows = _c(rows, np.int64)
    cols = _c(cols, np.int32)
    assert rows.shape == cols.shape and (rows < int(off[E])).all() and (cols < N).all()
    n = rows.size
    y = np.zeros(n, np.uint16)
    y64 = np.zeros(n, np.float64)
    mag = np.zeros(n, np.float64)
    _load().oracle_grouped_gemm_fp8_at(_p(a), _p(a_scales), _p(off), E, _p(w), _p(w_scales), N, K,
                                       _p(rows), _p(cols), n, _p(y), _p(y64), _p(mag))
    return Gemm(y, y64, mag)
