"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
binding and the CPU oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import sys
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

import oracle
from moe_synth import bf16_bits_to_f32, gen_logits, gen_x_bf16


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev_bf16(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).view(torch.bfloat16).to(dev)


def bf16_to_np(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


# the combine tolerance: |gpu - oracle| <= 1e-2 * max(1, |oracle|)
def combine_within_tolerance(y_gpu: np.ndarray, y_ref: np.ndarray):
    g = bf16_bits_to_f32(y_gpu).astype(np.float64)
    o = bf16_bits_to_f32(y_ref).astype(np.float64)
    err = np.abs(g - o)
    ok = err <= 1e-2 * np.maximum(1.0, np.abs(o))
    # tighter, internal: within one bf16 unit of the oracle value
    ulp = np.spacing(np.abs(o).astype(np.float32)).astype(np.float64) * 2.0 ** 16
    ulp = np.maximum(ulp, 2.0 ** -133)
    within_ulp = err <= ulp
    return ok, within_ulp, float(np.mean(g == o)) if g.size else 1.0


@dataclass
class Case:
    T: int
    H: int
    E: int
    k: int
    groups: int = 1
    row_align: int = 1
    fp8: bool = False
    seed: int = 0
    zipf_s: Optional[float] = None

    def label(self):
        return (f"T{self.T}_H{self.H}_E{self.E}_k{self.k}_G{self.groups}_A{self.row_align}"
                f"_{'fp8' if self.fp8 else 'bf16'}_s{self.seed}")


def route_parity(logits_np: np.ndarray, k: int, dev):
    from combine_moe_route_amd import moe_route_topk
    idx_ref, w_ref = oracle.route_topk(logits_np, k)
    gi, gw = moe_route_topk(torch.from_numpy(logits_np).to(dev), k)
    torch.cuda.synchronize()
    gi, gw = gi.cpu().numpy(), gw.cpu().numpy()
    assert np.array_equal(gi, idx_ref), "topk_idx differs from the oracle"
    rel = np.abs(gw.astype(np.float64) - w_ref) / np.maximum(np.abs(w_ref), 1e-30)
    assert np.all(rel <= 1e-5), f"topk_w max rel err {rel.max()}"
    if k == 1:
        assert np.all(gw == 1.0)
    return idx_ref, w_ref


def dispatch_parity(x_np, idx_np, E, groups, row_align, fp8, dev, check_rows=True):
    """GPU dispatch on the oracle's routing; every output compared bit for bit."""
    from combine_moe_route_amd import moe_dispatch
    ref = oracle.dispatch(x_np, idx_np, E, groups, row_align, fp8)
    x = to_dev_bf16(x_np, dev)
    idx = torch.from_numpy(np.ascontiguousarray(idx_np, np.int32)).to(dev)
    bufs = moe_dispatch(x, idx, E, groups, row_align, fp8)
    torch.cuda.synchronize()
    R = ref.num_rows
    assert np.array_equal(bufs.expert_counts.cpu().numpy(), ref.expert_counts), "expert_counts"
    assert np.array_equal(bufs.expert_offsets.cpu().numpy(), ref.expert_offsets), "expert_offsets"
    assert np.array_equal(bufs.group_offsets.cpu().numpy(), ref.group_offsets), "group_offsets"
    assert np.array_equal(bufs.dst_row.cpu().numpy(), ref.dst_row), "dst_row"
    assert np.array_equal(bufs.row_src[:R].cpu().numpy(), ref.row_src), "row_src"
    if check_rows:
        if fp8:
            assert np.array_equal(bufs.out[:R].cpu().numpy(), ref.out), "FP8 payload"
            assert np.array_equal(bufs.out_scales[:R].cpu().numpy().view(np.uint32),
                                  ref.scales.view(np.uint32)), "FP8 scales"
        else:
            assert np.array_equal(bf16_to_np(bufs.out[:R]), ref.out), "bf16 payload"
    return ref, bufs


def experts_and_combine_parity(ref, bufs, idx_np, w_np, E, fp8, dev, identity=False):
    """Stand-in experts compared bitwise; combine compared within tolerance, with
    both sides reading the oracle's expert rows."""
    from combine_moe_route_amd import moe_combine, moe_harness_expert_scale
    idx = torch.from_numpy(np.ascontiguousarray(idx_np, np.int32)).to(dev)
    eo_gpu = moe_harness_expert_scale(bufs, idx, E, fp8, identity)
    eo_ref = oracle.expert_scale(ref, idx_np, E, fp8, identity)
    torch.cuda.synchronize()
    R = ref.num_rows
    assert np.array_equal(bf16_to_np(eo_gpu[:R]), eo_ref), "stand-in expert rows"
    # combine on the oracle's expert rows
    eo_in = torch.zeros_like(eo_gpu)
    if R:
        eo_in[:R] = to_dev_bf16(eo_ref, dev)
    y_ref = oracle.combine(eo_ref if R else np.zeros((1, eo_gpu.shape[1]), np.uint16),
                           ref.dst_row, w_np)
    y = moe_combine(eo_in, torch.from_numpy(ref.dst_row).to(dev),
                    torch.from_numpy(np.ascontiguousarray(w_np, np.float32)).to(dev))
    torch.cuda.synchronize()
    ok, within_ulp, exact = combine_within_tolerance(bf16_to_np(y), y_ref)
    assert ok.all(), f"combine outside tolerance at {np.argwhere(~ok)[:5]}"
    assert within_ulp.all(), f"combine more than 1 bf16 ulp off at {np.argwhere(~within_ulp)[:5]}"
    return y, y_ref, exact


def full_case(c: Case, dev, identity=False, idx_np=None, logits_np=None):
    log(f"[case] {c.label()}")
    x_np = gen_x_bf16(c.T, c.H, c.seed)
    if idx_np is None:
        if logits_np is None:
            logits_np = gen_logits(c.T, c.E, c.seed, c.zipf_s)
        idx_np, w_np = route_parity(logits_np, c.k, dev)
    else:
        rng = np.random.default_rng([c.seed, 9])
        w_np = rng.uniform(0.0, 1.0, idx_np.shape).astype(np.float32)
    ref, bufs = dispatch_parity(x_np, idx_np, c.E, c.groups, c.row_align, c.fp8, dev)
    y, y_ref, exact = experts_and_combine_parity(ref, bufs, idx_np, w_np, c.E, c.fp8, dev, identity)
    return dict(ref=ref, bufs=bufs, x=x_np, idx=idx_np, w=w_np, y=y, y_ref=y_ref, exact=exact)
