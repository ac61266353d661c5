"""The path under a CU budget: route + dispatch + stand-in experts + combine
on CU-masked streams (hipExtStreamCreateWithCUMask; 32, 64 and 128 of the
GPU's CUs) give the same bits as on the unmasked stream, and stay
oracle-exact; so do they while the grouped FP8 GEMM of a second micro-batch
runs at the same time on the other CUs, and that GEMM's output equals its own
unmasked run. This is the overlap the posts describe ("Efficient and portable
mixture-of-experts communication", Portable kernels: dispatch and combine
split so other work overlaps them; the DeepSeek-V3 excerpt on the third page
gives communication a fixed share of the SMs). Streams keep the default
priority."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from moe_synth import gen_fp8_weight_codes, gen_logits, gen_weight_scales, gen_x_bf16
from parity_util import bf16_to_np, combine_within_tolerance, log, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hip():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import combine_moe_route_amd  # noqa: F401
    return ctypes.CDLL("libamdhip64.so")


class MaskedStreams:
    """CU-masked HIP streams wrapped for torch; destroyed on close."""

    def __init__(self, hip, dev):
        self.hip, self.dev, self.made = hip, dev, []
        self.n_cu = torch.cuda.get_device_properties(dev).multi_processor_count

    def make(self, cus):
        mask = (ctypes.c_uint32 * ((self.n_cu + 31) // 32))()
        for c in cus:
            mask[c // 32] |= 1 << (c % 32)
        h = ctypes.c_void_p()
        err = self.hip.hipExtStreamCreateWithCUMask(ctypes.byref(h), len(mask), mask)
        assert err == 0, f"hipExtStreamCreateWithCUMask failed: {err}"
        self.made.append(h)
        return torch.cuda.ExternalStream(h.value, device=self.dev)

    def close(self):
        torch.cuda.synchronize()
        while self.made:
            self.hip.hipStreamDestroy(self.made.pop())


T, H, E, K, G, A = 2048, 1024, 256, 8, 32, 128


def _inputs(seed, dev):
    x_np = gen_x_bf16(T, H, seed)
    l_np = gen_logits(T, E, seed)
    return x_np, l_np, to_dev_bf16(x_np, dev), torch.from_numpy(l_np).to(dev)


def _chain(x, logits, dev):
    """One pass of the path on torch's current stream; returns its outputs."""
    from combine_moe_route_amd import (alloc_dispatch, moe_combine, moe_harness_expert_scale,
                                       moe_route_dispatch)
    bufs = alloc_dispatch(T, H, E, K, G, A, True, dev)
    idx, w, bufs = moe_route_dispatch(logits, x, K, G, A, True, bufs)
    eo = moe_harness_expert_scale(bufs, idx, E, fp8=True)
    y = moe_combine(eo, bufs.dst_row, w)
    return dict(idx=idx, w=w, bufs=bufs, y=y)


def _host(r):
    b = r["bufs"]
    R = int(b.expert_offsets[-1].item())
    return [t.contiguous().view(torch.uint8).cpu().numpy() for t in
            (r["idx"], r["w"], b.expert_counts, b.expert_offsets, b.group_offsets, b.dst_row,
             b.row_src[:R], b.out[:R], b.out_scales[:R], r["y"])]


def _check_oracle(x_np, l_np, r):
    ri, rw = oracle.route_topk(l_np, K)
    assert np.array_equal(r["idx"].cpu().numpy(), ri)
    ref = oracle.dispatch(x_np, ri, E, G, A, True)
    R = ref.num_rows
    b = r["bufs"]
    assert np.array_equal(b.expert_offsets.cpu().numpy(), ref.expert_offsets)
    assert np.array_equal(b.dst_row.cpu().numpy(), ref.dst_row)
    assert np.array_equal(b.out[:R].cpu().numpy(), ref.out)
    assert np.array_equal(b.out_scales[:R].cpu().numpy().view(np.uint32), ref.scales.view(np.uint32))
    eo_ref = oracle.expert_scale(ref, ri, E, True)
    y_ref = oracle.combine(eo_ref, ref.dst_row, r["w"].cpu().numpy())
    ok, ulp, _ = combine_within_tolerance(bf16_to_np(r["y"]), y_ref)
    assert ok.all() and ulp.all()


@pytest.mark.parametrize("n_cus", [32, 64, 128])
def test_chain_on_masked_stream(hip, n_cus):
    dev = torch.device("cuda:0")
    log(f"[cu budget] {n_cus} CUs")
    x_np, l_np, x, logits = _inputs(1, dev)
    want = _host(_chain(x, logits, dev))
    torch.cuda.synchronize()
    ms = MaskedStreams(hip, dev)
    try:
        s = ms.make(range(min(n_cus, ms.n_cu)))
        with torch.cuda.stream(s):
            r = _chain(x, logits, dev)
        s.synchronize()
        got = _host(r)
        for a, b in zip(want, got):
            assert np.array_equal(a, b)
        _check_oracle(x_np, l_np, r)
    finally:
        ms.close()


def test_chain_beside_grouped_gemm(hip):
    """64 CUs for the path, the rest for the grouped FP8 GEMM of a second
    micro-batch, launched together; then both on plain streams sharing every
    CU. Every output equals its unmasked run."""
    from combine_moe_route_amd import (alloc_dispatch, moe_grouped_gemm_fp8, moe_route_dispatch)
    dev = torch.device("cuda:0")
    N = 512
    x_np, l_np, x, logits = _inputs(2, dev)
    x2_np, l2_np, x2, logits2 = _inputs(3, dev)
    want = _host(_chain(x, logits, dev))
    # the co-runner: the second micro-batch's dispatch output through its experts
    b2 = alloc_dispatch(T, H, E, K, G, A, True, dev)
    moe_route_dispatch(logits2, x2, K, G, A, True, b2)
    wq = torch.from_numpy(gen_fp8_weight_codes(E, N, H, seed=3)).to(dev)
    ws = torch.from_numpy(gen_weight_scales(E, N, H, seed=3)).to(dev)
    y2_want = moe_grouped_gemm_fp8(b2.out, b2.out_scales, b2.expert_offsets, wq, ws).clone()
    torch.cuda.synchronize()
    R2 = int(b2.expert_offsets[-1].item())
    ms = MaskedStreams(hip, dev)
    try:
        for label, (s_path, s_gemm) in (
                ("64 + rest CUs", (ms.make(range(64)), ms.make(range(64, ms.n_cu)))),
                ("shared CUs", (torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)))):
            log(f"[cu budget] path beside the grouped GEMM, {label}")
            start = torch.cuda.Event()
            start.record()
            s_path.wait_event(start)
            s_gemm.wait_event(start)
            y2 = torch.empty_like(y2_want)
            with torch.cuda.stream(s_gemm):
                for _ in range(3):
                    moe_grouped_gemm_fp8(b2.out, b2.out_scales, b2.expert_offsets, wq, ws, y2)
            with torch.cuda.stream(s_path):
                runs = [_chain(x, logits, dev) for _ in range(3)]
            torch.cuda.synchronize()
            for r in runs:
                for a, b in zip(want, _host(r)):
                    assert np.array_equal(a, b)
            assert torch.equal(y2[:R2].view(torch.int16), y2_want[:R2].view(torch.int16))
            _check_oracle(x_np, l_np, runs[-1])
    finally:
        ms.close()
