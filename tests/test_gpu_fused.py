"""moe_route_dispatch (routing inside the counting kernel, or the separate
route kernel first when the sorting-network path does not apply) against the
CPU oracle and against moe_route_topk followed by moe_dispatch.

Routing, counts, offsets, group offsets, both row maps, rows and FP8 scales
must be bit-exact; router weights within 1e-5 relative of the oracle and
bitwise equal to moe_route_topk's. Reuse of one workspace across calls of
different sizes and across both entry points is checked too."""
import numpy as np
import pytest
import torch

import oracle
from moe_synth import WORKLOADS, gen_logits, gen_x_bf16
from parity_util import bf16_to_np, log, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import combine_moe_route_amd  # noqa: F401
    return torch.device("cuda:0")


def _host(b, R, fp8):
    out = dict(counts=b.expert_counts.cpu().numpy(), offsets=b.expert_offsets.cpu().numpy(),
               goffs=b.group_offsets.cpu().numpy(), dst_row=b.dst_row.cpu().numpy(),
               row_src=b.row_src[:R].cpu().numpy())
    if fp8:
        out["out"] = b.out[:R].cpu().numpy()
        out["scales"] = b.out_scales[:R].cpu().numpy().view(np.uint32)
    else:
        out["out"] = bf16_to_np(b.out[:R])
    return out


def fused_case(T, H, E, k, groups=1, row_align=1, fp8=False, seed=0, zipf_s=None, dev=None,
               bufs=None, logits_t=None, check_two_call=True, logits_np=None):
    from combine_moe_route_amd import alloc_dispatch, moe_dispatch, moe_route_dispatch, moe_route_topk
    log(f"[fused] T={T} H={H} E={E} k={k} G={groups} A={row_align} fp8={fp8} seed={seed}")
    x_np = gen_x_bf16(T, H, seed)
    l_np = gen_logits(T, E, seed, zipf_s) if logits_np is None else logits_np
    x = to_dev_bf16(x_np, dev)
    logits = torch.from_numpy(l_np).to(dev) if logits_t is None else logits_t
    if bufs is None:
        bufs = alloc_dispatch(T, H, E, k, groups, row_align, fp8, dev)
    gi, gw, b = moe_route_dispatch(logits, x, k, groups, row_align, fp8, bufs)
    torch.cuda.synchronize()
    # against the oracle
    ri, rw = oracle.route_topk(l_np, k)
    assert np.array_equal(gi.cpu().numpy(), ri), "topk_idx"
    gwn = gw.cpu().numpy()
    assert np.all(np.abs(gwn.astype(np.float64) - rw) <= 1e-5 * np.abs(rw)), "topk_w"
    ref = oracle.dispatch(x_np, ri, E, groups, row_align, fp8)
    R = ref.num_rows
    g = _host(b, R, fp8)
    assert np.array_equal(g["counts"], ref.expert_counts), "expert_counts"
    assert np.array_equal(g["offsets"], ref.expert_offsets), "expert_offsets"
    assert np.array_equal(g["goffs"], ref.group_offsets), "group_offsets"
    assert np.array_equal(g["dst_row"], ref.dst_row), "dst_row"
    assert np.array_equal(g["row_src"], ref.row_src), "row_src"
    assert np.array_equal(g["out"], ref.out), "payload"
    if fp8:
        assert np.array_equal(g["scales"], ref.scales.view(np.uint32)), "scales"
    if check_two_call:
        i2, w2 = moe_route_topk(logits, k)
        b2 = moe_dispatch(x, i2, E, groups, row_align, fp8)
        torch.cuda.synchronize()
        assert torch.equal(i2, gi) and torch.equal(w2.view(torch.int32), gw.view(torch.int32))
        g2 = _host(b2, R, fp8)
        for key in g:
            assert np.array_equal(g[key], g2[key]), f"two-call path differs in {key}"
    return b


@pytest.mark.parametrize("name", ["tiny", "mixtral_decode", "dsv3_decode", "kimi_prefill",
                                  "dsv3_prefill"])
def test_fused_workloads(dev, name):
    w = WORKLOADS[name]
    fused_case(w.T, w.H, w.E, w.k, w.groups, w.row_align, w.fp8, w.seed, w.zipf_s, dev)
    if w.T <= 4096:
        fused_case(w.T, w.H, w.E, w.k, w.groups, w.row_align, w.fp8, 3, w.zipf_s, dev)


@pytest.mark.parametrize("T,H,E,k,G,A,fp8", [
    (1, 128, 8, 2, 1, 1, False),          # one token, one tile
    (17, 256, 12, 3, 3, 4, True),         # ragged tile, E = 12 (one lane per token)
    (1025, 256, 64, 5, 8, 8, False),      # 32-token tiles, two lanes per token
    (4097, 128, 128, 8, 4, 128, True),    # 64-token tiles, four lanes per token
    (333, 512, 512, 8, 16, 1, True),      # 16 lanes per token
    (700, 256, 768, 7, 1, 2, False),      # largest E of the sorting path
    (200, 256, 1000, 8, 8, 1, False),     # E > 768: route kernel first
    (300, 256, 64, 9, 2, 1, True),        # k > 8: route kernel first
    (257, 256, 65, 4, 5, 1, False),       # E % 4 != 0: route kernel first
    (100, 256, 256, 1, 32, 128, True),    # k = 1
], ids=lambda v: str(v))
def test_fused_shapes(dev, T, H, E, k, G, A, fp8):
    fused_case(T, H, E, k, G, A, fp8, seed=T + E, dev=dev)


@pytest.mark.parametrize("T,H,E,k,G,A,fp8", [
    (256, 256, 48, 4, 4, 8, True),        # largest T and E of the single-launch path, pad rows
    (128, 4096, 8, 8, 2, 1, False),       # k == E, T * k = 1024 pairs (the limit)
    (200, 136, 16, 5, 1, 1, False),       # ragged row units, K = 8 list with k = 5
    (64, 128, 4, 4, 1, 128, True),        # k == E == 4, 124 pad rows per expert
    (1, 8, 4, 1, 1, 1, False),            # one token, k = 1
    (257, 256, 48, 4, 4, 8, True),        # one token over: counting kernel + inline scan
    (128, 256, 52, 2, 1, 1, False),       # E over 48: counting kernel + inline scan
], ids=lambda v: str(v))
def test_single_launch_shapes(dev, T, H, E, k, G, A, fp8):
    """Small batches with few experts: moe_route_dispatch is one launch in
    which every block routes the whole batch (the last two cases sit just past
    its limits)."""
    fused_case(T, H, E, k, G, A, fp8, seed=7 * T + E, dev=dev)


def test_single_launch_ties(dev):
    """Tied and signed-zero logits on the single-launch path: the lower
    expert ranks first and the stable row order holds."""
    from combine_moe_route_amd import alloc_dispatch, moe_route_dispatch
    rng = np.random.default_rng(5)
    for E, k, T in [(8, 2, 256), (16, 4, 200), (48, 8, 128)]:
        l = (np.round(rng.standard_normal((T, E)) * 2) / 4).astype(np.float32)
        l[0] = 0.0
        l[1, ::2] = -0.0
        x_np = gen_x_bf16(T, 128, 5)
        ri, rw = oracle.route_topk(l, k)
        gi, gw, b = moe_route_dispatch(torch.from_numpy(l).to(dev), to_dev_bf16(x_np, dev), k,
                                       1, 1, False, alloc_dispatch(T, 128, E, k, 1, 1, False, dev))
        torch.cuda.synchronize()
        assert np.array_equal(gi.cpu().numpy(), ri), (E, k)
        assert np.all(np.abs(gw.cpu().numpy() - rw) <= 1e-5 * np.abs(rw))
        ref = oracle.dispatch(x_np, ri, E)
        assert np.array_equal(b.dst_row.cpu().numpy(), ref.dst_row)
        assert np.array_equal(b.row_src[:ref.num_rows].cpu().numpy(), ref.row_src)
        assert np.array_equal(bf16_to_np(b.out[:ref.num_rows]), ref.out)


def test_fused_empty_batch_writes_zero_offsets(dev):
    """T = 0: no routing happens, and the counts and offsets are still
    written (as zeros) over whatever the buffers held."""
    from combine_moe_route_amd import alloc_dispatch, moe_route_dispatch
    for E, k, G, A, fp8 in [(8, 2, 1, 1, False), (256, 8, 32, 128, True)]:
        bufs = alloc_dispatch(0, 256, E, k, G, A, fp8, dev)
        bufs.expert_counts.fill_(7)
        bufs.expert_offsets.fill_(7)
        bufs.group_offsets.fill_(7)
        logits = torch.empty((0, E), dtype=torch.float32, device=dev)
        x = torch.empty((0, 256), dtype=torch.bfloat16, device=dev)
        moe_route_dispatch(logits, x, k, G, A, fp8, bufs)
        torch.cuda.synchronize()
        assert bufs.expert_counts.cpu().tolist() == [0] * E
        assert bufs.expert_offsets.cpu().tolist() == [0] * (E + 1)
        assert bufs.group_offsets.cpu().tolist() == [0] * (G + 1)


def test_fused_unaligned_logits_fall_back(dev):
    """Logits not 16-byte aligned: the route kernel runs first."""
    T, E, k = 300, 256, 8
    l_np = gen_logits(T, E, 5)
    flat = torch.empty(T * E + 1, dtype=torch.float32, device=dev)
    view = flat[1:].view(T, E)
    view.copy_(torch.from_numpy(l_np))
    assert view.data_ptr() % 16 == 4
    fused_case(T, 256, E, k, 8, 1, True, seed=5, dev=dev, logits_t=view)


def test_fused_ties_and_signed_zero(dev):
    from combine_moe_route_amd import alloc_dispatch, moe_route_dispatch
    rng = np.random.default_rng(71)
    for E, k in [(8, 2), (64, 8), (256, 8), (384, 8), (16, 4)]:
        T = 300
        l = (np.round(rng.standard_normal((T, E)) * 2) / 4).astype(np.float32)
        l[0] = 0.0
        l[1, ::2] = -0.0
        l[2] = 1.25
        x_np = gen_x_bf16(T, 128, 71)
        ri, rw = oracle.route_topk(l, k)
        gi, gw, b = moe_route_dispatch(torch.from_numpy(l).to(dev), to_dev_bf16(x_np, dev), k,
                                       1, 1, False, alloc_dispatch(T, 128, E, k, 1, 1, False, dev))
        torch.cuda.synchronize()
        assert np.array_equal(gi.cpu().numpy(), ri), (E, k)
        assert np.all(np.abs(gw.cpu().numpy() - rw) <= 1e-5 * np.abs(rw))
        ref = oracle.dispatch(x_np, ri, E)
        assert np.array_equal(b.dst_row.cpu().numpy(), ref.dst_row)


def test_one_workspace_across_calls_and_sizes(dev):
    """One workspace (and one set of buffers, sized for the largest call)
    serves calls of different sizes and both entry points in a row; every
    result matches the oracle."""
    from combine_moe_route_amd import DispatchBuffers, alloc_dispatch, moe_dispatch
    E, k, H, G, A = 256, 8, 256, 32, 128
    big = alloc_dispatch(4096, H, E, k, G, A, True, dev)

    def view(T):
        from combine_moe_route_amd import moe_dispatch_max_rows
        R = moe_dispatch_max_rows(T, E, k, A)
        return DispatchBuffers(big.out[:R], big.out_scales[:R], big.expert_counts,
                               big.expert_offsets, big.group_offsets, big.row_src[:R],
                               big.dst_row.view(-1)[:T * k].view(T, k), big.workspace)

    for i, T in enumerate([4096, 16, 1000, 1, 2049, 4096, 0]):
        if T == 0:
            x = torch.empty((0, H), dtype=torch.bfloat16, device=dev)
            idx = torch.empty((0, k), dtype=torch.int32, device=dev)
            moe_dispatch(x, idx, E, G, A, True, view(0))
            torch.cuda.synchronize()
            assert big.expert_offsets.cpu().tolist() == [0] * (E + 1)
            continue
        if i % 2 == 0:
            fused_case(T, H, E, k, G, A, True, seed=i, dev=dev, bufs=view(T), check_two_call=False)
        else:
            x_np = gen_x_bf16(T, H, i)
            ri, _ = oracle.route_topk(gen_logits(T, E, i), k)
            b = moe_dispatch(to_dev_bf16(x_np, dev), torch.from_numpy(ri).to(dev), E, G, A, True,
                             view(T))
            torch.cuda.synchronize()
            ref = oracle.dispatch(x_np, ri, E, G, A, True)
            assert np.array_equal(b.expert_offsets.cpu().numpy(), ref.expert_offsets)
            assert np.array_equal(b.dst_row.cpu().numpy(), ref.dst_row)
            assert np.array_equal(b.out[:ref.num_rows].cpu().numpy(), ref.out)


def test_fused_repeat_bit_identical(dev):
    from combine_moe_route_amd import alloc_dispatch, moe_route_dispatch
    w = WORKLOADS["dsv3_decode"]
    T = 1500
    x = to_dev_bf16(gen_x_bf16(T, w.H, 16), dev)
    logits = torch.from_numpy(gen_logits(T, w.E, 16)).to(dev)
    bufs = alloc_dispatch(T, w.H, w.E, w.k, w.groups, 128, True, dev)
    first = None
    for it in range(20):
        gi, gw, b = moe_route_dispatch(logits, x, w.k, w.groups, 128, True, bufs)
        R = int(b.expert_offsets[-1])
        cur = [t.clone().contiguous().view(torch.uint8) for t in
               (gi, gw, b.out[:R], b.out_scales[:R], b.row_src[:R], b.dst_row, b.expert_offsets)]
        if first is None:
            first = cur
        else:
            for a, bb in zip(first, cur):
                assert torch.equal(a, bb), f"run {it} differs"


@pytest.mark.parametrize("i", range(40))
def test_fused_fuzz(dev, i):
    """Seeded random shapes across the three dispatch modes (one launch for
    small batches with few experts, inline scan for small batches, scan
    kernel) and the route-kernel fallbacks, with ties across the top-k
    boundary in some cases; oracle-exact and bitwise equal to the two-call
    path."""
    rng = np.random.default_rng([4242, i])
    E = int(rng.choice([4, 8, 12, 16, 44, 48, 52, 64, 65, 128, 256, 384, 768, 1000]))
    k = int(rng.integers(1, min(E, 10) + 1))
    G = int(rng.choice([g for g in (1, 2, 4, 8) if E % g == 0]))
    A = int(rng.choice([1, 1, 8, 128]))
    fp8 = bool(rng.random() < 0.5)
    H = int(rng.choice([128, 256, 1024])) if fp8 else int(rng.choice([8, 64, 200, 1024]))
    T = int(rng.choice([1, 7, 64, 128, 255, 256, 257, 1000, 1025, 4097]))
    logits = gen_logits(T, E, i)
    if rng.random() < 0.4:
        logits = (np.round(logits * 2.0) / 2.0).astype(np.float32)
    fused_case(T, H, E, k, G, A, fp8, seed=i, dev=dev, logits_np=logits)
