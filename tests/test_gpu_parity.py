"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Routing indices, counts, offsets, group offsets, both row maps, bf16 rows,
FP8 codes and scales must match bit for bit; router weights within 1e-5
relative; combine within |gpu - oracle| <= 1e-2 * max(1, |oracle|) (and, as
a tighter internal check, within one bf16 unit).
"""
import numpy as np
import pytest
import torch

import oracle
from moe_synth import WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits, gen_logits, gen_x_bf16
from parity_util import (Case, bf16_to_np, combine_within_tolerance, dispatch_parity,
                         experts_and_combine_parity, full_case, log, route_parity, to_dev_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import combine_moe_route_amd  # noqa: F401  (raises if the HIP library is missing)
    return torch.device("cuda:0")


def case_of(name, **kw):
    w = WORKLOADS[name]
    d = dict(T=w.T, H=w.H, E=w.E, k=w.k, groups=w.groups, row_align=w.row_align, fp8=w.fp8,
             seed=w.seed, zipf_s=w.zipf_s)
    d.update(kw)
    return Case(**d)


# ----------------------------------------------------------------- the five workloads

@pytest.mark.parametrize("name", ["tiny", "mixtral_decode", "dsv3_decode"])
@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_decode_workloads_full_parity(dev, name, seed):
    r = full_case(case_of(name, seed=seed), dev)
    log(f"  combine bit-exact fraction {r['exact']:.5f}")


def test_kimi_prefill_full_parity(dev):
    r = full_case(case_of("kimi_prefill"), dev)
    counts = r["ref"].expert_counts
    log(f"  skew: hottest expert {counts.max()} of {r['ref'].num_rows} rows, "
        f"{int(np.sum(counts == 0))} empty; combine exact {r['exact']:.5f}")


def test_dsv3_prefill_full_size(dev):
    """Full 16384-token FP8 workload: routing, the whole dispatch layout and
    payload, every stand-in expert row and every combined token, bit for bit
    (combine within its tolerance). The oracle's combine runs in its OpenMP
    build."""
    from combine_moe_route_amd import moe_combine, moe_harness_expert_scale
    c = case_of("dsv3_prefill")
    log(f"[case] {c.label()}")
    x_np = gen_x_bf16(c.T, c.H, c.seed)
    logits = gen_logits(c.T, c.E, c.seed)
    idx_np, w_np = route_parity(logits, c.k, dev)
    ref, bufs = dispatch_parity(x_np, idx_np, c.E, c.groups, c.row_align, c.fp8, dev)
    assert ref.num_rows == 147584
    idx = torch.from_numpy(idx_np).to(dev)
    eo = moe_harness_expert_scale(bufs, idx, c.E, fp8=True)
    y = moe_combine(eo, bufs.dst_row, torch.from_numpy(w_np).to(dev))
    with oracle.using("omp"):
        eo_ref = oracle.expert_scale(ref, idx_np, c.E, fp8=True)
        assert np.array_equal(bf16_to_np(eo[:ref.num_rows]), eo_ref)
        log("  stand-in experts: every row equal")
        y_ref = oracle.combine(eo_ref, ref.dst_row, w_np)
    ok, within_ulp, exact = combine_within_tolerance(bf16_to_np(y), y_ref)
    assert ok.all() and within_ulp.all()
    log(f"  combine: all {c.T} tokens within tolerance, exact {exact:.5f}")


# ----------------------------------------------------------------- edge cases

@pytest.mark.parametrize("c", [
    Case(T=300, H=136, E=8, k=2, seed=1),                       # ragged tile, 17 units per row
    Case(T=257, H=384, E=16, k=4, groups=4, row_align=8, fp8=True, seed=2),  # ragged, 24 units
    Case(T=1, H=128, E=4, k=4, groups=2, row_align=128, fp8=True),
    Case(T=1, H=8, E=1, k=1),                                   # smallest everything
    Case(T=513, H=64, E=8, k=8, seed=3),                        # k == E
    Case(T=200, H=256, E=65, k=5, seed=4),                      # two logits per lane
    Case(T=100, H=128, E=1024, k=3, groups=1024, seed=5),       # largest E, G == E
    Case(T=600, H=512, E=384, k=8, zipf_s=1.1, seed=6),         # skew, many empty experts
    Case(T=100, H=256, E=16, k=12, row_align=1024, seed=7),     # k > 8, biggest padding
    Case(T=3, H=65536, E=4, k=2, seed=8),                       # longest row
    Case(T=2048, H=1024, E=256, k=8, groups=32, row_align=128, fp8=True, seed=9),
], ids=lambda c: c.label())
def test_edge_shapes(dev, c):
    full_case(c, dev)


def test_identity_experts_round_trip(dev):
    for fp8 in (False, True):
        r = full_case(Case(T=256, H=512, E=32, k=4, groups=4, row_align=16 if fp8 else 1,
                           fp8=fp8, seed=11), dev, identity=True)
        y = bf16_bits_to_f32(bf16_to_np(r["y"])).astype(np.float64)
        x = bf16_bits_to_f32(r["x"]).astype(np.float64)
        if fp8:
            amax = np.abs(x).reshape(x.shape[0], -1, 128).max(-1).repeat(128, axis=1)
            assert np.all(np.abs(y - x) <= 2 ** -4 * np.abs(x) + 2 ** -10 * amax / 448 + 2 ** -7 * np.abs(x))
        else:
            assert np.all(np.abs(y - x) <= np.spacing(np.abs(x).astype(np.float32)) * 2 ** 16)


def test_k1_combine_returns_expert_row_bitwise(dev):
    r = full_case(Case(T=300, H=256, E=8, k=1, seed=12), dev)
    assert np.array_equal(bf16_to_np(r["y"]), r["y_ref"])


def test_router_ties_and_signed_zero(dev):
    rng = np.random.default_rng(13)
    for E, k in [(8, 2), (64, 8), (256, 8), (384, 8), (1000, 16)]:
        l = (np.round(rng.standard_normal((300, E)) * 2) / 4).astype(np.float32)
        l[0] = 0.0
        l[1, ::2] = -0.0
        l[2] = 1.25
        idx, w = route_parity(l, k, dev)
        assert np.allclose(w[2], 1.0 / k)


def test_all_tokens_one_expert_and_dropped_slots(dev):
    T, E, k = 1000, 8, 3
    idx = np.zeros((T, k), np.int32)
    idx[:, 1] = 5
    idx[:, 2] = np.where(np.arange(T) % 3 == 0, -1, 7)           # dropped every third
    idx[::7, 2] = E                                               # out of range: dropped
    full_case(Case(T=T, H=256, E=E, k=k, groups=2, row_align=4, seed=14), dev, idx_np=idx)
    full_case(Case(T=T, H=256, E=E, k=k, groups=2, row_align=128, fp8=True, seed=14), dev, idx_np=idx)


def test_zero_tokens_writes_empty_layout(dev):
    from combine_moe_route_amd import moe_combine, moe_dispatch, moe_route_topk
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((0, 2), dtype=torch.int32, device=dev)
    bufs = moe_dispatch(x, idx, 8, groups=4, row_align=128, fp8=True)
    i, w = moe_route_topk(torch.empty((0, 8), device=dev), 2)
    y = moe_combine(torch.empty((8 * 127, 256), dtype=torch.bfloat16, device=dev), bufs.dst_row, w)
    torch.cuda.synchronize()
    assert bufs.expert_counts.cpu().tolist() == [0] * 8
    assert bufs.expert_offsets.cpu().tolist() == [0] * 9
    assert bufs.group_offsets.cpu().tolist() == [0] * 5
    assert y.shape == (0, 256) and i.shape == (0, 2)


def test_zero_blocks_and_negative_zero_fp8(dev):
    T, H, E, k = 64, 512, 4, 2
    x = gen_x_bf16(T, H, 15)
    x[0] = 0                          # whole row zero
    x[1, :128] = 0x8000               # a block of -0.0
    x[2, 5] = 0x8000
    x[3, 128:256] = f32_to_bf16_bits(np.full(128, 1e-38, np.float32))   # tiny block
    x[4, 256:384] = f32_to_bf16_bits(np.full(128, 3e38, np.float32))    # huge block
    idx, _ = oracle.route_topk(gen_logits(T, E, 15), k)
    dispatch_parity(x, idx, E, 2, 8, True, dev)


def test_repeat_runs_bit_identical(dev):
    from combine_moe_route_amd import moe_combine, moe_dispatch, moe_route_topk
    c = case_of("dsv3_decode", T=1500)
    x = to_dev_bf16(gen_x_bf16(c.T, c.H, 16), dev)
    logits = torch.from_numpy(gen_logits(c.T, c.E, 16)).to(dev)
    first = None
    for it in range(20):
        i, w = moe_route_topk(logits, c.k)
        b = moe_dispatch(x, i, c.E, c.groups, 128, True)
        eo = torch.zeros((b.out.shape[0], c.H), dtype=torch.bfloat16, device=dev)
        R = int(b.expert_offsets[-1])
        eo[:R] = b.out[:R].view(torch.float8_e4m3fn).float().to(torch.bfloat16)
        y = moe_combine(eo, b.dst_row, w)
        cur = [i.clone(), w.clone(), b.out[:R].clone(), b.out_scales[:R].clone(), b.row_src[:R].clone(),
               b.dst_row.clone(), y.clone()]
        cur = [t.contiguous().view(torch.uint8) for t in cur]
        if first is None:
            first = cur
        else:
            for a, bb in zip(first, cur):
                assert torch.equal(a, bb), f"run {it} differs"


def _fp8_domain_rows(amax_bits: np.ndarray, rng, per_amax_blocks: int):
    """Blocks whose first element is the block maximum and whose other 127
    elements are bf16 values drawn uniformly over the bit patterns below it."""
    blocks = []
    for a in amax_bits:
        vals = rng.integers(0, int(a) + 1, size=(per_amax_blocks, 127), dtype=np.int64).astype(np.uint16)
        sign = rng.integers(0, 2, size=vals.shape).astype(np.uint16) << 15
        b = np.concatenate([np.full((per_amax_blocks, 1), a, np.uint16), vals | sign], axis=1)
        blocks.append(b)
    return np.concatenate(blocks)


def test_fp8_quantiser_domain_sweep(dev):
    """The FP8 element path over the (x, amax) domain: every bf16 binade of the
    block maximum (normal and subnormal), x spread over all smaller patterns."""
    rng = np.random.default_rng(17)
    amax = np.concatenate([
        np.arange(1, 128, dtype=np.uint16),                       # subnormal amax
        (np.arange(1, 255, dtype=np.uint16) << 7) | 0,            # every exponent, mantissa 0
        (np.arange(1, 255, dtype=np.uint16) << 7) | 0x55,
        (np.arange(1, 255, dtype=np.uint16) << 7) | 0x7F,
        rng.integers(0x0080, 0x7F80, 512).astype(np.uint16),
    ])
    blocks = _fp8_domain_rows(amax, rng, 16)
    H = 1024
    n = blocks.shape[0] // (H // 128) * (H // 128)
    x = blocks[:n].reshape(-1, H)
    idx = np.zeros((x.shape[0], 1), np.int32)
    log(f"  sweep: {x.size} elements, {n} blocks")
    dispatch_parity(x, idx, 1, 1, 1, True, dev)


@pytest.mark.parametrize("E", [1, 2, 3, 4, 5, 7, 8, 9, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128,
                               129, 200, 256, 257, 384, 511, 512, 513, 777, 1000, 1024])
def test_router_every_group_width(dev, E):
    """Every lane-group width (1..64 lanes per token) and candidates per lane
    (1..16), with k from 1 to E, against the oracle."""
    T = 333
    ks = sorted({1, min(E, 2), min(E, 3), min(E, 8), min(E, 16)} | ({E} if E <= 64 else set()))
    l = gen_logits(T, E, seed=E)
    lt = np.round(l * 2) / 2                              # many ties
    for k in ks:
        route_parity(l, k, dev)
        route_parity(lt.astype(np.float32), k, dev)


@pytest.mark.parametrize("E,k", [(128, 65), (128, 128), (300, 100), (1024, 200), (1024, 1024),
                                 (65, 65), (777, 129)])
def test_router_more_than_64_experts_per_token(dev, E, k):
    """Rounds past the 64th are kept in per-slot registers of the lanes."""
    l = gen_logits(200, E, seed=E + k)
    route_parity(l, k, dev)
    route_parity((np.round(l * 2) / 2).astype(np.float32), k, dev)


@pytest.mark.parametrize("c", [
    Case(T=300, H=512, E=128, k=65, groups=4, row_align=8, seed=21),                 # bf16, k > 64
    Case(T=257, H=1024, E=64, k=12, groups=8, row_align=128, fp8=True, seed=22),     # FP8, k > 8
    Case(T=100, H=256, E=512, k=100, groups=16, row_align=4, fp8=True, seed=23),     # FP8, k > 64
    Case(T=50, H=16384, E=32, k=8, groups=4, row_align=128, fp8=True, seed=24),     # FP8, > 16 chunks per row
    Case(T=33, H=16384, E=16, k=4, seed=25),                                          # bf16, 16 K wide rows
    Case(T=50, H=20480, E=16, k=4, groups=2, row_align=2, fp8=True, seed=24),        # FP8, > 16 waves per row
], ids=lambda c: c.label())
def test_many_slots_and_wide_rows(dev, c):
    full_case(c, dev)


def _ulps_apart(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 units between bit patterns (sign-magnitude aware)."""
    def key(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x & 0x7FFF)
    return np.abs(key(a) - key(b))


@pytest.mark.parametrize("c,G", [
    (Case(T=700, H=1024, E=256, k=8, seed=41), 32),        # DeepSeek-like groups
    (Case(T=300, H=512, E=64, k=8, seed=42), 1),           # one group: same as receiver-only
    (Case(T=300, H=136, E=16, k=4, seed=43), 16),          # one expert per group, ragged row
    (Case(T=200, H=256, E=128, k=12, seed=44), 8),         # k > 8: generic path
    (Case(T=257, H=7168, E=256, k=8, seed=45), 32),        # full hidden size
], ids=lambda v: v.label() if isinstance(v, Case) else f"G{v}")
def test_combine_sender_side(dev, c, G):
    from combine_moe_route_amd import moe_combine_recv, moe_combine_send
    log(f"[case] sender-side {c.label()} G={G}")
    x = gen_x_bf16(c.T, c.H, c.seed)
    idx, w = oracle.route_topk(gen_logits(c.T, c.E, c.seed), c.k)
    idx[::5, 1] = -1                                         # some dropped slots
    ref = oracle.dispatch(x, idx, c.E)
    eo = oracle.expert_scale(ref, idx, c.E, fp8=False)
    P_ref, cnt_ref, y_ref = oracle.combine_sender(eo, ref.dst_row, w, idx, c.E, G)
    eo_d = to_dev_bf16(eo, dev)
    dr = torch.from_numpy(ref.dst_row).to(dev)
    P, cnt = moe_combine_send(eo_d, dr, torch.from_numpy(w).to(dev),
                              torch.from_numpy(idx).to(dev), c.E, G)
    y = moe_combine_recv(P, cnt)
    # the receiving half alone, on the oracle's partial rows
    y_iso = moe_combine_recv(to_dev_bf16(P_ref, dev), torch.from_numpy(cnt_ref).to(dev))
    torch.cuda.synchronize()
    cnt_g = cnt.cpu().numpy()
    assert np.array_equal(cnt_g, cnt_ref)
    Pg = bf16_to_np(P)
    live = np.arange(c.k)[None, :] < cnt_ref[:, None]
    d = _ulps_apart(Pg[live], P_ref[live])
    assert d.max() <= 1, f"partial rows differ by {d.max()} ulp"
    log(f"  partial rows bit-exact {np.mean(d == 0):.5f}; rows per token "
        f"{cnt_ref.mean():.2f} of k={c.k}")
    assert _ulps_apart(bf16_to_np(y_iso), y_ref).max() <= 1
    ok, _, exact = combine_within_tolerance(bf16_to_np(y), y_ref)
    assert ok.all()
    assert _ulps_apart(bf16_to_np(y), y_ref).max() <= 2
    # accuracy consequence: distance from the exact weighted sum, both ways
    eof = bf16_bits_to_f32(eo).astype(np.float64)
    wl = np.where(ref.dst_row >= 0, w, 0).astype(np.float64)
    exact_sum = (wl[:, :, None] * eof[np.maximum(ref.dst_row, 0)]).sum(1)
    recv = bf16_bits_to_f32(oracle.combine(eo, ref.dst_row, w)).astype(np.float64)
    send = bf16_bits_to_f32(y_ref).astype(np.float64)
    log(f"  mean |error|: receiver-only {np.mean(np.abs(recv - exact_sum)):.3e}, "
        f"sender-side {np.mean(np.abs(send - exact_sum)):.3e}")


@pytest.mark.parametrize("E,k,n_shared,sw", [(8, 2, 1, 1.0), (256, 8, 1, 1.0), (384, 8, 2, 0.5),
                                             (16, 16, 3, 1.0), (100, 7, 64, 2.0)])
def test_route_shared_experts(dev, E, k, n_shared, sw):
    """Shared experts as always-chosen slots, then the full chain with E + n_shared experts."""
    from combine_moe_route_amd import moe_route_topk_shared
    T = 300
    l = gen_logits(T, E, seed=E + n_shared)
    ri, rw = oracle.route_topk_shared(l, k, n_shared, sw)
    gi, gw = moe_route_topk_shared(torch.from_numpy(l).to(dev), k, n_shared, sw)
    torch.cuda.synchronize()
    assert np.array_equal(gi.cpu().numpy(), ri)
    gw = gw.cpu().numpy()
    assert np.all(np.abs(gw - rw) <= 1e-5 * np.abs(rw))
    assert np.all(gw[:, k:] == np.float32(sw))
    if E + n_shared <= 1024:
        full_case(Case(T=T, H=256, E=E + n_shared, k=k + n_shared, groups=1, row_align=4,
                       seed=E), dev, idx_np=ri)


def test_route_replicas(dev):
    from combine_moe_route_amd import moe_route_replicas
    rng = np.random.default_rng(61)
    E, T, k = 64, 1000, 6
    copies = rng.integers(1, 5, E)
    base = np.concatenate([[0], np.cumsum(copies)]).astype(np.int32)
    idx, w = oracle.route_topk(gen_logits(T, E, seed=61, zipf_s=1.1), k)
    idx[::13, 2] = -1
    want = oracle.route_replicas(idx, E, base)
    g = torch.from_numpy(idx.copy()).to(dev)
    moe_route_replicas(g, E, torch.from_numpy(base).to(dev))
    torch.cuda.synchronize()
    assert np.array_equal(g.cpu().numpy(), want)
    # the chain on physical experts
    full_case(Case(T=T, H=512, E=int(base[-1]), k=k, groups=1, row_align=8, fp8=True, seed=62),
              dev, idx_np=want)
