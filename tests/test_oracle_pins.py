"""Pins of the CPU oracle against things other than itself.

Each test checks an oracle function against brute force, a library routine,
a closed form, a hand-worked example or an invariant, so that a plausible
slip in the oracle (a dropped term, a wrong sign, index or tie rule, a
transposed operand, a wrong scale constant) fails at least one of them.
No GPU is needed.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from moe_synth import bf16_bits_to_f32, f32_to_bf16_bits, gen_logits, gen_x_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- helpers

def ocp_e4m3_table():
    """Value of each of the 256 E4M3 codes from the OCP definition."""
    vals = np.empty(256, np.float64)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            v = np.nan
        elif e == 0:
            v = m / 8 * 2.0 ** -6
        else:
            v = (1 + m / 8) * 2.0 ** (e - 7)
        vals[c] = -v if s else v
    return vals


TABLE = ocp_e4m3_table()
POS_CODES = np.arange(0, 0x7F)           # finite non-negative codes 0x00..0x7E
POS_VALS = TABLE[POS_CODES]               # strictly increasing


def nearest_code(v: np.ndarray) -> np.ndarray:
    """Nearest finite E4M3 code by search over the code table.

    Ties go to the code with an even mantissa (even code); magnitudes above
    448 saturate to 448. Sign is carried separately (so -0 -> 0x80).
    """
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    hi = np.searchsorted(POS_VALS, a, side="left")        # first value >= a
    hi = np.clip(hi, 0, len(POS_VALS) - 1)
    lo = np.clip(hi - 1, 0, len(POS_VALS) - 1)
    dlo = a - POS_VALS[lo]
    dhi = POS_VALS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, POS_CODES[hi], POS_CODES[lo])
    code = np.where(a >= POS_VALS[hi], POS_CODES[hi], code)   # exact hit / above top
    code = np.where(a > 448.0, 0x7E, code)
    sign = np.signbit(v)
    return (code | np.where(sign, 0x80, 0)).astype(np.uint8)


def fp32_patterns_rounding_classes():
    """fp32 values covering every E4M3 rounding decision.

    For each sign, each exponent from 2^-12 to 2^9 and each top-4 mantissa
    bit pattern, the low 19 mantissa bits take values below, at and above the
    rounding midpoint and at the ends. Also the subnormal E4M3 range at a fine
    grid, zeros, and the saturation range.
    """
    lows = np.array([0, 1, 2, 0x3FFFF, 0x40000 - 1, 0x40000, 0x40001, 0x7FFFE, 0x7FFFF,
                     0x12345, 0x6789A], np.uint32)
    out = []
    for sgn in (0, 1):
        for ex in range(127 - 12, 127 + 10):
            for top in range(16):
                base = (sgn << 31) | (ex << 23) | (top << 19)
                out.append(base | lows)
    arr = np.concatenate(out).astype(np.uint32)
    extra = np.array([0x00000000, 0x80000000, 0x43E00000, 0x43E00001, 0x43E7FFFF,
                      0x43E80000, 0x43E80001, 0x43F00000, 0x7F7FFFFF, 0x00000001],
                     np.uint32)
    arr = np.concatenate([arr, extra, extra | np.uint32(0x80000000)])
    return arr.view(np.float32)


# ----------------------------------------------------------------- E4M3

def test_e4m3_value_matches_ocp_points():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e4m3_ocp_points.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) >= 10
    for code, val in rows:
        c = int(code, 16)
        assert oracle.e4m3_value(c) == float(val), code
        assert TABLE[c] == float(val)
    assert math.isnan(oracle.e4m3_value(0x7F)) and math.isnan(oracle.e4m3_value(0xFF))


def test_e4m3_value_all_codes_match_definition_table():
    for c in range(256):
        v = oracle.e4m3_value(c)
        if np.isnan(TABLE[c]):
            assert math.isnan(v)
        else:
            assert v == TABLE[c] and math.copysign(1, v) == math.copysign(1, TABLE[c])


def test_e4m3_encode_rounding_classes_vs_nearest_search():
    v = fp32_patterns_rounding_classes()
    got = oracle.e4m3_encode_array(v)
    want = nearest_code(v.astype(np.float64))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


def test_e4m3_encode_random_patterns_vs_nearest_search():
    rng = np.random.default_rng(123)
    bits = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    got = oracle.e4m3_encode_array(v)
    want = nearest_code(v.astype(np.float64))
    assert np.array_equal(got, want)


def test_e4m3_encode_vs_torch_in_range():
    # torch's float8_e4m3fn cast rounds to nearest even; it does not saturate,
    # so compare only where |v| <= 448.
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.uniform(-448, 448, 500_000).astype(np.float32),
        (rng.standard_normal(500_000) * 10.0 ** rng.uniform(-5, 2, 500_000)).astype(np.float32),
        fp32_patterns_rounding_classes(),
    ])
    v = v[np.abs(v) <= 448]
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode_array(v)
    assert np.array_equal(got, want)


def test_e4m3_encode_saturates_and_keeps_sign():
    assert oracle.e4m3_encode(448.0) == 0x7E
    assert oracle.e4m3_encode(463.99) == 0x7E
    assert oracle.e4m3_encode(464.0) == 0x7E
    assert oracle.e4m3_encode(1e30) == 0x7E
    assert oracle.e4m3_encode(-1e30) == 0xFE
    assert oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(-1e-9) == 0x80
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00       # tie between 0 and 2^-9 -> even 0
    assert oracle.e4m3_encode(3 * 2.0 ** -10) == 0x02    # tie between 1 and 2 (x 2^-9) -> 2


def test_e4m3_encode_all_fp32_patterns():
    """All 2^32 fp32 bit patterns (the finite ones) through the encoder.
    Magnitudes below 2^-10 (under half the smallest subnormal code, 2^-9) must
    give a signed zero and magnitudes above 448 the saturated code; every
    pattern in between goes through the nearest-code search. The encoder runs
    in the oracle's OpenMP build (same source)."""
    step = 1 << 26                                   # a chunk never straddles the sign bit
    lo_mag, hi_mag, inf_mag = 0x3A800000, 0x43E00000, 0x7F800000   # 2^-10, 448, inf
    with oracle.using("omp"):
        for start in range(0, 1 << 32, step):
            got = oracle.e4m3_encode_bits(start, step)
            sign = 0x80 if start >> 31 else 0x00
            m0 = start & 0x7FFFFFFF                      # magnitudes m0 .. m0 + step - 1, in order
            i_lo = min(max(lo_mag - m0, 0), step)        # first index with magnitude >= 2^-10
            i_hi = min(max(hi_mag + 1 - m0, 0), step)    # first index with magnitude > 448
            i_inf = min(max(inf_mag - m0, 0), step)      # first non-finite index
            assert np.all(got[:i_lo] == sign), hex(start)
            assert np.all(got[i_hi:i_inf] == (0x7E | sign)), hex(start)
            if i_hi > i_lo:
                u = np.arange(i_lo, i_hi, dtype=np.uint32) + np.uint32(start)
                want = nearest_code(u.view(np.float32).astype(np.float64))
                bad = np.flatnonzero(got[i_lo:i_hi] != want)
                assert bad.size == 0, hex(start + i_lo + int(bad[0]))


# ----------------------------------------------------------------- bf16

def test_bf16_from_double_vs_torch_on_float_values():
    rng = np.random.default_rng(5)
    f = np.concatenate([
        (rng.standard_normal(200_000) * 10.0 ** rng.uniform(-40, 38, 200_000)).astype(np.float32),
        rng.integers(0, 2 ** 32, 200_000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    f = f[np.isfinite(f) & (np.abs(f) < 3.3e38)]
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_from_double(float(x)) for x in f[:20000]], np.uint16)
    assert np.array_equal(got, want[:20000])


def _bf16_exact(b):
    return Fraction(float(bf16_bits_to_f32(np.array([b], np.uint16))[0]))


def test_bf16_from_double_exact_nearest_on_doubles():
    """Doubles that are not floats: compare against exact rational search."""
    rng = np.random.default_rng(11)
    for _ in range(3000):
        d = float(rng.standard_normal() * 2.0 ** rng.integers(-130, 120))
        b = oracle.bf16_from_double(d)
        cand = f32_to_bf16_bits(np.array([d], np.float32))[0]
        best = None
        for c in (int(cand) - 1, int(cand), int(cand) + 1):
            c &= 0xFFFF
            if (c & 0x7F80) == 0x7F80:
                continue
            err = abs(_bf16_exact(c) - Fraction(d))
            key = (err, c & 1)
            if best is None or key < best[0]:
                best = (key, c)
        # same magnitude neighbours; ties broken towards the even pattern
        assert b == best[1] or abs(_bf16_exact(b) - Fraction(d)) == best[0][0] and b % 2 == 0, d


def test_bf16_from_double_midpoints_round_to_even():
    # 1 + 2^-8 lies halfway between bf16 1.0 (0x3F80) and 1.0078125 (0x3F81)
    assert oracle.bf16_from_double(1 + 2 ** -8) == 0x3F80
    assert oracle.bf16_from_double(1 + 3 * 2 ** -8) == 0x3F82
    # just above the midpoint must round up (a float detour would lose this)
    assert oracle.bf16_from_double(1 + 2 ** -8 + 2 ** -40) == 0x3F81
    assert oracle.bf16_from_double(-(1 + 2 ** -8 + 2 ** -40)) == 0xBF81
    assert oracle.bf16_from_double(0.0) == 0 and oracle.bf16_from_double(-0.0) == 0x8000


# ----------------------------------------------------------------- FP8 block

def test_fp8_block_hand_worked_example():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "fp8_block_example.txt"))
            if l.strip() and not l.startswith("#")]
    xb = np.zeros(128, np.uint16)
    want = np.zeros(128, np.uint8)
    for i, xb_hex, c_hex in rows:
        xb[int(i)] = int(xb_hex, 16)
        want[int(i)] = int(c_hex, 16)
    q, s = oracle.quantize_block(xb)
    assert np.array_equal(q, want), [hex(v) for v in q[:8]]
    assert abs(float(s) - 2.0 / 448) <= 2.0 / 448 * 2 ** -24


def test_fp8_block_properties_random():
    rng = np.random.default_rng(3)
    for trial in range(400):
        scale = 10.0 ** rng.uniform(-30, 30)
        x = f32_to_bf16_bits((rng.standard_normal(128) * scale).astype(np.float32))
        if trial % 7 == 0:
            x[rng.integers(0, 128, 20)] = 0x8000   # some -0.0
        q, s = oracle.quantize_block(x)
        xf = bf16_bits_to_f32(x).astype(np.float64)
        amax = np.max(np.abs(xf))
        # the block maximum maps onto +-448 exactly
        imax = np.argmax(np.abs(xf))
        assert q[imax] & 0x7F == 0x7E
        # dequantisation error bound: half a unit of the 3-bit mantissa in the
        # normal range, half the subnormal spacing below it
        deq = TABLE[q] * float(s)
        y = np.abs(xf) / float(s)
        bound = np.where(y >= 2.0 ** -6, 2.0 ** -4 * np.abs(xf), 2.0 ** -10 * float(s)) * (1 + 2 ** -20)
        assert np.all(np.abs(deq - xf) <= bound + 1e-300)
        assert float(s) > 0 and abs(float(s) * 448 - amax) <= amax * 2 ** -23
        # negative zero keeps its sign
        assert np.all(q[x == 0x8000] == 0x80)


def test_fp8_block_vs_torch_library_path():
    """x / s in torch float32 then torch's e4m3 cast gives the same codes."""
    rng = np.random.default_rng(4)
    for _ in range(200):
        x = f32_to_bf16_bits((rng.standard_normal(128) * 10.0 ** rng.uniform(-6, 6)).astype(np.float32))
        q, s = oracle.quantize_block(x)
        xt = torch.from_numpy(bf16_bits_to_f32(x).copy())
        st = torch.tensor(float(s), dtype=torch.float32)
        assert float(st) == float(xt.abs().max() / 448.0)
        want = (xt / st).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(q, want)


def test_block_quantiser_batch_matches_single_and_torch():
    """quantize_blocks, the reference of the whole-domain GPU sweep, on blocks
    built like that sweep's (amax first, every other |x| <= amax, both signs,
    amax from bf16 subnormals up to the largest finite bf16): per block the
    same codes and scale as quantize_block, and the codes of torch's E4M3 cast
    of the fp32 quotient x / (amax / 448), in the plain and the OpenMP build."""
    rng = np.random.default_rng(9)
    n = 3000
    amax = np.concatenate([np.arange(1, 9), rng.integers(1, 0x7F80, n - 16),
                           np.arange(0x7F78, 0x7F80)]).astype(np.uint16)
    mags = np.floor(rng.random((n, 127)) * (amax[:, None].astype(np.float64) + 1)).astype(np.uint32)
    mags = np.minimum(mags, amax[:, None].astype(np.uint32))
    signs = rng.integers(0, 2, (n, 127)).astype(np.uint32) << 15
    blocks = np.empty((n, 128), np.uint16)
    blocks[:, 0] = amax
    blocks[:, 1:] = (mags | signs).astype(np.uint16)
    xt = torch.from_numpy(bf16_bits_to_f32(blocks).copy())
    st = (xt[:, :1].abs() / 448.0)
    want = (xt / st).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for v in ("plain", "omp"):
        with oracle.using(v):
            q, s = oracle.quantize_blocks(blocks)
        assert np.array_equal(s.view(np.uint32), st[:, 0].numpy().view(np.uint32)), v
        assert np.array_equal(q, want), v
    for i in range(0, n, 97):
        qi, si = oracle.quantize_block(blocks[i])
        assert np.array_equal(qi, q[i]) and np.float32(si).view(np.uint32) == s[i].view(np.uint32)


def test_fp8_block_all_zero():
    q, s = oracle.quantize_block(np.zeros(128, np.uint16))
    assert s == 0.0 and np.all(q == 0)
    z = np.full(128, 0x8000, np.uint16)
    q, s = oracle.quantize_block(z)
    assert s == 0.0 and np.all(q == 0)


# ----------------------------------------------------------------- routing

def _golden_example():
    d = {}
    for l in open(os.path.join(GOLDEN, "worked_example.txt")):
        if not l.strip() or l.startswith("#"):
            continue
        key, *vals = l.split()
        d.setdefault(key, []).append(vals)
    return d


def test_routing_hand_worked_example():
    g = _golden_example()
    logits = np.array([[float(v) for v in r[1:]] for r in g["logits"]], np.float32)
    idx, w = oracle.route_topk(logits, 2)
    assert idx.tolist() == [[int(v) for v in r[1:]] for r in g["idx"]]
    want_w = np.array([[float(v) for v in r[1:]] for r in g["w"]])
    assert np.allclose(w, want_w, rtol=2e-7, atol=0)


def test_dispatch_hand_worked_example():
    g = _golden_example()
    idx = np.array([[int(v) for v in r[1:]] for r in g["idx"]], np.int32)
    x = np.tile(f32_to_bf16_bits(np.ones(8, np.float32)), (3, 1))
    for a in (1, 2):
        d = oracle.dispatch(x, idx, E=4, groups=2, row_align=a)
        assert d.expert_counts.tolist() == [int(v) for v in g["counts"][0]]
        assert d.expert_offsets.tolist() == [int(v) for v in g[f"offsets_a{a}"][0]]
        assert d.row_src.tolist() == [int(v) for v in g[f"row_src_a{a}"][0]]
        assert d.dst_row.ravel().tolist() == [int(v) for v in g[f"dst_row_a{a}"][0]]
        assert d.group_offsets.tolist() == [int(v) for v in g[f"groups2_a{a}"][0]]


def test_combine_hand_worked_example():
    g = _golden_example()
    logits = np.array([[float(v) for v in r[1:]] for r in g["logits"]], np.float32)
    idx, w = oracle.route_topk(logits, 2)
    x = np.tile(f32_to_bf16_bits(np.ones(8, np.float32)), (3, 1))
    d = oracle.dispatch(x, idx, E=4)
    eo = oracle.expert_scale(d, idx, E=4, fp8=False)
    y = bf16_bits_to_f32(oracle.combine(eo, d.dst_row, w))
    for t, v in g["y_scaled"]:
        assert np.all(y[int(t)] == float(v))


def _stable_ref_idx(logits, k):
    return np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :k].astype(np.int32)


@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (33, 6, 6), (20, 64, 8), (9, 384, 8), (5, 1024, 3), (7, 1, 1)])
def test_route_topk_indices_vs_stable_argsort(T, E, k):
    l = gen_logits(T, E, seed=T + E)
    idx, _ = oracle.route_topk(l, k)
    assert np.array_equal(idx, _stable_ref_idx(l, k))


def test_route_topk_ties_vs_stable_argsort():
    rng = np.random.default_rng(9)
    for E, k in [(8, 2), (8, 8), (12, 5), (256, 8)]:
        l = (np.round(rng.standard_normal((50, E)) * 2) / 4).astype(np.float32)   # multiples of 0.25
        l[0, :] = 0.0
        l[1, ::2] = -0.0                                                          # -0 == +0
        l[2, :] = 1.5
        idx, w = oracle.route_topk(l, k)
        assert np.array_equal(idx, _stable_ref_idx(l, k))
        assert np.allclose(w[0], 1.0 / k, rtol=0, atol=0) and np.all(w[2] == np.float32(1.0 / k))


def test_route_topk_brute_force_permutations():
    rng = np.random.default_rng(21)
    for trial in range(60):
        E = int(rng.integers(1, 7))
        k = int(rng.integers(1, E + 1))
        l = (np.round(rng.standard_normal(E) * 2) / 2).astype(np.float32)   # frequent ties
        # the unique ordering in which every neighbour pair is in order
        # (larger logit first, equal logits by lower index)
        valid = [p for p in itertools.permutations(range(E))
                 if all(l[p[i]] > l[p[i + 1]] or (l[p[i]] == l[p[i + 1]] and p[i] < p[i + 1])
                        for i in range(E - 1))]
        assert len(valid) == 1
        idx, _ = oracle.route_topk(l[None, :], k)
        assert idx[0].tolist() == list(valid[0][:k])


def test_route_topk_weights_closed_forms():
    l = gen_logits(300, 16, seed=1)
    # k = 1: the renormalised weight is exactly one
    _, w1 = oracle.route_topk(l, 1)
    assert np.all(w1 == 1.0)
    # k = 2: logistic function of the logit gap
    idx, w2 = oracle.route_topk(l, 2)
    gap = l[np.arange(300), idx[:, 0]].astype(np.float64) - l[np.arange(300), idx[:, 1]]
    assert np.allclose(w2[:, 0], 1 / (1 + np.exp(-gap)), rtol=1.2e-7, atol=0)
    assert np.allclose(w2[:, 1], 1 / (1 + np.exp(gap)), rtol=1.2e-7, atol=0)
    assert np.all(w2[:, 0] >= w2[:, 1])
    # k = E: the full softmax (scipy's), in slot order
    from scipy.special import softmax
    idxE, wE = oracle.route_topk(l, 16)
    ref = softmax(l.astype(np.float64), axis=1)
    ref = np.take_along_axis(ref, idxE, axis=1).astype(np.float32)
    ulp = np.spacing(ref)
    assert np.all(np.abs(wE - ref) <= ulp)
    # weights sum to one and are non-increasing along the slots
    for k in (2, 4, 8):
        _, w = oracle.route_topk(l, k)
        assert np.allclose(w.astype(np.float64).sum(1), 1.0, atol=k * 2 ** -24)
        assert np.all(np.diff(w, axis=1) <= 0)


def test_route_topk_shift_invariance():
    l = gen_logits(200, 32, seed=2)
    idx0, w0 = oracle.route_topk(l, 4)
    idx1, w1 = oracle.route_topk((l.astype(np.float64) + 0.5).astype(np.float32), 4)
    assert np.array_equal(idx0, idx1)
    assert np.allclose(w0, w1, rtol=2e-6)


# ----------------------------------------------------------------- dispatch

def _routing(T, E, k, seed, zipf=None):
    idx, w = oracle.route_topk(gen_logits(T, E, seed, zipf), k)
    return idx, w


@pytest.mark.parametrize("T,H,E,k,G,A", [
    (64, 256, 8, 2, 1, 1), (300, 128, 16, 4, 4, 1), (300, 128, 16, 4, 4, 128),
    (513, 64, 384, 8, 1, 1), (100, 256, 256, 8, 32, 128), (1, 128, 4, 4, 2, 8),
])
def test_dispatch_layout_vs_library_routines(T, H, E, k, G, A):
    idx, _ = _routing(T, E, k, seed=T, zipf=1.1 if E == 384 else None)
    x = gen_x_bf16(T, H, seed=T)
    d = oracle.dispatch(x, idx, E, groups=G, row_align=A)
    counts = np.bincount(idx.ravel(), minlength=E)
    assert np.array_equal(d.expert_counts, counts) and counts.sum() == T * k
    padded = -(-counts // A) * A
    offs = np.concatenate([[0], np.cumsum(padded)])
    assert np.array_equal(d.expert_offsets, offs)
    assert np.array_equal(d.group_offsets, offs[:: E // G])
    assert d.num_rows == offs[-1]
    real = d.row_src[d.row_src >= 0]
    # stable counting sort == stable argsort of the expert keys
    assert np.array_equal(real, np.argsort(idx.ravel(), kind="stable"))
    # pad rows sit at the end of each segment, and only there
    for e in range(E):
        seg = d.row_src[offs[e]:offs[e + 1]]
        assert np.all(seg[:counts[e]] >= 0) and np.all(seg[counts[e]:] == -1)
    # inverse maps
    assert np.array_equal(d.dst_row.ravel()[real], np.nonzero(d.row_src >= 0)[0])
    # bf16 payload is the token's row
    assert np.array_equal(d.out[d.row_src >= 0], x[real // k])
    assert np.all(d.out[d.row_src < 0] == 0)


def test_dispatch_fp8_rows_are_token_block_quantisation():
    T, H, E, k = 40, 384, 16, 4
    idx, _ = _routing(T, E, k, seed=8)
    x = gen_x_bf16(T, H, seed=8)
    x[3, :128] = 0                      # an all-zero block
    d = oracle.dispatch(x, idx, E, groups=4, row_align=8, fp8=True)
    xt = torch.from_numpy(bf16_bits_to_f32(x).copy()).view(T, H // 128, 128)
    s_ref = (xt.abs().amax(-1) / 448.0)
    q_ref = torch.where(s_ref[..., None] > 0, xt / s_ref[..., None], torch.zeros(()))
    q_ref = q_ref.to(torch.float8_e4m3fn).view(torch.uint8).view(T, H).numpy()
    live = d.row_src >= 0
    t_of_row = d.row_src[live] // k
    assert np.array_equal(d.out[live], q_ref[t_of_row])
    assert np.array_equal(d.scales[live], s_ref.numpy()[t_of_row])
    assert np.all(d.out[~live] == 0) and np.all(d.scales[~live] == 0)


def test_dispatch_dropped_slots():
    idx = np.array([[0, 5], [-1, 1], [1, 2]], np.int32)   # 5 and -1 are outside [0, 3)
    x = gen_x_bf16(3, 8, seed=0)
    d = oracle.dispatch(x, idx, E=3)
    assert d.expert_counts.tolist() == [1, 2, 1]
    assert d.dst_row.tolist() == [[0, -1], [-1, 1], [2, 3]]
    assert d.row_src.tolist() == [0, 3, 4, 5]


def test_dispatch_empty_and_single_expert():
    x = gen_x_bf16(0, 128, seed=0)
    d = oracle.dispatch(x, np.zeros((0, 2), np.int32), E=4, groups=2, row_align=128)
    assert d.num_rows == 0 and d.expert_counts.tolist() == [0] * 4
    assert d.expert_offsets.tolist() == [0] * 5 and d.group_offsets.tolist() == [0, 0, 0]
    x = gen_x_bf16(10, 128, seed=1)
    d = oracle.dispatch(x, np.zeros((10, 1), np.int32), E=3, row_align=4)
    assert d.expert_offsets.tolist() == [0, 12, 12, 12]
    assert d.row_src.tolist() == list(range(10)) + [-1, -1]


# ----------------------------------------------------------------- experts + combine

def test_expert_scale_vs_torch():
    T, H, E, k = 30, 256, 8, 2
    idx, _ = _routing(T, E, k, seed=4)
    x = gen_x_bf16(T, H, seed=4)
    for fp8 in (False, True):
        d = oracle.dispatch(x, idx, E, row_align=4, fp8=fp8)
        eo = oracle.expert_scale(d, idx, E, fp8)
        live = d.row_src >= 0
        e_of_row = idx.ravel()[d.row_src[live]]
        c = torch.tensor((e_of_row + 1).astype(np.float32)) / float(E)
        if fp8:
            v = torch.from_numpy(d.out[live].copy()).view(torch.float8_e4m3fn).float()
            v = (v.view(-1, H // 128, 128) * torch.from_numpy(d.scales[live].copy())[..., None]).view(-1, H)
        else:
            v = torch.from_numpy(bf16_bits_to_f32(d.out[live]).copy())
        want = (v * c[:, None]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(eo[live], want)
        assert np.all(eo[~live] == 0)


def test_combine_k1_returns_expert_row_bitwise():
    T, H, E = 50, 128, 8
    idx, w = _routing(T, E, 1, seed=5)
    x = gen_x_bf16(T, H, seed=5)
    d = oracle.dispatch(x, idx, E)
    eo = oracle.expert_scale(d, idx, E, fp8=False)
    y = oracle.combine(eo, d.dst_row, w)
    assert np.array_equal(y, eo[d.dst_row[:, 0]])


def test_combine_identity_experts_round_trip():
    T, H, E, k = 64, 256, 16, 4
    idx, w = _routing(T, E, k, seed=6)
    x = gen_x_bf16(T, H, seed=6)
    d = oracle.dispatch(x, idx, E, row_align=8)
    eo = oracle.expert_scale(d, idx, E, fp8=False, identity=True)
    y = bf16_bits_to_f32(oracle.combine(eo, d.dst_row, w))
    xf = bf16_bits_to_f32(x)
    assert np.all(np.abs(y - xf) <= np.spacing(np.abs(xf).astype(np.float32)) * 2 ** 16 + 0)  # within 1 bf16 ulp
    assert np.mean(y == xf) > 0.99


def test_combine_scalar_experts_closed_form():
    T, H, E, k = 64, 256, 16, 4
    idx, w = _routing(T, E, k, seed=7)
    x = gen_x_bf16(T, H, seed=7)
    d = oracle.dispatch(x, idx, E)
    eo = oracle.expert_scale(d, idx, E, fp8=False)
    y = bf16_bits_to_f32(oracle.combine(eo, d.dst_row, w)).astype(np.float64)
    factor = (w.astype(np.float64) * (idx + 1) / E).sum(1)
    want = bf16_bits_to_f32(x).astype(np.float64) * factor[:, None]
    assert np.all(np.abs(y - want) <= 2 ** -7 * np.abs(want) + 1e-30)


def test_combine_dropped_slot_equals_zero_weight():
    T, H, E, k = 20, 128, 8, 3
    idx, w = _routing(T, E, k, seed=9)
    x = gen_x_bf16(T, H, seed=9)
    d = oracle.dispatch(x, idx, E)
    eo = oracle.expert_scale(d, idx, E, fp8=False)
    dr = d.dst_row.copy()
    dr[::2, 1] = -1
    w0 = w.copy()
    w0[::2, 1] = 0.0
    assert np.array_equal(oracle.combine(eo, dr, w), oracle.combine(eo, d.dst_row, w0))


def test_chain_fp8_round_trip_error_bound():
    T, H, E, k = 32, 512, 8, 2
    idx, w = _routing(T, E, k, seed=10)
    x = gen_x_bf16(T, H, seed=10)
    d = oracle.dispatch(x, idx, E, groups=2, row_align=128, fp8=True)
    eo = oracle.expert_scale(d, idx, E, fp8=True, identity=True)
    y = bf16_bits_to_f32(oracle.combine(eo, d.dst_row, w)).astype(np.float64)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    amax = np.abs(xf).reshape(T, -1, 128).max(-1).repeat(128, axis=1)
    # E4M3 relative error 2^-4 (normals), subnormal floor 2^-10 * amax/448, two bf16 roundings
    bound = 2 ** -4 * np.abs(xf) + 2 ** -10 * amax / 448 + 2 ** -7 * np.abs(xf)
    assert np.all(np.abs(y - xf) <= bound)


# ----------------------------------------------------------------- sender-side combine

def _live_groups(idx, dst_row, E, G):
    per = E // G
    return [sorted({int(e) // per for e, r in zip(idx[t], dst_row[t]) if r >= 0 and 0 <= e < E})
            for t in range(idx.shape[0])]


def test_sender_single_group_equals_receiver_combine():
    T, H, E, k = 60, 256, 16, 4
    idx, w = _routing(T, E, k, seed=31)
    x = gen_x_bf16(T, H, seed=31)
    d = oracle.dispatch(x, idx, E)
    eo = oracle.expert_scale(d, idx, E, fp8=False)
    part, cnt, y = oracle.combine_sender(eo, d.dst_row, w, idx, E, groups=1)
    assert np.all(cnt == 1)
    assert np.array_equal(y, oracle.combine(eo, d.dst_row, w))
    assert np.array_equal(part[:, 0], y) and np.all(part[:, 1:] == 0)


def test_sender_counts_are_distinct_groups():
    T, H, E, k = 200, 64, 32, 6
    idx, w = _routing(T, E, k, seed=32)
    idx[::9, 2] = -1                                   # dropped slots do not count
    x = gen_x_bf16(T, H, seed=32)
    d = oracle.dispatch(x, idx, E)
    eo = oracle.expert_scale(d, idx, E, fp8=False)
    for G in (2, 4, 8, 32):
        _, cnt, _ = oracle.combine_sender(eo, d.dst_row, w, idx, E, G)
        assert cnt.tolist() == [len(g) for g in _live_groups(idx, d.dst_row, E, G)]


def test_sender_partials_are_nearest_bf16_of_group_sums():
    """One expert per group: each partial is the nearest bf16 of w * v."""
    T, H, E, k = 40, 128, 8, 3
    idx, w = _routing(T, E, k, seed=33)
    x = gen_x_bf16(T, H, seed=33)
    d = oracle.dispatch(x, idx, E)
    eo = oracle.expert_scale(d, idx, E, fp8=False)
    part, cnt, _ = oracle.combine_sender(eo, d.dst_row, w, idx, E, groups=E)
    eof = bf16_bits_to_f32(eo).astype(np.float64)
    for t in range(T):
        order = np.argsort(idx[t])                     # groups ascending = experts ascending
        for p, j in enumerate(order):
            exact = float(w[t, j]) * eof[d.dst_row[t, j]]
            got = bf16_bits_to_f32(part[t, p]).astype(np.float64)
            up = bf16_bits_to_f32(part[t, p] + np.uint16(1)).astype(np.float64)
            dn = bf16_bits_to_f32(part[t, p] - np.uint16(1)).astype(np.float64)
            err = np.abs(got - exact)
            assert np.all((err <= np.abs(up - exact)) & (err <= np.abs(dn - exact)) | (part[t, p] & 0x7FFF == 0))


def test_sender_equals_receiver_when_sums_are_exact():
    """Power-of-two weights and small-integer rows make every partial exact."""
    T, H, E, k = 30, 64, 16, 4
    rng = np.random.default_rng(34)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = (2.0 ** -rng.integers(0, 4, (T, k))).astype(np.float32)
    x = f32_to_bf16_bits(rng.integers(-8, 9, (T, H)).astype(np.float32))
    d = oracle.dispatch(x, idx, E)
    eo = oracle.expert_scale(d, idx, E, fp8=False, identity=True)
    want = oracle.combine(eo, d.dst_row, w)
    for G in (1, 2, 4, 16):
        _, _, y = oracle.combine_sender(eo, d.dst_row, w, idx, E, G)
        assert np.array_equal(y, want), G


def test_sender_error_bound():
    """|y - exact| <= (n_groups + 1) half-units of bf16 relative to the sum of |terms|."""
    T, H, E, k = 100, 256, 64, 8
    idx, w = _routing(T, E, k, seed=35)
    x = gen_x_bf16(T, H, seed=35)
    d = oracle.dispatch(x, idx, E)
    eo = oracle.expert_scale(d, idx, E, fp8=False)
    _, cnt, y = oracle.combine_sender(eo, d.dst_row, w, idx, E, groups=8)
    eof = bf16_bits_to_f32(eo).astype(np.float64)
    terms = w[:, :, None].astype(np.float64) * eof[d.dst_row]
    exact = terms.sum(1)
    mag = np.abs(terms).sum(1)
    err = np.abs(bf16_bits_to_f32(y).astype(np.float64) - exact)
    assert np.all(err <= (cnt[:, None] + 1) * 2.0 ** -8 * mag + 1e-30)


def test_sender_receiver_half_sums_the_rounded_partials():
    """y is the nearest bf16 of the sum of the (bf16) partial rows."""
    T, H, E, k = 80, 128, 32, 8
    idx, w = _routing(T, E, k, seed=36)
    x = gen_x_bf16(T, H, seed=36)
    d = oracle.dispatch(x, idx, E)
    eo = oracle.expert_scale(d, idx, E, fp8=False)
    part, cnt, y = oracle.combine_sender(eo, d.dst_row, w, idx, E, groups=8)
    s = bf16_bits_to_f32(part).astype(np.float64).sum(1)          # unused rows are zero
    got = bf16_bits_to_f32(y).astype(np.float64)
    up = bf16_bits_to_f32((y + np.uint16(1)) & np.uint16(0xFFFF)).astype(np.float64)
    dn = bf16_bits_to_f32((y - np.uint16(1)) & np.uint16(0xFFFF)).astype(np.float64)
    err = np.abs(got - s)
    ok = ((err <= np.abs(up - s)) & (err <= np.abs(dn - s))) | ((y & 0x7FFF) == 0)
    assert ok.all()


# ----------------------------------------------------------------- routing variants

def test_route_shared_experts_extend_the_routed_slots():
    l = gen_logits(120, 64, seed=51)
    for n_shared, sw in [(1, 1.0), (2, 0.5)]:
        idx, w = oracle.route_topk_shared(l, 8, n_shared, sw)
        ri, rw = oracle.route_topk(l, 8)
        assert np.array_equal(idx[:, :8], ri) and np.array_equal(w[:, :8], rw)
        assert np.all(idx[:, 8:] == 64 + np.arange(n_shared)) and np.all(w[:, 8:] == np.float32(sw))
        # dispatch puts every token into each shared expert's segment, in token order
        x = gen_x_bf16(120, 64, seed=51)
        d = oracle.dispatch(x, idx, 64 + n_shared)
        for s in range(n_shared):
            seg = d.row_src[d.expert_offsets[64 + s]:d.expert_offsets[65 + s]]
            assert np.array_equal(seg, np.arange(120) * (8 + n_shared) + 8 + s)


def test_route_replicas_map_back_and_spread():
    rng = np.random.default_rng(52)
    E, T, k = 16, 500, 4
    copies = rng.integers(1, 4, E)
    base = np.concatenate([[0], np.cumsum(copies)]).astype(np.int32)
    idx, _ = oracle.route_topk(gen_logits(T, E, seed=52), k)
    idx[::11, 0] = -1
    phys = oracle.route_replicas(idx, E, base)
    live = idx >= 0
    # each physical id maps back to its logical expert (library search)
    back = np.searchsorted(base, phys[live], side="right") - 1
    assert np.array_equal(back, idx[live])
    assert np.array_equal(phys[~live], idx[~live])
    # the copy used by token t is t mod copies
    t_of = np.broadcast_to(np.arange(T)[:, None], idx.shape)[live]
    assert np.array_equal(phys[live] - base[idx[live]], t_of % copies[idx[live]])
    # one copy everywhere is the identity
    assert np.array_equal(oracle.route_replicas(idx, E, np.arange(E + 1, dtype=np.int32)), idx)
