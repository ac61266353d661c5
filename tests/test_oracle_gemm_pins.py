"""Pins for the oracle's grouped GEMM consumer of the padded FP8 segments.

The DeepSeek-V3 excerpts (fine-grained quantisation: 1x128 activation tiles,
128x128 weight blocks, per-interval promotion into a high-precision
accumulator) define what it computes. Because every scale is constant over one
128-element interval of the inner dimension, the sum of scaled interval
partials equals the plain matrix product of the dequantised operands. That
identity lets a library matmul on library-decoded operands pin the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_synth import gen_logits, gen_x_bf16

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes -> float64 through torch's float8_e4m3fn type (library)."""
    t = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _random_codes(rng, shape):
    """Uniform over the 254 finite E4M3 codes (0x7F and 0xFF are NaN)."""
    c = rng.integers(0, 254, size=shape, dtype=np.int64)
    c = np.where(c >= 0x7F, c + 1, c)
    return c.astype(np.uint8)


def _segments(rng, E, rows_per_expert_max, align):
    counts = rng.integers(0, rows_per_expert_max + 1, size=E)
    padded = -(-counts // align) * align
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(padded)
    return counts, off


def _library_gemm(a, a_s, off, w, w_s):
    """Dequantise with the library decode and np.repeat'ed scales, then one
    float64 matmul per expert."""
    E, N, K = w.shape
    ad = _decode(a) * np.repeat(a_s.astype(np.float64), 128, axis=1)
    wd = _decode(w) * np.repeat(np.repeat(w_s.astype(np.float64), 128, axis=1), 128, axis=2)
    y = np.zeros((a.shape[0], N))
    mag = np.zeros((a.shape[0], N))
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        y[r0:r1] = ad[r0:r1] @ wd[e].T
        mag[r0:r1] = np.abs(ad[r0:r1]) @ np.abs(wd[e]).T
    return y, mag


@pytest.mark.parametrize("E,N,K,align,seed", [(3, 128, 128, 1, 0), (4, 256, 384, 128, 1),
                                              (5, 128, 512, 8, 2), (1, 384, 256, 1, 3)])
def test_gemm_equals_dequantised_library_matmul(E, N, K, align, seed):
    rng = np.random.default_rng(seed)
    _, off = _segments(rng, E, 40, align)
    rows = int(off[E]) + 5
    a = _random_codes(rng, (rows, K))
    a_s = rng.uniform(0.5, 2.0, size=(rows, K // 128)).astype(np.float32) * 1e-3
    w = _random_codes(rng, (E, N, K))
    w_s = rng.uniform(0.5, 2.0, size=(E, N // 128, K // 128)).astype(np.float32) * 1e-2
    # The formula holds for any fp32 scale; negative ones exercise the
    # absolute-value sum (quantisation itself only makes scales >= 0).
    w_s *= np.where(rng.random(w_s.shape) < 0.3, -1.0, 1.0).astype(np.float32)
    g = oracle.grouped_gemm_fp8(a, a_s, off, w, w_s)
    y_lib, mag_lib = _library_gemm(a, a_s, off, w, w_s)
    live = slice(0, int(off[E]))
    # Two fp64 evaluations of the same real-number sum in different orders.
    assert np.all(np.abs(g.y64[live] - y_lib[live]) <= 1e-12 * mag_lib[live] + 1e-300)
    assert np.all(np.abs(g.mag[live] - mag_lib[live]) <= 1e-12 * mag_lib[live] + 1e-300)
    # The bf16 output is the nearest bf16 of the library value: within half a
    # bf16 spacing (2^-8 relative to the value's binade, so 2^-8 |v| bounds it).
    yb = g.y[live].astype(np.uint32) << 16
    yv = yb.view(np.float32).astype(np.float64)
    assert np.all(np.abs(yv - y_lib[live]) <= 2.0 ** -8 * np.abs(y_lib[live]) + 1e-30)
    # Rows past the last segment are not written.
    assert not g.y[int(off[E]):].any()


def test_gemm_identity_weights_return_dequantised_rows():
    rng = np.random.default_rng(5)
    E, K = 2, 256
    _, off = _segments(rng, E, 30, 1)
    rows = int(off[E])
    a = _random_codes(rng, (rows, K))
    a_s = rng.uniform(0.1, 4.0, size=(rows, K // 128)).astype(np.float32)
    w = np.zeros((E, K, K), np.uint8)
    w[:, np.arange(K), np.arange(K)] = 0x38          # 1.0
    w_s = np.ones((E, K // 128, K // 128), np.float32)
    g = oracle.grouped_gemm_fp8(a, a_s, off, w, w_s)
    # + 0.0: a sum that starts at +0 and meets only a -0 term stays +0.
    want = _decode(a) * np.repeat(a_s.astype(np.float64), 128, axis=1) + 0.0
    np.testing.assert_array_equal(g.y64, want)
    wbits = np.array([oracle.bf16_from_double(v) for v in want.ravel()], np.uint16)
    np.testing.assert_array_equal(g.y.ravel(), wbits)


def test_gemm_segments_use_their_own_expert():
    rng = np.random.default_rng(6)
    E, K = 6, 128
    counts, off = _segments(rng, E, 9, 4)
    rows = int(off[E])
    a = _random_codes(rng, (rows, K))
    a_s = np.ones((rows, 1), np.float32)
    w = np.zeros((E, K, K), np.uint8)
    w[:, np.arange(K), np.arange(K)] = 0x38
    w_s = (np.arange(E, dtype=np.float32) + 1.0).reshape(E, 1, 1)
    g = oracle.grouped_gemm_fp8(a, a_s, off, w, w_s)
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        np.testing.assert_array_equal(g.y64[r0:r1], (e + 1.0) * _decode(a[r0:r1]))


def test_gemm_interval_scales_brute_force_fractions():
    """Exact rational evaluation of sum_b s_a s_w sum_k a w on a tiny case."""
    from fractions import Fraction
    rng = np.random.default_rng(7)
    E, N, K = 1, 128, 256
    off = np.array([0, 3], np.int32)
    a = _random_codes(rng, (3, K))
    a_s = rng.uniform(0.5, 2.0, size=(3, 2)).astype(np.float32)
    w = _random_codes(rng, (E, N, K))
    w_s = rng.uniform(0.5, 2.0, size=(E, 1, 2)).astype(np.float32)
    g = oracle.grouped_gemm_fp8(a, a_s, off, w, w_s)
    ad, wd = _decode(a), _decode(w)
    for r in range(3):
        for n in (0, 17, 127):
            exact = Fraction(0)
            for b in range(2):
                part = sum(Fraction(ad[r, k]) * Fraction(wd[0, n, k]) for k in range(b * 128, b * 128 + 128))
                exact += Fraction(float(a_s[r, b])) * Fraction(float(w_s[0, 0, b])) * part
            assert abs(Fraction(g.y64[r, n]) - exact) <= Fraction(2) ** -40 * abs(Fraction(g.mag[r, n]))


def test_gemm_pad_rows_of_dispatch_are_zero():
    """FP8 dispatch with 128-row alignment: pad rows have zero codes and zero
    scales, so their GEMM output is exactly +0."""
    T, H, E, k = 40, 256, 4, 2
    x = gen_x_bf16(T, H, 0)
    idx, _ = oracle.route_topk(gen_logits(T, E, 0), k)
    d = oracle.dispatch(x, idx, E, 1, 128, True)
    rng = np.random.default_rng(8)
    w = _random_codes(rng, (E, 128, H))
    w_s = rng.uniform(0.5, 2.0, size=(E, 1, H // 128)).astype(np.float32)
    g = oracle.grouped_gemm_fp8(d.out, d.scales, d.expert_offsets, w, w_s)
    pad = d.row_src[:d.num_rows] < 0
    assert pad.any()
    assert not g.y[:d.num_rows][pad].any()
    assert (g.y[:d.num_rows][~pad] != 0).any()


def test_gemm_sampled_positions_equal_full():
    rng = np.random.default_rng(9)
    E, N, K = 3, 256, 256
    _, off = _segments(rng, E, 20, 1)
    rows = int(off[E])
    a = _random_codes(rng, (rows, K))
    a_s = rng.uniform(0.5, 2.0, size=(rows, K // 128)).astype(np.float32)
    w = _random_codes(rng, (E, N, K))
    w_s = rng.uniform(0.5, 2.0, size=(E, N // 128, K // 128)).astype(np.float32)
    full = oracle.grouped_gemm_fp8(a, a_s, off, w, w_s)
    rr = rng.integers(0, rows, 200)
    cc = rng.integers(0, N, 200).astype(np.int32)
    at = oracle.grouped_gemm_fp8_at(a, a_s, off, w, w_s, rr, cc)
    np.testing.assert_array_equal(at.y, full.y[rr, cc])
    np.testing.assert_array_equal(at.y64, full.y64[rr, cc])
    np.testing.assert_array_equal(at.mag, full.mag[rr, cc])


def test_quantize_weights_block_scales_and_codes():
    rng = np.random.default_rng(10)
    N, K = 256, 384
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    w[128:256, 256:384] = 0.0                     # one all-zero block
    q, s = oracle.quantize_weights(w)
    assert s.shape == (2, 3)
    for nb in range(2):
        for kb in range(3):
            blk = w[nb * 128:nb * 128 + 128, kb * 128:kb * 128 + 128]
            amax = np.float32(np.abs(blk).max())
            assert s[nb, kb] == np.float32(amax / np.float32(448.0))
            qb = q[nb * 128:nb * 128 + 128, kb * 128:kb * 128 + 128]
            if amax == 0:
                assert s[nb, kb] == 0 and not qb.any()
                continue
            quot = (torch.from_numpy(blk) / torch.tensor(s[nb, kb])).float()
            want = quot.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            np.testing.assert_array_equal(qb, want)
            i = np.unravel_index(np.abs(blk).argmax(), blk.shape)
            assert qb[i] & 0x7F == 0x7E                 # the block maximum maps to 448
            deq = _decode(qb) * float(s[nb, kb])
            nz = np.abs(blk) >= 2.0 ** -6 * float(s[nb, kb])
            assert np.all(np.abs(deq[nz] - blk[nz]) <= 2.0 ** -4 * np.abs(blk[nz]))


def test_quantize_weights_divides_exactly():
    """Block amax 3136 gives s = 7 exactly. 0.68359375 / 7 = 0.09765625 is the
    midpoint of the E4M3 values 0.09375 (0x1C, even) and 0.1015625 (0x1D), so
    the correctly rounded quotient takes 0x1C; fp32(1/7) is above 1/7, and a
    reciprocal multiply lands above the midpoint and takes 0x1D."""
    w = np.zeros((128, 128), np.float32)
    w[0, 0] = 3136.0
    w[5, 7] = 0.68359375
    w[9, 9] = -0.68359375
    q, s = oracle.quantize_weights(w)
    assert s[0, 0] == np.float32(7.0)
    assert q[0, 0] == 0x7E and q[5, 7] == 0x1C and q[9, 9] == 0x9C
    assert np.float32(0.68359375) * (np.float32(1.0) / np.float32(7.0)) > np.float32(0.09765625)


def test_quantized_weights_gemm_close_to_fp32_product():
    """End to end on realistic operands: quantised activations (dispatch) and
    quantised weights give a product close to the unquantised one."""
    T, H, E, k, N = 32, 256, 2, 1, 128
    x = gen_x_bf16(T, H, 1)
    idx, _ = oracle.route_topk(gen_logits(T, E, 1), k)
    d = oracle.dispatch(x, idx, E, 1, 1, True)
    rng = np.random.default_rng(11)
    wf = (rng.standard_normal((E, N, H)) * 0.05).astype(np.float32)
    q, s = oracle.quantize_weights(wf)
    g = oracle.grouped_gemm_fp8(d.out, d.scales, d.expert_offsets, q, s)
    xs = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for e in range(E):
        r0, r1 = d.expert_offsets[e], d.expert_offsets[e + 1]
        src = d.row_src[r0:r1] // k
        ref = xs[src] @ wf[e].astype(np.float64).T
        err = np.abs(g.y64[r0:r1] - ref)
        # Two E4M3 roundings (2^-4 relative each) bound the error by ~2^-3 of
        # the absolute-value product.
        assert np.all(err <= 2.0 ** -3 * (np.abs(xs[src]) @ np.abs(wf[e]).astype(np.float64).T))
