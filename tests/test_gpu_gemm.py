"""GPU parity of the grouped FP8 GEMM (moe_grouped_gemm_fp8, through the C ABI)
against the oracle, on the same seeded inputs.

Tolerance, derived from the arithmetic (the pages print no values). Let y be
the oracle's fp64 sum and M the same sum over absolute values. The GPU
  - sums each 128-element interval on the matrix cores. On quantised data
    their internal summation error stays below 2^-15.5 of the interval's sum
    of |products|; the bound used is 2^-12 of it. Where every product is an
    integer of at most 225 and the interval sum fits 24 bits, the sum is
    exact;
  - forms the fp32 product of the two scales (one rounding) and adds the
    scaled partial into an fp32 accumulator (one rounding per interval), so
    the error is at most (K/128 + 2) * 2^-24 * M;
  - rounds once to bf16 (8 significant bits): at most half a unit, which is
    at most 2^-8 of the magnitude.
With e = (K/128 + 2) 2^-24 M (+ 2^-12 M unless the intervals are exact):
  |gpu - y| <= 2^-8 (|y| + e) + e.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_synth import (bf16_bits_to_f32, gen_fp8_weight_codes, gen_logits, gen_weight_scales,
                       gen_weights_f32, gen_x_bf16, workload)
from parity_util import bf16_to_np, log

pytestmark = pytest.mark.gpu

MFMA_INTERVAL_REL = 2.0 ** -12
SENTINEL = 0x7FC1          # a bf16 NaN pattern the kernel never produces


def dev():
    return torch.device("cuda:0")


def tolerance(y64, mag, K, exact_intervals=False):
    e = (K // 128 + 2) * 2.0 ** -24 * mag
    if not exact_intervals:
        e = e + MFMA_INTERVAL_REL * mag
    return 2.0 ** -8 * (np.abs(y64) + e) + e + 2.0 ** -133


def dispatched(T, H, E, k, row_align, seed):
    """The oracle's FP8 dispatch of seeded inputs, padded to the capacity with
    rows that no segment covers (filled with codes and scales that would
    show up if they were read)."""
    x = gen_x_bf16(T, H, seed)
    idx, _ = oracle.route_topk(gen_logits(T, E, seed), k)
    d = oracle.dispatch(x, idx, E, 1, row_align, True)
    cap = oracle.max_rows(T, E, k, row_align)
    a = np.full((cap, H), 0x48, np.uint8)          # 4.0
    a[:d.num_rows] = d.out
    a_s = np.full((cap, H // 128), 1.0, np.float32)
    a_s[:d.num_rows] = d.scales
    return a, a_s, d.expert_offsets.copy(), d


def run_gpu(a, a_s, off, w, w_s):
    from combine_moe_route_amd import moe_grouped_gemm_fp8
    d = dev()
    R = a.shape[0]
    N = w.shape[1]
    y = torch.full((R, N), SENTINEL, dtype=torch.int16, device=d).view(torch.bfloat16)
    moe_grouped_gemm_fp8(torch.from_numpy(a).to(d), torch.from_numpy(a_s).to(d),
                         torch.from_numpy(off.astype(np.int32)).to(d), torch.from_numpy(w).to(d),
                         torch.from_numpy(w_s).to(d), y=y)
    torch.cuda.synchronize()
    return bf16_to_np(y)


def check(y_gpu, g, off, K, exact_intervals=False):
    live = int(off[-1])
    yg = bf16_bits_to_f32(y_gpu[:live]).astype(np.float64)
    tol = tolerance(g.y64[:live], g.mag[:live], K, exact_intervals)
    err = np.abs(yg - g.y64[:live])
    bad = ~(err <= tol)
    if bad.any():
        r, n = np.argwhere(bad)[0]
        raise AssertionError(f"{bad.sum()} outputs out of tolerance; first at ({r},{n}): "
                             f"gpu {yg[r, n]!r} oracle {g.y64[r, n]!r} tol {tol[r, n]!r}")
    # rows past the last segment keep their previous contents
    assert (y_gpu[live:] == SENTINEL).all()
    same = float(np.mean(y_gpu[:live] == g.y[:live])) if live else 1.0
    worst = float((err / tol).max()) if live else 0.0
    log(f"  rows {live}: bitwise-equal to the oracle's bf16 {same:.4f}, max err/tol {worst:.3f}")
    return same


@pytest.mark.parametrize("T,H,E,k,A,N,seed", [
    (300, 512, 8, 2, 128, 512, 0),      # 128-row aligned segments, several tiles
    (300, 512, 8, 2, 1, 512, 1),        # ragged segments: partial tiles
    (200, 256, 16, 4, 8, 256, 2),
    (97, 384, 5, 3, 1, 768, 3),         # odd sizes, three column tiles
])
def test_gemm_parity_quantised_weights(T, H, E, k, A, N, seed):
    log(f"gemm parity T={T} H={H} E={E} k={k} A={A} N={N} seed={seed}")
    a, a_s, off, _ = dispatched(T, H, E, k, A, seed)
    w, w_s = oracle.quantize_weights(gen_weights_f32(E, N, H, seed))
    g = oracle.grouped_gemm_fp8(a, a_s, off, w, w_s)
    y = run_gpu(a, a_s, off, w, w_s)
    same = check(y, g, off, H)
    assert same > 0.5


def _integer_codes():
    vals = np.array([oracle.e4m3_value(c) for c in range(256)])
    ok = np.isfinite(vals) & (np.abs(vals) <= 15) & (vals == np.round(vals))
    return np.nonzero(ok)[0].astype(np.uint8)


@pytest.mark.parametrize("E,K,N,seed", [(3, 512, 256, 0), (6, 1024, 512, 1)])
def test_gemm_exact_intervals_tight_tolerance(E, K, N, seed):
    """Integer codes of magnitude <= 15: every interval sum is an integer
    below 2^15, which the matrix cores produce exactly, so only the fp32
    scaling, the accumulation and the bf16 rounding remain."""
    log(f"gemm exact intervals E={E} K={K} N={N}")
    rng = np.random.default_rng(100 + seed)
    codes = _integer_codes()
    counts = rng.integers(0, 300, size=E)
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(counts)
    R = int(off[E]) + 7
    a = codes[rng.integers(0, codes.size, size=(R, K))]
    w = codes[rng.integers(0, codes.size, size=(E, N, K))]
    a_s = rng.uniform(0.25, 4.0, size=(R, K // 128)).astype(np.float32)
    w_s = rng.uniform(0.25, 4.0, size=(E, N // 128, K // 128)).astype(np.float32)
    g = oracle.grouped_gemm_fp8(a, a_s, off, w, w_s)
    y = run_gpu(a, a_s, off, w, w_s)
    same = check(y, g, off, K, exact_intervals=True)
    # With exact intervals the fp32 result differs from y by far less than a
    # bf16 unit, so the bf16 outputs match except next to a rounding midpoint.
    assert same >= 0.999


@pytest.mark.parametrize("counts,N,K,seed", [([600, 450], 512, 512, 0),      # ragged: partial 256-row tiles
                                              ([1024, 0, 256], 256, 384, 1),  # aligned, an empty expert
                                              ([513, 1, 700], 768, 256, 2)])
def test_gemm_256_row_tiles(counts, N, K, seed):
    """Capacities of at least 512 rows per expert select 256-row tiles."""
    rng = np.random.default_rng(40 + seed)
    E = len(counts)
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(counts)
    R = max(int(off[E]) + 5, 512 * E)
    log(f"gemm 256-row tiles: segments {counts}, rows {R}")
    a = gen_fp8_weight_codes(1, R, K, 50 + seed)[0]
    a_s = rng.uniform(0.5, 1.5, size=(R, K // 128)).astype(np.float32)
    w = gen_fp8_weight_codes(E, N, K, 60 + seed)
    w_s = gen_weight_scales(E, N, K, 60 + seed)
    g = oracle.grouped_gemm_fp8(a, a_s, off, w, w_s)
    y = run_gpu(a, a_s, off, w, w_s)
    check(y, g, off, K)


def test_gemm_deep_inner_dimension():
    """K = 16384 (128 k-blocks: many rounds of the three-stage ring)."""
    rng = np.random.default_rng(12)
    E, K, N = 2, 16384, 256
    off = np.array([0, 40, 64], np.int32)
    R = 70
    a = gen_fp8_weight_codes(1, R, K, 31)[0]
    a_s = rng.uniform(0.5, 1.5, size=(R, K // 128)).astype(np.float32)
    w = gen_fp8_weight_codes(E, N, K, 32)
    w_s = gen_weight_scales(E, N, K, 32)
    g = oracle.grouped_gemm_fp8(a, a_s, off, w, w_s)
    y = run_gpu(a, a_s, off, w, w_s)
    check(y, g, off, K)


def test_gemm_empty_experts_and_single_expert():
    rng = np.random.default_rng(7)
    K, N = 256, 256
    for counts in ([0, 130, 0, 5], [260], [0, 0, 0], [128, 128, 1, 127]):
        E = len(counts)
        log(f"gemm segments {counts}")
        off = np.zeros(E + 1, np.int32)
        off[1:] = np.cumsum(counts)
        R = max(int(off[E]), 1) + 3
        a = gen_fp8_weight_codes(1, R, K, 11)[0]
        a_s = rng.uniform(0.5, 1.5, size=(R, K // 128)).astype(np.float32)
        w = gen_fp8_weight_codes(E, N, K, 12)
        w_s = gen_weight_scales(E, N, K, 12)
        g = oracle.grouped_gemm_fp8(a, a_s, off, w, w_s)
        y = run_gpu(a, a_s, off, w, w_s)
        check(y, g, off, K)


def test_gemm_pad_rows_are_exact_zero_and_runs_repeat_bitwise():
    a, a_s, off, d = dispatched(257, 256, 4, 2, 128, 5)
    w, w_s = oracle.quantize_weights(gen_weights_f32(4, 256, 256, 5))
    y1 = run_gpu(a, a_s, off, w, w_s)
    y2 = run_gpu(a, a_s, off, w, w_s)
    np.testing.assert_array_equal(y1, y2)
    pad = d.row_src < 0
    assert pad.any()
    assert not y1[:d.num_rows][pad].any()          # +0 exactly


def test_gemm_uniform_codes_full_exponent_range():
    """Codes uniform over all finite E4M3 values (subnormals to 448)."""
    rng = np.random.default_rng(8)
    E, K, N = 4, 768, 512
    counts = rng.integers(50, 200, size=E)
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(counts)
    R = int(off[E])
    a = gen_fp8_weight_codes(1, R, K, 21)[0]
    a_s = rng.uniform(0.5, 1.5, size=(R, K // 128)).astype(np.float32)
    w = gen_fp8_weight_codes(E, N, K, 22)
    w_s = gen_weight_scales(E, N, K, 22)
    g = oracle.grouped_gemm_fp8(a, a_s, off, w, w_s)
    y = run_gpu(a, a_s, off, w, w_s)
    check(y, g, off, K)


def test_gemm_full_size_dsv3_prefill_sampled():
    """The benchmark's configuration: the DSV3-like prefill dispatch (16384
    tokens, H = K = 7168, 256 experts, top-8, 128-row alignment) into a
    4096-wide expert projection. Outputs are checked at sampled positions
    (every tile's first and last rows among them) against the oracle."""
    wl = workload("dsv3_prefill")
    N = 4096
    log("gemm full size: oracle dispatch")
    a, a_s, off, d = dispatched(wl.T, wl.H, wl.E, wl.k, wl.row_align, wl.seed)
    log(f"gemm full size: rows {d.num_rows} of {a.shape[0]}; weight codes")
    w = gen_fp8_weight_codes(wl.E, N, wl.H, wl.seed)
    w_s = gen_weight_scales(wl.E, N, wl.H, wl.seed)
    from combine_moe_route_amd import moe_grouped_gemm_fp8
    dv = dev()
    R = a.shape[0]
    y = torch.full((R, N), SENTINEL, dtype=torch.int16, device=dv).view(torch.bfloat16)
    log("gemm full size: GPU")
    moe_grouped_gemm_fp8(torch.from_numpy(a).to(dv), torch.from_numpy(a_s).to(dv),
                         torch.from_numpy(off).to(dv), torch.from_numpy(w).to(dv),
                         torch.from_numpy(w_s).to(dv), y=y)
    torch.cuda.synchronize()
    live = int(off[-1])
    yi = y.view(torch.int16)
    assert bool((yi[live:] == SENTINEL).all())
    pad = torch.from_numpy(d.row_src < 0).to(dv)
    assert bool((yi[:live][pad] == 0).all())
    assert bool(torch.isfinite(y[:live].float()).all())
    rng = np.random.default_rng(3)
    tile_rows = np.arange(0, live, 128)
    rows = np.concatenate([tile_rows, np.minimum(tile_rows + 127, live - 1),
                           rng.integers(0, live, 4000)])
    cols = rng.integers(0, N, rows.size).astype(np.int32)
    cols[:tile_rows.size] = rng.integers(0, 16, tile_rows.size) * 256          # tile edges
    cols[tile_rows.size:2 * tile_rows.size] = rng.integers(1, 17, tile_rows.size) * 256 - 1
    got = yi[torch.from_numpy(rows).to(dv), torch.from_numpy(cols.astype(np.int64)).to(dv)]
    got = got.cpu().numpy().view(np.uint16)
    log(f"gemm full size: oracle at {rows.size} positions")
    g = oracle.grouped_gemm_fp8_at(a, a_s, off, w, w_s, rows, cols)
    yg = bf16_bits_to_f32(got).astype(np.float64)
    tol = tolerance(g.y64, g.mag, wl.H)
    err = np.abs(yg - g.y64)
    assert (err <= tol).all(), f"{(err > tol).sum()} sampled outputs out of tolerance"
    log(f"  bitwise-equal {np.mean(got == g.y):.4f}, max err/tol {(err / tol).max():.3f}")
