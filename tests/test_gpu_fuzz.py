"""Seeded fuzz of the whole chain (route, dispatch, stand-in experts, combine)
against the oracle over random shapes and options: token counts including 0
and ragged tails, expert counts 1..1024, k up to 80, destination groups,
row alignments, bf16 and FP8, and logits rounded to a coarse grid so that
ties straddle the top-k boundary. Every case runs the same bitwise checks as
the hand-picked parity cases."""
import numpy as np
import pytest
import torch

from moe_synth import gen_logits
from parity_util import Case, full_case, log

pytestmark = pytest.mark.gpu

N_CASES = 40


def _case(i):
    rng = np.random.default_rng([2024, i])
    E = int(rng.choice([1, 2, 3, 8, 17, 64, 100, 256, 384, 512, 1024]))
    if rng.random() < 0.1:
        k = int(rng.integers(65, min(E, 80) + 1)) if E > 64 else E
    else:
        k = int(rng.integers(1, min(E, 16) + 1))
    divisors = [g for g in (1, 2, 4, 8, 16, 32) if E % g == 0]
    G = int(rng.choice(divisors))
    A = int(rng.choice([1, 1, 8, 128]))
    fp8 = bool(rng.random() < 0.5)
    H = int(rng.choice([128, 256, 640, 1024])) if fp8 else int(rng.choice([8, 64, 200, 512, 1024]))
    T = int(rng.choice([0, 1, 7, 64, 255, 256, 257, 600]))
    return Case(T=T, H=H, E=E, k=k, groups=G, row_align=A, fp8=fp8, seed=i), rng


@pytest.mark.parametrize("i", range(N_CASES))
def test_fuzz_chain(i):
    c, rng = _case(i)
    dev = torch.device("cuda:0")
    logits = gen_logits(c.T, c.E, c.seed)
    if rng.random() < 0.4:
        # a coarse grid makes equal logits common, so ties cross the k boundary
        logits = (np.round(logits * 2.0) / 2.0).astype(np.float32)
    log(f"fuzz case {i}: {c.label()}")
    full_case(c, dev, logits_np=logits)


@pytest.mark.parametrize("i", range(10))
def test_fuzz_grouped_gemm(i):
    """Random segment layouts (empty, ragged, 128-aligned), widths and depths
    for the grouped FP8 GEMM, uniform finite codes, against the oracle."""
    import oracle
    from moe_synth import gen_fp8_weight_codes, gen_weight_scales
    from test_gpu_gemm import check, run_gpu
    rng = np.random.default_rng([77, i])
    E = int(rng.choice([1, 3, 8, 33]))
    N = 256 * int(rng.integers(1, 4))
    K = 128 * int(rng.integers(1, 9))
    align = int(rng.choice([1, 8, 128]))
    counts = rng.integers(0, 300, size=E)
    counts[rng.random(E) < 0.25] = 0
    padded = -(-counts // align) * align
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(padded)
    R = int(off[E]) + int(rng.integers(0, 40))
    log(f"gemm fuzz {i}: E={E} N={N} K={K} align={align} rows={int(off[E])} of {R}")
    a = gen_fp8_weight_codes(1, max(R, 1), K, 100 + i)[0][:R]
    a_s = rng.uniform(0.25, 4.0, size=(R, K // 128)).astype(np.float32)
    w = gen_fp8_weight_codes(E, N, K, 200 + i)
    w_s = gen_weight_scales(E, N, K, 200 + i)
    g = oracle.grouped_gemm_fp8(a, a_s, off, w, w_s)
    y = run_gpu(np.ascontiguousarray(a), a_s, off, w, w_s)
    check(y, g, off, K)
