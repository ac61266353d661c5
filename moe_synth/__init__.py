"""Seeded synthetic inputs for the MoE dispatch/combine path.

This module is shared by the tests, the benchmark and the smoke check. It
holds only input generation: workload shapes, random streams and the
rounding of the generated float32 activations to bfloat16 bit patterns. It
contains none of the routing, dispatch or combine arithmetic, so the CPU
oracle and the HIP library stay independent of each other and of it.

Workloads stand in for the shapes the Perplexity posts ("Enabling
trillion-parameter models on AWS EFA", section Evaluation / dispatch and
combine latency: hidden size 7168, block-scaled FP8 dispatch, bf16 combine,
128-token decode and 4096-token prefill batches) and the DeepSeek-V3 and
Kimi-K2 / Mixtral expert counts. No public dataset is involved; every array
is drawn from numpy's PCG64 generator with the stream layout below.

Streams: ``np.random.default_rng([seed, s])`` with s = 0 for activations,
s = 1 for router logits, s = 2 for the Zipf popularity permutation, s = 3
for fp32 expert weights, s = 4 for E4M3 weight codes, s = 5 for weight
block scales.

Expert weights for the grouped GEMM that consumes the FP8 segments come in
two forms: fp32 normal weights with standard deviation 1/sqrt(K) (the tests
quantise them), and already-quantised weights drawn directly as E4M3 codes,
uniform over the 254 finite codes, with block scales uniform in
[0.5, 1.5) * 2^-8 (for full-size runs, where quantising 7.5 GB on the host
would take minutes; the GEMM's speed does not depend on the values).
"""
from __future__ import annotations

from dataclasses import dataclass, asdict
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "workload",
    "gen_x_bf16",
    "gen_logits",
    "zipf_bias",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "gen_weights_f32",
    "gen_fp8_weight_codes",
    "gen_weight_scales",
]


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes plus the options of the dispatch call."""

    name: str
    T: int              # tokens on this GPU
    H: int              # hidden size
    E: int              # experts
    k: int              # experts per token (top-k)
    groups: int = 1     # destination groups (stand-in for EP send buffers)
    row_align: int = 1  # expert segments padded to a multiple of this many rows
    fp8: bool = False   # FP8 e4m3 payload with 1x128 fp32 scales
    zipf_s: Optional[float] = None  # skewed router prior, or None
    seed: int = 0

    def with_(self, **kw) -> "Workload":
        d = asdict(self)
        d.update(kw)
        return Workload(**d)


# The five workloads, smallest first. Names describe the shape they mimic.
WORKLOADS = {
    "tiny": Workload("tiny", T=64, H=256, E=8, k=2),
    "mixtral_decode": Workload("mixtral_decode", T=128, H=4096, E=8, k=2),
    "dsv3_decode": Workload("dsv3_decode", T=128, H=7168, E=256, k=8,
                            groups=32, fp8=True),
    "kimi_prefill": Workload("kimi_prefill", T=4096, H=7168, E=384, k=8,
                             zipf_s=1.1),
    "dsv3_prefill": Workload("dsv3_prefill", T=16384, H=7168, E=256, k=8,
                             groups=32, row_align=128, fp8=True),
}


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return w.with_(**overrides) if overrides else w


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); finite input.

    Returns the 16-bit patterns as uint16.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def gen_x_bf16(T: int, H: int, seed: int = 0) -> np.ndarray:
    """Activations x ~ N(0, 1) drawn in float32, rounded to bf16; uint16 [T, H]."""
    x = _rng(seed, 0).standard_normal((T, H), dtype=np.float32)
    return f32_to_bf16_bits(x)


def zipf_bias(E: int, s: float, seed: int = 0) -> np.ndarray:
    """Per-expert logit bias giving a Zipf(s) popularity prior.

    bias_e = -s * ln(rank_e), where rank is a seeded permutation of 1..E. Added
    to N(0,1) logits, the softmax prior of expert e is proportional to
    rank_e ** -s.
    """
    rank = _rng(seed, 2).permutation(E) + 1
    return (-s * np.log(rank.astype(np.float64))).astype(np.float32)


def gen_logits(T: int, E: int, seed: int = 0, zipf_s: Optional[float] = None) -> np.ndarray:
    """Router logits ~ N(0, 1) in float32 [T, E], optionally plus a Zipf bias."""
    l = _rng(seed, 1).standard_normal((T, E), dtype=np.float32)
    if zipf_s is not None:
        l = (l + zipf_bias(E, zipf_s, seed)[None, :]).astype(np.float32)
    return np.ascontiguousarray(l)


def gen_inputs(w: Workload):
    """(x_bf16 uint16 [T,H], logits float32 [T,E]) for a workload."""
    return gen_x_bf16(w.T, w.H, w.seed), gen_logits(w.T, w.E, w.seed, w.zipf_s)


def gen_weights_f32(E: int, N: int, K: int, seed: int = 0) -> np.ndarray:
    """fp32 expert weights [E, N, K], N(0, 1/K) (a fan-in-scaled linear layer)."""
    w = _rng(seed, 3).standard_normal((E, N, K), dtype=np.float32)
    w *= np.float32(1.0 / np.sqrt(K))
    return w


def gen_fp8_weight_codes(E: int, N: int, K: int, seed: int = 0) -> np.ndarray:
    """E4M3 codes [E, N, K], uniform over the 254 finite codes (0x7F and 0xFF,
    the two NaN codes, never occur)."""
    c = _rng(seed, 4).integers(0, 254, size=(E, N, K), dtype=np.uint8)
    for ce in c:                      # per expert: no full-size temporaries
        ce += (ce >= 0x7F).astype(np.uint8)
    return c


def gen_weight_scales(E: int, N: int, K: int, seed: int = 0) -> np.ndarray:
    """fp32 block scales [E, N/128, K/128], uniform in [0.5, 1.5) * 2^-8."""
    s = _rng(seed, 5).random((E, N // 128, K // 128), dtype=np.float32) + np.float32(0.5)
    return s * np.float32(2.0 ** -8)
