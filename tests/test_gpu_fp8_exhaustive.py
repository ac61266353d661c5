"""The FP8 quantiser over its whole input domain: every pair of bf16 values
(x, amax) with amax finite and positive and |x| <= amax, both signs of x and
-0 included (1.07e9 pairs). Each 1x128 block holds amax first (so it is the
block maximum) and 127 values below it; the blocks go through moe_dispatch
(FP8, one expert, so rows keep token order) and every E4M3 code and every
block scale must equal the oracle's quantisation of the same block (1x128
tiles, s = amax / 448, codes = RNE E4M3 of the fp32 quotient, saturating:
the DeepSeek-V3 excerpt on fine-grained 1x128 activation tiles; "Enabling
trillion-parameter models on AWS EFA", Evaluation, block-scaled FP8
dispatch). The oracle runs in its OpenMP build, spread over the host cores."""
import time

import numpy as np
import pytest
import torch

import oracle
from parity_util import log, to_dev_bf16


AMAX_LAST = 0x7F7F             # largest finite bf16
BLOCKS_PER_ROW = 64            # rows of 8192 values
CHUNK_VALUES = 1 << 25         # values per chunk (before packing)


# every bf16 pattern of magnitude m, then its negation: 0, -0, 1, -1, ...
_SIGNED = ((np.arange(2 * 0x7F80, dtype=np.uint32) >> 1) |
           ((np.arange(2 * 0x7F80, dtype=np.uint32) & 1) << 15)).astype(np.uint16)


def domain_blocks(a0: int, a1: int) -> np.ndarray:
    """Blocks [n, 128] uint16 for the amax bit patterns a0 .. a1-1: for each
    amax, its values x = m | sign (m = 0 .. amax, both signs) in groups of
    127, each group led by amax; the last group of an amax is padded with +0."""
    parts, nbs = [], []
    for a in range(a0, a1):
        L = 2 * (a + 1)
        nb = (L + 126) // 127
        parts.append(_SIGNED[:L])
        parts.append(np.zeros(nb * 127 - L, np.uint16))
        nbs.append(nb)
    blocks = np.empty((sum(nbs), 128), np.uint16)
    blocks[:, 0] = np.repeat(np.arange(a0, a1, dtype=np.uint16), nbs)
    blocks[:, 1:] = np.concatenate(parts).reshape(-1, 127)
    return blocks


def chunks():
    a0 = 1
    while a0 <= AMAX_LAST:
        a1, n = a0, 0
        while a1 <= AMAX_LAST and n < CHUNK_VALUES:
            n += 2 * (a1 + 1)
            a1 += 1
        yield a0, a1
        a0 = a1


def test_domain_blocks_cover_every_pair():
    """The enumeration itself (CPU): for a few amax values every |x| <= amax
    appears once with each sign, nothing larger appears, and padding is +0."""
    for a0, a1 in [(1, 5), (0x3F80, 0x3F83), (0x7F7D, 0x7F80)]:
        b = domain_blocks(a0, a1)
        assert np.all(np.abs(b.view(np.int16).astype(np.int32) & 0x7FFF) <= b[:, :1].astype(np.int32))
        for a in range(a0, a1):
            rows = b[b[:, 0] == a, 1:].ravel()
            want = np.concatenate([np.arange(a + 1), np.arange(a + 1) | 0x8000]).astype(np.uint16)
            got = np.sort(rows)
            pad = len(got) - len(want)
            assert pad >= 0 and np.array_equal(np.sort(np.concatenate([want, np.zeros(pad, np.uint16)])), got)


@pytest.mark.gpu
def test_fp8_quantiser_every_x_amax_pair():
    from combine_moe_route_amd import moe_dispatch
    assert torch.cuda.is_available()
    dev = torch.device("cuda:0")
    with oracle.using("omp"):
        done, t0 = 0, time.time()
        for a0, a1 in chunks():
            blocks = domain_blocks(a0, a1)
            n = len(blocks)
            rows = (n + BLOCKS_PER_ROW - 1) // BLOCKS_PER_ROW
            padded = np.zeros((rows * BLOCKS_PER_ROW, 128), np.uint16)
            padded[:n] = blocks
            x = to_dev_bf16(padded.reshape(rows, BLOCKS_PER_ROW * 128), dev)
            idx = torch.zeros((rows, 1), dtype=torch.int32, device=dev)
            b = moe_dispatch(x, idx, 1, 1, 1, True)
            q_ref, s_ref = oracle.quantize_blocks(padded)
            torch.cuda.synchronize()
            q = b.out[:rows].cpu().numpy().reshape(-1, 128)
            s = b.out_scales[:rows].cpu().numpy().reshape(-1)
            bad = np.flatnonzero((q != q_ref).any(axis=1) | (s.view(np.uint32) != s_ref.view(np.uint32)))
            assert bad.size == 0, (f"amax {a0:#06x}..{a1 - 1:#06x}: {bad.size} blocks differ, first "
                                   f"amax {padded[bad[0], 0]:#06x}")
            done += n
            log(f"  amax {a0:#06x}..{a1 - 1:#06x}: {n} blocks, {done} total, {time.time() - t0:.1f} s")
        assert done > 8_400_000
