"""The launches moe_route_dispatch makes for each kind of batch, read from
the library's launch log (MOE_ROUTE_LOG=1) in one child process: one for
small batches with few experts, two (counting, scan + rows) for small
batches, three for large ones, and the route kernel first when the
sorting-network top-k does not apply."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys, torch
sys.path.insert(0, "tests")
from combine_moe_route_amd import alloc_dispatch, moe_route_dispatch
from moe_synth import gen_logits, gen_x_bf16
from parity_util import to_dev_bf16
dev = torch.device("cuda:0")
for name, T, H, E, k, G, A, fp8 in CASES:
    x = to_dev_bf16(gen_x_bf16(T, H, 0), dev)
    logits = torch.from_numpy(gen_logits(T, E, 0)).to(dev)
    torch.cuda.synchronize()
    print("@case " + name, file=sys.stderr, flush=True)
    moe_route_dispatch(logits, x, k, G, A, fp8, alloc_dispatch(T, H, E, k, G, A, fp8, dev))
    torch.cuda.synchronize()
    print("@end", file=sys.stderr, flush=True)
"""

CASES = [
    # name, T, H, E, k, groups, row_align, fp8 -> launches
    ("mixtral_decode", 128, 4096, 8, 2, 1, 1, False),
    ("dsv3_decode", 128, 7168, 256, 8, 32, 1, True),
    ("kimi_prefill", 4096, 1024, 384, 8, 1, 1, False),
    ("dsv3_prefill", 16384, 1024, 256, 8, 32, 128, True),
    ("k9", 300, 256, 64, 9, 1, 1, False),
]
WANT = {
    "mixtral_decode": ["route+scan+scatter"],
    "dsv3_decode": ["route_count", "scan+scatter"],
    "kimi_prefill": ["route_count", "scan", "scatter"],
    "dsv3_prefill": ["route_count", "scan", "scatter"],
    "k9": ["route", "count", "scan+scatter"],
}


def test_launch_plan_per_batch_kind():
    assert __import__("torch").cuda.is_available()
    env = dict(os.environ, MOE_ROUTE_LOG="1")
    code = "CASES = " + repr(CASES) + "\n" + CHILD
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    got, cur = {}, None
    for line in r.stderr.splitlines():
        if line.startswith("@case "):
            cur = line.split()[1]
            got[cur] = []
        elif line.startswith("@end"):
            cur = None
        elif cur and line.startswith("[moe_route] "):
            got[cur].append(line.split()[1])
    assert got == WANT, got


MASKED = r"""
import ctypes, sys, torch
sys.path.insert(0, "tests")
from combine_moe_route_amd import alloc_dispatch, moe_route_dispatch
from moe_synth import gen_logits, gen_x_bf16
from parity_util import to_dev_bf16
hip = ctypes.CDLL("libamdhip64.so")
dev = torch.device("cuda:0")
n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
T, H, E, k, G, A = 16384, 1024, 256, 8, 32, 128
x = to_dev_bf16(gen_x_bf16(T, H, 0), dev)
logits = torch.from_numpy(gen_logits(T, E, 0)).to(dev)
bufs = alloc_dispatch(T, H, E, k, G, A, True, dev)
torch.cuda.synchronize()
for n in (0, 32, 64):
    print("@case %d" % n, file=sys.stderr, flush=True)
    if n:
        mask = (ctypes.c_uint32 * ((n_cu + 31) // 32))()
        for c in range(n):
            mask[c // 32] |= 1 << (c % 32)
        h = ctypes.c_void_p()
        assert hip.hipExtStreamCreateWithCUMask(ctypes.byref(h), len(mask), mask) == 0
        s = torch.cuda.ExternalStream(h.value, device=dev)
    else:
        h, s = None, torch.cuda.current_stream(dev)
    with torch.cuda.stream(s):
        moe_route_dispatch(logits, x, k, G, A, True, bufs)
    torch.cuda.synchronize()
    if h is not None:
        hip.hipStreamDestroy(h)
    print("@end", file=sys.stderr, flush=True)
"""


def test_scan_grid_follows_cu_mask():
    """The scan takes one block per CU of the stream's CU mask (its blocks
    each hold over half a CU's LDS), up to 128 blocks."""
    assert __import__("torch").cuda.is_available()
    env = dict(os.environ, MOE_ROUTE_LOG="1")
    r = subprocess.run([sys.executable, "-c", MASKED], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    grids, cur = {}, None
    for line in r.stderr.splitlines():
        if line.startswith("@case "):
            cur = int(line.split()[1])
        elif line.startswith("@end"):
            cur = None
        elif cur is not None and line.startswith("[moe_route] scan "):
            grids[cur] = int(line.split()[2].split("=")[1])
    assert grids == {0: 128, 32: 32, 64: 64}, r.stderr[-3000:]
