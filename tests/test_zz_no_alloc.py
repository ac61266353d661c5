"""moe_dispatch_no_alloc (the library's static scratch instead of a caller
workspace) gives exactly moe_dispatch's results, on two calls in a row, the
second on a smaller input, for bf16 and FP8 rows, padding and groups."""
import numpy as np
import pytest
import torch

from moe_synth import gen_logits, gen_x_bf16
from parity_util import log, to_dev_bf16

pytestmark = pytest.mark.gpu


def _outputs(b, R):
    out = [b.expert_counts, b.expert_offsets, b.group_offsets, b.dst_row, b.row_src[:R],
           b.out[:R].contiguous().view(torch.uint8)]
    if b.out_scales is not None:
        out.append(b.out_scales[:R].contiguous().view(torch.int32))
    return [t.cpu().numpy() for t in out]


def _one(T, H, E, k, groups, row_align, fp8, seed, dev):
    from combine_moe_route_amd import moe_dispatch, moe_dispatch_no_alloc, moe_route_topk
    log(f"[no_alloc] T={T} H={H} E={E} k={k} G={groups} A={row_align} fp8={fp8} seed={seed}")
    x = to_dev_bf16(gen_x_bf16(T, H, seed), dev)
    idx, _ = moe_route_topk(torch.from_numpy(gen_logits(T, E, seed)).to(dev), k)
    ref = moe_dispatch(x, idx, E, groups, row_align, fp8)
    got = moe_dispatch_no_alloc(x, idx, E, groups, row_align, fp8)
    torch.cuda.synchronize()
    R = int(ref.expert_offsets[-1].item())
    for name, a, b in zip(("counts", "offsets", "group_offsets", "dst_row", "row_src", "out",
                           "scales"), _outputs(ref, R), _outputs(got, R)):
        assert np.array_equal(a, b), name
    return R


@pytest.mark.parametrize("fp8", [True, False])
def test_no_alloc_matches_dispatch_twice_second_smaller(fp8):
    dev = torch.device("cuda:0")
    if fp8:
        big = dict(T=2048, H=1024, E=256, k=8, groups=32, row_align=128, fp8=True)
        small = dict(T=300, H=512, E=64, k=4, groups=8, row_align=16, fp8=True)
    else:
        big = dict(T=4096, H=512, E=384, k=8, groups=1, row_align=1, fp8=False)
        small = dict(T=77, H=256, E=8, k=2, groups=2, row_align=4, fp8=False)
    _one(**big, seed=1, dev=dev)
    _one(**small, seed=2, dev=dev)


def test_no_alloc_full_prefill_size():
    dev = torch.device("cuda:0")
    _one(T=16384, H=7168, E=256, k=8, groups=32, row_align=128, fp8=True, seed=0, dev=dev)
    _one(T=128, H=7168, E=256, k=8, groups=32, row_align=1, fp8=True, seed=3, dev=dev)


def test_no_alloc_rejects_oversize_without_launch():
    from combine_moe_route_amd import MoeRouteError, alloc_dispatch, moe_dispatch_no_alloc
    from combine_moe_route_amd.binding import MOE_ENOSPC
    dev = torch.device("cuda:0")
    T, H, E, k = 2_000_000, 8, 64, 8
    x = torch.zeros((T, H), dtype=torch.bfloat16, device=dev)
    idx = torch.zeros((T, k), dtype=torch.int32, device=dev)
    bufs = alloc_dispatch(T, H, E, k, 1, 1, False, dev, workspace=False)
    with pytest.raises(MoeRouteError) as e:
        moe_dispatch_no_alloc(x, idx, E, 1, 1, False, bufs)
    assert e.value.status == MOE_ENOSPC
