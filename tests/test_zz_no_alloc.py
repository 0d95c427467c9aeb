"""moe_permute_noalloc (the allocation-free permute, for callers that cannot allocate) against moe_permute,
through the C ABI: identical bits on two calls in a row, the second smaller (fewer tokens, fewer experts)
so that it runs over the first call's scratch contents; and a shape past the fixed scratch is refused
before anything is enqueued."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_group_amd as moe

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(T, emb, E, k, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((T, emb), generator=g).to(torch.bfloat16).to(DEV)
    idx = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).to(torch.int32).to(DEV)
    return x, idx


def _equal(a, b):
    for n in ("group_sizes", "group_offsets", "sorted_slot", "slot_row"):
        assert torch.equal(a[n], b[n]), n
    if a["xs"] is not None:
        assert torch.equal(a["xs"].view(torch.int16), b["xs"].view(torch.int16)), "xs"


@pytest.mark.parametrize("rows", [True, False])
def test_permute_noalloc_equals_permute_twice_second_smaller(rows):
    for T, emb, E, k, seed in ((20000, 256, 128, 8, 1), (3000, 128, 40, 6, 2)):
        x, idx = _case(T, emb, E, k, seed)
        got = moe.permute(x, idx, E, rows=rows, noalloc=True)
        ref = moe.permute(x, idx, E, rows=rows)
        torch.cuda.synchronize()
        _equal(got, ref)
        assert int(got["group_sizes"].sum()) == T * k


def test_permute_noalloc_refuses_shapes_past_its_scratch():
    E, k = 256, 8
    T = 87360 + 64  # one 64-token block more than 4 MiB of masks and bases hold at E = 256
    x = torch.zeros((T, 64), dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros((T, k), dtype=torch.int32, device=DEV)
    with pytest.raises(moe.MoeError) as ei:
        moe.permute(x, idx, E, rows=False, noalloc=True)
    assert ei.value.status == moe._lib.MOE_ERR_WORKSPACE
    # the largest shape that fits runs
    T = 87360
    x, idx = _case(T, 64, E, k, 3)
    _equal(moe.permute(x, idx, E, rows=False, noalloc=True), moe.permute(x, idx, E, rows=False))
