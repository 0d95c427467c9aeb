"""The layer at seeded random shapes across the supported range: emb and mlp multiples of 64 up to 1024,
E up to 256, k up to 64 (more than 8 in about a third of the cases), T up to 3000, the oracle's work bounded.
Every case checks routing and the sort order bit for bit and y on every token against the oracle, and that the
inference forward (x rows gathered in place) equals the training forward bit for bit; half of them also run
the backward (dx, dtopk_w on every token, dW of every expert)."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_group_amd as moe
import oracle
import workloads
from parity_util import W_ABS, assert_close, assert_close_bf16_out, bits, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _shapes(n=16, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        emb, mlp = 64 * int(rng.integers(1, 17)), 64 * int(rng.integers(1, 17))
        E = int(rng.integers(1, 17)) if rng.random() < 0.5 else int(rng.integers(17, 257))
        k = int(min(E, rng.choice([1, 2, 3, 4, 6, 8])))
        if E > 8 and rng.random() < 0.35:
            k = int(rng.integers(9, min(E, 64) + 1))
        T = int(min(3000, rng.integers(1, max(2, int(4e8 / (k * emb * mlp))) + 1)))
        out.append((i, T, emb, mlp, E, k, bool(rng.random() < 0.5)))
    return out


@pytest.mark.parametrize("i,T,emb,mlp,E,k,bwd", _shapes(), ids=lambda v: str(v))
def test_layer_at_random_shape(i, T, emb, mlp, E, k, bwd):
    wl = workloads.custom(T, emb, mlp, E, k, seed=5000 + i, sigma_w=0.5 / np.sqrt(max(emb, mlp)), backward=bwd)
    h = workloads.make_inputs(wl)
    d = {n: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for n, v in h.items()}
    y, saved = moe.ffn_fwd(d["x"], d["wi"], d["wo"], k, wr=d["wr"], save=True)
    y_inf, _ = moe.ffn_fwd(d["x"], d["wi"], d["wo"], k, wr=d["wr"], save=False)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_inf.view(torch.int16)), "inference and training forward differ"
    x, wi, wo = bits(h["x"]), bits(h["wi"]), bits(h["wo"])
    idx, w, _ = oracle.route(x, h["wr"].numpy(), None, k)
    assert np.array_equal(saved["topk_idx"].cpu().numpy(), idx), "topk_idx"
    assert np.abs(saved["topk_w"].cpu().numpy() - w).max() <= W_ABS, "topk_w"
    _, go, ss, sr = oracle.dispatch(idx, E)
    assert np.array_equal(saved["group_offsets"].cpu().numpy(), go), "group_offsets"
    assert np.array_equal(saved["sorted_slot"].cpu().numpy(), ss), "sorted_slot"
    assert np.array_equal(saved["slot_row"].cpu().numpy(), sr), "slot_row"
    assert_close(to_np(y), oracle.ffn_fwd_tokens(x, idx, w, wi, wo), "y")
    if not bwd:
        return
    g = moe.ffn_bwd(d["dy"], saved, d["wi"], d["wo"], k)
    dy = bits(h["dy"])
    dx, dtw = oracle.ffn_bwd_tokens(x, idx, w, wi, wo, dy, stored_bf16=True)
    assert_close(to_np(g["dx"]), dx, "dx")
    assert_close(g["dtopk_w"].cpu().numpy(), dtw, "dtopk_w")
    ref = oracle.ffn_wgrad_experts(x, idx, w, wi, wo, dy, range(E), stored_bf16=True)
    assert_close_bf16_out(to_np(g["dwi"]), np.stack([ref[e][0] for e in range(E)]), "dwi")
    assert_close_bf16_out(to_np(g["dwo"]), np.stack([ref[e][1] for e in range(E)]), "dwo")
