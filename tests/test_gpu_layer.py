"""GPU parity of the whole MoE FFN layer (moe_ffn_fwd / moe_ffn_bwd) against the oracle.

Small workloads are compared element by element on every token. Full-size
workloads (the Gemma4-class layer, the Zipf token sweep, the DeepSeek-V3-shaped
forward+backward) are generated on the device; routing, group sizes, sort
order and the permuted rows are compared bit for bit on every token. The
forward output of the Gemma4-class layer and of the sweep is compared on
every token; the DeepSeek-V3-shaped output and gradients on 64 sampled tokens
and nine experts that the oracle computes one by one. At the largest token count
the boundary takes (T * emb just under 2^31) routing and the sort order are
compared on every token and the output on sampled ones, the last tokens among
them.
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_group_amd as moe
import oracle
import workloads
from parity_util import W_ABS, assert_close, assert_close_bf16_out, bits, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev(inp, device=DEV):
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def _fwd(d, save=True, out=None):
    wl = d["workload"]
    return moe.ffn_fwd(d["x"], d["wi"], d["wo"], wl.k, wr=d["wr"], bias=d["bias"], logits=d["logits_in"], save=save,
                       out=out)


def _np32(t):
    return None if t is None else t.detach().cpu().numpy()


def _oracle_route(h):
    wl = h["workload"]
    return oracle.route(bits(h["x"]), _np32(h["wr"]), _np32(h["bias"]), wl.k, logits_in=_np32(h["logits_in"]))


def _check_routing_and_permute(saved, h, check_xs_rows=None):
    wl = h["workload"]
    r_idx, r_w, _ = _oracle_route(h)
    assert np.array_equal(saved["topk_idx"].cpu().numpy(), r_idx), "topk_idx differs"
    assert np.abs(saved["topk_w"].cpu().numpy() - r_w).max() <= W_ABS
    gs, go, ss, sr = oracle.dispatch(r_idx, wl.E)
    assert np.array_equal(saved["group_sizes"].cpu().numpy(), gs)
    assert np.array_equal(saved["group_offsets"].cpu().numpy(), go)
    assert np.array_equal(saved["sorted_slot"].cpu().numpy(), ss)
    assert np.array_equal(saved["slot_row"].cpu().numpy(), sr)
    xs = bits(saved["xs"])
    xb = bits(h["x"])
    rows = np.arange(wl.S) if check_xs_rows is None else check_xs_rows
    assert np.array_equal(xs[rows], xb[ss[rows] // wl.k])
    return r_idx, r_w, gs, go, ss, sr


@pytest.mark.parametrize("name", ["tiny", "mid_skewed"])
def test_layer_forward_every_token(name):
    h = workloads.make_inputs(name)
    d = _dev(h)
    y, saved = _fwd(d)
    r_idx, r_w, gs, *_ = _check_routing_and_permute(saved, h)
    if name == "mid_skewed":
        assert gs[-1] == 0 and gs[:4].min() > 1000
    ref = oracle.ffn_fwd_tokens(bits(h["x"]), r_idx, r_w, bits(h["wi"]), bits(h["wo"]))
    assert_close(to_np(y), ref, f"{name} y")


@pytest.mark.parametrize("T,emb,mlp,E,k", [(1, 64, 64, 4, 2), (300, 192, 320, 12, 3), (257, 256, 128, 64, 8),
                                           (100, 128, 64, 2, 2), (0, 128, 128, 8, 2), (20, 64, 64, 64, 64),
                                           (200, 192, 320, 37, 3)])
def test_layer_forward_edge_shapes(T, emb, mlp, E, k):
    wl = workloads.custom(T, emb, mlp, E, k, seed=T + E, sigma_w=0.05)
    h = workloads.make_inputs(wl)
    y, saved = _fwd(_dev(h))
    assert y.shape == (T, emb)
    if T == 0:
        assert saved["group_sizes"].sum().item() == 0
        return
    r_idx, r_w, *_ = _check_routing_and_permute(saved, h)
    ref = oracle.ffn_fwd_tokens(bits(h["x"]), r_idx, r_w, bits(h["wi"]), bits(h["wo"]))
    assert_close(to_np(y), ref, "y")


def test_layer_forward_is_deterministic_and_writes_every_output():
    h = workloads.make_inputs("mid_skewed")
    d = _dev(h)
    canary = torch.full((h["workload"].T, h["workload"].emb), float("nan"), dtype=torch.bfloat16, device=DEV)
    y1, _ = _fwd(d, save=False, out=canary)
    assert torch.isfinite(y1).all()
    y2, _ = _fwd(d, save=False)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("name", ["tiny", "mid_skewed"])
def test_layer_forward_inference_gather_equals_training_forward_bitwise(name):
    """Inference reads x rows in place through sorted_slot; training materialises xs first. The GEMM
    arithmetic is the same, so y must agree bit for bit."""
    h = workloads.make_inputs(name)
    d = _dev(h)
    y_inf, _ = _fwd(d, save=False)
    y_trn, saved = _fwd(d, save=True)
    assert saved is not None
    assert torch.equal(y_inf.view(torch.int16), y_trn.view(torch.int16))


def test_layer_forward_wo_times_two_doubles_y_exactly():
    h = workloads.make_inputs("tiny")
    d = _dev(h)
    y1, _ = _fwd(d, save=False)
    d["wo"] = (d["wo"].float() * 2).to(torch.bfloat16)
    y2, _ = _fwd(d, save=False)
    assert torch.equal((y1.float() * 2).to(torch.bfloat16).view(torch.int16), y2.view(torch.int16))


def test_layer_forward_token_shuffle_shuffles_rows():
    h = workloads.make_inputs("tiny")
    d = _dev(h)
    y, _ = _fwd(d, save=False)
    perm = torch.randperm(h["workload"].T, generator=torch.Generator().manual_seed(0)).to(DEV)
    d2 = dict(d)
    d2["x"] = d["x"][perm].contiguous()
    y2, _ = _fwd(d2, save=False)
    assert torch.equal(y[perm].view(torch.int16), y2.view(torch.int16))


def _small_bwd_case():
    wl = workloads.custom(384, 256, 128, 8, 2, seed=77, sigma_w=0.02, backward=True)
    return workloads.make_inputs(wl)


def test_layer_backward_every_token_and_expert():
    h = _small_bwd_case()
    wl = h["workload"]
    d = _dev(h)
    y, saved = _fwd(d)
    g = moe.ffn_bwd(d["dy"], saved, d["wi"], d["wo"], wl.k)
    r_idx, r_w, *_ = _check_routing_and_permute(saved, h)
    x, wi, wo, dy = bits(h["x"]), bits(h["wi"]), bits(h["wo"]), bits(h["dy"])
    # o, dh and dxs are stored in bf16 between stages (R9): the reference rounds them there too
    dx, dtw = oracle.ffn_bwd_tokens(x, r_idx, r_w, wi, wo, dy, stored_bf16=True)
    assert_close(to_np(g["dx"]), dx, "dx")
    assert_close(g["dtopk_w"].cpu().numpy(), dtw, "dtopk_w")
    # dW = X^T dH multiplies factors the layer stores in bf16 (a, do, dh): the reference rounds them
    # where the layer stores them and is held to the fixed bound
    ref = oracle.ffn_wgrad_experts(x, r_idx, r_w, wi, wo, dy, range(wl.E), stored_bf16=True)
    assert_close_bf16_out(to_np(g["dwi"]), np.stack([ref[e][0] for e in range(wl.E)]), "dwi")
    assert_close_bf16_out(to_np(g["dwo"]), np.stack([ref[e][1] for e in range(wl.E)]), "dwo")
    # skipping outputs leaves the others unchanged
    g2 = moe.ffn_bwd(d["dy"], saved, d["wi"], d["wo"], wl.k, need=("dx",))
    assert torch.equal(g2["dx"].view(torch.int16), g["dx"].view(torch.int16))


@pytest.mark.parametrize("T,emb,mlp,E,k", [(1, 64, 64, 4, 2), (100, 128, 64, 2, 2), (257, 256, 128, 64, 8),
                                           (0, 128, 128, 8, 2), (20, 64, 64, 64, 64), (200, 192, 320, 37, 3)])
def test_layer_backward_edge_shapes(T, emb, mlp, E, k):
    """One token (two of its four experts get no rows); k = E; 64 experts of about 32 rows each (every row
    block partial); no tokens at all; the largest k (every token picks all 64 experts); 37 experts (not a
    multiple of the 8 XCDs the weight-gradient tiles are dealt over) with emb and mlp that leave partial
    tiles in every weight-gradient dimension. Every gradient on every token and expert against the oracle, and an
    expert with no rows gets dW exactly 0."""
    wl = workloads.custom(T, emb, mlp, E, k, seed=T + 3 * E, sigma_w=0.05, backward=True)
    h = workloads.make_inputs(wl)
    d = _dev(h)
    y, saved = _fwd(d)
    g = moe.ffn_bwd(d["dy"], saved, d["wi"], d["wo"], k)
    assert tuple(g["dx"].shape) == (T, emb) and tuple(g["dtopk_w"].shape) == (T, k)
    gs = saved["group_sizes"].cpu().numpy()
    for e in np.flatnonzero(gs == 0):
        assert not g["dwi"][e].any() and not g["dwo"][e].any(), f"expert {e} has no rows but a nonzero dW"
    if T == 0:
        return
    r_idx, r_w, *_ = _check_routing_and_permute(saved, h)
    x, wi, wo, dy = bits(h["x"]), bits(h["wi"]), bits(h["wo"]), bits(h["dy"])
    dx, dtw = oracle.ffn_bwd_tokens(x, r_idx, r_w, wi, wo, dy, stored_bf16=True)
    assert_close(to_np(g["dx"]), dx, "dx")
    assert_close(g["dtopk_w"].cpu().numpy(), dtw, "dtopk_w")
    ref = oracle.ffn_wgrad_experts(x, r_idx, r_w, wi, wo, dy, range(E), stored_bf16=True)
    assert_close_bf16_out(to_np(g["dwi"]), np.stack([ref[e][0] for e in range(E)]), "dwi")
    assert_close_bf16_out(to_np(g["dwo"]), np.stack([ref[e][1] for e in range(E)]), "dwo")


@pytest.mark.parametrize("T,emb,mlp,E,k", [(384, 256, 128, 8, 2), (300, 128, 256, 6, 3)])
def test_layer_backward_recomputing_h_equals_kept_h_bitwise(T, emb, mlp, E, k):
    """Full rematerialisation of h: the forward keeps no h and the backward recomputes it with the forward's
    own GEMM, so every gradient and every other kept activation is bit-identical to the run that keeps h
    (mlp > emb in the second case puts the recomputed SwiGLU output in a buffer of its own)."""
    wl = workloads.custom(T, emb, mlp, E, k, seed=91, sigma_w=0.02, backward=True)
    d = _dev(workloads.make_inputs(wl))
    y1, s1 = moe.ffn_fwd(d["x"], d["wi"], d["wo"], k, wr=d["wr"], bias=d["bias"], save=True)
    y2, s2 = moe.ffn_fwd(d["x"], d["wi"], d["wo"], k, wr=d["wr"], bias=d["bias"], save=True, keep_h=False)
    assert s2["h"] is None
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    for n, v in s1.items():
        if n != "h":
            assert torch.equal(v.view(torch.uint8), s2[n].view(torch.uint8)), n
    g1 = moe.ffn_bwd(d["dy"], s1, d["wi"], d["wo"], k)
    g2 = moe.ffn_bwd(d["dy"], s2, d["wi"], d["wo"], k)
    for n in ("dx", "dwi", "dwo", "dtopk_w"):
        assert torch.equal(g1[n].view(torch.uint8), g2[n].view(torch.uint8)), n


# ---------------------------------------------------------------- full-size workloads

def _sample_tokens(T, n, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, T - 1], rng.choice(T, n - 2, replace=False)])).astype(np.int64)


def _host(d):
    return {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


_FULL: dict = {}
FULL_FWD = ["gemma4_class"] + [f"sweep_zipf_T{t}" for t in workloads.SWEEP_T]
CHUNK = 4096  # tokens per oracle comparison (one test each, so a long check reports as it goes)


def _full_forward(name):
    """The full-size forward in the launch configuration the benchmark times (inference: x rows gathered
    in place), cached for the module; routing, sort order and xs of the training forward checked bit for
    bit on every row, and the two forwards' outputs bit for bit against each other."""
    if name not in _FULL:
        _FULL.clear()
        d = workloads.make_inputs(name, device=DEV)
        y_inf, _ = _fwd(d, save=False)
        y_trn, saved = _fwd(d)
        torch.cuda.synchronize()
        assert torch.equal(y_inf.view(torch.int16), y_trn.view(torch.int16))
        h = _host(d)
        routing = _check_routing_and_permute(saved, h)
        _FULL[name] = (h, to_np(y_inf), routing)
    return _FULL[name]


@pytest.mark.slow
@pytest.mark.parametrize("name,chunk", [(n, c) for n in FULL_FWD
                                        for c in range(-(-workloads.WORKLOADS[n].T // CHUNK))])
def test_full_size_forward_every_token(name, chunk):
    h, y, (r_idx, r_w, *_) = _full_forward(name)
    T = h["workload"].T
    toks = np.arange(chunk * CHUNK, min(T, (chunk + 1) * CHUNK), dtype=np.int64)
    ref = oracle.ffn_fwd_tokens(bits(h["x"]), r_idx, r_w, bits(h["wi"]), bits(h["wo"]), tokens=toks)
    assert_close(y[toks], ref, f"{name} y[{toks[0]}:{toks[-1] + 1}]")


@pytest.mark.slow
def test_layer_forward_at_the_largest_token_count():
    """The largest T * emb the boundary takes: token rows are gathered through 32-bit byte offsets, so
    T * emb < 2^31. 33,554,431 tokens of width 64, 4 experts, top-2, in the inference launch configuration:
    GEMM 1 gathers the rows of x in place, the last ones almost 4 GiB into it. Routing and the sort order
    are compared with the oracle bit for bit on every token, y on sampled tokens, the last 64 among them."""
    T, emb, mlp, E, k = (2 ** 31 - 1) // 64, 64, 64, 4, 2
    d = workloads.make_inputs(workloads.custom(T, emb, mlp, E, k, seed=4242, sigma_w=0.05), device=DEV)
    y, _ = _fwd(d, save=False)
    idx_d, w_d = moe.route(k, x=d["x"], wr=d["wr"])
    perm = moe.permute(d["x"], idx_d, E, rows=False)
    torch.cuda.synchronize()
    xb = bits(d["x"])
    idx, w, _ = oracle.route(xb, d["wr"].cpu().numpy(), None, k)
    assert np.array_equal(idx_d.cpu().numpy(), idx), "topk_idx differs"
    assert np.abs(w_d.cpu().numpy() - w).max() <= W_ABS
    gs, go, ss, sr = oracle.dispatch(idx, E)
    assert np.array_equal(perm["group_sizes"].cpu().numpy(), gs)
    assert np.array_equal(perm["group_offsets"].cpu().numpy(), go)
    assert np.array_equal(perm["sorted_slot"].cpu().numpy(), ss)
    assert np.array_equal(perm["slot_row"].cpu().numpy(), sr)
    toks = np.unique(np.concatenate([np.arange(T - 64, T), [0, T // 2],
                                     np.random.default_rng(1).choice(T, 62, replace=False)])).astype(np.int64)
    ref = oracle.ffn_fwd_tokens(np.ascontiguousarray(xb[toks]), np.ascontiguousarray(idx[toks]),
                                np.ascontiguousarray(w[toks]), bits(d["wi"]), bits(d["wo"]))
    assert_close(to_np(y[torch.from_numpy(toks).to(DEV)]), ref, "y (sampled, the last 64 tokens among them)")
    del d, y, idx_d, w_d, perm
    torch.cuda.empty_cache()


@pytest.mark.slow
def test_layer_forward_at_the_largest_expert_weight():
    """The largest expert weight the boundary takes: emb * 2 * mlp < 2^31 elements, so that offsets inside one
    expert's weight fit 32 bits. emb 16384, mlp 65472 (a 4.3 GB prefused wi, a partial SwiGLU column tile,
    GEMM 2 contracting over 65472), 16 tokens, every output element against the oracle."""
    T, emb, mlp, E, k = 16, 16384, 65472, 1, 1
    assert emb * 2 * mlp < 2 ** 31 and emb * 2 * (mlp + 64) >= 2 ** 31
    h = workloads.make_inputs(workloads.custom(T, emb, mlp, E, k, seed=77, sigma_w=0.004), device=DEV)
    y, _ = _fwd(h, save=False)
    torch.cuda.synchronize()
    idx = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    ref = oracle.ffn_fwd_tokens(bits(h["x"]), idx, w, bits(h["wi"]), bits(h["wo"]))
    assert_close(to_np(y), ref, "y")
    del h, y
    torch.cuda.empty_cache()


@pytest.mark.slow
def test_full_size_deepseek_v3_shape_forward_backward_sampled():
    d = workloads.make_inputs("deepseek_v3_shape", device=DEV)
    wl = d["workload"]
    y, saved = _fwd(d)
    g = moe.ffn_bwd(d["dy"], saved, d["wi"], d["wo"], wl.k)
    torch.cuda.synchronize()
    h = _host(d)
    r_idx, r_w, gs, go, ss, sr = _check_routing_and_permute(saved, h)
    x, wi, wo, dy = bits(h["x"]), bits(h["wi"]), bits(h["wo"]), bits(h["dy"])
    toks = _sample_tokens(wl.T, 64, 5)
    ref_y = oracle.ffn_fwd_tokens(x, r_idx, r_w, wi, wo, tokens=toks)
    assert_close(to_np(y)[toks], ref_y, "y[sampled]")
    dx, dtw = oracle.ffn_bwd_tokens(x, r_idx, r_w, wi, wo, dy, tokens=toks, stored_bf16=True)
    assert_close(to_np(g["dx"])[toks], dx, "dx[sampled]")
    assert_close(g["dtopk_w"].cpu().numpy()[toks], dtw, "dtopk_w[sampled]")
    # dW on the most- and least-loaded experts (longest and shortest reductions), the median one and six
    # drawn at random, against the reference with the layer's bf16-stored factors, at the fixed bound
    order = np.argsort(gs, kind="stable")
    experts = {int(order[-1]), int(order[0]), int(order[len(order) // 2])}
    rng = np.random.default_rng(7)
    while len(experts) < 9:
        experts.add(int(rng.integers(0, wl.E)))
    experts = sorted(experts)
    ref = oracle.ffn_wgrad_experts(x, r_idx, r_w, wi, wo, dy, experts, stored_bf16=True)
    for e in experts:
        assert_close_bf16_out(to_np(g["dwi"][e]), ref[e][0], f"dwi[{e}] ({gs[e]} rows)")
        assert_close_bf16_out(to_np(g["dwo"][e]), ref[e][1], f"dwo[{e}] ({gs[e]} rows)")
