"""Pins of the CPU oracle against facts outside itself (CPU only).

Each test ties one oracle function to something the oracle does not compute
the same way: brute force over every expert, a closed form (dense SwiGLU FFN,
full softmax mixture), an exact-rational emulation of the fp32 fma chain,
library sorts and softmax, permutation invariants, exact power-of-two
identities, or central finite differences. A dropped term, a wrong sign, a
swapped gate/up half, a transposed operand or an off-by-one index fails at
least one of them.
"""
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import workloads


def _bf16(a: np.ndarray) -> np.ndarray:
    """Round float data to bf16 (RNE) and return the bit patterns."""
    return workloads.bf16_bits(torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16))


def _val(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _silu(g):
    return g / (1.0 + np.exp(-g))


def _case(T, emb, mlp, E, k, seed, sigma=0.3):
    rng = np.random.default_rng(seed)
    x = _bf16(rng.standard_normal((T, emb)))
    wr = (rng.standard_normal((emb, E)) * 0.3).astype(np.float32)
    wi = _bf16(rng.standard_normal((E, emb, 2 * mlp)) * sigma)
    wo = _bf16(rng.standard_normal((E, mlp, emb)) * sigma)
    return x, wr, wi, wo


def _dense_expert(xv, wiv, wov, e):
    """Textbook SwiGLU FFN of expert e on all tokens, float64, gate = first half."""
    mlp = wov.shape[1]
    h = xv @ wiv[e]
    return (_silu(h[:, :mlp]) * h[:, mlp:]) @ wov[e]


# ---------------------------------------------------------------- full forward

@pytest.mark.parametrize("shape", [(8, 16, 16, 4, 2), (64, 128, 256, 8, 2), (16, 32, 24, 6, 3)])
def test_forward_matches_brute_force_dense_then_mask(shape):
    """Every expert computed densely on every token, then masked by the routing."""
    T, emb, mlp, E, k = shape
    x, wr, wi, wo = _case(T, emb, mlp, E, k, seed=sum(shape))
    idx, w, _ = oracle.route(x, wr, None, k)
    xv, wiv, wov = _val(x), _val(wi), _val(wo)
    dense = np.stack([_dense_expert(xv, wiv, wov, e) for e in range(E)])  # [E, T, emb]
    want = np.zeros((T, emb))
    for t in range(T):
        for j in range(k):
            want[t] += float(w[t, j]) * dense[idx[t, j], t]
    got64 = oracle.ffn_fwd_tokens(x, idx, w, wi, wo, real="f64")
    np.testing.assert_allclose(got64, want, rtol=1e-10, atol=1e-12)
    got32 = oracle.ffn_fwd_tokens(x, idx, w, wi, wo, real="f32")
    assert np.linalg.norm(got32 - want) / np.linalg.norm(want) < 1e-5


def test_single_expert_is_dense_swiglu_ffn():
    """E = 1, k = 1: weight exactly 1 and the layer is the dense FFN (silu(xWg) * xWu) Wo."""
    x, wr, wi, wo = _case(12, 32, 40, 1, 1, seed=7)
    idx, w, _ = oracle.route(x, wr, None, 1)
    assert (idx == 0).all() and (w == 1.0).all()
    xv, wiv, wov = _val(x), _val(wi), _val(wo)
    g, u = xv @ wiv[0][:, :40], xv @ wiv[0][:, 40:]
    want = (g * scipy.special.expit(g) * u) @ wov[0]
    np.testing.assert_allclose(oracle.ffn_fwd_tokens(x, idx, w, wi, wo, real="f64"), want, rtol=1e-10, atol=1e-12)


def test_all_experts_is_full_softmax_mixture():
    """k = E: the renormalised weights are the full softmax, y = sum_e softmax(l)_e FFN_e(x)."""
    T, emb, mlp, E = 10, 24, 16, 5
    x, wr, wi, wo = _case(T, emb, mlp, E, E, seed=11)
    idx, w, logits = oracle.route(x, wr, None, E)
    p = scipy.special.softmax(logits.astype(np.float64), axis=1)
    xv, wiv, wov = _val(x), _val(wi), _val(wo)
    parts = [_dense_expert(xv, wiv, wov, e) for e in range(E)]
    want = sum(p[:, e:e + 1] * parts[e] for e in range(E))
    # the weights are stored as fp32: each carries a relative rounding of at most 2^-24
    bound = 2.0 ** -24 * sum(p[:, e:e + 1] * np.abs(parts[e]) for e in range(E)) + 1e-12
    got = oracle.ffn_fwd_tokens(x, idx, w, wi, wo, real="f64")
    assert (np.abs(got - want) <= bound).all()


def test_power_of_two_scaling_is_exact():
    """y(2 wo) == 2 y(wo) bit for bit (scaling by 2 is exact in every operation)."""
    x, wr, wi, wo = _case(16, 32, 32, 4, 2, seed=3)
    idx, w, _ = oracle.route(x, wr, None, 2)
    wo2 = _bf16(_val(wo) * 2.0)
    y1 = oracle.ffn_fwd_tokens(x, idx, w, wi, wo)
    y2 = oracle.ffn_fwd_tokens(x, idx, w, wi, wo2)
    assert np.array_equal(y2, 2 * y1)


def test_token_shuffle_shuffles_rows():
    x, wr, wi, wo = _case(24, 32, 16, 6, 3, seed=5)
    idx, w, _ = oracle.route(x, wr, None, 3)
    y = oracle.ffn_fwd_tokens(x, idx, w, wi, wo)
    perm = np.random.default_rng(0).permutation(24)
    idx2, w2, _ = oracle.route(x[perm], wr, None, 3)
    assert np.array_equal(idx2, idx[perm]) and np.array_equal(w2, w[perm])
    assert np.array_equal(oracle.ffn_fwd_tokens(x[perm], idx2, w2, wi, wo), y[perm])


def test_token_subset_and_thread_count_do_not_change_results():
    x, wr, wi, wo = _case(40, 32, 16, 6, 2, seed=9)
    idx, w, _ = oracle.route(x, wr, None, 2)
    full = oracle.ffn_fwd_tokens(x, idx, w, wi, wo, threads=1)
    sub = np.array([39, 0, 17, 17, 5])
    assert np.array_equal(oracle.ffn_fwd_tokens(x, idx, w, wi, wo, tokens=sub, threads=3), full[sub])
    assert np.array_equal(oracle.router_logits(x, wr, threads=1), oracle.router_logits(x, wr, threads=7))


# ---------------------------------------------------------------- router

def _round_f32(q: Fraction) -> float:
    """Correctly rounded (nearest, ties to even) fp32 value of an exact rational."""
    if q == 0:
        return 0.0
    sign = -1.0 if q < 0 else 1.0
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    ulp = Fraction(2) ** (max(e, -126) - 23)
    s = q / ulp
    n = s.numerator // s.denominator
    rem = s - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * float(n * ulp)


def test_router_logits_are_the_exact_fp32_fma_chain():
    """Each logit equals the chain acc = fl32(x*w + acc) over emb ascending, emulated with exact rationals."""
    T, emb, E = 3, 40, 5
    rng = np.random.default_rng(1)
    x = _bf16(rng.standard_normal((T, emb)))
    wr = (rng.standard_normal((emb, E)) * 0.3).astype(np.float32)
    bias = np.array([0.0, 2.0, -1.5, 0.25, 0.0], np.float32)
    got = oracle.router_logits(x, wr, bias)
    xv = _val(x)
    for t in range(T):
        for e in range(E):
            acc = 0.0
            for i in range(emb):
                acc = _round_f32(Fraction(float(xv[t, i])) * Fraction(float(wr[i, e])) + Fraction(acc))
            acc = _round_f32(Fraction(acc) + Fraction(float(bias[e])))
            assert np.float32(acc) == got[t, e], (t, e)


def test_router_logits_close_to_float64_matmul():
    x, wr, _, _ = _case(50, 256, 8, 16, 2, seed=2)
    got = oracle.router_logits(x, wr).astype(np.float64)
    ref = _val(x) @ wr.astype(np.float64)
    bound = 256 * 2.0 ** -24 * (np.abs(_val(x)) @ np.abs(wr.astype(np.float64)))
    assert (np.abs(got - ref) <= bound + 1e-30).all()


def test_topk_matches_stable_sort_and_softmax():
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((200, 16)).astype(np.float32)
    logits[:, 3] = logits[:, 7]  # plant ties
    logits[::5, 11] = logits[::5, 2]
    for k in (1, 2, 5, 16):
        idx, w = oracle.topk(logits, k)
        want = np.argsort(-logits, axis=1, kind="stable")[:, :k]
        assert np.array_equal(idx, want)
        picked = np.take_along_axis(logits, idx, 1).astype(np.float64)
        np.testing.assert_allclose(w, scipy.special.softmax(picked, axis=1), rtol=0, atol=1e-7)
        # renormalising the full softmax over the picks gives the same weights
        full = scipy.special.softmax(logits.astype(np.float64), axis=1)
        sel = np.take_along_axis(full, idx, 1)
        np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=0, atol=1e-7)


def test_topk_crafted_cases():
    # all equal -> experts 0..k-1 with weight exactly 1/k
    idx, w = oracle.topk(np.full((3, 8), 0.7, np.float32), 4)
    assert (idx == np.arange(4)).all() and (w == 0.25).all()
    # +0 and -0 are equal: lower id first
    idx, _ = oracle.topk(np.array([[-0.0, 0.0, -1.0, 0.0]], np.float32), 2)
    assert idx.tolist() == [[0, 1]]
    # -inf is never picked while finite logits remain, and is picked last (lowest id first) otherwise
    l = np.array([[-np.inf, 1.0, -np.inf, 0.5]], np.float32)
    idx, w = oracle.topk(l, 2)
    assert idx.tolist() == [[1, 3]]
    idx, w = oracle.topk(l, 3)
    assert idx.tolist() == [[1, 3, 0]] and w[0, 2] == 0.0
    # k = 1 -> weight exactly 1; k = E -> every expert once
    _, w = oracle.topk(np.random.default_rng(0).standard_normal((5, 6)).astype(np.float32), 1)
    assert (w == 1.0).all()
    idx, _ = oracle.topk(np.random.default_rng(1).standard_normal((5, 6)).astype(np.float32), 6)
    assert (np.sort(idx, 1) == np.arange(6)).all()
    # known weights: logits 0 and ln 3 -> weights 1/4 and 3/4
    idx, w = oracle.topk(np.array([[0.0, np.log(3.0), -5.0]], np.float32), 2)
    assert idx.tolist() == [[1, 0]]
    np.testing.assert_allclose(w[0], [0.75, 0.25], atol=1e-7)
    with pytest.raises(oracle.OracleError):
        oracle.topk(np.array([[0.0, np.nan]], np.float32), 1)


def test_skewed_bias_and_empty_expert_workload_routing():
    """Mid workload: bias -inf on the last expert empties it, +2 on four experts makes them hot."""
    inp = workloads.make_inputs("mid_skewed", with_weights=False)
    x = workloads.bf16_bits(inp["x"])[:512]
    idx, w, logits = oracle.route(x, inp["wr"].numpy(), inp["bias"].numpy(), 4)
    gs, go, ss, sr = oracle.dispatch(idx, 32)
    assert gs[31] == 0 and gs[:4].min() > 5 * gs[4:31].max()
    assert np.isinf(logits[:, 31]).all()


# ---------------------------------------------------------------- dispatch / permute

@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (300, 32, 4), (257, 128, 8), (5, 4, 4), (0, 4, 2)])
def test_dispatch_is_the_expert_then_token_order(T, E, k):
    rng = np.random.default_rng(T + E)
    idx = np.array([rng.permutation(E)[:k] for _ in range(T)], np.int32).reshape(T, k)
    if T >= 3:
        idx[:3] = np.arange(k)  # several tokens on the same experts
    gs, go, ss, sr = oracle.dispatch(idx, E)
    S = T * k
    assert np.array_equal(gs, np.bincount(idx.reshape(-1), minlength=E))
    assert go[0] == 0 and np.array_equal(np.diff(go), gs) and go[-1] == S
    flat_e = idx.reshape(-1)
    flat_t = np.repeat(np.arange(T), k)
    order = np.lexsort((flat_t, flat_e))  # library sort by (expert, token)
    assert np.array_equal(ss, order)
    assert np.array_equal(sr[ss], np.arange(S))  # bijection
    assert np.array_equal(ss[sr], np.arange(S))
    if S:
        assert np.all(np.diff(flat_e[ss]) >= 0)
        for e in range(E):
            assert np.all(flat_e[ss[go[e]:go[e + 1]]] == e)


def test_dispatch_rejects_bad_indices():
    with pytest.raises(oracle.OracleError):
        oracle.dispatch(np.array([[0, 4]], np.int32), 4)
    with pytest.raises(oracle.OracleError):
        oracle.dispatch(np.array([[1, 1]], np.int32), 4)


def test_permute_copies_rows_bitwise_and_combine_with_unit_weights_is_k_x():
    for T, emb, E, k in [(64, 128, 8, 2), (33, 64, 16, 4), (20, 32, 8, 8)]:
        rng = np.random.default_rng(k)
        x = _bf16(rng.standard_normal((T, emb)))
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        gs, go, ss, sr = oracle.dispatch(idx, E)
        xs = oracle.permute(x, ss, k)
        assert np.array_equal(xs, x[ss // k])
        y = oracle.combine(xs, sr, None, T, k)  # permute backward = combine with unit weights
        assert np.array_equal(y, (k * _val(x)).astype(np.float32))


# ---------------------------------------------------------------- stage oracles

def _offsets(rng, M, E, empty=(1,)):
    cuts = np.sort(rng.integers(0, M + 1, E - 1))
    sizes = np.diff(np.concatenate([[0], cuts, [M]]))
    for e in empty:
        if e < E:
            sizes[e + 1 if e + 1 < E else 0] += sizes[e]
            sizes[e] = 0
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)


def test_grouped_gemm_stage_matches_per_group_matmul():
    rng = np.random.default_rng(6)
    M, K, N, E = 37, 24, 20, 5
    off = _offsets(rng, M, E)
    A = _bf16(rng.standard_normal((M, K)))
    Bnn = _bf16(rng.standard_normal((E, K, N)))
    Bnt = _bf16(rng.standard_normal((E, N, K)))
    Av = _val(A)
    got = oracle.grouped_gemm(0, 0, A, Bnn, off, real="f64")
    got_t = oracle.grouped_gemm(1, 0, A, Bnt, off, real="f64")
    got_s = oracle.grouped_gemm(0, 1, A, Bnn, off, real="f64")
    for e in range(E):
        r = slice(off[e], off[e + 1])
        h = Av[r] @ _val(Bnn)[e]
        np.testing.assert_allclose(got[r], h, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(got_t[r], Av[r] @ _val(Bnt)[e].T, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(got_s[r], _silu(h[:, :N // 2]) * h[:, N // 2:], rtol=1e-12, atol=1e-12)
    part = oracle.grouped_gemm(0, 0, A, Bnn, off, rows=(5, 30), real="f64")
    assert np.array_equal(part, got[5:30])


def test_swiglu_backward_epilogue_matches_finite_differences():
    """epi 2 returns d/d[h] of sum(da * silu(g) * u) for h = [g | u]."""
    rng = np.random.default_rng(8)
    M, K, N, E = 6, 5, 4, 2
    off = np.array([0, 2, 6], np.int32)
    A = rng.standard_normal((M, K))
    B = rng.standard_normal((E, N, K))  # NT
    h = rng.standard_normal((M, 2 * N))
    dh = oracle.grouped_gemm(1, 2, A, B, off, aux=h, real="f64")
    da = np.concatenate([A[off[e]:off[e + 1]] @ B[e].T for e in range(E)])
    f = lambda hh: np.sum(da * _silu(hh[:, :N]) * hh[:, N:])  # noqa: E731
    eps = 1e-6
    fd = np.zeros_like(h)
    for i in np.ndindex(h.shape):
        hp, hm = h.copy(), h.copy()
        hp[i] += eps
        hm[i] -= eps
        fd[i] = (f(hp) - f(hm)) / (2 * eps)
    np.testing.assert_allclose(dh, fd, rtol=1e-7, atol=1e-8)


def test_wgrad_stage_matches_transposed_matmul():
    rng = np.random.default_rng(10)
    M, P, Q, E = 29, 12, 9, 4
    off = _offsets(rng, M, E, empty=(2,))
    A = _bf16(rng.standard_normal((M, P)))
    D = _bf16(rng.standard_normal((M, Q)))
    for e in range(E):
        got = oracle.grouped_wgrad(A, D, off, e, real="f64")
        r = slice(off[e], off[e + 1])
        want = _val(A)[r].T @ _val(D)[r]
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
        if off[e] == off[e + 1]:
            assert (got == 0).all()


def test_combine_and_combine_backward_stages():
    rng = np.random.default_rng(12)
    T, emb, E, k = 21, 16, 6, 3
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    _, _, ss, sr = oracle.dispatch(idx, E)
    ys = _bf16(rng.standard_normal((T * k, emb)))
    dy = _bf16(rng.standard_normal((T, emb)))
    y = oracle.combine(ys, sr, w, T, k, real="f64")
    want = np.einsum("tj,tjn->tn", w.astype(np.float64), _val(ys)[sr.reshape(T, k)])
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12)
    dys, dw = oracle.combine_bwd(dy, ys, sr, w, k, real="f64")
    # adjoint identity: <combine(ys), dy> == <ys, dys> and dw = d<combine, dy>/dw
    assert abs(np.sum(y * _val(dy)) - np.sum(_val(ys) * dys)) < 1e-9 * np.abs(y).sum()
    want_dw = np.einsum("tjn,tn->tj", _val(ys)[sr.reshape(T, k)], _val(dy))
    np.testing.assert_allclose(dw, want_dw, rtol=1e-12, atol=1e-12)


def test_stage_composition_equals_per_token_forward():
    """route -> dispatch -> permute -> GEMM1(SwiGLU) -> GEMM2 -> combine == the per-token loop."""
    T, emb, mlp, E, k = 48, 32, 24, 6, 2
    x, wr, wi, wo = _case(T, emb, mlp, E, k, seed=13)
    idx, w, _ = oracle.route(x, wr, None, k)
    gs, go, ss, sr = oracle.dispatch(idx, E)
    xs = oracle.permute(x, ss, k)
    a = oracle.grouped_gemm(0, 1, xs, wi, go, real="f64")
    o = oracle.grouped_gemm(0, 0, a, _val(wo), go, real="f64")
    y = oracle.combine(o, sr, w, T, k, real="f64")
    np.testing.assert_allclose(y, oracle.ffn_fwd_tokens(x, idx, w, wi, wo, real="f64"), rtol=1e-10, atol=1e-13)


# ---------------------------------------------------------------- backward

def _fd_case():
    T, emb, mlp, E, k = 4, 8, 8, 4, 2
    rng = np.random.default_rng(21)
    x = rng.standard_normal((T, emb))
    wi = rng.standard_normal((E, emb, 2 * mlp)) * 0.4
    wo = rng.standard_normal((E, mlp, emb)) * 0.4
    dy = rng.standard_normal((T, emb))
    idx = np.array([[0, 2], [1, 3], [2, 0], [0, 1]], np.int32)
    w = rng.random((T, k)).astype(np.float32)
    return x, wi, wo, dy, idx, w


def _loss(x, wi, wo, dy, idx, w):
    return float(np.sum(oracle.ffn_fwd_tokens(x, idx, w, wi, wo, real="f64") * dy))


def _central(f, arr, eps=1e-5):
    g = np.zeros_like(arr)
    for i in np.ndindex(arr.shape):
        old = arr[i]
        arr[i] = old + eps
        fp = f()
        arr[i] = old - eps
        fm = f()
        arr[i] = old
        g[i] = (fp - fm) / (2 * eps)
    return g


def test_backward_matches_central_finite_differences():
    x, wi, wo, dy, idx, w = _fd_case()
    dx, dw = oracle.ffn_bwd_tokens(x, idx, w, wi, wo, dy, real="f64")
    grads = oracle.ffn_wgrad_experts(x, idx, w, wi, wo, dy, range(4), real="f64")
    dwi = np.stack([grads[e][0] for e in range(4)])
    dwo = np.stack([grads[e][1] for e in range(4)])
    f = lambda: _loss(x, wi, wo, dy, idx, w)  # noqa: E731
    np.testing.assert_allclose(dx, _central(f, x), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dwi, _central(f, wi), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dwo, _central(f, wo), rtol=1e-6, atol=1e-8)
    wd = w.astype(np.float64)
    fw = lambda: float(np.sum(oracle.ffn_fwd_tokens(x, idx, wd.astype(np.float32), wi, wo, real="f64") * dy))  # noqa: E731
    # topk_w is stored fp32, so differentiate by linearity instead: y is linear in each weight
    y_parts = oracle.ffn_fwd_tokens(x, idx, w, wi, wo, real="f64", want_intermediates=True)[3]  # o [T,k,emb]
    np.testing.assert_allclose(dw, np.einsum("tjn,tn->tj", y_parts, dy), rtol=1e-12, atol=1e-12)
    assert np.isfinite(fw())


def test_unrouted_expert_gets_zero_weight_gradient():
    x, wi, wo, dy, idx, w = _fd_case()
    idx = np.where(idx == 3, 1, idx).astype(np.int32)
    idx[1] = [1, 2]
    g = oracle.ffn_wgrad_experts(x, idx, w, wi, wo, dy, [3], real="f64")[3]
    assert (g[0] == 0).all() and (g[1] == 0).all()


def _bf16_round(v):
    """Nearest bf16 value (ties to even) of float64 data, through torch's own conversion from float32."""
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16).double().numpy()


def test_weight_gradient_with_stored_bf16_factors():
    """stored_bf16 rounds a, do = w * dy and dh to bf16 before the dW products (reading R9). Reference:
    float64 numpy per expert on the picked rows, the three factors rounded by torch, dh from the
    unrounded do. Rounding a different factor (h instead of dh, or none) moves dW by ~2^-9 relative,
    far outside the 1e-4 the two fp32/f64 paths keep."""
    T, emb, mlp, E, k = 40, 32, 24, 4, 2
    x, wr, wi, wo = _case(T, emb, mlp, E, k, seed=33, sigma=0.4)
    dy = _bf16(np.random.default_rng(4).standard_normal((T, emb)))
    idx, w, _ = oracle.route(x, wr, None, k)
    got = oracle.ffn_wgrad_experts(x, idx, w, wi, wo, dy, range(E), stored_bf16=True)
    plain = oracle.ffn_wgrad_experts(x, idx, w, wi, wo, dy, range(E))
    xv, wiv, wov, dyv = _val(x), _val(wi), _val(wo), _val(dy)
    for e in range(E):
        t_, j_ = np.nonzero(idx == e)                        # ascending token: expert-sorted order
        h = xv[t_] @ wiv[e]
        g, u = h[:, :mlp], h[:, mlp:]
        a = _silu(g) * u
        do = (w[t_, j_].astype(np.float32)[:, None] * dyv[t_].astype(np.float32)).astype(np.float64)
        da = do @ wov[e].T
        sg = scipy.special.expit(g)
        dh = np.concatenate([da * u * sg * (1 + g * (1 - sg)), da * g * sg], axis=1)
        dwo = _bf16_round(a).T @ _bf16_round(do)
        dwi = xv[t_].T @ _bf16_round(dh)
        for name, gv, pv, rv in (("dwi", got[e][0], plain[e][0], dwi), ("dwo", got[e][1], plain[e][1], dwo)):
            rel = np.linalg.norm(gv - rv) / np.linalg.norm(rv)
            assert rel <= 1e-4, (e, name, rel)
            # the unrounded reference is measurably elsewhere: the check sees the rounding
            assert np.linalg.norm(pv - rv) / np.linalg.norm(rv) > 1e-3, (e, name)


def test_backward_with_stored_bf16_activations():
    """ffn_bwd_tokens with stored_bf16 (reading R9): o from a rounded to bf16, dtopk_w from o rounded to
    bf16, dxs from dh rounded to bf16, dx the sum of the rounded dxs. Reference: float64 numpy per token and pick, roundings by torch;
    the unrounded oracle is measurably elsewhere."""
    T, emb, mlp, E, k = 24, 64, 32, 4, 2
    x, wr, wi, wo = _case(T, emb, mlp, E, k, seed=35, sigma=0.4)
    dy = _bf16(np.random.default_rng(6).standard_normal((T, emb)))
    idx, w, _ = oracle.route(x, wr, None, k)
    dx, dtw = oracle.ffn_bwd_tokens(x, idx, w, wi, wo, dy, stored_bf16=True)
    dx0, dtw0 = oracle.ffn_bwd_tokens(x, idx, w, wi, wo, dy)
    xv, wiv, wov, dyv = _val(x), _val(wi), _val(wo), _val(dy)
    rdx = np.zeros((T, emb))
    rdw = np.zeros((T, k))
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            h = xv[t] @ wiv[e]
            g, u = h[:mlp], h[mlp:]
            o = _bf16_round(_silu(g) * u) @ wov[e]
            rdw[t, j] = _bf16_round(o) @ dyv[t]
            da = (float(w[t, j]) * dyv[t]) @ wov[e].T
            sg = scipy.special.expit(g)
            dh = _bf16_round(np.concatenate([da * u * sg * (1 + g * (1 - sg)), da * g * sg]))
            rdx[t] += _bf16_round(dh @ wiv[e].T)
    # dxs sums 2*mlp products with cancellation, so the fp32 oracle and the float64 reference round a
    # few dxs elements to neighbouring bf16 values (one unit in the last place each); an element is
    # counted as differing beyond 1e-5 of the largest |dx|
    def off(a, ref):
        return np.mean(np.abs(a - ref) > 1e-5 * np.abs(ref).max())
    assert np.linalg.norm(dx - rdx) / np.linalg.norm(rdx) <= 1e-3 and off(dx, rdx) <= 0.05
    assert off(dx0, rdx) >= 0.5                      # without the roundings nearly every element differs
    assert np.linalg.norm(dtw - rdw) / np.linalg.norm(rdw) <= 1e-6
    assert np.linalg.norm(dtw0 - rdw) / np.linalg.norm(rdw) > 1e-4


def test_backward_stage_composition_equals_per_token_backward():
    """combine-bwd -> NT GEMM + SwiGLU-bwd -> NT GEMM -> permute-bwd == the per-token backward;
    wgrad stage on the sorted activations == the per-expert weight gradients."""
    T, emb, mlp, E, k = 12, 16, 8, 4, 2
    x, wr, wi, wo = _case(T, emb, mlp, E, k, seed=17)
    dy = _bf16(np.random.default_rng(3).standard_normal((T, emb)))
    idx, w, _ = oracle.route(x, wr, None, k)
    gs, go, ss, sr = oracle.dispatch(idx, E)
    xs = oracle.permute(x, ss, k)
    h = oracle.grouped_gemm(0, 0, xs, wi, go, real="f64")
    a = _silu(h[:, :mlp]) * h[:, mlp:]
    o = oracle.grouped_gemm(0, 0, a, _val(wo), go, real="f64")
    do, dwt = oracle.combine_bwd(dy, o, sr, w, k, real="f64")
    wo_t = np.ascontiguousarray(_val(wo))  # NT: B[e] = wo[e] is [mlp, emb] = [N, K]
    dh = oracle.grouped_gemm(1, 2, do, wo_t, go, aux=h, real="f64")
    dxs = oracle.grouped_gemm(1, 0, dh, np.ascontiguousarray(_val(wi)), go, real="f64")  # wi[e] = [emb, 2mlp] = [N, K]
    dx = oracle.combine(dxs, sr, None, T, k, real="f64")
    dx_ref, dw_ref = oracle.ffn_bwd_tokens(x, idx, w, wi, wo, dy, real="f64")
    np.testing.assert_allclose(dx, dx_ref, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dwt, dw_ref, rtol=1e-9, atol=1e-12)
    ref = oracle.ffn_wgrad_experts(x, idx, w, wi, wo, dy, range(E), real="f64")
    for e in range(E):
        np.testing.assert_allclose(oracle.grouped_wgrad(a, do, go, e, real="f64"), ref[e][1], rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(oracle.grouped_wgrad(_val(xs), dh, go, e, real="f64"), ref[e][0], rtol=1e-9,
                                   atol=1e-12)


# ---------------------------------------------------------------- router backward

def _router_loss(x, wr, bias, idx, g):
    """sum_t sum_j g[t,j] w[t,j] with w = softmax over each token's picked logits, picks fixed; numpy fp64,
    written independently of the oracle."""
    logits = x @ wr + bias
    picked = np.take_along_axis(logits, idx, axis=1)
    w = scipy.special.softmax(picked, axis=1)
    return float((g * w).sum()), w


def _router_case(T, emb, E, k, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, emb))
    wr = rng.standard_normal((emb, E)) * 0.3
    bias = rng.standard_normal(E) * 0.1
    logits = x @ wr + bias
    idx = np.argsort(-logits, axis=1, kind="stable")[:, :k].astype(np.int32)
    g = rng.standard_normal((T, k))
    return x, wr, bias, idx, g


@pytest.mark.parametrize("T,emb,E,k,seed", [(6, 16, 8, 3, 1), (4, 8, 16, 5, 2), (3, 12, 4, 4, 3)])
def test_router_backward_matches_central_finite_differences(T, emb, E, k, seed):
    x, wr, bias, idx, g = _router_case(T, emb, E, k, seed)
    _, w = _router_loss(x, wr, bias, idx, g)
    dl, dwr, db, dx = oracle.router_bwd(x, wr.astype(np.float32), idx, w.astype(np.float32), g)
    rng = np.random.default_rng(seed + 100)
    h = 1e-5

    def fd(fn, arr, pos):
        a1, a2 = arr.copy(), arr.copy()
        a1[pos] += h
        a2[pos] -= h
        return (fn(a1) - fn(a2)) / (2 * h)

    wr32 = wr.astype(np.float32).astype(np.float64)  # the oracle reads Wr as fp32
    for _ in range(12):
        i, e = rng.integers(emb), rng.integers(E)
        num = fd(lambda a: _router_loss(x, a, bias, idx, g)[0], wr32, (i, e))
        assert abs(num - dwr[i, e]) <= 1e-6 + 1e-5 * abs(num), ("dWr", i, e, num, dwr[i, e])
        e = rng.integers(E)
        num = fd(lambda a: _router_loss(x, wr32, a, idx, g)[0], bias, (e,))
        assert abs(num - db[e]) <= 1e-6 + 1e-5 * abs(num), ("dbias", e, num, db[e])
        t, i = rng.integers(T), rng.integers(emb)
        num = fd(lambda a: _router_loss(a, wr32, bias, idx, g)[0], x, (t, i))
        assert abs(num - dx[t, i]) <= 1e-6 + 1e-5 * abs(num), ("dx", t, i, num, dx[t, i])
    # unpicked experts get no logit gradient; each token's logit gradient sums to zero
    mask = np.zeros((T, E), bool)
    np.put_along_axis(mask, idx, True, axis=1)
    assert (dl[~mask] == 0).all()
    assert np.abs(dl.sum(axis=1)).max() <= 1e-6 * np.abs(dl).sum(axis=1).max()


def test_router_backward_closed_forms():
    # k = 1: the single weight is 1 whatever the logit -> no router gradient
    x, wr, bias, idx, g = _router_case(5, 8, 6, 1, 7)
    dl, dwr, db, dx = oracle.router_bwd(x, wr.astype(np.float32), idx, np.ones((5, 1), np.float32), g)
    assert not dl.any() and not dwr.any() and not db.any() and not dx.any()
    # a gradient equal across a token's picks moves nothing (the weights sum to 1)
    x, wr, bias, idx, g = _router_case(5, 8, 6, 3, 8)
    _, w = _router_loss(x, wr, bias, idx, g)
    g = np.repeat(np.arange(1.0, 6.0)[:, None], 3, axis=1)
    w32 = w.astype(np.float32)
    dl, _, _, _ = oracle.router_bwd(x, wr.astype(np.float32), idx, w32, g)
    assert np.abs(dl).max() <= 1e-6 * g.max()  # only the fp32 rounding of sum(w) = 1 remains
    # dWr is the exact matrix product x^T dl, and dx is dl Wr^T
    x, wr, bias, idx, g = _router_case(7, 5, 4, 2, 9)
    _, w = _router_loss(x, wr, bias, idx, g)
    dl, dwr, db, dx = oracle.router_bwd(x, wr.astype(np.float32), idx, w.astype(np.float32), g)
    np.testing.assert_allclose(dwr, x.T @ dl, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(db, dl.sum(axis=0), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dx, dl @ wr.astype(np.float32).astype(np.float64).T, rtol=1e-12, atol=1e-14)


def test_layer_router_gradient_matches_finite_differences_of_the_layer_output():
    """y = sum_j w_j(Wr) o_j with the expert outputs o from the oracle forward; L = <y, dy>. The weight gradient
    reaching the router is the combine backward's dtopk_w, and the router backward turns it into dWr."""
    T, emb, mlp, E, k = 5, 16, 32, 6, 3
    x_b, wr, wi, wo = _case(T, emb, mlp, E, k, 21)[:4]
    x = _val(x_b)
    rng = np.random.default_rng(22)
    bias = np.zeros(E)
    logits = x @ wr.astype(np.float64)
    idx = np.argsort(-logits, axis=1, kind="stable")[:, :k].astype(np.int32)
    _, w = _router_loss(x, wr.astype(np.float64), bias, idx, np.zeros((T, k)))
    y, _, _, o = oracle.ffn_fwd_tokens(x_b, idx, w.astype(np.float32), wi, wo, real="f64", want_intermediates=True)
    dy = rng.standard_normal((T, emb))
    g = np.einsum("tjn,tn->tj", o, dy)  # dL/dw_j = <o_j, dy>
    _, dwr, _, _ = oracle.router_bwd(x_b, wr, idx, w.astype(np.float32), g)

    def loss(wr_):
        _, w_ = _router_loss(x, wr_, bias, idx, np.zeros((T, k)))
        return float(np.einsum("tj,tjn,tn->", w_, o, dy))

    wr64 = wr.astype(np.float64)
    h = 1e-5
    for i, e in [(0, 0), (3, 2), (15, 5), (7, 1)]:
        a1, a2 = wr64.copy(), wr64.copy()
        a1[i, e] += h
        a2[i, e] -= h
        num = (loss(a1) - loss(a2)) / (2 * h)
        assert abs(num - dwr[i, e]) <= 1e-6 + 1e-5 * abs(num), (i, e, num, dwr[i, e])


# ---------------------------------------------------------------- MXFP8 (reading R8 of moe_oracle.c)

def _e4m3_table():
    return np.array([oracle.e4m3_value(c) for c in range(256)])


def _bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_e4m3_code_table_matches_the_format():
    t = _e4m3_table()
    pos = t[:0x7F]
    # OCP E4M3 ("FN"): 1.0 is 0x38, the largest finite value 448 is 0x7e, the smallest subnormal is 2^-9
    # (0x01), the smallest normal 2^-6 (0x08); 0x7f / 0xff are NaN; the negative half mirrors the positive
    assert t[0x38] == 1.0 and t[0x7E] == 448.0 and t[0x01] == 2.0 ** -9 and t[0x08] == 2.0 ** -6
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.array_equal(t[0x80:0xFF], -pos) and np.signbit(t[0x80])
    assert np.all(np.diff(pos) > 0)  # codes in magnitude order
    # eight values per binade above 2^-6, spacing 2^-9 below it
    for e in range(-6, 9):
        assert np.count_nonzero((pos >= 2.0 ** e) & (pos < 2.0 ** (e + 1))) == (7 if e == 8 else 8)
    assert np.allclose(np.diff(pos[:9]), 2.0 ** -9)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_mx_quantize_picks_the_nearest_code_by_search(seed):
    rng = np.random.default_rng(seed)
    M, K = 24, 96
    x = rng.standard_normal((M, K)) * np.exp(rng.uniform(-12, 12, (M, 1)))  # a different magnitude per row
    x[0, :32] = 0.0                      # an all-zero block
    x[1, 5] = -0.0
    x[2, :32] = np.linspace(-1, 1, 32)   # exact zero inside a block
    xb = _bf16_bits(x)
    xv = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).double().numpy()
    codes, scales = oracle.mx_quantize(xb)
    t = _e4m3_table()
    finite = np.array([c for c in range(256) if not np.isnan(t[c])])
    for r in range(M):
        for b in range(K // 32):
            blk = xv[r, 32 * b: 32 * b + 32]
            amax = np.abs(blk).max()
            sc = float(2.0 ** (int(scales[r, b]) - 127))
            if amax == 0:
                assert scales[r, b] == 0 and np.all(t[codes[r, 32 * b: 32 * b + 32]] == 0)
                continue
            assert 256 <= amax / sc < 512  # scale = 2^(floor(log2 amax) - 8)
            for i in range(32):
                v = blk[i] / sc
                c = int(codes[r, 32 * b + i])
                d = np.abs(t[finite] - v)
                best = finite[d == d.min()]
                if len(best) > 1:  # tie: the even mantissa (for zero, the sign of v)
                    best = [cc for cc in best if (cc & 1) == 0 and (t[cc] != 0 or np.signbit(t[cc]) == np.signbit(v))]
                if abs(v) > 448:
                    best = [0x7E | (0x80 if v < 0 else 0)]
                assert c in best, (r, b, i, v, c, best)
                assert np.signbit(t[c]) == np.signbit(v)


def test_mx_quantize_round_trips_representable_values_and_bounds_the_error():
    rng = np.random.default_rng(5)
    t = _e4m3_table()
    # values that are E4M3 codes times the block's own scale come back exactly
    c = rng.choice([cc for cc in range(0x7F) if not np.isnan(t[cc])], (8, 64))
    c[:, 0] = 0x7E                                   # pins each block's amax to 448 * 2^s
    c[:, 32] = 0x7E
    s = rng.integers(100, 150, (8, 1))
    x = t[c] * np.ldexp(1.0, s - 127)
    x *= rng.choice([-1.0, 1.0], x.shape)
    codes, scales = oracle.mx_quantize(_bf16_bits(x))
    assert np.array_equal(oracle.mx_dequantize(codes, scales), x)
    # otherwise the error is at most half a grid step: 2^-4 of the value in the normal range, 2^-10 of the
    # scale below it; a block maximum in [464, 512) x scale (past 448 and its rounding interval) saturates
    y = rng.standard_normal((16, 128))
    yb = _bf16_bits(y)
    yv = torch.from_numpy(yb.view(np.int16)).view(torch.bfloat16).double().numpy()
    cq, sq = oracle.mx_quantize(yb)
    dq = oracle.mx_dequantize(cq, sq)
    scale = np.repeat(np.ldexp(1.0, sq.astype(np.int64) - 127), 32, axis=1)
    sat = np.abs(yv) >= 464 * scale
    assert sat.any()  # the sample has some
    assert np.array_equal(dq[sat], np.sign(yv[sat]) * 448 * scale[sat])
    normal = (np.abs(yv) >= scale * 2.0 ** -6) & ~sat
    assert np.all(np.abs(dq - yv)[normal] <= 2.0 ** -4 * np.abs(yv)[normal])
    assert np.all(np.abs(dq - yv)[~normal & ~sat] <= scale[~normal & ~sat] * 2.0 ** -10)


def test_mx_quantize_rejects_non_finite_input():
    x = np.zeros((1, 32), np.float32)
    x[0, 3] = np.inf
    with pytest.raises(RuntimeError):
        oracle.mx_quantize(_bf16_bits(x))


def test_mx_grouped_gemm_on_integer_codes_is_the_integer_product():
    rng = np.random.default_rng(9)
    t = _e4m3_table()
    ints = [cc for cc in range(0x7F) if t[cc] == int(t[cc]) and t[cc] <= 16]  # 0, 1, ..., 16 and a few more
    M, K, N, E = 40, 64, 24, 3
    ac = rng.choice(ints, (M, K)).astype(np.uint8) | (rng.integers(0, 2, (M, K)) * 0x80).astype(np.uint8)
    bc = rng.choice(ints, (E, N, K)).astype(np.uint8)
    a_s = np.full((M, K // 32), 127, np.uint8)
    b_s = np.full((E, N, K // 32), 127, np.uint8)
    off = np.array([0, 7, 7, 40])
    got = oracle.mx_grouped_gemm_nt(ac, a_s, bc, b_s, off)
    A = t[ac].astype(np.int64)
    B = t[bc].astype(np.int64)
    ref = np.zeros((M, N), np.int64)
    for e in range(E):
        ref[off[e]:off[e + 1]] = A[off[e]:off[e + 1]] @ B[e].T
    assert np.array_equal(got, ref)


def _mx_integer_case(rng, M, K, N, E, t):
    """Integer-valued E4M3 codes (signed, |v| <= 16) with power-of-two block scales that differ from
    block to block and from row to row, so every product and every partial sum is exact in float64."""
    ints = [cc for cc in range(0x7F) if t[cc] == int(t[cc]) and t[cc] <= 16]
    sign = lambda shape: (rng.integers(0, 2, shape) * 0x80).astype(np.uint8)  # noqa: E731
    ac = rng.choice(ints, (M, K)).astype(np.uint8) | sign((M, K))
    bc = rng.choice(ints, (E, N, K)).astype(np.uint8) | sign((E, N, K))
    a_s = rng.integers(121, 127, (M, K // 32)).astype(np.uint8)
    b_s = rng.integers(121, 127, (E, N, K // 32)).astype(np.uint8)
    return ac, a_s, bc, b_s


def _mx_exact_product(t, ac, a_s, bc, b_s, off):
    """float64 C = A . B[e]^T per group, summed one 32-block at a time from exact int64 block sums, each
    block sum scaled by 2^(sa + sb - 254)."""
    M, K = ac.shape
    E, N, _ = bc.shape
    A = t[ac].astype(np.int64)
    B = t[bc].astype(np.int64)
    C_ = np.zeros((M, N), np.float64)
    for e in range(E):
        for m in range(off[e], off[e + 1]):
            for blk in range(K // 32):
                s = slice(32 * blk, 32 * blk + 32)
                part = B[e][:, s] @ A[m, s]                       # exact int64, [N]
                C_[m] += np.ldexp(part.astype(np.float64), a_s[m, blk].astype(np.int64) + b_s[e, :, blk] - 254)
    return C_


def test_mx_grouped_gemm_swiglu_epilogue_on_exact_products():
    """The MXFP8 SwiGLU reference (epi=1): gate is the first N/2 product columns and up the last N/2
    ("Gemma4 26B MoE on TPU v6e", Code Review: the split VJP concatenates [grad_gate, grad_up]), and
    SwiGLU is silu(gate) * up with silu(g) = g * sigmoid(g), applied to the split GMM output ("Keep fused
    MoE weights intact through FSDP gather", Description) of the MXFP8 MoE block ("[DRAFT][JAX] Optimize
    MoE block", Changes). The expected value is built from exact integer block
    sums with scipy's logistic sigmoid; a gate/up swap or a scale applied to the wrong 32-block is far
    outside the comparison."""
    rng = np.random.default_rng(21)
    t = _e4m3_table()
    M, K, N, E = 48, 128, 32, 4
    ac, a_s, bc, b_s = _mx_integer_case(rng, M, K, N, E, t)
    off = np.array([0, 13, 13, 40, 48])                          # an empty group among them
    got = oracle.mx_grouped_gemm_nt(ac, a_s, bc, b_s, off, epi=1)
    prod = _mx_exact_product(t, ac, a_s, bc, b_s, off)
    g, u = prod[:, : N // 2], prod[:, N // 2:]
    assert 0.5 < np.abs(g).mean() < 50                             # the sigmoid is neither saturated nor linear
    ref = g * scipy.special.expit(g) * u
    assert got.shape == (M, N // 2)
    assert np.allclose(got, ref, rtol=1e-12, atol=0)
    # the same comparison tells the plausible mistakes apart
    swapped = u * scipy.special.expit(u) * g
    assert np.abs(swapped - ref).max() > 1e-2 * np.abs(ref).max()
    wrong_blk = _mx_exact_product(t, ac, a_s[:, ::-1].copy(), bc, b_s, off)
    gw, uw = wrong_blk[:, : N // 2], wrong_blk[:, N // 2:]
    assert np.abs(gw * scipy.special.expit(gw) * uw - ref).max() > 1e-2 * np.abs(ref).max()
    # a single group covering all rows is the dense SwiGLU of the dequantized operands
    dense = oracle.mx_grouped_gemm_nt(ac, a_s, bc[:1], b_s[:1], np.array([0, M]), epi=1)
    A = t[ac] * np.repeat(np.ldexp(1.0, a_s.astype(np.int64) - 127), 32, axis=1)
    B = t[bc[0]] * np.repeat(np.ldexp(1.0, b_s[0].astype(np.int64) - 127), 32, axis=1)
    h = A @ B.T
    assert np.allclose(dense, scipy.special.expit(h[:, : N // 2]) * h[:, : N // 2] * h[:, N // 2:], rtol=1e-12, atol=0)
