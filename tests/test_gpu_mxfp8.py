"""MXFP8 quantizers and grouped GEMM on the GPU against the oracle (reading R8 of the oracle).

Quantization decides integers (codes and scales) from exact operations (a maximum, a power-of-two
rescaling, a rounding), so the device and the oracle must agree bit for bit."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_group_amd as moe
import oracle
from parity_util import bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16)


def _oracle_scales_to_device_layout(sc):
    """oracle scales [M, K/32] -> device layout [K/64, M, 4] (bytes 2, 3 zero)."""
    M, nb = sc.shape
    out = np.zeros((nb // 2, M, 4), np.uint8)
    out[:, :, 0] = sc[:, 0::2].T
    out[:, :, 1] = sc[:, 1::2].T
    return out


def _rows_case(M, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)) * np.exp(rng.uniform(-20, 20, (M, 1)))
    x[0, :32] = 0.0
    x[0, 40] = -0.0
    x[1, :] = np.where(rng.random(K) < 0.5, 1e-30, -3e30)  # far-apart magnitudes in one row
    x[2, 64:128] = 448.0 * 2.0 ** 5                          # exactly representable, saturating boundary
    x[3, :] = rng.choice([-1.0, 1.0], K) * 2.0 ** rng.integers(-20, 20, K)
    return _bf16(x)


@pytest.mark.parametrize("M,K,seed", [(5, 64, 0), (37, 192, 1), (300, 2048, 2), (129, 7168, 3)])
def test_mx_quantize_rows_bit_exact(M, K, seed):
    x = _rows_case(M, K, seed)
    codes, scales = moe.mx_quantize_rows(x.to(DEV))
    rc, rs = oracle.mx_quantize(bits(x))
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy(), _oracle_scales_to_device_layout(rs))


def test_mx_quantize_rows_gather_through_sorted_slot():
    T, K, k = 200, 256, 4
    rng = np.random.default_rng(7)
    x = _bf16(rng.standard_normal((T, K)))
    slots = rng.permutation(T * k).astype(np.int32)  # row r comes from token slots[r] // k
    codes, scales = moe.mx_quantize_rows(x.to(DEV), torch.from_numpy(slots).to(DEV), k)
    rc, rs = oracle.mx_quantize(bits(x)[slots // k])
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy(), _oracle_scales_to_device_layout(rs))


@pytest.mark.parametrize("E,K,N,seed", [(3, 64, 40, 0), (4, 192, 72, 1), (2, 2048, 256, 2)])
def test_mx_quantize_weight_bit_exact(E, K, N, seed):
    rng = np.random.default_rng(seed)
    w = _bf16(rng.standard_normal((E, K, N)) * np.exp(rng.uniform(-10, 10, (E, 1, N))))
    codes, scales = moe.mx_quantize_weight(w.to(DEV))
    wt = np.ascontiguousarray(np.transpose(bits(w), (0, 2, 1)))  # [E, N, K]
    for e in range(E):
        rc, rs = oracle.mx_quantize(wt[e])
        assert np.array_equal(codes[e].cpu().numpy(), rc)
        assert np.array_equal(scales[e].cpu().numpy(), _oracle_scales_to_device_layout(rs))


# ---------------------------------------------------------------- grouped GEMM

def _mx_step_bound(ac, as_, bc, bs, off, epi_width_N):
    """Per output element: the hardware's in-step summation (up to 2^-10 of the step's largest |product|, 8x the
    largest seen in probes; bounded here by max|a| * max|b| over the step) summed over the 64-element K steps,
    plus fp32 accumulation across steps."""
    A = oracle.mx_dequantize(ac, as_)
    B = oracle.mx_dequantize(bc, bs)
    M, K = A.shape
    N = B.shape[1]
    step = np.zeros((M, N))
    mag = np.zeros((M, N))
    for e in range(B.shape[0]):
        lo, hi = off[e], off[e + 1]
        if hi <= lo:
            continue
        a, b = np.abs(A[lo:hi]), np.abs(B[e])
        mag[lo:hi] = a @ b.T
        for s0 in range(0, K, 64):  # the step's largest product is at most max|a| * max|b| over the step
            step[lo:hi] += np.outer(a[:, s0:s0 + 64].max(axis=1), b[:, s0:s0 + 64].max(axis=1))
    return 2.0 ** -10 * step + (K // 64 + 2) * 2.0 ** -24 * mag, mag


def _mx_case(M, K, N, E, seed, empty=()):
    rng = np.random.default_rng(seed)
    sizes = rng.multinomial(M, rng.dirichlet(np.ones(E) * 2)).astype(np.int64)
    for e in empty:
        sizes[(e + 1) % E] += sizes[e]
        sizes[e] = 0
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    x = _bf16(rng.standard_normal((M, K)))
    w = _bf16(rng.standard_normal((E, K, N)) * (1.0 / np.sqrt(K)))
    return x, w, off


@pytest.mark.parametrize("M,K,N,E,empty", [(700, 128, 512, 4, (2,)), (1500, 256, 768, 6, (0, 5)),
                                           (300, 1024, 200, 3, ()), (64, 64, 64, 8, (1, 3, 6)),
                                           (2600, 512, 1536, 2, ())])
@pytest.mark.parametrize("epi", ["none", "swiglu"])
def test_grouped_gemm_mx_matches_oracle(M, K, N, E, empty, epi):
    if epi == "swiglu" and N % 16:
        N += 8
    x, w, off = _mx_case(M, K, N, E, M + K, empty)
    _check_mx_gemm(x, w, off, epi)


# Groups whose last 256-row tile ends at every 32-row block boundary of either half of the tile, and just past
# them, plus an empty group: every k-loop form of the tile (one to four blocks, none).
MX_PARTIAL_SIZES = [1, 32, 33, 64, 65, 96, 97, 128, 129, 160, 161, 192, 193, 224, 225, 255, 256, 257, 300, 384, 385,
                    448, 449, 512, 543, 0]


@pytest.mark.parametrize("epi", ["none", "swiglu"])
def test_grouped_gemm_mx_partial_tiles_every_block_count(epi):
    rng = np.random.default_rng(11)
    sizes = np.array(MX_PARTIAL_SIZES, np.int64)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M, K, N, E = int(off[-1]), 128, 256, len(sizes)
    x = _bf16(rng.standard_normal((M, K)))
    w = _bf16(rng.standard_normal((E, K, N)) * (1.0 / np.sqrt(K)))
    _check_mx_gemm(x, w, off, epi)


def _check_mx_gemm(x, w, off, epi):
    M, K = x.shape
    E, _, N = w.shape
    ac, as_ = moe.mx_quantize_rows(x.to(DEV))
    bc, bs = moe.mx_quantize_weight(w.to(DEV))
    offd = torch.from_numpy(off).to(DEV)
    got = moe.grouped_gemm_mx(ac, as_, bc, bs, offd, epilogue=epi).float().cpu().numpy().astype(np.float64)
    # oracle layouts: scales [rows, K/32]
    ac_n = ac.cpu().numpy()
    as_n = np.stack([as_.cpu().numpy()[:, :, 0].T, as_.cpu().numpy()[:, :, 1].T], axis=2).reshape(M, K // 32)
    bc_n = bc.cpu().numpy()
    bs_d = bs.cpu().numpy()
    bs_n = np.stack([np.transpose(bs_d[:, :, :, 0], (0, 2, 1)), np.transpose(bs_d[:, :, :, 1], (0, 2, 1))],
                    axis=3).reshape(E, N, K // 32)
    # the device scales are the oracle's (checked bit for bit above); use them in the reference
    rc, rs = oracle.mx_quantize(bits(x))
    assert np.array_equal(ac_n, rc) and np.array_equal(as_n, rs)
    ref = oracle.mx_grouped_gemm_nt(ac_n, as_n, bc_n, bs_n, off, epi=1 if epi == "swiglu" else 0)
    bound, mag = _mx_step_bound(ac_n, as_n, bc_n, bs_n, off, N)
    if epi == "swiglu":
        # SwiGLU of the two fp32 sums: propagate the bound of gate g and up u through silu(g) * u
        Cg = oracle.mx_grouped_gemm_nt(ac_n, as_n, bc_n, bs_n, off)
        g, u = Cg[:, : N // 2], Cg[:, N // 2:]
        dg, du = bound[:, : N // 2], bound[:, N // 2:]
        sg = 1.0 / (1.0 + np.exp(-g))
        dsilu = np.abs(sg * (1.0 + g * (1.0 - sg)))  # |d silu/dg|
        bound = np.abs(u) * (dsilu * dg + 1e-7 * np.abs(g)) + np.abs(g * sg) * du + dg * du + 1e-6 * np.abs(ref)
    rows = np.zeros(M, bool)
    rows[off[0]:off[-1]] = True
    err = np.abs(got[rows] - ref[rows])
    tol = bound[rows] + 2.0 ** -8 * np.abs(ref[rows]) + 1e-30  # + half a bf16 ulp of the output
    assert np.all(err <= tol), (float((err / tol).max()), np.unravel_index(np.argmax(err / tol), err.shape))


@pytest.mark.parametrize("epi", ["none", "swiglu"])
def test_grouped_gemm_mx_row_gather_equals_sorted_rows_bitwise(epi):
    """Token rows quantized once and read through sorted_slot give the same bits as the expert-sorted rows
    quantized one by one (the same codes and scales reach the same kernel arithmetic)."""
    T, K, N, E, k = 500, 256, 320, 6, 3
    rng = np.random.default_rng(17)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    gs, off, ss, sr = oracle.dispatch(idx, E)
    x = _bf16(rng.standard_normal((T, K)))
    w = _bf16(rng.standard_normal((E, K, N)) * (1.0 / np.sqrt(K)))
    bc, bs = moe.mx_quantize_weight(w.to(DEV))
    offd = torch.from_numpy(off.astype(np.int32)).to(DEV)
    ssd = torch.from_numpy(ss.astype(np.int32)).to(DEV)
    tq, ts = moe.mx_quantize_rows(x.to(DEV))                        # T token rows
    got = moe.grouped_gemm_mx(tq, ts, bc, bs, offd, epilogue=epi, row_slot=ssd, slot_div=k)
    sq, sqs = moe.mx_quantize_rows(x.to(DEV), ssd, k)               # T*k sorted rows
    ref = moe.grouped_gemm_mx(sq, sqs, bc, bs, offd, epilogue=epi)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("M,K,N,E,empty", [(700, 128, 512, 4, (2,)), (1500, 256, 768, 6, (0, 5)),
                                           (2600, 512, 1536, 2, ())])
def test_grouped_gemm_mx_swiglu_writes_the_mxfp8_of_its_bf16_output(M, K, N, E, empty):
    """The SwiGLU epilogue's MXFP8 output is the quantization of its own bf16 output, bit for bit, and it does
    not depend on whether the bf16 output is written too."""
    x, w, off = _mx_case(M, K, N, E, M + 2 * K, empty)
    ac, as_ = moe.mx_quantize_rows(x.to(DEV))
    bc, bs = moe.mx_quantize_weight(w.to(DEV))
    offd = torch.from_numpy(off).to(DEV)
    c, cq, cqs = moe.grouped_gemm_mx(ac, as_, bc, bs, offd, epilogue="swiglu", mx_out=True)
    rq, rqs = moe.mx_quantize_rows(c)
    assert torch.equal(cq, rq)
    assert torch.equal(cqs[:, :, :2], rqs[:, :, :2])
    _, cq2, cqs2 = moe.grouped_gemm_mx(ac, as_, bc, bs, offd, epilogue="swiglu", mx_out=True, bf16_out=False)
    assert torch.equal(cq2, cq) and torch.equal(cqs2[:, :, :2], cqs[:, :, :2])


# ---------------------------------------------------------------- MXFP8 layer forward

import workloads  # noqa: E402


def _mx_layer_inputs(name):
    h = workloads.make_inputs(workloads.WORKLOADS[name] if isinstance(name, str) else name)
    d = {kk: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for kk, v in h.items()}
    return h, d


@pytest.mark.parametrize("name", ["tiny", "mid_skewed", "sweep_zipf_T1024"])
def test_ffn_fwd_mx_equals_its_stages_bitwise(name):
    h, d = _mx_layer_inputs(name)
    wl = h["workload"]
    T, k = wl.T, wl.k
    wq = moe.mx_quantize_expert_weights(d["wi"], d["wo"])
    y = moe.ffn_fwd_mx(d["x"], wq, k, wr=d["wr"], bias=d["bias"], logits=d["logits_in"])
    if d["logits_in"] is not None:
        idx, w = moe.route(k, logits=d["logits_in"])
    else:
        idx, w = moe.route(k, x=d["x"], wr=d["wr"], bias=d["bias"])
    perm = moe.permute(d["x"], idx, wl.E, rows=False)
    xq, xqs = moe.mx_quantize_rows(d["x"])
    _, aq, aqs = moe.grouped_gemm_mx(xq, xqs, wq["wi_codes"], wq["wi_scales"], perm["group_offsets"],
                                     epilogue="swiglu", row_slot=perm["sorted_slot"], slot_div=k, mx_out=True,
                                     bf16_out=False)
    o = moe.grouped_gemm_mx(aq, aqs, wq["wo_codes"], wq["wo_scales"], perm["group_offsets"])
    y_ref = moe.combine(o, perm["slot_row"], w, T, k)
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))


# one token (two of its four experts get no rows); k = E; 64 experts of about 32 rows each (every row block
# partial); the largest k (every token picks all 64 experts)
MX_EDGE = [workloads.custom(1, 64, 64, 4, 2, seed=5, sigma_w=0.05),
           workloads.custom(100, 128, 64, 2, 2, seed=6, sigma_w=0.05),
           workloads.custom(257, 256, 128, 64, 8, seed=7, sigma_w=0.05),
           workloads.custom(20, 64, 64, 64, 64, seed=8, sigma_w=0.05)]


def _mx_random(n=6, seed=77):
    """Seeded random shapes across the supported range (emb and mlp multiples of 64 up to 1024, E up to 256,
    k up to 64), the oracle's work bounded."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        emb, mlp = 64 * int(rng.integers(1, 17)), 64 * int(rng.integers(1, 17))
        E = int(rng.integers(1, 17)) if rng.random() < 0.5 else int(rng.integers(17, 257))
        k = int(min(E, rng.choice([1, 2, 3, 4, 6, 8])))
        if E > 8 and rng.random() < 0.35:
            k = int(rng.integers(9, min(E, 64) + 1))
        T = int(min(2000, rng.integers(1, max(2, int(2e8 / (k * emb * mlp))) + 1)))
        out.append(workloads.custom(T, emb, mlp, E, k, seed=7100 + i, sigma_w=0.5 / np.sqrt(max(emb, mlp))))
    return out


@pytest.mark.parametrize("name", ["tiny", "mid_skewed"] + MX_EDGE + _mx_random(),
                         ids=lambda n: n if isinstance(n, str) else n.name)
def test_ffn_fwd_mx_matches_the_oracle_composition(name):
    """Each stage from the oracle: routing, token quantization, float64 GEMM 1 on the dequantized operands,
    SwiGLU rounded to bf16 and quantized, float64 GEMM 2, bf16 rounding, combine. The device and the oracle
    quantize the same token rows and weights bit for bit; the SwiGLU output can round to a neighbouring bf16
    value on either side and then to a neighbouring code, which the layer tolerance covers."""
    from parity_util import assert_close, to_np
    h, d = _mx_layer_inputs(name)
    wl = h["workload"]
    T, emb, mlp, E, k = wl.T, wl.emb, wl.mlp, wl.E, wl.k
    wq = moe.mx_quantize_expert_weights(d["wi"], d["wo"])
    y = moe.ffn_fwd_mx(d["x"], wq, k, wr=d["wr"], bias=d["bias"])
    xb = bits(h["x"])
    idx, w, _ = oracle.route(xb, h["wr"].numpy(), None if h["bias"] is None else h["bias"].numpy(), k)
    gs, off, ss, sr = oracle.dispatch(idx, E)
    xc, xs_ = oracle.mx_quantize(xb)
    wi_t = np.ascontiguousarray(np.transpose(bits(h["wi"]), (0, 2, 1)))   # [E, 2mlp, emb]
    wo_t = np.ascontiguousarray(np.transpose(bits(h["wo"]), (0, 2, 1)))   # [E, emb, mlp]
    wic = np.stack([oracle.mx_quantize(wi_t[e])[0] for e in range(E)])
    wis = np.stack([oracle.mx_quantize(wi_t[e])[1] for e in range(E)])
    woc = np.stack([oracle.mx_quantize(wo_t[e])[0] for e in range(E)])
    wos = np.stack([oracle.mx_quantize(wo_t[e])[1] for e in range(E)])
    a = oracle.mx_grouped_gemm_nt(xc[ss // k], xs_[ss // k], wic, wis, off, epi=1)
    a_b = bits(torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16))
    ac, as_ = oracle.mx_quantize(a_b)
    o = oracle.mx_grouped_gemm_nt(ac, as_, woc, wos, off)
    o_b = bits(torch.from_numpy(o.astype(np.float32)).to(torch.bfloat16))
    y_ref = oracle.combine(o_b, sr, w, T, k)
    assert_close(to_np(y), y_ref, "y")


def test_ffn_fwd_mx_with_no_tokens_is_a_no_op():
    h, d = _mx_layer_inputs("tiny")
    wq = moe.mx_quantize_expert_weights(d["wi"], d["wo"])
    y = moe.ffn_fwd_mx(d["x"][:0], wq, h["workload"].k, wr=d["wr"])
    assert y.shape == (0, d["x"].shape[1])


@pytest.mark.slow
@pytest.mark.parametrize("name,extra", [("gemma4_class", 22), ("deepseek_v3_shape", 10)])
def test_ffn_fwd_mx_full_size_sampled(name, extra):
    """A full-size workload through moe_ffn_fwd_mx (the kernels and launch configuration that the MXFP8
    bench times) against the oracle composition on sampled tokens. Every stage of the reference is the
    oracle's: routing of the sampled tokens, quantization of their rows and of the picked experts' weights,
    float64 GEMMs on the dequantized operands, the SwiGLU output rounded to bf16 and quantized, bf16
    rounding of GEMM 2, and the combine. Routing, the row quantization and the GEMMs act per token row
    and per expert, so taking them one sampled token and one expert at a time gives the values the
    whole-workload computation has for those tokens."""
    from parity_util import assert_close, to_np
    d = workloads.make_inputs(name, device=DEV)
    wl = d["workload"]
    T, k = wl.T, wl.k
    wq = moe.mx_quantize_expert_weights(d["wi"], d["wo"])
    y = moe.ffn_fwd_mx(d["x"], wq, k, wr=d["wr"], bias=d["bias"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(wl.seed)
    toks = np.unique(np.concatenate([[0, T - 1], rng.choice(T, extra, replace=False)])).astype(np.int64)
    xb = bits(d["x"][torch.from_numpy(toks).to(DEV)])
    idx, w, _ = oracle.route(xb, d["wr"].cpu().numpy(), None if d["bias"] is None else d["bias"].cpu().numpy(), k)
    # the sampled (token, pick) pairs, ordered by expert (then token), as group rows of the reference GEMMs
    pairs = sorted(((int(idx[i, j]), i, j) for i in range(len(toks)) for j in range(k)))
    xc, xs_ = oracle.mx_quantize(xb)  # per-row quantization: the same as quantizing every row
    o_b = np.empty((len(pairs), wl.emb), np.uint16)
    for u in sorted({e for e, _, _ in pairs}):
        rows = [r for r, (e, _, _) in enumerate(pairs) if e == u]
        src = [pairs[r][1] for r in rows]
        off = np.array([0, len(rows)], np.int32)
        wic, wis = oracle.mx_quantize(np.ascontiguousarray(bits(d["wi"][u]).T))  # [2mlp, emb] rows
        woc, wos = oracle.mx_quantize(np.ascontiguousarray(bits(d["wo"][u]).T))  # [emb, mlp] rows
        a = oracle.mx_grouped_gemm_nt(xc[src], xs_[src], wic[None], wis[None], off, epi=1)
        ac, as2 = oracle.mx_quantize(bits(torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)))
        o = oracle.mx_grouped_gemm_nt(ac, as2, woc[None], wos[None], off)
        o_b[rows] = bits(torch.from_numpy(o.astype(np.float32)).to(torch.bfloat16))
    slot_row = np.empty(len(toks) * k, np.int32)
    for r, (_, i, j) in enumerate(pairs):
        slot_row[i * k + j] = r
    y_ref = oracle.combine(o_b, slot_row, w, len(toks), k)
    assert_close(to_np(y)[toks], y_ref, "y[sampled]")
