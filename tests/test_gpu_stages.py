"""GPU parity of each hot-path stage against the CPU oracle, through the C ABI.

Integer and byte outputs (routing indices, group sizes/offsets, sort order,
the permuted rows) must match bit for bit; fp32 top-k weights within 1e-6;
bf16 outputs within relative Frobenius 1e-2 and max-abs 2e-2 (combine: at
most 1 bf16 ulp from the oracle's fp32 result).
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_group_amd as moe
import oracle
import workloads
from parity_util import W_ABS, assert_close, bf16_values, bits, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bf16_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).to(DEV)


def _route_case(T, emb, E, k, seed, bias=None):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((T, emb), generator=g).to(torch.bfloat16)
    wr = torch.randn((emb, E), generator=g) * 0.02
    return x, wr, bias


# ---------------------------------------------------------------- route

@pytest.mark.parametrize("T,emb,E,k,seed", [(64, 128, 8, 2, 1), (1000, 256, 32, 4, 2), (333, 512, 128, 8, 3),
                                            (130, 64, 256, 8, 4), (77, 128, 192, 6, 8), (70, 128, 5, 5, 5),
                                            (17, 64, 64, 1, 6), (0, 64, 8, 2, 7),
                                            # k > 16: one token per wave in the top-k (E % 4 != 0: register-staged kernel)
                                            (100, 128, 64, 20, 9), (50, 64, 256, 24, 10), (40, 64, 37, 17, 11),
                                            # the largest k: every expert (k = E = 64), and 64 of 256
                                            (40, 64, 64, 64, 12), (30, 128, 256, 64, 13)])
def test_route_bit_exact(T, emb, E, k, seed):
    x, wr, _ = _route_case(T, emb, E, k, seed)
    idx, w = moe.route(k, x=x.to(DEV), wr=wr.to(DEV))
    r_idx, r_w, _ = oracle.route(bits(x), wr.numpy(), None, k)
    assert np.array_equal(idx.cpu().numpy(), r_idx)
    assert np.abs(w.cpu().numpy() - r_w).max(initial=0) <= W_ABS


def test_route_with_bias_empty_and_hot_experts():
    inp = workloads.make_inputs("mid_skewed", with_weights=False)
    k = inp["workload"].k
    idx, w = moe.route(k, x=inp["x"].to(DEV), wr=inp["wr"].to(DEV), bias=inp["bias"].to(DEV))
    r_idx, r_w, _ = oracle.route(bits(inp["x"]), inp["wr"].numpy(), inp["bias"].numpy(), k)
    assert np.array_equal(idx.cpu().numpy(), r_idx)
    assert np.abs(w.cpu().numpy() - r_w).max() <= W_ABS
    assert not (r_idx == 31).any()


@pytest.mark.parametrize("E", [64, 200])
def test_route_bit_exact_with_subnormal_products_and_logits(E):
    """Products x*wr and the chains' partial sums in the fp32 subnormal range: the chain must still equal
    the oracle's fmaf chain bitwise (no flush to zero), so the top-k and its tie order match."""
    rng = np.random.default_rng(E)
    T, emb, k = 150, 256, 4
    x = torch.from_numpy((rng.standard_normal((T, emb)) * 1e-20).astype(np.float32)).to(torch.bfloat16)
    wr = torch.from_numpy((rng.standard_normal((emb, E)) * 1e-19).astype(np.float32))
    wr[:, 7] = 0.0                          # a zero column: logits exactly 0 -> ties broken by expert id
    idx, w = moe.route(k, x=x.to(DEV), wr=wr.to(DEV))
    r_idx, r_w, logits = oracle.route(bits(x), wr.numpy(), None, k)
    assert np.abs(logits).max() < 2e-37      # the workload really is in the subnormal range
    assert np.array_equal(idx.cpu().numpy(), r_idx)
    assert np.abs(w.cpu().numpy() - r_w).max(initial=0) <= W_ABS


@pytest.mark.parametrize("E,k", [(40, 6), (256, 16), (130, 16), (128, 8)])
def test_route_logits_in_with_ties_zero_signs_and_minus_inf(E, k):
    """Both lane layouts of the k <= 16 top-k (8 candidates per lane for E <= 128, 16 above), with ties
    inside a lane, across lanes of a row and in whole rows."""
    rng = np.random.default_rng(11 + E)
    T = 300
    l = rng.standard_normal((T, E)).astype(np.float32)
    l[:, 5] = l[:, 9]                      # exact ties -> lower id first
    l[::3, 1] = 0.0
    l[::3, 2] = -0.0                       # +0 == -0
    l[::3, 3:8] = 0.0
    l[::7, 0] = -np.inf                    # never picked while finite logits remain
    l[5] = 0.25                            # all equal -> experts 0..k-1
    l[6, ::16] = 3.0                       # equal maxima in one lane (experts r + 16q share lane r)
    l[7, :16] = 2.0                        # equal maxima across the 16 lanes of a row
    l[8, 1::2] = -np.inf                   # half the experts at -inf
    idx, w = moe.route(k, logits=torch.from_numpy(l).to(DEV))
    r_idx, r_w = oracle.topk(l, k)
    assert np.array_equal(idx.cpu().numpy(), r_idx)
    assert np.abs(w.cpu().numpy() - r_w).max() <= W_ABS
    assert np.abs(w[5].cpu().numpy() - 1 / k).max() < 1e-7


def test_route_zipf_logits_workload():
    inp = workloads.make_inputs("sweep_zipf_T1024", with_weights=False)
    idx, w = moe.route(8, logits=inp["logits_in"].to(DEV))
    r_idx, r_w = oracle.topk(inp["logits_in"].numpy(), 8)
    assert np.array_equal(idx.cpu().numpy(), r_idx)
    assert np.abs(w.cpu().numpy() - r_w).max() <= W_ABS
    loads = np.bincount(r_idx.reshape(-1), minlength=128)
    assert loads[0] > 5 * np.median(loads)  # skewed head


# ---------------------------------------------------------------- permute

def _random_idx(T, E, k, seed, skew=False):
    rng = np.random.default_rng(seed)
    if skew:
        p = 1.0 / np.arange(1, E + 1) ** 1.5
        return np.array([rng.choice(E, k, replace=False, p=p / p.sum()) for _ in range(T)], np.int32).reshape(T, k)
    return np.array([rng.permutation(E)[:k] for _ in range(T)], np.int32).reshape(T, k)


@pytest.mark.parametrize("T,emb,E,k,skew", [(64, 128, 8, 2, False), (1000, 256, 16, 4, True), (129, 64, 256, 8, False),
                                            (4096, 1024, 32, 4, True), (1, 64, 4, 4, False), (0, 64, 8, 2, False)])
def test_permute_bit_exact(T, emb, E, k, skew):
    rng = np.random.default_rng(T + E)
    x = torch.from_numpy(rng.standard_normal((T, emb)).astype(np.float32)).to(torch.bfloat16)
    idx = _random_idx(T, E, k, T, skew)
    out = moe.permute(x.to(DEV), torch.from_numpy(idx).to(DEV), E)
    gs, go, ss, sr = oracle.dispatch(idx, E)
    assert np.array_equal(out["group_sizes"].cpu().numpy(), gs)
    assert np.array_equal(out["group_offsets"].cpu().numpy(), go)
    assert np.array_equal(out["sorted_slot"].cpu().numpy(), ss)
    assert np.array_equal(out["slot_row"].cpu().numpy(), sr)
    assert np.array_equal(bits(out["xs"]), oracle.permute(bits(x), ss, k))


@pytest.mark.parametrize("T,emb,E,k,skew", [(1000, 256, 16, 4, True), (129, 64, 256, 8, False), (1, 64, 4, 4, False),
                                            (5000, 128, 128, 8, True), (0, 64, 8, 2, False)])
def test_permute_index_only_matches_the_oracle_dispatch(T, emb, E, k, skew):
    """With no xs the permute builds the same index by its own per-slot kernel, and copies no row."""
    rng = np.random.default_rng(T + 3 * E)
    x = torch.from_numpy(rng.standard_normal((T, emb)).astype(np.float32)).to(torch.bfloat16)
    idx = _random_idx(T, E, k, T + 1, skew)
    out = moe.permute(x.to(DEV), torch.from_numpy(idx).to(DEV), E, rows=False)
    assert out["xs"] is None
    gs, go, ss, sr = oracle.dispatch(idx, E)
    assert np.array_equal(out["group_sizes"].cpu().numpy(), gs)
    assert np.array_equal(out["group_offsets"].cpu().numpy(), go)
    assert np.array_equal(out["sorted_slot"].cpu().numpy(), ss)
    assert np.array_equal(out["slot_row"].cpu().numpy(), sr)


def test_permute_empty_expert_and_single_hot_expert():
    T, emb, E, k = 500, 128, 8, 2
    idx = np.zeros((T, k), np.int32)
    idx[:, 0] = 3
    idx[:, 1] = np.where(np.arange(T) % 2 == 0, 5, 6)  # experts 0,1,2,4,7 empty
    x = torch.randn((T, emb)).to(torch.bfloat16)
    out = moe.permute(x.to(DEV), torch.from_numpy(idx).to(DEV), E)
    gs, go, ss, sr = oracle.dispatch(idx, E)
    assert np.array_equal(out["group_sizes"].cpu().numpy(), gs)
    assert np.array_equal(out["sorted_slot"].cpu().numpy(), ss)
    assert np.array_equal(bits(out["xs"]), oracle.permute(bits(x), ss, k))


# ---------------------------------------------------------------- combine

def _combine_bound(exact, mag, k):
    """Error bound of k fused multiply-adds in fp32 followed by one rounding to bf16:
    k * 2^-24 * sum_j |w_j v_j| for the fp32 chain, plus half a bf16 ulp of the result."""
    chain = k * 2.0 ** -24 * mag
    top = np.abs(exact) + chain
    ulp = np.where(top > 0, 2.0 ** (np.floor(np.log2(np.maximum(top, 1e-300))) - 7), 0.0)
    return chain + 0.5 * ulp


# the last two: more picks than 16-byte chunks in a row (emb 64, k 64) and in its last round of
# chunks (emb 576: 72 chunks, a round of 64 and one of 8, with k 16)
@pytest.mark.parametrize("T,emb,k", [(64, 128, 2), (777, 1024, 4), (300, 2048, 8), (5, 7168, 8), (40, 64, 64),
                                     (50, 576, 16)])
def test_combine_within_rounding_bound_of_exact_sum(T, emb, k):
    E = max(8, k)
    rng = np.random.default_rng(T)
    idx = _random_idx(T, E, k, T)
    _, _, ss, sr = oracle.dispatch(idx, E)
    ys = torch.from_numpy(rng.standard_normal((T * k, emb)).astype(np.float32)).to(torch.bfloat16)
    w = rng.random((T, k))
    w = torch.from_numpy((w / w.sum(1, keepdims=True)).astype(np.float32))  # top-k weights sum to 1
    y = moe.combine(ys.to(DEV), torch.from_numpy(sr).to(DEV), w.to(DEV), T, k)
    exact = oracle.combine(bits(ys), sr, w.numpy(), T, k, real="f64")
    mag = oracle.combine(bits(ys) & np.uint16(0x7fff), sr, w.numpy(), T, k, real="f64")
    err = np.abs(bf16_values(bits(y)) - exact)
    assert (err <= _combine_bound(exact, mag, k) * (1 + 1e-9)).all(), float(err.max())
    assert_close(bf16_values(bits(y)), exact, "y")


@pytest.mark.parametrize("k", [2, 3, 4, 8, 16, 64])
def test_combine_of_permute_with_unit_weights_is_k_x(k):
    """permute then combine with unit weights: y == bf16(k * x) exactly (exact for k a power of two)."""
    T, emb, E = 513, 256, max(16, k)
    x = torch.randn((T, emb)).to(torch.bfloat16)
    idx = torch.from_numpy(_random_idx(T, E, k, k)).to(DEV)
    out = moe.permute(x.to(DEV), idx, E)
    y = moe.combine(out["xs"], out["slot_row"], None, T, k)
    want = (x.float() * k).to(torch.bfloat16)
    assert np.array_equal(bits(y), bits(want))
    if k in (2, 4, 8, 16, 64):
        assert np.array_equal(bf16_values(bits(y)), k * bf16_values(bits(x)))


def test_combine_bwd_matches_oracle():
    T, emb, E, k = 400, 512, 16, 4
    rng = np.random.default_rng(3)
    idx = _random_idx(T, E, k, 3)
    _, _, ss, sr = oracle.dispatch(idx, E)
    dy = torch.from_numpy(rng.standard_normal((T, emb)).astype(np.float32)).to(torch.bfloat16)
    ys = torch.from_numpy(rng.standard_normal((T * k, emb)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy(rng.random((T, k)).astype(np.float32))
    dys, dw = moe.combine_bwd(dy.to(DEV), ys.to(DEV), torch.from_numpy(sr).to(DEV), w.to(DEV), k)
    r_dys, r_dw = oracle.combine_bwd(bits(dy), bits(ys), sr, w.numpy(), k)
    # do = bf16(fp32(w * dy)) on both sides: the same fp32 product, the same rounding
    assert np.array_equal(bits(dys), bits(torch.from_numpy(r_dys).to(torch.bfloat16)))
    np.testing.assert_allclose(dw.cpu().numpy(), r_dw, rtol=1e-4, atol=1e-3)


# ---------------------------------------------------------------- grouped GEMM

def _offsets(M, E, seed, empty=()):
    rng = np.random.default_rng(seed)
    sizes = rng.multinomial(M, rng.dirichlet(np.ones(E) * 2)).astype(np.int64)
    for e in empty:
        j = (e + 1) % E
        sizes[j] += sizes[e]
        sizes[e] = 0
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)


GEMM_CASES = [  # (M, K, N, E, empty groups)
    (700, 128, 512, 4, (2,)),
    (1500, 256, 1536, 6, (0, 5)),
    (300, 1024, 200, 3, ()),
    (64, 64, 64, 8, (1, 3, 6)),
    (2600, 512, 768, 2, ()),
]


@pytest.mark.parametrize("M,K,N,E,empty", GEMM_CASES)
def test_grouped_gemm_nn_none(M, K, N, E, empty):
    rng = np.random.default_rng(M)
    off = _offsets(M, E, M, empty)
    A = _bf16_dev(rng.standard_normal((M, K)))
    B = _bf16_dev(rng.standard_normal((E, K, N)) * (0.5 / np.sqrt(K)))
    C_ = moe.grouped_gemm(A, B, torch.from_numpy(off).to(DEV), op="nn")
    ref = oracle.grouped_gemm(0, 0, bits(A), bits(B), off)
    assert_close(to_np(C_), ref, "C")


@pytest.mark.parametrize("M,K,N,E,empty", GEMM_CASES)
def test_grouped_gemm_nn_swiglu_on_prefused_weight(M, K, N, E, empty):
    N2 = 2 * N
    rng = np.random.default_rng(M + 1)
    off = _offsets(M, E, M + 1, empty)
    A = _bf16_dev(rng.standard_normal((M, K)))
    B = _bf16_dev(rng.standard_normal((E, K, N2)) * (0.5 / np.sqrt(K)))
    a, h = moe.grouped_gemm(A, B, torch.from_numpy(off).to(DEV), op="nn", epilogue="swiglu", save_h=True)
    ref_a = oracle.grouped_gemm(0, 1, bits(A), bits(B), off)
    ref_h = oracle.grouped_gemm(0, 0, bits(A), bits(B), off)
    assert_close(to_np(a), ref_a, "a")
    assert_close(to_np(h), ref_h, "h")


@pytest.mark.parametrize("M,K,N,E,empty", GEMM_CASES)
def test_grouped_gemm_nt_none(M, K, N, E, empty):
    rng = np.random.default_rng(M + 2)
    off = _offsets(M, E, M + 2, empty)
    A = _bf16_dev(rng.standard_normal((M, K)))
    B = _bf16_dev(rng.standard_normal((E, N, K)) * (0.5 / np.sqrt(K)))
    C_ = moe.grouped_gemm(A, B, torch.from_numpy(off).to(DEV), op="nt")
    ref = oracle.grouped_gemm(1, 0, bits(A), bits(B), off)
    assert_close(to_np(C_), ref, "C")


@pytest.mark.parametrize("M,K,N,E,empty", GEMM_CASES)
def test_grouped_gemm_nt_swiglu_bwd(M, K, N, E, empty):
    rng = np.random.default_rng(M + 3)
    off = _offsets(M, E, M + 3, empty)
    A = _bf16_dev(rng.standard_normal((M, K)))
    B = _bf16_dev(rng.standard_normal((E, N, K)) * (0.5 / np.sqrt(K)))
    h = (rng.standard_normal((M, 2 * N)) * 0.5).astype(np.float32)  # saved h is fp32
    dh = moe.grouped_gemm(A, B, torch.from_numpy(off).to(DEV), op="nt", epilogue="swiglu_bwd",
                          aux_in=torch.from_numpy(h).to(DEV))
    ref = oracle.grouped_gemm(1, 2, bits(A), bits(B), off, aux=h)
    assert_close(to_np(dh), ref, "dh")


# Groups whose last 256-row tile ends at every 32-row block boundary of either half of the tile, and just past
# it (a tile multiplies only its blocks that hold rows of the group); groups of 257-512 rows, which run as two
# halves multiplied as ceil(n/2) rows, whose second row half ends at and just past its 64- and 96-row block
# boundaries (384/385, 448/449) or fills it (512); and an empty group.
PARTIAL_SIZES = [1, 32, 33, 64, 65, 96, 97, 128, 129, 160, 161, 192, 193, 224, 225, 255, 256, 257, 300, 384, 385,
                 448, 449, 512, 543, 0]


@pytest.mark.parametrize("op,epi", [("nn", "none"), ("nn", "swiglu"), ("nt", "none"), ("nt", "swiglu_bwd")])
def test_grouped_gemm_partial_tiles_every_block_count(op, epi):
    K, N = 192, 320
    sizes = np.array(PARTIAL_SIZES, np.int64)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M, E = int(off[-1]), len(sizes)
    rng = np.random.default_rng(31)
    A = _bf16_dev(rng.standard_normal((M, K)))
    Nb = 2 * N if epi == "swiglu" else N
    B = _bf16_dev(rng.standard_normal((E, K, Nb) if op == "nn" else (E, Nb, K)) * (0.5 / np.sqrt(K)))
    h = (rng.standard_normal((M, 2 * N)) * 0.5).astype(np.float32)
    got = moe.grouped_gemm(A, B, torch.from_numpy(off).to(DEV), op=op, epilogue=epi,
                           aux_in=torch.from_numpy(h).to(DEV) if epi == "swiglu_bwd" else None)
    ref = oracle.grouped_gemm(0 if op == "nn" else 1, {"none": 0, "swiglu": 1, "swiglu_bwd": 2}[epi], bits(A),
                              bits(B), off, aux=h if epi == "swiglu_bwd" else None)
    assert_close(to_np(got), ref, f"{op}/{epi}")


@pytest.mark.parametrize("op,epi", [("nn", "none"), ("nn", "swiglu"), ("nt", "none"), ("nt", "swiglu_bwd")])
def test_grouped_gemm_row_gather_and_row_scale(op, epi):
    """Rows read in place from A [T, K] through slots t*k + j, each output row scaled by w[slot] in fp32:
    equal to the oracle GEMM on the gathered, scaled rows (scaling a bf16 value is exact in fp64)."""
    T, K, N, E, k = 400, 256, 320, 6, 3
    rng = np.random.default_rng(21)
    idx = _random_idx(T, E, k, 21)
    gs, off, ss, sr = oracle.dispatch(idx, E)
    A = _bf16_dev(rng.standard_normal((T, K)))
    Nb = 2 * N if epi == "swiglu" else N
    B = _bf16_dev(rng.standard_normal((E, K, Nb) if op == "nn" else (E, Nb, K)) * (0.5 / np.sqrt(K)))
    w = rng.random(T * k).astype(np.float32)
    h = (rng.standard_normal((T * k, 2 * N)) * 0.5).astype(np.float32)
    got = moe.grouped_gemm(A, B, torch.from_numpy(off).to(DEV), op=op, epilogue=epi,
                           aux_in=torch.from_numpy(h).to(DEV) if epi == "swiglu_bwd" else None,
                           row_slot=torch.from_numpy(ss).to(DEV), slot_div=k, slot_scale=torch.from_numpy(w).to(DEV))
    A_rows = bf16_values(bits(A))[ss // k] * w[ss].astype(np.float64)[:, None]
    ref = oracle.grouped_gemm(0 if op == "nn" else 1, {"none": 0, "swiglu": 1, "swiglu_bwd": 2}[epi],
                              np.ascontiguousarray(A_rows), bits(B), off, aux=h if epi == "swiglu_bwd" else None,
                              real="f64")
    assert_close(to_np(got), ref, f"{op}/{epi}")


@pytest.mark.parametrize("op,epi", [("nn", "none"), ("nn", "swiglu"), ("nt", "none"), ("nt", "swiglu_bwd")])
def test_grouped_gemm_row_scale_without_gather(op, epi):
    """A per-row fp32 scale with no row gather (slot_scale indexed by the output row, A read as it is):
    equal to the oracle GEMM on the scaled rows."""
    M, K, N, E = 700, 256, 320, 5
    rng = np.random.default_rng(23)
    sizes = rng.multinomial(M, np.ones(E) / E)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    A = _bf16_dev(rng.standard_normal((M, K)))
    Nb = 2 * N if epi == "swiglu" else N
    B = _bf16_dev(rng.standard_normal((E, K, Nb) if op == "nn" else (E, Nb, K)) * (0.5 / np.sqrt(K)))
    w = rng.random(M).astype(np.float32)
    h = (rng.standard_normal((M, 2 * N)) * 0.5).astype(np.float32)
    got = moe.grouped_gemm(A, B, torch.from_numpy(off).to(DEV), op=op, epilogue=epi,
                           aux_in=torch.from_numpy(h).to(DEV) if epi == "swiglu_bwd" else None,
                           slot_scale=torch.from_numpy(w).to(DEV))
    A_rows = bf16_values(bits(A)) * w.astype(np.float64)[:, None]
    ref = oracle.grouped_gemm(0 if op == "nn" else 1, {"none": 0, "swiglu": 1, "swiglu_bwd": 2}[epi],
                              np.ascontiguousarray(A_rows), bits(B), off, aux=h if epi == "swiglu_bwd" else None,
                              real="f64")
    assert_close(to_np(got), ref, f"{op}/{epi}")


def test_grouped_gemm_rows_past_last_group_untouched():
    M, K, N, E = 600, 128, 256, 3
    off = np.array([0, 100, 100, 450], np.int32)  # rows 450.. belong to no group
    A = _bf16_dev(np.random.default_rng(0).standard_normal((M, K)))
    B = _bf16_dev(np.random.default_rng(1).standard_normal((E, K, N)) * (0.5 / np.sqrt(K)))
    out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    moe.grouped_gemm(A, B, torch.from_numpy(off).to(DEV), op="nn", out=out)
    got = to_np(out)
    assert np.isnan(got[450:]).all() and np.isfinite(got[:450]).all()
    assert_close(got[:450], oracle.grouped_gemm(0, 0, bits(A), bits(B), off)[:450], "C")


# The last two cases have 16 experts of 32 tiles each, so every workgroup runs several tiles of the experts
# its XCD is dealt, with groups of ~150 rows (5 k-slices) and of ~37 rows (2 k-slices).
@pytest.mark.parametrize("M,P,Q,E,empty", [(700, 128, 512, 4, (2,)), (1000, 256, 200, 5, (0,)),
                                           (90, 64, 64, 8, (1, 2, 3)), (3000, 768, 256, 3, ()),
                                           (2400, 2048, 1024, 16, (3,)), (600, 1024, 2048, 16, (5,))])
def test_wgrad_matches_oracle_and_zeros_empty_groups(M, P, Q, E, empty):
    rng = np.random.default_rng(P + Q)
    off = _offsets(M, E, P + Q, empty)
    # scaled so that |dW| stays O(1) for groups of up to ~1000 rows
    A = _bf16_dev(rng.standard_normal((M, P)) * 0.03)
    D = _bf16_dev(rng.standard_normal((M, Q)) * 0.5)
    C_ = moe.grouped_gemm_wgrad(A, D, torch.from_numpy(off).to(DEV), E)
    Cn = to_np(C_)
    for e in range(E):
        ref = oracle.grouped_wgrad(bits(A), bits(D), off, e)
        if off[e] == off[e + 1]:
            assert (Cn[e] == 0).all()
        else:
            assert_close(Cn[e], ref, f"dW[{e}]")


# ---------------------------------------------------------------- router backward

def _route_bwd_case(T, emb, E, k, seed, empty=()):
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.standard_normal((T, emb)).astype(np.float32)).to(torch.bfloat16)
    wr = torch.from_numpy((rng.standard_normal((emb, E)) * 0.05).astype(np.float32))
    bias = torch.zeros(E)
    bias[list(empty)] = -float("inf")
    idx, w = moe.route(k, x=x.to(DEV), wr=wr.to(DEV), bias=bias.to(DEV))
    perm = moe.permute(x.to(DEV), idx, E, rows=False)
    g = torch.from_numpy(rng.standard_normal((T, k)).astype(np.float32)).to(DEV)
    dx0 = torch.from_numpy(rng.standard_normal((T, emb)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    return x, wr, idx, w, g, perm, dx0


def _check_route_bwd(x, wr, idx, w, g, perm, dx0, out, dx, want_dx=True):
    T, emb = x.shape
    E = wr.shape[1]
    k = idx.shape[1]
    xb = bits(x)
    dl, dwr, db, dxr = oracle.router_bwd(xb, wr.numpy(), idx.cpu().numpy(), w.cpu().numpy(),
                                         g.cpu().numpy().astype(np.float64), want_dx=want_dx)
    n_max = int(np.diff(perm["group_offsets"].cpu().numpy()).max(initial=0))
    eps = 2.0 ** -24
    xa = np.abs(bf16_values(xb))
    # Error of the fp32 logit gradient dl_j = w_j (g_j - s), s = sum_i w_i g_i: the fp32 chain for s errs by up to
    # k eps sum|w g|, which the subtraction turns into an absolute error of dl (g_j ~ s cancels), plus three
    # roundings relative to dl itself.
    wn = w.cpu().numpy().astype(np.float64)
    gn = g.cpu().numpy().astype(np.float64)
    s_mag = (np.abs(wn) * np.abs(gn)).sum(axis=1, keepdims=True)
    ddl_slot = wn * (k + 2) * eps * s_mag + 3 * eps * np.abs(np.take_along_axis(dl, idx.cpu().numpy(), axis=1))
    ddl = np.zeros_like(dl)
    np.put_along_axis(ddl, idx.cpu().numpy(), ddl_slot, axis=1)
    # dWr, dbias: fp32 chain over a group's rows, plus the propagated error of dl
    bound = (n_max + 8) * eps * (xa.T @ np.abs(dl)) + xa.T @ ddl + 1e-30
    got = out["dwr"].cpu().numpy().astype(np.float64)
    assert (np.abs(got - dwr) <= bound).all(), np.abs(got - dwr).max()
    got_b = out["dbias"].cpu().numpy().astype(np.float64)
    assert (np.abs(got_b - db) <= (n_max + 8) * eps * np.abs(dl).sum(axis=0) + ddl.sum(axis=0) + 1e-30).all()
    if want_dx:
        d0 = to_np(dx0)
        exact = d0 + dxr
        wra = np.abs(wr.numpy().astype(np.float64))
        mag = np.abs(d0) + np.abs(dl) @ wra.T
        assert np.all(np.abs(to_np(dx) - exact) <= _combine_bound(exact, mag, k + 1) + ddl @ wra.T + 1e-30)


def _rb_random(n=6, seed=91):
    """Seeded random router-backward shapes: emb up to 1024, E up to 256, k up to 64, up to two experts
    that no token picks."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        emb = 64 * int(rng.integers(1, 17))
        E = int(rng.integers(1, 17)) if rng.random() < 0.5 else int(rng.integers(17, 257))
        k = int(min(E, rng.choice([1, 2, 3, 4, 6, 8])))
        if E > 8 and rng.random() < 0.35:
            k = int(rng.integers(9, min(E, 64) + 1))
        T = int(rng.integers(1, 1500))
        empty = tuple(int(e) for e in rng.choice(E, min(E - k, int(rng.integers(0, 3))), replace=False)) \
            if E > k else ()
        out.append((T, emb, E, k, 100 + i, empty))
    return out


@pytest.mark.parametrize("T,emb,E,k,seed,empty", _rb_random() + [(300, 256, 16, 4, 1, ()), (129, 64, 256, 8, 2, (3, 77)),
                                                  (1000, 1024, 128, 8, 3, (0,)), (77, 7168, 200, 6, 4, ()),
                                                  (50, 128, 8, 8, 5, ()), (40, 64, 64, 64, 6, ()),
                                                  (60, 128, 37, 5, 7, (36,))])
def test_route_bwd_matches_oracle(T, emb, E, k, seed, empty):
    x, wr, idx, w, g, perm, dx0 = _route_bwd_case(T, emb, E, k, seed, empty)
    dx = dx0.clone()
    out = moe.route_bwd(x.to(DEV), wr.to(DEV), idx, w, g, perm["sorted_slot"], perm["group_offsets"], dx=dx)
    _check_route_bwd(x, wr, idx, w, g, perm, dx0, out, dx)
    for e in empty:  # an expert no token picked gets exact zeros
        assert (out["dwr"][:, e] == 0).all() and out["dbias"][e] == 0


def test_route_bwd_single_pick_and_no_tokens():
    x, wr, idx, w, g, perm, dx0 = _route_bwd_case(200, 128, 16, 1, 6)
    dx = dx0.clone()
    out = moe.route_bwd(x.to(DEV), wr.to(DEV), idx, w, g, perm["sorted_slot"], perm["group_offsets"], dx=dx)
    assert (out["dwr"] == 0).all() and (out["dbias"] == 0).all()  # one pick: its weight is 1 whatever the logit
    assert torch.equal(dx.view(torch.int16), dx0.view(torch.int16))
    e0 = torch.empty((0, 128), dtype=torch.bfloat16, device=DEV)
    i0 = torch.empty((0, 4), dtype=torch.int32, device=DEV)
    f0 = torch.empty((0, 4), dtype=torch.float32, device=DEV)
    s0 = torch.empty(0, dtype=torch.int32, device=DEV)
    go = torch.zeros(17, dtype=torch.int32, device=DEV)
    out = moe.route_bwd(e0, wr.to(DEV), i0, f0, f0, s0, go)
    assert (out["dwr"] == 0).all() and (out["dbias"] == 0).all()


def test_route_bwd_full_size_gemma4_class():
    inp = workloads.make_inputs("gemma4_class", with_weights=False)
    wl = inp["workload"]
    x, wr = inp["x"], inp["wr"]
    idx, w = moe.route(wl.k, x=x.to(DEV), wr=wr.to(DEV))
    perm = moe.permute(x.to(DEV), idx, wl.E, rows=False)
    g = torch.from_numpy(np.random.default_rng(5).standard_normal((wl.T, wl.k)).astype(np.float32)).to(DEV)
    out = moe.route_bwd(x.to(DEV), wr.to(DEV), idx, w, g, perm["sorted_slot"], perm["group_offsets"])
    _check_route_bwd(x, wr, idx, w, g, perm, None, out, None, want_dx=False)


@pytest.mark.parametrize("op,epi", [("nn", "swiglu"), ("nt", "swiglu_bwd")])
def test_swiglu_epilogues_with_saturating_gates(op, epi):
    """Gate values far into both tails (|g| up to ~200): the sigmoid's exponential overflows to inf or
    underflows to 0 and its reciprocal must still give silu -> -0 / g and sigmoid -> 0 / 1, as in the
    oracle's double-precision evaluation."""
    M, K, N, E = 512, 64, 128, 2
    rng = np.random.default_rng(99)
    off = np.array([0, 200, M], np.int32)
    A = rng.standard_normal((M, K))
    A[:, 0] = np.linspace(-60.0, 60.0, M)              # one large input column drives the gates
    A = _bf16_dev(A)
    Nb = 2 * N if epi == "swiglu" else N
    Bn = rng.standard_normal((E, K, Nb) if op == "nn" else (E, Nb, K)) * (0.5 / np.sqrt(K))
    if op == "nn":
        Bn[:, 0, :] = 3.0                               # gate and up both see 3 * A[:, 0]
    else:
        Bn[:, :, 0] = 3.0
    B = _bf16_dev(Bn)
    h = None
    if epi == "swiglu_bwd":
        hv = rng.standard_normal((M, 2 * N)) * 0.5
        hv[:, :N] = np.linspace(-200.0, 200.0, M)[:, None]  # saved gate values in both tails
        h = hv.astype(np.float32)
    got = moe.grouped_gemm(A, B, torch.from_numpy(off).to(DEV), op=op, epilogue=epi,
                           aux_in=None if h is None else torch.from_numpy(h).to(DEV))
    g = to_np(got)
    assert np.isfinite(g).all()
    ref = oracle.grouped_gemm(0 if op == "nn" else 1, 1 if epi == "swiglu" else 2, bits(A), bits(B), off, aux=h)
    rel = np.linalg.norm(g - ref) / np.linalg.norm(ref)
    assert rel <= 1e-2, rel
    # elementwise: one bf16 rounding of the result, plus the fp32 sums' own error
    assert np.all(np.abs(g - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-3 * np.abs(ref).max()), np.abs(g - ref).max()


# ---------------------------------------------------------------- index data out of range

def test_out_of_range_index_data_never_leaves_the_buffers():
    """Index data made on the device is not checked on the host: out-of-range values give unspecified
    results, but no kernel reads or writes outside the buffers. Expert ids out of range and repeated within
    a token (permute), group offsets past M, negative and decreasing (grouped GEMM, weight gradient, router
    backward), rows out of range (combine and its backward, the GEMM's row gather) and sorted slots out of
    range (router backward): every output and workspace sits at the start of a larger allocation whose
    tail must come back untouched."""
    import ctypes as C

    from mixture_experts_ffn_group_amd import _lib

    L = _lib.lib()
    st = torch.cuda.current_stream().cuda_stream
    fills = {torch.int16: 0x2EAD, torch.int32: 0x2EADBEEF, torch.uint8: 0x5A}
    guards = []

    def guarded(shape, dtype, init=None):
        n = int(np.prod(shape))
        raw = {torch.bfloat16: torch.int16, torch.float32: torch.int32}.get(dtype, dtype)
        buf = torch.full((n + 4096,), fills[raw], dtype=raw, device=DEV)
        view = buf[:n].view(dtype).view(shape)
        if init is not None:
            view.copy_(init)
        guards.append((buf, n, fills[raw]))
        return view

    def p(t):
        return C.c_void_p(t.data_ptr())

    rng = np.random.default_rng(5)
    T, emb, E, k = 300, 128, 16, 4
    S = T * k
    s = _lib.shape(T, emb, 64, E, k)
    x = _bf16_dev(rng.standard_normal((T, emb)))
    bad_idx = torch.from_numpy(_random_idx(T, E, k, 5)).to(DEV)
    bad_idx[::7, 0] = -1
    bad_idx[1::7, 1] = E
    bad_idx[2::7, 2] = 100000
    bad_idx[3::7, 3] = bad_idx[3::7, 0]  # the same expert twice in one token
    gs, go = guarded((E,), torch.int32), guarded((E + 1,), torch.int32)
    ss, sr = guarded((S,), torch.int32), guarded((S,), torch.int32)
    xs = guarded((S, emb), torch.bfloat16)
    ws_n = int(L.moe_permute_workspace_bytes(C.byref(s)))
    ws = guarded((ws_n,), torch.uint8)
    _lib.check(L.moe_permute(C.byref(s), p(x), p(bad_idx), p(gs), p(go), p(ss), p(sr), p(xs), p(ws), ws_n, st),
               "moe_permute")

    row = torch.from_numpy(rng.integers(0, S, S).astype(np.int32)).to(DEV)
    row[::5] = -3
    row[1::5] = S
    row[2::5] = 2 ** 31 - 1
    ys = _bf16_dev(rng.standard_normal((S, emb)))
    dy = _bf16_dev(rng.standard_normal((T, emb)))
    w = torch.rand((T, k), device=DEV)
    y = guarded((T, emb), torch.bfloat16)
    _lib.check(L.moe_combine(C.byref(s), p(ys), p(row), p(w), p(y), st), "moe_combine")
    dys, dtw = guarded((S, emb), torch.bfloat16), guarded((T, k), torch.float32)
    _lib.check(L.moe_combine_bwd(C.byref(s), p(dy), p(ys), p(row), p(w), p(dys), p(dtw), st), "moe_combine_bwd")

    M, K, N, Eg = 300, 128, 256, 6
    off = torch.tensor([0, 120, 80, 400, -20, 290, 10 ** 6], dtype=torch.int32, device=DEV)
    A = _bf16_dev(rng.standard_normal((M, K)))
    B = _bf16_dev(rng.standard_normal((Eg, K, N)) * 0.05)
    moe.grouped_gemm(A, B, off, out=guarded((M, N), torch.bfloat16))
    moe.grouped_gemm(A, B, off, out=guarded((M, N), torch.bfloat16), row_slot=row[:M].contiguous())
    D = _bf16_dev(rng.standard_normal((M, N)))
    cw = guarded((Eg, K, N), torch.bfloat16)
    _lib.check(L.moe_grouped_gemm_wgrad(p(A), p(D), p(off), Eg, M, K, N, p(cw), st), "moe_grouped_gemm_wgrad")

    wr = torch.from_numpy((rng.standard_normal((emb, E)) * 0.05).astype(np.float32)).to(DEV)
    g = torch.from_numpy(rng.standard_normal((T, k)).astype(np.float32)).to(DEV)
    go_bad = torch.tensor([0, 500, 100, -7] + [S + 99] * (E - 3), dtype=torch.int32, device=DEV)
    dwr, dbias = guarded((emb, E), torch.float32), guarded((E,), torch.float32)
    dx = guarded((T, emb), torch.bfloat16, init=dy)
    rb_n = int(L.moe_route_bwd_workspace_bytes(C.byref(s)))
    rb_ws = guarded((rb_n,), torch.uint8)
    _lib.check(L.moe_route_bwd(C.byref(s), p(x), p(wr), p(bad_idx), p(w), p(g), p(row), p(go_bad), p(dwr),
                               p(dbias), p(dx), p(rb_ws), rb_n, st), "moe_route_bwd")

    torch.cuda.synchronize()
    for i, (buf, n, fill) in enumerate(guards):
        assert torch.equal(buf[n:], torch.full_like(buf[n:], fill)), f"guarded buffer {i}: tail overwritten"
