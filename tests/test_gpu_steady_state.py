"""GPU parity of the persistent GEMMs' steady state, element by element.

A persistent workgroup loads the first k-slices of its next tile while it
finishes the current one (epilogue, copying-to-storing wave hand-over). At the
default grid, small shapes give each workgroup one or two tiles, so that path
would only be seen on the sampled full-size checks. Here it is compared on
every element:
  - the stage GEMMs with a grid of 8 workgroups (moe_grouped_gemm_grid,
    moe_grouped_gemm_wgrad_grid): dozens of tiles per workgroup, bitwise
    equal to the default grid (each tile is computed whole, in the same k
    order, whichever workgroup takes it) and within tolerance of the oracle;
  - the whole layer at the default grid on a shape where every workgroup runs
    8 tiles of each forward GEMM (T = 65536, emb = 512, mlp = 256, E = 16,
    k = 4): the forward on every token, the backward's dx and dtopk_w on every
    token and dW on four experts (the most- and least-loaded among them).
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_group_amd as moe
import oracle
import workloads
from parity_util import assert_close, assert_close_bf16_out, bf16_values, bits, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SMALL_GRID = 8


def _bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).to(DEV)


def _offsets(M, E, seed, empty=()):
    rng = np.random.default_rng(seed)
    sizes = rng.multinomial(M, rng.dirichlet(np.ones(E) * 2)).astype(np.int64)
    for e in empty:
        sizes[(e + 1) % E] += sizes[e]
        sizes[e] = 0
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)


def _same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.int16), b.contiguous().view(torch.int16))


@pytest.mark.parametrize("op,epi,K,N", [("nn", "none", 512, 1024), ("nn", "swiglu", 512, 1024),
                                         ("nt", "none", 1024, 1024), ("nt", "swiglu_bwd", 512, 1024)])
def test_grouped_gemm_small_grid_runs_many_tiles_per_workgroup(op, epi, K, N):
    M, E = 6000, 12
    rng = np.random.default_rng(K + N)
    off = _offsets(M, E, K + N, empty=(4,))
    # the SwiGLU GEMM runs on the prefused [K, 2N] weight with N output columns; the others tile N columns
    tiles = moe.tile_schedule("swiglu" if epi == "swiglu" else "gemm", off, M, 2 * N if epi == "swiglu" else N,
                              SMALL_GRID)
    assert tiles[:, 1].max() >= 10
    Nb = 2 * N if epi == "swiglu" else N
    A = _bf16_dev(rng.standard_normal((M, K)))
    B = _bf16_dev(rng.standard_normal((E, K, Nb) if op == "nn" else (E, Nb, K)) * (0.5 / np.sqrt(K)))
    h = (rng.standard_normal((M, 2 * N)) * 0.5).astype(np.float32)
    aux = torch.from_numpy(h).to(DEV) if epi == "swiglu_bwd" else None
    go = torch.from_numpy(off).to(DEV)
    small = moe.grouped_gemm(A, B, go, op=op, epilogue=epi, aux_in=aux, grid=SMALL_GRID)
    full = moe.grouped_gemm(A, B, go, op=op, epilogue=epi, aux_in=aux)
    torch.cuda.synchronize()
    assert _same_bits(small, full), "the result depends on the grid"
    code = {"none": 0, "swiglu": 1, "swiglu_bwd": 2}[epi]
    ref = oracle.grouped_gemm(0 if op == "nn" else 1, code, bits(A), bits(B), off,
                              aux=h if epi == "swiglu_bwd" else None)
    assert_close(to_np(small), ref, f"{op}/{epi} grid {SMALL_GRID}")


@pytest.mark.parametrize("grid", [SMALL_GRID, 24])
def test_row_gathered_swiglu_gemm_small_grid(grid):
    """The inference GEMM1: token rows read in place through sorted slots, many tiles per workgroup."""
    T, K, N, E, k = 2000, 512, 512, 16, 4
    rng = np.random.default_rng(grid)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    gs, off, ss, sr = oracle.dispatch(idx, E)
    A = _bf16_dev(rng.standard_normal((T, K)))
    B = _bf16_dev(rng.standard_normal((E, K, 2 * N)) * (0.5 / np.sqrt(K)))
    args = dict(op="nn", epilogue="swiglu", row_slot=torch.from_numpy(ss).to(DEV), slot_div=k)
    small = moe.grouped_gemm(A, B, torch.from_numpy(off).to(DEV), grid=grid, **args)
    full = moe.grouped_gemm(A, B, torch.from_numpy(off).to(DEV), **args)
    torch.cuda.synchronize()
    assert _same_bits(small, full)
    A_rows = np.ascontiguousarray(bf16_values(bits(A))[ss // k])
    ref = oracle.grouped_gemm(0, 1, A_rows, bits(B), off, real="f64")
    assert_close(to_np(small), ref, f"gathered swiglu grid {grid}")


def test_wgrad_small_grid_runs_many_tiles_per_workgroup():
    M, P, Q, E = 3000, 1024, 512, 16
    rng = np.random.default_rng(5)
    off = _offsets(M, E, 5, empty=(9,))
    tiles = moe.tile_schedule("wgrad", off, M, P, SMALL_GRID, Q=Q)
    assert tiles[:, 1].max() >= 15
    A = _bf16_dev(rng.standard_normal((M, P)) * 0.03)
    D = _bf16_dev(rng.standard_normal((M, Q)) * 0.5)
    go = torch.from_numpy(off).to(DEV)
    small = moe.grouped_gemm_wgrad(A, D, go, E, grid=SMALL_GRID)
    full = moe.grouped_gemm_wgrad(A, D, go, E)
    torch.cuda.synchronize()
    assert _same_bits(small, full)
    Cn = to_np(small)
    for e in range(E):
        if off[e] == off[e + 1]:
            assert (Cn[e] == 0).all()
        else:
            assert_close(Cn[e], oracle.grouped_wgrad(bits(A), bits(D), off, e), f"dW[{e}]")


def test_grid_argument_is_validated():
    A = torch.zeros((16, 64), dtype=torch.bfloat16, device=DEV)
    B = torch.zeros((1, 64, 64), dtype=torch.bfloat16, device=DEV)
    go = torch.tensor([0, 16], dtype=torch.int32, device=DEV)
    for g in (-8, 12, 65544):
        with pytest.raises(moe.MoeError):
            moe.grouped_gemm(A, B, go, grid=g)


# ---------------------------------------------------------------- the layer, many tiles per workgroup

# weights ~ N(0, 0.02), as in the pages' model settings
MANY = workloads.custom(65536, 512, 256, 16, 4, seed=4242, sigma_w=0.02, backward=True)


@pytest.fixture(scope="module")
def many_tiles():
    h = workloads.make_inputs(MANY)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in h.items()}
    return h, d


@pytest.mark.slow
def test_layer_forward_many_tiles_per_workgroup_every_token(many_tiles):
    h, d = many_tiles
    wl = MANY
    y, _ = moe.ffn_fwd(d["x"], d["wi"], d["wo"], wl.k, wr=d["wr"], save=False)
    torch.cuda.synchronize()
    idx, w, _ = oracle.route(bits(h["x"]), h["wr"].numpy(), None, wl.k)
    gs, off, *_ = oracle.dispatch(idx, wl.E)
    for kind, n, ntn in (("swiglu", 2 * wl.mlp, -(-wl.mlp // 128)), ("gemm", wl.emb, -(-wl.emb // 256))):
        per_wg = sum(-(-int(g) // 256) * ntn for g in gs) / moe_grid()
        assert per_wg >= 8, (kind, per_wg)
    ref = oracle.ffn_fwd_tokens(bits(h["x"]), idx, w, bits(h["wi"]), bits(h["wo"]))
    assert_close(to_np(y), ref, "y (every token)")


@pytest.mark.slow
def test_layer_backward_many_tiles_per_workgroup(many_tiles):
    h, d = many_tiles
    wl = MANY
    y, saved = moe.ffn_fwd(d["x"], d["wi"], d["wo"], wl.k, wr=d["wr"], save=True)
    g = moe.ffn_bwd(d["dy"], saved, d["wi"], d["wo"], wl.k)
    torch.cuda.synchronize()
    x, wi, wo, dy = bits(h["x"]), bits(h["wi"]), bits(h["wo"]), bits(h["dy"])
    idx, w, _ = oracle.route(x, h["wr"].numpy(), None, wl.k)
    assert np.array_equal(saved["topk_idx"].cpu().numpy(), idx)
    dx, dtw = oracle.ffn_bwd_tokens(x, idx, w, wi, wo, dy, stored_bf16=True)
    assert_close(to_np(g["dx"]), dx, "dx (every token)")
    assert_close(g["dtopk_w"].cpu().numpy(), dtw, "dtopk_w (every token)")
    gs = np.bincount(idx.reshape(-1), minlength=wl.E)
    experts = sorted({int(np.argmax(gs)), int(np.argmin(gs)), 3, 11})
    ref = oracle.ffn_wgrad_experts(x, idx, w, wi, wo, dy, experts, stored_bf16=True)
    for e in experts:
        assert_close_bf16_out(to_np(g["dwi"][e]), ref[e][0], f"dwi[{e}]")
        assert_close_bf16_out(to_np(g["dwo"][e]), ref[e][1], f"dwo[{e}]")


def moe_grid():
    props = torch.cuda.get_device_properties(0)
    n = props.multi_processor_count
    return max(8, n - n % 8)
