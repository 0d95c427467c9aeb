"""CPU checks of the persistent grouped GEMMs' ragged tile lists (no GPU).

moe_tile_schedule runs, on the host, the same tile functions the kernels call
(csrc/tiles.h) and lists what every workgroup computes on every turn. The
pages' grouped GEMM runs only the tiles a group needs and masks the partial
tile at a group edge ("MoE: fused TensorCore Pallas permute/combine kernels
and split-expert wi layout for TPU v6e", Tests: boundary-tile masking;
"[DRAFT][JAX] Optimize MoE block", Changes: group-aware kernels). Checked
here, for ragged, empty, clamped and single-row groups and several grid sizes:
every row of every group and every output column is covered exactly once, no
tile reaches past its group's end or the output width, empty groups get no
tile, rows past the last offset none, each workgroup runs consecutive turns,
and the deal balances tiles over workgroups to within one.
"""
import numpy as np
import pytest

import mixture_experts_ffn_group_amd as moe


def _offsets(sizes):
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)


def _check_turns(tiles, grid, total, balanced=True):
    assert len(tiles) == total
    w, it = tiles[:, 0], tiles[:, 1]
    assert w.min(initial=0) >= 0 and w.max(initial=0) < grid
    per_w = np.bincount(w, minlength=grid)
    if total and balanced:
        assert per_w.max() - per_w.min() <= 1, per_w
    for g in range(grid):
        turns = np.sort(it[w == g])
        assert np.array_equal(turns, np.arange(len(turns))), (g, turns)


def _check_gemm(kind, off, M, N, grid):
    tiles = moe.tile_schedule(kind, off, M, N, grid)
    swiglu = kind == "swiglu"
    width, tile_n = (N // 2, 128) if swiglu else (N, 256)
    ntn = -(-width // tile_n)
    lo = np.clip(off, 0, M)
    sizes = np.maximum(lo[1:] - lo[:-1], 0)
    total = int(sum(-(-n // 256) * ntn for n in sizes))
    _check_turns(tiles, grid, total)
    cover = np.zeros((M, ntn), np.int32)
    for (_, _, e, r0, r1, c0, c1) in tiles:
        assert sizes[e] > 0, "a tile for an empty group"
        assert lo[e] <= r0 < r1 <= lo[e + 1], (e, r0, r1, lo[e], lo[e + 1])
        n = sizes[e]
        if 256 < n <= 512:  # two equal halves: the first ceil(n/2) rows, then the rest
            h = (n + 1) // 2
            assert (r0, r1) in ((lo[e], lo[e] + h), (lo[e] + h, lo[e] + n)), (e, r0, r1, lo[e], n)
        else:
            assert r1 - r0 <= 256 and (r0 - lo[e]) % 256 == 0
        assert c0 % tile_n == 0 and c1 == min(c0 + tile_n, width)
        cover[r0:r1, c0 // tile_n] += 1
    in_group = np.zeros(M, bool)
    for e in range(len(sizes)):
        in_group[lo[e]:lo[e] + sizes[e]] = True
    assert (cover[in_group] == 1).all(), "a row/column block not covered exactly once"
    assert (cover[~in_group] == 0).all(), "a row outside every group covered"
    return tiles


CASES = [
    ("ragged + empty", [300, 0, 17, 256, 257, 0, 1, 900], 0),
    ("one group", [1000], 0),
    ("all empty", [0, 0, 0, 0], 0),
    ("single rows", [1] * 40, 0),
    ("uniform", [2048] * 16, 0),
    ("offsets past M (clamped)", [100, 100, 100, 100], -150),
]


@pytest.mark.parametrize("kind,N", [("gemm", 2048), ("gemm", 200), ("swiglu", 1536), ("swiglu", 2 * 96)])
@pytest.mark.parametrize("grid", [8, 16, 256])
@pytest.mark.parametrize("name,sizes,trim", CASES, ids=[c[0] for c in CASES])
def test_gemm_tiles_cover_each_group_once(kind, N, grid, name, sizes, trim):
    off = _offsets(sizes)
    M = int(off[-1]) + trim
    _check_gemm(kind, off, max(M, 0), N, grid)


def test_gemm_tiles_zipf_like_128_experts_many_turns():
    rng = np.random.default_rng(0)
    p = (np.arange(128) + 1.0) ** -1.1
    sizes = rng.multinomial(8192 * 8, p / p.sum())
    sizes[5] = 0
    off = _offsets(sizes)
    t = _check_gemm("swiglu", off, int(off[-1]), 1536, 8)
    assert t[:, 1].max() >= 30  # a small grid: dozens of turns per workgroup
    _check_gemm("gemm", off, int(off[-1]), 2048, 256)


def test_gemm_two_block_group_runs_as_equal_halves():
    # a group of 257 rows runs as halves of 129 and 128 rows for every column tile, and a group of
    # 513 rows as three 256-row blocks (the last of one row)
    off = _offsets([257])
    t = _check_gemm("gemm", off, 257, 512, 8)
    assert sorted((t[:, 4] - t[:, 3]).tolist()) == [128, 128, 129, 129]
    off = _offsets([513])
    t = _check_gemm("gemm", off, 513, 512, 8)
    assert sorted((t[:, 4] - t[:, 3]).tolist()) == [1, 1, 256, 256, 256, 256]


@pytest.mark.parametrize("kind,N", [("swiglu", 2 * 2048), ("gemm", 7168)])
def test_gemm_two_block_halves_run_side_by_side(kind, N):
    """256 groups of 256 +- 16 rows (the DeepSeek-V3 shape): both halves of a column of a 257-272-row
    group run on the same turn, on workgroups w and w + 8 (the same XCD, neighbouring slots). Every
    expert then has an even tile count, so workgroups 16i + x and 16i + 8 + x get tiles of equal
    height (+-1 row) on every turn, and stay in step."""
    rng = np.random.default_rng(3)
    sizes = 256 + rng.integers(-16, 17, 256)
    off = _offsets(sizes)
    t = _check_gemm(kind, off, int(off[-1]), N, 256)
    by = {}
    for (w, it, e, r0, r1, c0, c1) in t:
        by[(int(w), int(it))] = (int(e), int(r0), int(r1), int(c0))
        if 256 < sizes[e]:
            by.setdefault(("pair", int(e), int(c0)), []).append((int(w), int(it)))
    pairs = [v for k, v in by.items() if k[0] == "pair"]
    assert len(pairs) == int((sizes > 256).sum()) * (-(-(N // 2 if kind == "swiglu" else N) // (128 if kind == "swiglu" else 256)))
    for (wa, ia), (wb, ib) in (sorted(v) for v in pairs):
        assert ia == ib and wb == wa + 8 and (wa // 8) % 2 == 0, (wa, ia, wb, ib)
    for (w, it), (e, r0, r1, c0) in [(k, v) for k, v in by.items() if k[0] != "pair"]:
        if (w // 8) % 2 == 0 and (w + 8, it) in by:
            _, q0, q1, _ = by[(w + 8, it)]
            assert abs((r1 - r0) - (q1 - q0)) <= 1, (w, it, r1 - r0, q1 - q0)


@pytest.mark.parametrize("E,P,Q,grid", [(8, 512, 1536, 8), (5, 296, 64, 16), (256, 7168, 4096, 256),
                                        (16, 256, 256, 8), (1, 1000, 2000, 256)])
def test_wgrad_tiles_cover_every_expert_once(E, P, Q, grid):
    rng = np.random.default_rng(E)
    off = _offsets(rng.integers(0, 50, E))
    tiles = moe.tile_schedule("wgrad", off, int(off[-1]), P, grid, Q=Q)
    tp, tq = -(-P // 256), -(-Q // 256)
    # whole experts per XCD: balanced when E is a multiple of 8
    _check_turns(tiles, grid, E * tp * tq, balanced=E % 8 == 0)
    cover = np.zeros((E, tp, tq), np.int32)
    for (w, _, e, p0, p1, q0, q1) in tiles:
        assert w % 8 == e % 8, "an expert's tiles stay on its XCD"
        assert p0 % 256 == 0 and p1 == min(p0 + 256, P) and q0 % 256 == 0 and q1 == min(q0 + 256, Q)
        cover[e, p0 // 256, q0 // 256] += 1
    assert (cover == 1).all()


def test_schedule_rejects_bad_arguments():
    off = _offsets([10, 20])
    for grid in (0, 12, -8):
        with pytest.raises(moe.MoeError):
            moe.tile_schedule("gemm", off, 30, 256, grid)
    assert len(moe.tile_schedule("gemm", _offsets([0]), 0, 256, 8)) == 0
