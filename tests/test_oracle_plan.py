"""Pins for the oracle's tile plan (CPU only).

Each test ties the oracle to something other than its own formula: numbers the
pages print, closed forms of the tiling, brute-force enumeration on tiny
grids, and the invariants the TDP page states (masks sum to one, generated
tokens start at zero after normalization with widths kept, negative-time
tokens kept by every tile, a token kept by k tiles weighted 1/k).
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import tdp_inputs as ti

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")

TILINGS_1D = [(16, 2, 4), (32, 2, 8), (64, 4, 8), (48, 3, 8), (80, 4, 8), (32, 2, 4),
              (96, 6, 16), (160, 10, 16), (17, 3, 5), (23, 4, 5), (10, 3, 3), (7, 7, 1),
              (9, 1, 0), (9, 1, 5), (13, 5, 0), (11, 4, 2), (31, 6, 5)]


@pytest.mark.parametrize("L,n,o", TILINGS_1D)
def test_boxes_closed_forms(L, n, o):
    boxes = oracle.dim_boxes(L, n, o)
    assert len(boxes) == n
    assert boxes[0][0] == 0 and boxes[-1][1] == L
    if n == 1:
        assert boxes == [(0, L)]
        return
    # adjacent boxes overlap by exactly o, sizes add up to L + (n-1) o
    for i in range(n - 1):
        assert boxes[i][1] - boxes[i + 1][0] == o
    assert sum(b - a for a, b in boxes) == L + (n - 1) * o
    # every position is covered, by at most two boxes
    cover = np.zeros(L, int)
    for a, b in boxes:
        cover[a:b] += 1
    assert cover.min() >= 1 and cover.max() <= 2
    # boxes are as equal as the integer split allows
    sizes = [b - a for a, b in boxes]
    interior = sizes[1:-1]
    if interior:
        assert max(interior) - min(interior) <= 1


@pytest.mark.parametrize("L,n,o", [(8, 0, 0), (8, 9, 0), (8, 2, -1), (8, 2, 5), (0, 1, 0)])
def test_boxes_reject_invalid(L, n, o):
    with pytest.raises(oracle.PlanError):
        oracle.dim_boxes(L, n, o)


def test_pages_round_robin_example():
    """16 tiles on 4 GPUs = 4 tiles per rank (TDP page, "What it is")."""
    facts = json.load(open(GOLDEN))["round_robin_example"]
    seen = []
    for r in range(facts["gpus"]):
        p = oracle.plan((2, 16, 16), ((1, 0), (4, 2), (4, 2)), world_size=facts["gpus"], rank=r)
        assert p.n_tiles_total == facts["tiles"]
        assert p.tile_id.size == facts["tiles_per_rank"]
        seen += list(p.tile_id)
    assert sorted(seen) == list(range(facts["tiles"]))


def test_interior_tile_size_16tile():
    facts = json.load(open(GOLDEN))["interior_tile_tokens_16tile"]
    p = oracle.plan(tuple(facts["grid"]), tuple(map(tuple, facts["tiling"])))
    assert p.max_tile_rows == facts["interior_tokens"]
    assert p.n_tiles_total == 16


def test_pages_overlap_5_is_valid():
    o = json.load(open(GOLDEN))["stage2_overlap"]["overlap"]
    p = oracle.plan((4, 24, 40), ((1, 0), (2, o), (3, o)))
    assert p.n_tiles_total == 6


def _brute_rows(grid, tiling):
    """Which tiles contain each token, by enumerating every box (no ordering logic)."""
    F, H, W = grid
    boxes = [oracle.dim_boxes(grid[d], tiling[d][0], tiling[d][1]) for d in range(3)]
    member = {}
    for t, (i, j, k) in enumerate(itertools.product(*[range(len(b)) for b in boxes])):
        for f in range(F):
            for h in range(H):
                for w in range(W):
                    if (boxes[0][i][0] <= f < boxes[0][i][1] and boxes[1][j][0] <= h < boxes[1][j][1]
                            and boxes[2][k][0] <= w < boxes[2][k][1]):
                        member.setdefault(t, []).append((f * H + h) * W + w)
    return member


@pytest.mark.parametrize("grid,tiling", [
    ((2, 16, 16), ((1, 0), (2, 4), (2, 4))),
    ((3, 17, 23), ((1, 0), (3, 5), (4, 5))),
    ((5, 6, 7), ((2, 1), (2, 2), (3, 1))),
    ((4, 9, 9), ((2, 2), (1, 0), (3, 3))),
])
def test_rows_brute_force(grid, tiling):
    p = oracle.plan(grid, tiling)
    member = _brute_rows(grid, tiling)
    for li, t in enumerate(p.tile_id):
        r0, r1 = p.tile_row_begin[li], p.tile_row_begin[li + 1]
        rows = list(p.row_src[r0:r1])
        assert rows == sorted(member[int(t)])       # row-major box order == ascending token id


def _mask_sums(p, n_gen):
    s = [Fraction(0)] * n_gen
    sf = np.zeros(n_gen, np.float32)
    for r in range(p.n_rows):
        n = int(p.row_src[r])
        if n < n_gen:
            s[n] += Fraction(float(p.row_weight[r]))
            sf[n] += p.row_weight[r]
    return s, sf


@pytest.mark.parametrize("name", list(ti.WORKLOADS))
def test_masks_sum_to_one_exactly(name):
    """Masks sum to 1 globally (TDP page, "What it is"), exactly in float32 for o in {4, 8, 16}."""
    wl = ti.WORKLOADS[name]
    p = oracle.plan(wl.grid, wl.tiling)
    gen = p.row_src < wl.n_gen
    sf = np.zeros(wl.n_gen, np.float32)
    np.add.at(sf, p.row_src[gen], p.row_weight[gen])
    assert np.all(sf == np.float32(1.0))
    # the float32 weights are dyadic here, so the float64 sum is exactly 1 too
    s64 = np.zeros(wl.n_gen, np.float64)
    np.add.at(s64, p.row_src[gen], p.row_weight[gen].astype(np.float64))
    assert np.all(s64 == 1.0)


@pytest.mark.parametrize("grid,tiling", [((3, 17, 23), ((1, 0), (3, 5), (4, 5))),
                                         ((6, 12, 10), ((2, 3), (3, 3), (2, 5)))])
def test_masks_sum_to_one_odd_overlap(grid, tiling):
    p = oracle.plan(grid, tiling)
    n_gen = grid[0] * grid[1] * grid[2]
    s, sf = _mask_sums(p, n_gen)
    for v in s:      # exact rational sum of the float32 weights: within float32 rounding of 1
        assert abs(v - 1) <= Fraction(3, 2 ** 24)
    assert np.abs(sf - 1).max() <= 3 * 2.0 ** -24


@pytest.mark.parametrize("L,n,o", [(64, 4, 8), (17, 3, 5), (160, 10, 16), (12, 3, 1)])
def test_trapezoid_shape(L, n, o):
    """1D factors: 1 away from overlaps, ramps monotone, neighbours complementary."""
    boxes = oracle.dim_boxes(L, n, o)
    ws = [oracle.dim_weights(L, n, o, i) for i in range(n)]
    for i, ((a, b), w) in enumerate(zip(boxes, ws)):
        assert np.all(w > 0) and np.all(w <= 1)
        assert np.all(np.diff(w[: (b - a) // 2]) >= 0) or i == 0
        # the value at each position, seen from the two tiles that share it, adds to 1
        if i + 1 < n:
            a2, _ = boxes[i + 1]
            for pos in range(a2, b):
                tot = Fraction(float(w[pos - a])) + Fraction(float(ws[i + 1][pos - a2]))
                assert abs(tot - 1) <= Fraction(1, 2 ** 24)
        # positions not shared with a neighbour weigh exactly 1
        shared = set()
        if i > 0:
            shared |= set(range(a, boxes[i - 1][1]))
        if i + 1 < n:
            shared |= set(range(boxes[i + 1][0], b))
        for pos in range(a, b):
            if pos not in shared:
                assert w[pos - a] == 1.0
    # the up-ramp of tile i+1 mirrors the down-ramp of tile i
    a2, _ = boxes[1]
    up = ws[1][: boxes[0][1] - a2]
    down = ws[0][a2 - boxes[0][0]:]
    assert np.all(up == down[::-1])


def test_single_tile_all_weights_one():
    p = oracle.plan((3, 8, 8), ((1, 0), (1, 0), (1, 0)))
    assert np.all(p.row_weight == 1.0) and p.n_rows == 3 * 8 * 8


@pytest.mark.parametrize("name", ["tiny_2x16x16", "d64_8x32x32", "audio_32x48x80"])
def test_normalization_invariants(name):
    """Generated tokens start at 0 in every dim; widths kept (TDP page, "Position normalization")."""
    inp = ti.make_inputs(name)
    wl = inp.workload
    p = oracle.plan(wl.grid, wl.tiling, inp.cond_pos)
    praw = oracle.plan(wl.grid, wl.tiling, inp.cond_pos, normalize_positions=False)
    assert np.all(praw.tile_offset == 0)
    for t in range(p.tile_id.size):
        r0, r1 = p.tile_row_begin[t], p.tile_row_begin[t + 1]
        g1 = r0 + p.tile_n_gen[t]
        pos, raw = p.row_pos[r0:r1], praw.row_pos[r0:r1]
        assert np.all(pos[: g1 - r0, :, 0].min(axis=0) == 0)
        assert np.all((pos[..., 1] - pos[..., 0]) == (raw[..., 1] - raw[..., 0]))
        # one shift per tile and dim, for generated and conditioning rows alike
        shift = raw - pos
        assert np.all(shift == shift[0:1])
        # unnormalized positions are the global ones: generated (f,h,w) cells, cond intervals
        F, H, W = wl.grid
        src = p.row_src[r0:g1]
        cells = np.stack([src // (H * W), (src // W) % H, src % W], axis=1)
        assert np.all(raw[: g1 - r0, :, 0] == cells) and np.all(raw[: g1 - r0, :, 1] == cells + 1)
        csrc = p.row_src[g1:r1] - wl.n_gen
        assert np.all(raw[g1 - r0:] == inp.cond_pos[csrc])


def _keep_brute(cond_pos, box):
    """Overlap by enumerating integer cells of the tile (intervals have integer ends)."""
    s, e = cond_pos[:, 0], cond_pos[:, 1]
    if s[0] < 0:
        return True
    for d in range(3):
        cells = range(int(box[d][0]), int(box[d][1]))
        if not any(s[d] <= x < e[d] for x in cells):
            return False
    return True


@pytest.mark.parametrize("name", ["tiny_2x16x16", "d64_8x32x32", "audio_32x48x80"])
def test_keep_rule_brute_force(name):
    inp = ti.make_inputs(name)
    wl = inp.workload
    p = oracle.plan(wl.grid, wl.tiling, inp.cond_pos)
    k = np.zeros(wl.n_cond, int)
    for t in range(p.tile_id.size):
        r0, r1 = p.tile_row_begin[t], p.tile_row_begin[t + 1]
        kept = [int(x) - wl.n_gen for x in p.row_src[r0 + p.tile_n_gen[t]:r1]]
        want = [j for j in range(wl.n_cond) if _keep_brute(inp.cond_pos[j], p.tile_box[t])]
        assert kept == want
        for j in kept:
            k[j] += 1
        # negative-time tokens are kept by every tile
        for j in range(wl.n_cond):
            if inp.cond_pos[j, 0, 0] < 0:
                assert j in kept
    assert np.all(k == p.cond_keep_count)


@pytest.mark.parametrize("name", ["tiny_2x16x16", "d64_8x32x32", "audio_32x48x80"])
def test_inverse_k_weights_sum_to_one(name):
    inp = ti.make_inputs(name)
    wl = inp.workload
    p = oracle.plan(wl.grid, wl.tiling, inp.cond_pos)
    cond = p.row_src >= wl.n_gen
    s = np.zeros(wl.n_cond, np.float64)
    np.add.at(s, p.row_src[cond] - wl.n_gen, p.row_weight[cond].astype(np.float64))
    kept = p.cond_keep_count > 0
    assert np.all(np.abs(s[kept] - 1) <= 4 * 2.0 ** -24)
    assert np.all(s[~kept] == 0)


def test_unkept_token_gets_no_row():
    cond = np.array([[[0, 1], [0, 1], [0, 1]], [[5, 6], [30, 31], [30, 31]]], np.float32)
    p = oracle.plan((8, 16, 16), ((1, 0), (2, 2), (2, 2)), cond)
    # token 1 lies outside the grid in h and w, at non-negative time: kept by no tile
    assert p.cond_keep_count.tolist() == [1, 0]
    assert (p.row_src == 8 * 16 * 16 + 1).sum() == 0
    assert p.dst_row_begin[-1] - p.dst_row_begin[-2] == 0


@pytest.mark.parametrize("W", [2, 3, 4])
def test_round_robin_partition(W):
    inp = ti.make_inputs("audio_32x48x80")
    wl = inp.workload
    full = oracle.plan(wl.grid, wl.tiling, inp.cond_pos)
    tiles, nrows = [], 0
    for r in range(W):
        p = oracle.plan(wl.grid, wl.tiling, inp.cond_pos, world_size=W, rank=r)
        assert all(int(t) % W == r for t in p.tile_id)
        assert np.all(p.cond_keep_count == full.cond_keep_count)
        tiles += list(p.tile_id)
        nrows += p.n_rows
    assert sorted(tiles) == list(range(full.n_tiles_total)) and nrows == full.n_rows


def test_inverse_map_lists_rows_in_tile_order():
    inp = ti.make_inputs("d64_8x32x32")
    wl = inp.workload
    p = oracle.plan(wl.grid, wl.tiling, inp.cond_pos)
    tile_of_row = np.repeat(np.arange(p.tile_id.size), np.diff(p.tile_row_begin))
    for n in range(p.n_dst_rows):
        rows = p.dst_rows[p.dst_row_begin[n]:p.dst_row_begin[n + 1]]
        assert np.all(p.row_src[rows] == n)
        assert np.all(np.diff(tile_of_row[rows]) > 0)
    assert sorted(p.dst_rows.tolist()) == list(range(p.n_rows))


# --------------------------------------------------------------------------
# balanced 2D split of a group ("Usage": balanced_tile_split)
# --------------------------------------------------------------------------

def _balanced_brute(n):
    # every factor pair with h <= w; the balanced one has the smallest gap
    pairs = [(h, n // h) for h in range(1, n + 1) if n % h == 0 and h <= n // h]
    return min(pairs, key=lambda p: p[1] - p[0])


def test_balanced_split_brute_force():
    for n in range(1, 1025):
        assert oracle.balanced_tile_split(n) == _balanced_brute(n), n


def test_balanced_split_special_cases():
    # primes have only the trivial split; squares split evenly
    for p in [2, 3, 5, 7, 11, 13, 97, 1009]:
        assert oracle.balanced_tile_split(p) == (1, p)
    for r in range(1, 40):
        assert oracle.balanced_tile_split(r * r) == (r, r)
    # the spatial tile grids of the 4-, 16- and 60-tile workloads
    assert oracle.balanced_tile_split(4) == (2, 2)
    assert oracle.balanced_tile_split(16) == (4, 4)
    assert oracle.balanced_tile_split(60) == (6, 10)
    with pytest.raises(oracle.PlanError):
        oracle.balanced_tile_split(0)


# --------------------------------------------------------------------------
# longest-first tile assignment
# --------------------------------------------------------------------------

def test_longest_first_textbook_case():
    """Costs 7, 6, 5, 4, 3 on two ranks: 7 -> 0, 6 -> 1, 5 -> 1, 4 -> 0, and 3
    to rank 0 on the 11/11 tie; loads 14 and 11."""
    owner = oracle.assign_tiles([7, 6, 5, 4, 3], 2, "longest_first")
    assert owner == [0, 1, 1, 0, 0]
    # ties in cost: lower index first
    assert oracle.assign_tiles([5, 9, 5, 9], 2, "longest_first") == [0, 0, 1, 1]


@pytest.mark.parametrize("T,W", [(16, 4), (7, 3), (5, 8), (24, 5)])
def test_longest_first_with_equal_costs_is_round_robin(T, W):
    assert oracle.assign_tiles([4] * T, W, "longest_first") == [t % W for t in range(T)]


@pytest.mark.parametrize("name,W", [("t16_16x64x64", 4), ("audio_32x48x80", 5),
                                    ("tiny_2x16x16", 3)])
def test_longest_first_partitions_and_balances(name, W):
    inp = ti.make_inputs(name)
    wl = inp.workload
    seen, rr_load, lf_load = [], [], []
    for r in range(W):
        p_lf = oracle.plan(wl.grid, wl.tiling, inp.cond_pos, True, W, r, "longest_first")
        p_rr = oracle.plan(wl.grid, wl.tiling, inp.cond_pos, True, W, r)
        seen += p_lf.tile_id.tolist()
        assert list(p_lf.tile_id) == sorted(p_lf.tile_id)
        lf_load.append(int(np.sum(np.diff(p_lf.tile_row_begin).astype(np.int64) ** 2)))
        rr_load.append(int(np.sum(np.diff(p_rr.tile_row_begin).astype(np.int64) ** 2)))
    assert sorted(seen) == list(range(wl.n_tiles))
    assert max(lf_load) <= max(rr_load)
    if name == "t16_16x64x64":
        assert max(lf_load) < max(rr_load)      # interior tiles carry 1.44x a corner's cost
