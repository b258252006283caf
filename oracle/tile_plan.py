"""Oracle tile plan: geometry, masks, normalized positions, conditioning keep.

Test infrastructure (see the package docstring).  Integer work is exact; the
float outputs are the float32 values the plan defines (masks, 1/k weights,
offsets and positions), so the GPU library's host plan must match them bit
for bit.
"""
from __future__ import annotations

import dataclasses

import numpy as np

F32 = np.float32


class PlanError(ValueError):
    """An invalid tiling or descriptor."""


def _cores(L: int, n: int) -> list:
    # Core partition of [0, L) into n nearly equal parts: core i = [c_i, c_{i+1}).
    return [(i * L) // n for i in range(n + 1)]


def dim_boxes(L: int, n: int, o: int) -> list:
    """Tile boxes ``[a, b)`` along one dimension of length ``L``.

    TDP page, "API / Tiling config": a dimension is configured by a tile COUNT
    and an overlap in latent grid units; the page gives no formula for the
    boxes.  Reading used: split [0, L) into ``n`` cores ``[c_i, c_{i+1})`` with
    ``c_i = floor(i L / n)`` and widen each core by ``floor(o/2)`` on the left
    and ``ceil(o/2)`` on the right, clipped to [0, L).  Adjacent boxes then
    overlap by exactly ``o``.  ``n == 1`` gives ``[0, L)`` whatever ``o``.
    Valid only for ``1 <= n <= L`` and ``0 <= o <= min core length``, so a
    grid position lies in at most two boxes per dimension.
    """
    if L < 1:
        raise PlanError(f"dimension length {L} < 1")
    if n < 1 or n > L:
        raise PlanError(f"num_tiles {n} not in [1, {L}]")
    if o < 0:
        raise PlanError(f"overlap {o} < 0")
    if n == 1:
        return [(0, L)]
    c = _cores(L, n)
    min_core = min(c[i + 1] - c[i] for i in range(n))
    if o > min_core:
        raise PlanError(f"overlap {o} exceeds the smallest core length {min_core}")
    lo, hi = o // 2, o - o // 2
    return [(max(0, c[i] - lo), min(L, c[i + 1] + hi)) for i in range(n)]


def dim_weights(L: int, n: int, o: int, i: int) -> np.ndarray:
    """Trapezoid mask factors (float32) of tile ``i`` over its box, one dimension.

    TDP page, "What it is": overlapping regions are blended with trapezoidal
    masks that sum to one globally.  Reading used: the overlap between tiles
    ``i-1`` and ``i`` is ``[c_i - floor(o/2), c_i + ceil(o/2))``; at its k-th
    position (k = 0 .. o-1) the right-hand tile ramps up with
    ``(2k+1)/(2o)`` and the left-hand tile ramps down with ``(2o-2k-1)/(2o)``,
    each rounded once to float32.  Everywhere else, including the global
    edges of the grid, the factor is 1.
    """
    boxes = dim_boxes(L, n, o)
    a, b = boxes[i]
    w = np.ones(b - a, dtype=F32)
    if n == 1 or o == 0:
        return w
    c = _cores(L, n)
    lo = o // 2
    two_o = F32(2 * o)
    for p in range(a, b):
        if i > 0:
            s = c[i] - lo                      # overlap with tile i-1 starts here
            if s <= p < s + o:
                k = p - s
                w[p - a] = F32(2 * k + 1) / two_o
                continue
        if i < n - 1:
            s = c[i + 1] - lo                  # overlap with tile i+1 starts here
            if s <= p < s + o:
                k = p - s
                w[p - a] = F32(2 * o - 2 * k - 1) / two_o
    return w


@dataclasses.dataclass
class Plan:
    """A rank's share of one TDP step.  Arrays mirror the GPU library's plan."""
    grid: tuple
    tiling: tuple
    n_cond: int
    world_size: int
    rank: int
    n_tiles_total: int
    tile_id: np.ndarray          # [T] int32 global tile index
    tile_box: np.ndarray         # [T][3][2] int32
    tile_offset: np.ndarray      # [T][3] float32
    tile_row_begin: np.ndarray   # [T+1] int64
    tile_n_gen: np.ndarray       # [T] int32
    row_src: np.ndarray          # [rows] int32 (>= N: conditioning token N + j)
    row_weight: np.ndarray       # [rows] float32
    row_pos: np.ndarray          # [rows][3][2] float32
    cond_keep_count: np.ndarray  # [M] int32, over all tiles of all ranks
    dst_row_begin: np.ndarray    # [N+M+1] int64
    dst_rows: np.ndarray         # [rows] int32

    @property
    def n_rows(self) -> int:
        return int(self.tile_row_begin[-1])

    @property
    def n_dst_rows(self) -> int:
        return int(self.dst_row_begin.shape[0] - 1)

    @property
    def max_tile_rows(self) -> int:
        if self.tile_id.size == 0:
            return 0
        return int(np.max(np.diff(self.tile_row_begin)))


def _tile_coords(t: int, counts) -> tuple:
    # Tile index t = (i_f * n_h + i_h) * n_w + i_w (width fastest).
    n_f, n_h, n_w = counts
    return (t // (n_h * n_w), (t // n_w) % n_h, t % n_w)


def _keeps(cond_pos: np.ndarray, j: int, ext_start, ext_end) -> bool:
    """Keep rule, TDP page, "Shared negative (reference) positions".

    A tile keeps conditioning token j when the token's [start, end) interval
    overlaps the tile in all three dimensions, or when its time start is
    negative.  Readings: overlap is strict half-open (``s < E and e > S``)
    against the tile's extent ``[S, E)`` = [min start, max end) of its
    generated tokens in global coordinates; "negative" means start < 0 in
    global coordinates.
    """
    s = cond_pos[j, :, 0]
    e = cond_pos[j, :, 1]
    if s[0] < 0:
        return True
    return all(s[d] < ext_end[d] and e[d] > ext_start[d] for d in range(3))


def assign_tiles(costs, world_size: int, assignment: str = "round_robin") -> list:
    """Owner rank of every tile.

    TDP page, "What it is": tiles are assigned round-robin, tile t to rank
    t mod world_size.  "longest_first" is a balancing alternative the page
    does not give (longest-processing-time-first): tiles in decreasing cost
    (ties: lower index first), each to the rank whose cost so far is least
    (ties: lower rank).
    """
    T = len(costs)
    if assignment == "round_robin":
        return [t % world_size for t in range(T)]
    if assignment != "longest_first":
        raise PlanError(f"unknown assignment {assignment!r}")
    order = sorted(range(T), key=lambda t: (-costs[t], t))
    load = [0] * world_size
    owner = [0] * T
    for t in order:
        r = min(range(world_size), key=lambda q: (load[q], q))
        owner[t] = r
        load[r] += costs[t]
    return owner


def plan(grid, tiling, cond_pos=None, normalize_positions: bool = True,
         world_size: int = 1, rank: int = 0, assignment: str = "round_robin") -> Plan:
    """Plan one rank's tiles of a TDP step.

    ``grid`` = (F, H, W); ``tiling`` = ((n_f, o_f), (n_h, o_h), (n_w, o_w));
    ``cond_pos`` = [M][3][2] float32 (start, end) intervals of the conditioning
    tokens, dims (time, height, width).

    Passages followed (TDP page):
      * "What it is": tiles of the patchified latent, assigned round-robin, so
        tile t goes to rank ``t mod world_size`` (or longest first, see
        ``assign_tiles``).  Tile order (a reading): row-major over
        (i_f, i_h, i_w), width fastest; a rank's tiles in ascending order.
      * Token order (a reading): generated token (f, h, w) is global row
        ``(f H + h) W + w``; conditioning token j is row ``N + j`` ("appended
        after the generated tokens").  A tile's rows are its generated tokens,
        row-major over its box, then its kept conditioning tokens, ascending j.
      * A generated token at (f, h, w) has the unit intervals [f, f+1),
        [h, h+1), [w, w+1) (a reading: latent grid units).
      * "Position normalization": offset = per-dimension minimum start over the
        tile's generated tokens; subtracted from both ends of every row of the
        tile, generated and conditioning.  Zero when normalization is off.
      * "Shared negative (reference) positions": keep rule (``_keeps``), and a
        kept token's blend weight ``1 / (number of tiles that kept it)``,
        counted over all tiles of all ranks.  A token no tile keeps gets no
        row (its output stays zero).
    """
    F, H, W = (int(v) for v in grid)
    counts = tuple(int(c) for c, _ in tiling)
    overl = tuple(int(o) for _, o in tiling)
    if world_size < 1 or not (0 <= rank < world_size):
        raise PlanError(f"rank {rank} not in [0, {world_size})")
    if cond_pos is None:
        cond_pos = np.zeros((0, 3, 2), dtype=F32)
    cond_pos = np.asarray(cond_pos, dtype=F32).reshape(-1, 3, 2)
    if not np.all(np.isfinite(cond_pos)) or np.any(cond_pos[..., 1] < cond_pos[..., 0]):
        raise PlanError("conditioning intervals must be finite with end >= start")
    M = int(cond_pos.shape[0])
    N = F * H * W
    dims = (F, H, W)
    boxes = [dim_boxes(dims[d], counts[d], overl[d]) for d in range(3)]
    wts = [[dim_weights(dims[d], counts[d], overl[d], i) for i in range(counts[d])]
           for d in range(3)]
    T = counts[0] * counts[1] * counts[2]

    # Generated tokens and extents of every tile (all ranks: k_j needs them).
    gen = []
    for t in range(T):
        ii = _tile_coords(t, counts)
        (af, bf), (ah, bh), (aw, bw) = (boxes[d][ii[d]] for d in range(3))
        f, h, w = np.meshgrid(np.arange(af, bf), np.arange(ah, bh), np.arange(aw, bw),
                              indexing="ij")
        f, h, w = f.ravel(), h.ravel(), w.ravel()
        src = ((f * H + h) * W + w).astype(np.int32)
        wf, wh, ww = (wts[d][ii[d]] for d in range(3))
        weight = (wf[f - af] * wh[h - ah]) * ww[w - aw]          # float32 products
        start = np.stack([f, h, w], axis=1).astype(F32)           # [n][3]
        end = start + F32(1)
        gen.append((ii, src, weight.astype(F32), start, end))

    keep = np.zeros((T, M), dtype=bool)
    for t in range(T):
        _, _, _, start, end = gen[t]
        ext_s, ext_e = start.min(axis=0), end.max(axis=0)
        for j in range(M):
            keep[t, j] = _keeps(cond_pos, j, ext_s, ext_e)
    k = keep.sum(axis=0).astype(np.int32)

    # Attention cost of a tile: (generated rows + kept conditioning rows)^2.
    costs = [(gen[t][1].size + int(keep[t].sum())) ** 2 for t in range(T)]
    owner = assign_tiles(costs, world_size, assignment)
    local = [t for t in range(T) if owner[t] == rank]
    tile_box = np.zeros((len(local), 3, 2), dtype=np.int32)
    tile_offset = np.zeros((len(local), 3), dtype=F32)
    begin = [0]
    n_gen = []
    srcs, weights, poss = [], [], []
    for li, t in enumerate(local):
        ii, src, weight, start, end = gen[t]
        for d in range(3):
            tile_box[li, d] = boxes[d][ii[d]]
        off = start.min(axis=0) if normalize_positions else np.zeros(3, dtype=F32)
        tile_offset[li] = off
        kept = [j for j in range(M) if keep[t, j]]
        c_src = np.array([N + j for j in kept], dtype=np.int32)
        c_w = np.array([F32(1) / F32(k[j]) for j in kept], dtype=F32)
        c_pos = cond_pos[kept].reshape(len(kept), 3, 2)
        g_pos = np.stack([start, end], axis=2)                    # [n][3][2]
        pos = np.concatenate([g_pos, c_pos], axis=0) - off[None, :, None]
        srcs.append(np.concatenate([src, c_src]))
        weights.append(np.concatenate([weight, c_w]))
        poss.append(pos.astype(F32))
        n_gen.append(src.size)
        begin.append(begin[-1] + src.size + c_src.size)

    row_src = np.concatenate(srcs).astype(np.int32) if srcs else np.zeros(0, np.int32)
    row_weight = np.concatenate(weights).astype(F32) if weights else np.zeros(0, F32)
    row_pos = (np.concatenate(poss).astype(F32) if poss
               else np.zeros((0, 3, 2), dtype=F32))
    # Inverse map: for each destination row, the rows feeding it in ascending
    # (tile, row) order.  A stable sort by destination keeps that order.
    n_dst = N + M
    dst_rows = np.argsort(row_src, kind="stable").astype(np.int32)
    per_dst = np.bincount(row_src, minlength=n_dst) if row_src.size else np.zeros(n_dst, int)
    dst_row_begin = np.concatenate([[0], np.cumsum(per_dst)]).astype(np.int64)
    return Plan(grid=(F, H, W), tiling=tuple(zip(counts, overl)), n_cond=M,
                world_size=world_size, rank=rank, n_tiles_total=T,
                tile_id=np.array(local, dtype=np.int32), tile_box=tile_box,
                tile_offset=tile_offset, tile_row_begin=np.array(begin, dtype=np.int64),
                tile_n_gen=np.array(n_gen, dtype=np.int32), row_src=row_src,
                row_weight=row_weight, row_pos=row_pos, cond_keep_count=k,
                dst_row_begin=dst_row_begin, dst_rows=dst_rows)


def balanced_tile_split(n: int) -> tuple:
    """(h_tiles, w_tiles) for ``n`` tiles on a 2D height x width grid.

    TDP page, "Usage": the full-resolution stage asks a ``balanced_tile_split``
    helper for a balanced 2D spatial (height x width) grid with one tile per
    rank of the group; the page does not define it.  Reading used: the factor
    pair h * w = n with h <= w and w - h as small as possible, i.e. h is the
    largest divisor of n not above sqrt(n) (width gets the larger count, as
    video latents are wider than tall).  Walks h down from floor(sqrt(n)).
    """
    if n < 1:
        raise PlanError("n must be >= 1")
    h = int(np.floor(np.sqrt(n)))
    while h * h > n:
        h -= 1
    while (h + 1) * (h + 1) <= n:
        h += 1
    while n % h:
        h -= 1
    return h, n // h
