"""Oracle gather and blend.  Float64 accumulation.

Test infrastructure (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .tile_plan import Plan

F64 = np.float64


def gather_tiles(x_global: np.ndarray, p: Plan) -> np.ndarray:
    """Copy each tile row from the global latent: ``x_tiles[b][r] = x_global[b][row_src[r]]``.

    TDP page, "What it is": each tile is a piece of the patchified latent;
    "Shared negative (reference) positions": the kept conditioning tokens,
    appended after the generated ones, follow the tile's generated rows.
    """
    return np.asarray(x_global)[:, p.row_src, :]


def blend_tiles(y_tiles: np.ndarray, p: Plan, n_dst: int | None = None,
                y_global: np.ndarray | None = None) -> np.ndarray:
    """Weighted sum of the tile outputs into the global latent (float64).

    TDP page, "What it is": overlapping regions are blended with trapezoidal
    masks and one all_reduce sums the blended tiles; "Shared negative
    (reference) positions": a conditioning token kept by k tiles is weighted
    1/k.  On one GPU the all_reduce becomes this sum.  Order: tiles ascending,
    then rows; a destination row receives at most one row per tile.  If
    ``y_global`` is given the sum is added to it (the sum over ranks).
    """
    y_tiles = np.asarray(y_tiles, dtype=F64)
    B, _, C = y_tiles.shape
    if n_dst is None:
        n_dst = p.n_dst_rows
    out = np.zeros((B, n_dst, C), dtype=F64) if y_global is None else \
        np.array(y_global, dtype=F64, copy=True)
    w = p.row_weight.astype(F64)
    for t in range(p.tile_id.size):
        r0, r1 = int(p.tile_row_begin[t]), int(p.tile_row_begin[t + 1])
        src = p.row_src[r0:r1]
        assert np.unique(src).size == src.size
        out[:, src, :] += w[r0:r1][None, :, None] * y_tiles[:, r0:r1, :]
    return out


def audio_mean(y_aud_tiles: np.ndarray, n_tiles_total: int) -> np.ndarray:
    """Average of the per-tile audio outputs: ``sum_t (1/T) y_aud_t`` (float64).

    TDP page, "What it is" and its warning box: the audio stream is not cut
    into tiles, it enters each tile's forward pass, and the tiles' audio
    results are averaged.  With
    several ranks each rank sums its own tiles with weight 1/T_total, so the
    sum over ranks is the mean over all tiles.
    """
    y = np.asarray(y_aud_tiles, dtype=F64)       # [T_local][B][A][C]
    return (y * (1.0 / n_tiles_total)).sum(axis=0)
