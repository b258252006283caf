"""Oracle TDP step: plan -> gather -> per-tile denoiser -> blend (+ audio mean).

Test infrastructure (see the package docstring).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from .blend import audio_mean, blend_tiles, gather_tiles
from .denoise import tile_forward
from .tile_plan import Plan, plan as make_plan


@dataclasses.dataclass
class StepResult:
    plan: Plan
    x_tiles: np.ndarray                 # [B][rows][C] as gathered
    y_tiles: np.ndarray                 # [B][rows][C] float64
    y_global: np.ndarray                # [B][N+M][C] float64
    y_aud_tiles: Optional[np.ndarray]   # [T_local][B][A][C] float64
    y_aud: Optional[np.ndarray]         # [B][A][C] float64


def step(inp, normalize_positions: bool = True, world_size: int = 1, rank: int = 0,
         identity: Optional[bool] = None, rope_base: float = 10000.0,
         p: Optional[Plan] = None) -> StepResult:
    """One TDP step over a rank's tiles (``inp`` is a ``tdp_inputs.Inputs``).

    TDP page, "What it is": tiles of the latent (round-robin over ranks), one
    denoiser forward per tile, trapezoid-weighted blend summed into the global
    latent, audio averaged over tiles.  With ``identity`` the denoiser returns
    its input (tile rows and audio), which makes the blend reconstruct the
    latent.
    """
    wl = inp.workload
    if identity is None:
        identity = wl.identity
    if p is None:
        p = make_plan(wl.grid, wl.tiling, inp.cond_pos, normalize_positions,
                      world_size, rank)
    x_tiles = gather_tiles(inp.x_global, p)
    B, rows, C = x_tiles.shape
    y_tiles = np.zeros((B, rows, C), dtype=np.float64)
    T = p.tile_id.size
    y_aud_tiles = None
    if inp.x_aud is not None:
        y_aud_tiles = np.zeros((T,) + inp.x_aud.shape, dtype=np.float64)
    for t in range(T):
        r0, r1 = int(p.tile_row_begin[t]), int(p.tile_row_begin[t + 1])
        for b in range(B):
            xa = None if inp.x_aud is None else inp.x_aud[b]
            if identity:
                y, ya = x_tiles[b, r0:r1].astype(np.float64), xa
            else:
                y, ya = tile_forward(x_tiles[b, r0:r1], p.row_pos[r0:r1], xa,
                                     inp.wq, inp.wk, inp.wv, inp.wo,
                                     wl.heads, wl.head_dim, rope_base)
            y_tiles[b, r0:r1] = y
            if ya is not None:
                y_aud_tiles[t, b] = ya
    y_global = blend_tiles(y_tiles, p)
    y_aud = None if y_aud_tiles is None else audio_mean(y_aud_tiles, p.n_tiles_total)
    return StepResult(p, x_tiles, y_tiles, y_global, y_aud_tiles, y_aud)
