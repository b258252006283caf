"""Oracle of the TDP upscale loop: re-noise, TDP velocity per step, Euler
update, and the seam spread of the tiles.  Float64 throughout.

Test infrastructure (see the package docstring).

TDP page, "When to use it" (the warning on stages): TDP is run as the upscale
stage, on a latent that a faithful full-frame first stage produced, not from
pure noise; the upscale stage re-injects noise up to its first sigma; tiles
drift apart more the larger that first sigma is, and conditioning on the
stage-1 result at negative time indices (or a smaller first sigma) keeps them
consistent.  The page names no sampler and no drift measure.  Readings used
(flow-matching form, the plainest one the page's "sigma" supports):

  U1  noise level sigma in [0, 1]; a latent at sigma is (1 - sigma) x0 +
      sigma eps; the tile transformer's blended output is the velocity
      v = eps - x0.
  U2  re-noise: x = (1 - sigma_0) x_stage1 + sigma_0 eps on the generated
      rows; the conditioning rows hold the clean stage-1 tokens and are never
      changed.
  U3  one step: x <- x + (sigma_{i+1} - sigma_i) v(x, sigma_i) on the
      generated rows (explicit Euler), v being the TDP step's blend of the
      tile outputs (gather, per-tile transformer, blend).
  U4  schedule: sigma_i = sigma_0 (1 - i / S), i = 0..S, rounded to float32.
  U5  the transformer's timestep is tau = 1000 sigma.
  U6  seam spread of a step: over the batch entries and the generated tokens
      that two or more tiles cover, S2 = sum over those tiles' rows r of
      w_r |y_r - ybar|^2 and S0 = sum |ybar|^2, ybar = sum_r w_r y_r being the
      blended output; the relative spread is sqrt(S2 / S0).  It is zero when
      every tile predicts the same values where tiles overlap.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, List, Optional, Tuple

import numpy as np

from .blend import blend_tiles, gather_tiles
from .tile_plan import Plan

F64 = np.float64

TAU_PER_SIGMA = 1000.0


def linear_sigmas(sigma0: float, n_steps: int) -> np.ndarray:
    """The schedule of U4: ``S + 1`` float32 values from sigma_0 down to 0
    (``[sigma_0]`` alone for S = 0)."""
    s0 = F64(np.float32(sigma0))
    if n_steps < 0 or not (0.0 <= s0 <= 1.0):
        raise ValueError("need n_steps >= 0 and 0 <= sigma0 <= 1")
    if n_steps == 0:
        return np.array([s0], dtype=np.float32)
    i = np.arange(n_steps + 1, dtype=F64)
    return (s0 * (1.0 - i / n_steps)).astype(np.float32)


def renoise(x_stage1: np.ndarray, noise: np.ndarray, sigma0: float, n_gen: int) -> np.ndarray:
    """U2: ``(1 - sigma_0) x_stage1 + sigma_0 eps`` on generated rows ``[0, n_gen)``;
    conditioning rows copied.  ``x_stage1 [B][N+M][C]``, ``noise [B][N][C]``."""
    x = np.array(x_stage1, dtype=F64, copy=True)
    s = F64(sigma0)
    x[:, :n_gen] = (1.0 - s) * x[:, :n_gen] + s * np.asarray(noise, dtype=F64)
    return x


def euler_step(x: np.ndarray, v: np.ndarray, sigma: float, sigma_next: float,
               n_gen: int) -> np.ndarray:
    """U3: ``x + (sigma_next - sigma) v`` on the generated rows only."""
    out = np.array(x, dtype=F64, copy=True)
    out[:, :n_gen] += (F64(sigma_next) - F64(sigma)) * np.asarray(v, dtype=F64)[:, :n_gen]
    return out


def seam_spread(y_tiles: np.ndarray, p: Plan, n_gen: int) -> Tuple[float, float]:
    """U6: ``(S2, S0)`` of one step's tile outputs ``y_tiles [B][rows][C]``."""
    y = np.asarray(y_tiles, dtype=F64)
    ybar = blend_tiles(y, p)
    w = p.row_weight.astype(F64)
    covered = np.bincount(p.row_src, minlength=p.n_dst_rows)
    rows = np.nonzero((p.row_src < n_gen) & (covered[p.row_src] >= 2))[0]
    d = y[:, rows] - ybar[:, p.row_src[rows]]
    s2 = float((w[rows][None, :, None] * d * d).sum())
    toks = np.nonzero(covered[:n_gen] >= 2)[0]
    s0 = float((ybar[:, toks] ** 2).sum())
    return s2, s0


def relative_spread(s2: float, s0: float) -> float:
    return float(np.sqrt(s2 / s0)) if s0 > 0 else 0.0


# A velocity field: (x [B][N+M][C], sigma) -> (v [B][N+M][C], (S2, S0) or None).
Velocity = Callable[[np.ndarray, float], Tuple[np.ndarray, Optional[Tuple[float, float]]]]


def tdp_velocity(binp, p: Plan) -> Velocity:
    """U3's velocity: gather, the per-tile transformer of every tile and batch
    entry at tau = 1000 sigma (``block.tile_transformer``), blend; with the
    step's seam spread."""
    from .block import model_from_inputs, tile_transformer

    model = model_from_inputs(binp)
    n_gen = int(np.prod(binp.base.workload.grid))

    def velocity(x, sigma):
        x_tiles = gather_tiles(x, p)
        y = np.zeros(x_tiles.shape, dtype=F64)
        tau = TAU_PER_SIGMA * F64(sigma)
        for t in range(p.tile_id.size):
            r0, r1 = int(p.tile_row_begin[t]), int(p.tile_row_begin[t + 1])
            for b in range(x_tiles.shape[0]):
                y[b, r0:r1] = tile_transformer(x_tiles[b, r0:r1], p.row_pos[r0:r1],
                                               binp.text[b], tau, model)
        return blend_tiles(y, p), seam_spread(y, p, n_gen)

    return velocity


@dataclasses.dataclass
class LoopResult:
    x: np.ndarray                  # the latent after the last step, [B][N+M][C]
    seam: List[Tuple[float, float]]   # (S2, S0) of every step that reported one
    states: List[np.ndarray]       # the latent before each step, then the result


def upscale_loop(x_stage1: np.ndarray, noise: np.ndarray, sigmas: np.ndarray, n_gen: int,
                 velocity: Velocity) -> LoopResult:
    """Re-noise to ``sigmas[0]`` (U2), then one Euler step (U3) per consecutive
    pair of ``sigmas``."""
    sig = np.asarray(sigmas, dtype=np.float32)
    x = renoise(x_stage1, noise, sig[0], n_gen)
    states, seam = [x], []
    for i in range(sig.size - 1):
        v, s = velocity(x, F64(sig[i]))
        if s is not None:
            seam.append(s)
        x = euler_step(x, v, sig[i], sig[i + 1], n_gen)
        states.append(x)
    return LoopResult(x, seam, states)
