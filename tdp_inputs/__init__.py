"""Seeded synthetic workloads for one Tiled Data Parallelism (TDP) upscale step.

This module is shared by the CPU oracle, the tests, the smoke check and the
benchmark.  It holds no arithmetic of the method itself: it only names the five
workloads and draws their random inputs.  Nothing here tiles, normalizes, keeps,
attends or blends.

The workloads stand in for the shapes that the TDP design page ("Tiled Data
Parallelism (TDP)", sections "What it is" and "Usage") describes: a patchified
(frames, height, width) latent, counts of tiles per dimension with an overlap in
latent units, conditioning tokens with [start, end) intervals of which some sit
at negative time, and an untiled audio stream.  The pages measure no public
dataset; these synthetic arrays replace real latents and trained weights.

Draw order per workload (``numpy.random.default_rng(seed)``):
  1. ``x_global [B][N+M][C]``  ~ N(0, 1)
  2. ``cond_pos [M][3][2]``    (see ``draw_cond_pos``)
  3. ``wq, wk, wv [C][hidden]`` ~ N(0, 1/sqrt(C))
  4. ``wo [hidden][C]``         ~ N(0, 1/sqrt(hidden))
  5. ``x_aud [B][A][C]``        ~ N(0, 1)
Arrays of a bf16 workload are rounded once to bf16 values (round to nearest,
ties to even) and kept as float32 arrays holding those values.  The weights
are always rounded to bf16: the attention consumes bf16 weights.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "workload", "Inputs", "make_inputs",
           "round_to_bf16", "draw_cond_pos", "BlockWorkload", "BLOCK_WORKLOADS",
           "UpscaleWorkload", "UPSCALE_WORKLOADS", "UpscaleInputs", "make_upscale_inputs",
           "BlockInputs", "make_block_inputs"]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic TDP step: geometry, tiling, denoiser shape and dtype."""
    name: str
    grid: tuple            # (F, H, W) patchified latent grid
    tiling: tuple          # ((n_f, o_f), (n_h, o_h), (n_w, o_w)) tile counts and overlaps
    batch: int
    channels: int          # C, channels per latent token
    heads: int
    head_dim: int
    n_cond: int            # M conditioning tokens appended after the N generated ones
    n_cond_neg: int        # how many of them (the last ones) sit at negative time
    n_audio: int           # A untiled audio tokens attended on every tile forward
    latent_dtype: str      # "f32" or "bf16"
    identity: bool         # identity denoiser (blend stress) instead of attention
    seed: int

    @property
    def n_gen(self) -> int:
        f, h, w = self.grid
        return f * h * w

    @property
    def hidden(self) -> int:
        return self.heads * self.head_dim

    @property
    def n_tiles(self) -> int:
        n = 1
        for c, _ in self.tiling:
            n *= c
        return n


# The workloads.  Sizes follow the TDP page's examples: 16 tiles (as in the
# "16 tiles on 4 GPUs" example), 2D H x W grids with an overlap in latent units,
# negative-time reference tokens, and an untiled audio stream.
WORKLOADS = {
    "tiny_2x16x16": Workload(
        "tiny_2x16x16", grid=(2, 16, 16), tiling=((1, 0), (2, 4), (2, 4)), batch=1,
        channels=128, heads=2, head_dim=64, n_cond=8, n_cond_neg=2, n_audio=0,
        latent_dtype="f32", identity=False, seed=0),
    "d64_8x32x32": Workload(
        "d64_8x32x32", grid=(8, 32, 32), tiling=((1, 0), (2, 8), (2, 8)), batch=1,
        channels=128, heads=32, head_dim=64, n_cond=16, n_cond_neg=4, n_audio=0,
        latent_dtype="bf16", identity=False, seed=1),
    "t16_16x64x64": Workload(
        "t16_16x64x64", grid=(16, 64, 64), tiling=((1, 0), (4, 8), (4, 8)), batch=1,
        channels=128, heads=32, head_dim=128, n_cond=0, n_cond_neg=0, n_audio=0,
        latent_dtype="bf16", identity=False, seed=2),
    "audio_32x48x80": Workload(
        "audio_32x48x80", grid=(32, 48, 80), tiling=((2, 4), (3, 8), (4, 8)), batch=2,
        channels=128, heads=16, head_dim=128, n_cond=64, n_cond_neg=16, n_audio=256,
        latent_dtype="bf16", identity=False, seed=3),
    "blend_32x96x160": Workload(
        "blend_32x96x160", grid=(32, 96, 160), tiling=((1, 0), (6, 16), (10, 16)), batch=1,
        channels=128, heads=0, head_dim=0, n_cond=0, n_cond_neg=0, n_audio=0,
        latent_dtype="f32", identity=True, seed=4),
    # Sequence parallelism for the first stage: the whole latent is one
    # sequence (a 1x1x1 "tiling"), its heads split over the ranks.  The
    # 16x16x24 grid is the 6144-token first-stage latent of the sequence-
    # parallel guide's table (512 x 768 pixels, 121 frames).
    "sp_small": Workload(
        "sp_small", grid=(2, 6, 10), tiling=((1, 0), (1, 0), (1, 0)), batch=1,
        channels=128, heads=8, head_dim=64, n_cond=0, n_cond_neg=0, n_audio=0,
        latent_dtype="bf16", identity=False, seed=5),
    "sp_16x16x24": Workload(
        "sp_16x16x24", grid=(16, 16, 24), tiling=((1, 0), (1, 0), (1, 0)), batch=1,
        channels=128, heads=32, head_dim=128, n_cond=0, n_cond_neg=0, n_audio=0,
        latent_dtype="bf16", identity=False, seed=6),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even).

    Returns float32 values that are exactly representable in bf16.  NaN/Inf do
    not occur in these synthetic inputs.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def draw_cond_pos(rng: np.random.Generator, grid, n_cond: int, n_neg: int) -> np.ndarray:
    """Conditioning token intervals ``[M][3][2]`` (start, end) in latent units.

    Non-negative tokens: per dim, start ~ U{0..L-1}, width ~ U{1..4} (time:
    U{1..2}), end = min(start + width, L).  The last ``n_neg`` tokens are
    negative-time reference tokens: time start ~ U{-4..-1}, end = start + 1,
    spatial dims drawn as above.
    """
    pos = np.zeros((n_cond, 3, 2), dtype=np.float32)
    for j in range(n_cond):
        for d in range(3):
            L = grid[d]
            s = int(rng.integers(0, L))
            wmax = 2 if d == 0 else 4
            width = int(rng.integers(1, wmax + 1))
            e = min(s + width, L)
            pos[j, d] = (s, e)
        if j >= n_cond - n_neg:
            s = int(rng.integers(-4, 0))
            pos[j, 0] = (s, s + 1)
    return pos


@dataclasses.dataclass
class Inputs:
    workload: Workload
    x_global: np.ndarray              # [B][N+M][C] float32 (bf16 values for bf16 workloads)
    cond_pos: np.ndarray              # [M][3][2] float32
    wq: Optional[np.ndarray]          # [C][hidden] float32 holding bf16 values
    wk: Optional[np.ndarray]
    wv: Optional[np.ndarray]
    wo: Optional[np.ndarray]          # [hidden][C]
    x_aud: Optional[np.ndarray]       # [B][A][C] or None


def make_inputs(wl: Workload | str, seed: Optional[int] = None) -> Inputs:
    """Draw the seeded inputs of a workload (seed defaults to the workload's)."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    B, C = wl.batch, wl.channels
    n_rows = wl.n_gen + wl.n_cond
    x = rng.standard_normal((B, n_rows, C), dtype=np.float32)
    if wl.latent_dtype == "bf16":
        x = round_to_bf16(x)
    cond = draw_cond_pos(rng, wl.grid, wl.n_cond, wl.n_cond_neg)
    wq = wk = wv = wo = xa = None
    if not wl.identity:
        hid = wl.hidden
        s_in = np.float32(1.0 / np.sqrt(C))
        s_out = np.float32(1.0 / np.sqrt(hid))
        wq = round_to_bf16(rng.standard_normal((C, hid), dtype=np.float32) * s_in)
        wk = round_to_bf16(rng.standard_normal((C, hid), dtype=np.float32) * s_in)
        wv = round_to_bf16(rng.standard_normal((C, hid), dtype=np.float32) * s_in)
        wo = round_to_bf16(rng.standard_normal((hid, C), dtype=np.float32) * s_out)
        if wl.n_audio > 0:
            xa = rng.standard_normal((B, wl.n_audio, C), dtype=np.float32)
            if wl.latent_dtype == "bf16":
                xa = round_to_bf16(xa)
    return Inputs(wl, x, cond, wq, wk, wv, wo, xa)



# ---------------------------------------------------------------------------
# The per-tile transformer block (the whole network each rank applies to its tiles)
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class BlockWorkload:
    """A TDP step whose tile denoiser is L transformer blocks of width
    D = heads * head_dim with text cross-attention and timestep modulation."""
    name: str
    base: str              # geometry, channels, heads and dtype from this workload
    layers: int
    n_text: int            # text tokens per batch entry, width D
    time_dim: int = 256    # timestep embedding width
    ffn_mult: int = 4
    heads: Optional[int] = None        # override the base workload's heads
    head_dim: Optional[int] = None

    def base_workload(self) -> Workload:
        wl = WORKLOADS[self.base]
        kw = {}
        if self.heads is not None:
            kw["heads"] = self.heads
        if self.head_dim is not None:
            kw["head_dim"] = self.head_dim
        if kw:
            wl = dataclasses.replace(wl, name=self.name, **kw)
        return wl


BLOCK_WORKLOADS = {
    # two blocks on the 4-tile 2x16x16 latent, D = 128: the oracle runs all of it
    "block_tiny": BlockWorkload("block_tiny", base="tiny_2x16x16", layers=2, n_text=16),
    # one block, head_dim 128, D = 256, bf16 latent with conditioning
    "block_d128": BlockWorkload("block_d128", base="d64_8x32x32", layers=1, n_text=24,
                                heads=2, head_dim=128),
    # one block at the 16-tile step's width (32 heads x 128 = 4096), 128 text tokens
    "block_t16": BlockWorkload("block_t16", base="t16_16x64x64", layers=1, n_text=128),
}


@dataclasses.dataclass
class BlockInputs:
    workload: BlockWorkload
    base: Inputs                      # latent, conditioning positions (no attention weights used)
    w_in: np.ndarray                  # [C][D]
    w_out: np.ndarray                 # [D][C]
    wt1: np.ndarray                   # [time_dim][D]
    wt2: np.ndarray                   # [D][6 D]
    layers: list                      # per layer: dict of wq wk wv wo cq ck cv co w1 w2 table
    text: np.ndarray                  # [B][n_text][D]
    tau: np.ndarray                   # [B] timesteps


def make_block_inputs(bw: BlockWorkload | str) -> BlockInputs:
    """Seeded inputs of a block workload.

    The latent and conditioning positions are those of ``make_inputs`` on the
    base workload.  The block's arrays come from a second generator,
    ``default_rng(seed + 1000)``, in this order: w_in [C][D]; w_out [D][C];
    wt1 [time_dim][D]; wt2 [D][6D]; then per layer wq, wk, wv, wo, cq, ck, cv,
    co [D][D], w1 [D][ffn D], w2 [ffn D][D], table [6][D]; text [B][n_text][D];
    tau [B].  Matrices are N(0, 1/sqrt(fan_in)), table N(0, 0.1), text
    N(0, 1), tau U(0, 1000).  Everything but tau is rounded once to bf16.
    """
    if isinstance(bw, str):
        bw = BLOCK_WORKLOADS[bw]
    wl = bw.base_workload()
    base = make_inputs(wl)
    rng = np.random.default_rng(wl.seed + 1000)
    C, D, B = wl.channels, wl.hidden, wl.batch
    F = bw.ffn_mult * D

    def mat(fan_in, fan_out):
        a = rng.standard_normal((fan_in, fan_out), dtype=np.float32)
        return round_to_bf16(a * np.float32(1.0 / np.sqrt(fan_in)))

    w_in = mat(C, D)
    w_out = mat(D, C)
    wt1 = mat(bw.time_dim, D)
    wt2 = mat(D, 6 * D)
    layers = []
    for _ in range(bw.layers):
        lay = {k: mat(D, D) for k in ("wq", "wk", "wv", "wo", "cq", "ck", "cv", "co")}
        lay["w1"] = mat(D, F)
        lay["w2"] = mat(F, D)
        lay["table"] = round_to_bf16(rng.standard_normal((6, D), dtype=np.float32)
                                     * np.float32(0.1))
        layers.append(lay)
    text = round_to_bf16(rng.standard_normal((B, bw.n_text, D), dtype=np.float32))
    tau = rng.uniform(0.0, 1000.0, size=B).astype(np.float32)
    return BlockInputs(bw, base, w_in, w_out, wt1, wt2, layers, text, tau)


# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class UpscaleWorkload:
    """The TDP upscale loop: a block workload's latent, taken as the clean
    stage-1 result at the target grid, re-noised to ``sigma0`` and denoised in
    ``n_steps`` steps."""
    name: str
    block: str             # a BLOCK_WORKLOADS name
    sigma0: float
    n_steps: int


UPSCALE_WORKLOADS = {
    # three steps from sigma 0.5 on the 4-tile 2x16x16 latent (with negative-time
    # conditioning): the oracle runs all of it
    "upscale_tiny": UpscaleWorkload("upscale_tiny", block="block_tiny", sigma0=0.5, n_steps=3),
    # two steps from sigma 0.3, D = 256
    "upscale_d128": UpscaleWorkload("upscale_d128", block="block_d128", sigma0=0.3, n_steps=2),
    # four steps from sigma 0.3 on the 16-tile step at D = 4096
    "upscale_t16": UpscaleWorkload("upscale_t16", block="block_t16", sigma0=0.3, n_steps=4),
}


@dataclasses.dataclass
class UpscaleInputs:
    workload: UpscaleWorkload
    block: BlockInputs                # weights, text; block.base.x_global is the stage-1 latent
    noise: np.ndarray                 # [B][N][C] float32, the re-injected noise


def make_upscale_inputs(uw: UpscaleWorkload | str) -> UpscaleInputs:
    """Seeded inputs of an upscale workload: the block workload's inputs and
    the noise, N(0, 1) float32 ``[B][N][C]`` from ``default_rng(seed + 2000)``
    (N generated tokens; conditioning rows get no noise)."""
    if isinstance(uw, str):
        uw = UPSCALE_WORKLOADS[uw]
    binp = make_block_inputs(uw.block)
    wl = binp.base.workload
    rng = np.random.default_rng(wl.seed + 2000)
    noise = rng.standard_normal((wl.batch, wl.n_gen, wl.channels), dtype=np.float32)
    return UpscaleInputs(uw, binp, noise)
