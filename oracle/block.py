"""Oracle transformer block per tile (the whole network a rank applies).

Test infrastructure (see the package docstring).  Float64 throughout.

TDP page, "What it is": each rank applies the whole denoising network to the
tiles it holds.  The pages describe neither the transformer nor its block, so the
block here is a reading, the diffusion-transformer layout with one shared
timestep modulation ("AdaLN-single"), written out step by step:

  h = rms_norm(x) * (1 + scale_a) + shift_a;  x = x + gate_a * self_attn(h)
  h = rms_norm(x);                            x = x + cross_attn(h, text)
  h = rms_norm(x) * (1 + scale_f) + shift_f;  x = x + gate_f * ffn(h)

with x the tile's residual stream of width D = heads * head_dim.  self_attn is
the hot path's attention layer (QKV projection, 3D RoPE on the tile's
normalized positions, softmax attention, output projection; see denoise.py).
Around L such blocks: x_0 = X_t W_in (latent channels C -> D) and
y_t = rms_norm(x_L) W_out (D -> C).  No linear layer has a bias.
"""
from __future__ import annotations

import dataclasses
from typing import List

import numpy as np

from .denoise import tile_forward

F64 = np.float64
RMS_EPS = 1e-6
TIME_DIM = 256          # sinusoidal timestep embedding width
FFN_MULT = 4            # FFN hidden width = FFN_MULT * D


def rms_norm(x: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """x / sqrt(mean over the feature axis of x^2 + eps), no affine weight."""
    x = np.asarray(x, dtype=F64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def gelu_tanh(u: np.ndarray) -> np.ndarray:
    """The tanh form of GELU: u/2 * (1 + tanh(sqrt(2/pi) * (u + 0.044715 u^3)))."""
    u = np.asarray(u, dtype=F64)
    return 0.5 * u * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (u + 0.044715 * u ** 3)))


def silu(u: np.ndarray) -> np.ndarray:
    u = np.asarray(u, dtype=F64)
    return u / (1.0 + np.exp(-u))


def timestep_embedding(tau: float, dim: int = TIME_DIM) -> np.ndarray:
    """[cos(tau w_i) for i < dim/2] followed by [sin(tau w_i)], w_i = 10000^(-i/(dim/2))."""
    half = dim // 2
    w = 10000.0 ** (-np.arange(half, dtype=F64) / half)
    return np.concatenate([np.cos(tau * w), np.sin(tau * w)])


def modulation(tau: float, wt1: np.ndarray, wt2: np.ndarray, table: np.ndarray) -> np.ndarray:
    """The six modulation vectors of one layer for one batch entry, [6][D].

    E = silu(emb(tau) Wt1) Wt2 (shared by all layers), reshaped [6][D], plus the
    layer's own table [6][D].  Rows: shift_a, scale_a, gate_a, shift_f,
    scale_f, gate_f.
    """
    e = silu(timestep_embedding(tau, np.asarray(wt1).shape[0]) @ np.asarray(wt1, dtype=F64))
    e = e @ np.asarray(wt2, dtype=F64)
    return e.reshape(6, -1) + np.asarray(table, dtype=F64)


def cross_attn(h: np.ndarray, text: np.ndarray, wq, wk, wv, wo, heads: int,
               head_dim: int) -> np.ndarray:
    """Softmax attention of the tile rows (queries) over the text tokens.

    Q = h Wq, K = text Wk, V = text Wv, per head softmax(Q K^T / sqrt(d)) V,
    then Wo.  No rotation, no mask: every tile sees every text token.
    """
    h = np.asarray(h, dtype=F64)
    text = np.asarray(text, dtype=F64)
    q = h @ np.asarray(wq, dtype=F64)
    k = text @ np.asarray(wk, dtype=F64)
    v = text @ np.asarray(wv, dtype=F64)
    d = head_dim
    out = np.zeros((h.shape[0], heads * d), dtype=F64)
    for hd in range(heads):
        cols = slice(hd * d, (hd + 1) * d)
        logits = (q[:, cols] @ k[:, cols].T) / np.sqrt(d)
        logits -= logits.max(axis=1, keepdims=True)
        p = np.exp(logits)
        p /= p.sum(axis=1, keepdims=True)
        out[:, cols] = p @ v[:, cols]
    return out @ np.asarray(wo, dtype=F64)


def ffn(h: np.ndarray, w1, w2) -> np.ndarray:
    """gelu_tanh(h W1) W2."""
    return gelu_tanh(np.asarray(h, dtype=F64) @ np.asarray(w1, dtype=F64)) @ np.asarray(w2, dtype=F64)


@dataclasses.dataclass
class Layer:
    """Weights of one block, [in][out] each."""
    wq: np.ndarray
    wk: np.ndarray
    wv: np.ndarray
    wo: np.ndarray
    cq: np.ndarray
    ck: np.ndarray
    cv: np.ndarray
    co: np.ndarray
    w1: np.ndarray
    w2: np.ndarray
    table: np.ndarray     # [6][D]


@dataclasses.dataclass
class Model:
    """Weights of the per-tile transformer."""
    w_in: np.ndarray      # [C][D]
    w_out: np.ndarray     # [D][C]
    wt1: np.ndarray       # [TIME_DIM][D]
    wt2: np.ndarray       # [D][6 D]
    layers: List[Layer]
    heads: int
    head_dim: int


def block_forward(x: np.ndarray, pos: np.ndarray, text: np.ndarray, mod: np.ndarray,
                  lay: Layer, heads: int, head_dim: int, query_rows=None) -> np.ndarray:
    """One block on one tile's residual stream x [n][D]; mod [6][D].

    ``query_rows`` restricts the rows returned (all rows still give keys and
    values to the self-attention); default all rows.
    """
    x = np.asarray(x, dtype=F64)
    shift_a, scale_a, gate_a, shift_f, scale_f, gate_f = mod
    h = rms_norm(x) * (1.0 + scale_a) + shift_a
    a, _ = tile_forward(h, pos, None, lay.wq, lay.wk, lay.wv, lay.wo, heads, head_dim,
                        query_rows=query_rows)
    if query_rows is not None:
        x = x[np.asarray(query_rows)]
    x = x + gate_a * a
    x = x + cross_attn(rms_norm(x), text, lay.cq, lay.ck, lay.cv, lay.co, heads, head_dim)
    h = rms_norm(x) * (1.0 + scale_f) + shift_f
    return x + gate_f * ffn(h, lay.w1, lay.w2)


def tile_transformer(x_tile: np.ndarray, pos: np.ndarray, text: np.ndarray, tau: float,
                     model: Model, query_rows=None) -> np.ndarray:
    """The per-tile transformer for one batch entry: [n][C] -> [n][C].

    ``query_rows`` (models of at most one layer) evaluates only those rows.
    """
    x = np.asarray(x_tile, dtype=F64) @ np.asarray(model.w_in, dtype=F64)
    if query_rows is not None and len(model.layers) > 1:
        raise ValueError("query_rows needs every row of the earlier layers")
    for lay in model.layers:
        mod = modulation(tau, model.wt1, model.wt2, lay.table)
        x = block_forward(x, pos, text, mod, lay, model.heads, model.head_dim, query_rows)
    if query_rows is not None and not model.layers:
        x = x[np.asarray(query_rows)]
    return rms_norm(x) @ np.asarray(model.w_out, dtype=F64)


def model_from_inputs(binp) -> Model:
    """The oracle's Model from a ``tdp_inputs.BlockInputs``."""
    wl = binp.base.workload
    layers = [Layer(**lay) for lay in binp.layers]
    return Model(binp.w_in, binp.w_out, binp.wt1, binp.wt2, layers, wl.heads, wl.head_dim)


def block_step(binp, normalize_positions: bool = True, world_size: int = 1, rank: int = 0):
    """One TDP step whose tile denoiser is the per-tile transformer.

    Same plan, gather and blend as ``tdp_step.step`` (TDP page, "What it
    is"); every tile of every batch entry runs ``tile_transformer`` with that
    entry's text tokens and timestep.  Block workloads have no audio.
    Returns a ``tdp_step.StepResult``.
    """
    from .blend import blend_tiles, gather_tiles
    from .tdp_step import StepResult
    from .tile_plan import plan as make_plan

    inp = binp.base
    wl = inp.workload
    if inp.x_aud is not None:
        raise ValueError("block workloads have no audio")
    p = make_plan(wl.grid, wl.tiling, inp.cond_pos, normalize_positions, world_size, rank)
    x_tiles = gather_tiles(inp.x_global, p)
    model = model_from_inputs(binp)
    y_tiles = np.zeros(x_tiles.shape, dtype=F64)
    for t in range(p.tile_id.size):
        r0, r1 = int(p.tile_row_begin[t]), int(p.tile_row_begin[t + 1])
        for b in range(x_tiles.shape[0]):
            y_tiles[b, r0:r1] = tile_transformer(x_tiles[b, r0:r1], p.row_pos[r0:r1],
                                                 binp.text[b], float(binp.tau[b]), model)
    return StepResult(p, x_tiles, y_tiles, blend_tiles(y_tiles, p), None, None)
