"""Oracle per-tile denoiser: QKV projection, 3D RoPE, softmax attention, output
projection.  Float64 throughout.

Test infrastructure (see the package docstring).

TDP page, "What it is": each rank applies the whole denoising network to the
tiles it holds; "When to use it": the cost of self-attention grows with the
square of a tile's token count, and that is where the time goes.  The pages do
not describe the transformer, so the denoiser here is one multi-head
self-attention layer (a reading): no bias, no norm, no residual, scale
1/sqrt(d), bidirectional, no mask.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

F64 = np.float64


def rope_angles(pos: np.ndarray, head_dim: int, base: float = 10000.0) -> np.ndarray:
    """Rotation angle of every (row, pair) for 3D RoPE; float64 ``[n][d/2]``.

    TDP page, "Position normalization": RoPE sees each tile's normalized
    position grid; the page does not give the RoPE layout.  Reading used: a
    head of size d has d/2 interleaved pairs (2i, 2i+1); with p = floor(d/6)
    pairs per axis, pairs [0, p) rotate with the time position, [p, 2p) with
    height, [2p, 3p) with width, and the rest are not rotated.  Pair j of an
    axis has frequency ``base**(-j/p)``; the position of a row on an axis is the
    midpoint (start + end) / 2 of its [start, end) interval, so both ends of
    the (normalized) interval count.
    """
    pos = np.asarray(pos, dtype=F64)
    n = pos.shape[0]
    half = head_dim // 2
    p = head_dim // 6
    ang = np.zeros((n, half), dtype=F64)
    mid = (pos[:, :, 0] + pos[:, :, 1]) / 2.0          # [n][3]
    for axis in range(3):
        for j in range(p):
            theta = base ** (-j / p)
            ang[:, axis * p + j] = mid[:, axis] * theta
    return ang


def apply_rope(x: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Rotate interleaved pairs: (x0, x1) -> (x0 cos - x1 sin, x0 sin + x1 cos)."""
    x = np.asarray(x, dtype=F64)
    c, s = np.cos(angles), np.sin(angles)
    x0, x1 = x[:, 0::2], x[:, 1::2]
    out = np.empty_like(x)
    out[:, 0::2] = x0 * c - x1 * s
    out[:, 1::2] = x0 * s + x1 * c
    return out


def _softmax_rows(logits: np.ndarray) -> np.ndarray:
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    return e / e.sum(axis=1, keepdims=True)


def tile_forward(x_tile: np.ndarray, pos: np.ndarray, x_aud: Optional[np.ndarray],
                 wq, wk, wv, wo, heads: int, head_dim: int, base: float = 10000.0,
                 query_rows: Optional[np.ndarray] = None,
                 audio_query_rows: Optional[np.ndarray] = None,
                 chunk: int = 2048):
    """One tile's (and one batch entry's) denoiser forward.

    The sequence is the tile's rows followed by the audio tokens, if any.
    TDP page, "What it is": the audio stream is not cut into tiles; it enters
    each tile's forward pass.
    Reading used: the audio tokens join each tile's self-attention as queries
    and as keys/values, with no rotation (they have no grid position).

    ``query_rows`` / ``audio_query_rows`` restrict the queries evaluated (all
    keys are always used); defaults are all tile rows / all audio rows.
    Returns ``(y_tile [q][C], y_aud [qa][C] or None)`` in float64.
    """
    x_tile = np.asarray(x_tile, dtype=F64)
    n = x_tile.shape[0]
    seq = x_tile
    n_aud = 0
    if x_aud is not None:
        seq = np.concatenate([x_tile, np.asarray(x_aud, dtype=F64)], axis=0)
        n_aud = x_aud.shape[0]
    if query_rows is None:
        query_rows = np.arange(n)
    if audio_query_rows is None:
        audio_query_rows = np.arange(n_aud)
    qidx = np.concatenate([np.asarray(query_rows, dtype=np.int64),
                           n + np.asarray(audio_query_rows, dtype=np.int64)])
    wq, wk, wv, wo = (np.asarray(w, dtype=F64) for w in (wq, wk, wv, wo))
    d = head_dim
    ang = rope_angles(pos, d, base)                      # tile rows only
    ang_all = np.concatenate([ang, np.zeros((n_aud, d // 2))], axis=0)

    q = seq[qidx] @ wq
    k = seq @ wk
    v = seq @ wv
    out = np.zeros((qidx.size, heads * d), dtype=F64)
    scale = 1.0 / np.sqrt(d)
    for h in range(heads):
        cols = slice(h * d, (h + 1) * d)
        qh = apply_rope(q[:, cols], ang_all[qidx])
        kh = apply_rope(k[:, cols], ang_all)
        vh = v[:, cols]
        for r0 in range(0, qidx.size, chunk):
            r1 = min(qidx.size, r0 + chunk)
            prob = _softmax_rows((qh[r0:r1] @ kh.T) * scale)
            out[r0:r1, cols] = prob @ vh
    y = out @ wo
    nq = len(query_rows)
    return y[:nq], (y[nq:] if x_aud is not None else None)
