"""Oracle of sequence parallelism (SP) for the first stage: the token
partition, the head exchange and its inverse, and the layer computed the SP
way.  Float64 for the arithmetic; the exchanges are plain copies.

Test infrastructure (see the package docstring).

The LTX-2 sequence-parallel guide (page 4: the section on how one denoising
step is split, and the section on the all2all kernel) describes SP as:
  * pad the video token dimension to a multiple of the world size W, with a
    key-only padding mask (padded tokens are never attended to; padded query
    rows attend to every valid key, and their outputs are cut off);
  * give rank r an equal contiguous slice of the padded tokens;
  * before self-attention, an all2all exchanges heads: afterwards every rank
    holds every token for H/W of the heads, attends over all tokens locally,
    and a second exchange returns each token slice's outputs for all heads;
  * gather the output tokens from all ranks and drop the padding.
The exchanges only move bytes, so gather(send(x)) == x exactly, and the
result is the single-GPU layer up to the order of floating-point sums.
Readings used (the page gives no more detail):
  SP1  rank r holds padded tokens [r T_pad / W, (r + 1) T_pad / W); rank s
       receives heads [s H / W, (s + 1) H / W); after the exchange the tokens
       are in global order (source rank, then position).
  SP2  the layer is the hot path's attention layer (QKV projection, 3D RoPE,
       softmax attention, output projection), per token slice outside the
       attention; the output projection of a token uses all heads.
"""
from __future__ import annotations

import numpy as np

from .denoise import apply_rope, rope_angles

F64 = np.float64


def padded_tokens(n_tokens: int, world: int) -> int:
    """T_pad: the smallest multiple of ``world`` that is >= n_tokens."""
    if n_tokens < 1 or world < 1:
        raise ValueError("need n_tokens >= 1 and world >= 1")
    return -(-n_tokens // world) * world


def send_heads(x_local: np.ndarray, rank: int, world: int, t_pad: int, dst: list) -> None:
    """Rank ``rank``'s part of the exchange: its token slice ``x_local``
    ``[t_loc][H][d]`` goes to ``dst[s]`` ``[t_pad][H/W][d]`` at tokens
    ``[rank t_loc, (rank + 1) t_loc)`` for the heads of rank s (SP1)."""
    t_loc, heads, d = x_local.shape
    if heads % world or t_loc * world != t_pad:
        raise ValueError("heads must divide by world and t_loc * world == t_pad")
    hw = heads // world
    for s in range(world):
        dst[s][rank * t_loc:(rank + 1) * t_loc] = x_local[:, s * hw:(s + 1) * hw]


def gather_heads(src: list, rank: int, world: int, t_loc: int) -> np.ndarray:
    """The inverse exchange for rank ``rank``: its tokens
    ``[rank t_loc, (rank + 1) t_loc)`` from every rank's ``[t_pad][H/W][d]``
    buffer, heads in order -> ``[t_loc][H][d]``."""
    return np.concatenate([src[s][rank * t_loc:(rank + 1) * t_loc] for s in range(world)],
                          axis=1)


def _softmax_masked(logits: np.ndarray, n_valid: int) -> np.ndarray:
    z = logits[:, :n_valid]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    p = np.zeros_like(logits)
    p[:, :n_valid] = e / e.sum(axis=1, keepdims=True)
    return p


def sp_layer(x: np.ndarray, pos: np.ndarray, wq, wk, wv, wo, heads: int, head_dim: int,
             world: int, rope_base: float = 10000.0) -> np.ndarray:
    """The attention layer computed the SP way on ``world`` emulated ranks:
    ``x [T][C]``, ``pos [T][3][2]`` -> ``y [T][C]`` (float64)."""
    x = np.asarray(x, dtype=F64)
    T, _ = x.shape
    t_pad = padded_tokens(T, world)
    t_loc = t_pad // world
    hw = heads // world
    if heads % world:
        raise ValueError("heads must divide by world")
    # pad: zero rows at the end, positions repeated from the last token (any
    # value does: padded keys are masked and padded outputs dropped)
    xp = np.zeros((t_pad, x.shape[1]), dtype=F64)
    xp[:T] = x
    pp = np.zeros((t_pad,) + pos.shape[1:], dtype=F64)
    pp[:T] = pos
    pp[T:] = pos[T - 1]
    ang = rope_angles(pp, head_dim, rope_base)
    # per rank: projection of its own tokens, all heads
    qkv = []
    for r in range(world):
        sl = slice(r * t_loc, (r + 1) * t_loc)
        q = (xp[sl] @ np.asarray(wq, F64)).reshape(t_loc, heads, head_dim)
        k = (xp[sl] @ np.asarray(wk, F64)).reshape(t_loc, heads, head_dim)
        v = (xp[sl] @ np.asarray(wv, F64)).reshape(t_loc, heads, head_dim)
        for h in range(heads):
            q[:, h] = apply_rope(q[:, h], ang[sl])
            k[:, h] = apply_rope(k[:, h], ang[sl])
        qkv.append((q, k, v))
    # exchange: every rank gets all tokens of its heads
    bufs = {n: [np.zeros((t_pad, hw, head_dim)) for _ in range(world)] for n in "qkv"}
    for r in range(world):
        for n, a in zip("qkv", qkv[r]):
            send_heads(a, r, world, t_pad, bufs[n])
    # local attention over all tokens for the rank's heads, padded keys masked
    outs = [np.zeros((t_pad, hw, head_dim)) for _ in range(world)]
    for s in range(world):
        for h in range(hw):
            q, k, v = bufs["q"][s][:, h], bufs["k"][s][:, h], bufs["v"][s][:, h]
            p = _softmax_masked(q @ k.T / np.sqrt(head_dim), T)
            outs[s][:, h] = p @ v
    # inverse exchange, output projection per token slice, gather, unpad
    y = np.zeros((t_pad, np.asarray(wo).shape[1]))
    for r in range(world):
        o = gather_heads(outs, r, world, t_loc).reshape(t_loc, heads * head_dim)
        y[r * t_loc:(r + 1) * t_loc] = o @ np.asarray(wo, F64)
    return y[:T]


def head_share(heads: int, world: int, rank: int) -> slice:
    """Heads of rank ``rank`` after the exchange (SP1)."""
    hw = heads // world
    return slice(rank * hw, (rank + 1) * hw)
