"""Pins for the oracle's per-tile denoiser (CPU only).

The oracle's attention is tied to: a pure-Python brute-force evaluation on tiny
inputs (complex-number RoPE, math.exp softmax), torch's scaled_dot_product_attention
on cases where RoPE cancels, closed forms (zero query weights give uniform
attention), and RoPE's own properties (norm preserving, relative, per-axis).
"""
import cmath
import math

import numpy as np
import pytest
import torch

import oracle
import tdp_inputs as ti

RNG = np.random.default_rng(1234)


def _rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def _brute_forward(x, pos, xa, wq, wk, wv, wo, heads, d, base=10000.0):
    """Pure-Python evaluation: lists, complex rotation, math.exp softmax."""
    seq = [list(r) for r in x] + ([list(r) for r in xa] if xa is not None else [])
    n_tile = len(x)
    C = len(seq[0])
    hid = heads * d
    p = d // 6

    def mat(rows, w):
        return [[sum(r[c] * w[c][o] for c in range(C)) for o in range(hid)] for r in rows]

    def rot(vec, i):
        if i >= n_tile:
            return vec
        out = list(vec)
        for pair in range(d // 2):
            axis = pair // p if p else 3
            if axis >= 3:
                continue
            j = pair % p
            mid = (pos[i][axis][0] + pos[i][axis][1]) / 2.0
            z = complex(vec[2 * pair], vec[2 * pair + 1]) * cmath.exp(1j * mid * base ** (-j / p))
            out[2 * pair], out[2 * pair + 1] = z.real, z.imag
        return out

    Q, K, V = mat(seq, wq), mat(seq, wk), mat(seq, wv)
    O = [[0.0] * hid for _ in seq]
    for h in range(heads):
        cs = slice(h * d, (h + 1) * d)
        qh = [rot(Q[i][cs], i) for i in range(len(seq))]
        kh = [rot(K[i][cs], i) for i in range(len(seq))]
        for i in range(len(seq)):
            logits = [sum(a * b for a, b in zip(qh[i], kh[j])) / math.sqrt(d) for j in range(len(seq))]
            m = max(logits)
            e = [math.exp(v - m) for v in logits]
            z = sum(e)
            for dd in range(d):
                O[i][h * d + dd] = sum(e[j] * V[j][h * d + dd] for j in range(len(seq))) / z
    Y = [[sum(O[i][k] * wo[k][c] for k in range(hid)) for c in range(C)] for i in range(len(seq))]
    return np.array(Y[:n_tile]), (np.array(Y[n_tile:]) if xa is not None else None)


@pytest.mark.parametrize("with_audio", [False, True])
@pytest.mark.parametrize("d", [6, 12, 14])
def test_attention_brute_force(with_audio, d):
    n, C, heads, A = 7, 5, 2, 3
    x = _rand(n, C)
    pos = RNG.integers(-3, 6, size=(n, 3, 1)).astype(np.float64)
    pos = np.concatenate([pos, pos + RNG.integers(1, 3, size=(n, 3, 1))], axis=2)
    xa = _rand(A, C) if with_audio else None
    w = [_rand(C, heads * d, scale=0.7) for _ in range(3)] + [_rand(heads * d, C, scale=0.5)]
    y, ya = oracle.tile_forward(x, pos, xa, *w, heads, d)
    yb, yab = _brute_forward(x, pos, xa, *w, heads, d)
    np.testing.assert_allclose(y, yb, rtol=1e-11, atol=1e-12)
    if with_audio:
        np.testing.assert_allclose(ya, yab, rtol=1e-11, atol=1e-12)
    # restricting the queries returns the same rows
    sel = np.array([5, 0, 3])
    ys, _ = oracle.tile_forward(x, pos, xa, *w, heads, d, query_rows=sel)
    np.testing.assert_allclose(ys, yb[sel], rtol=1e-11, atol=1e-12)


def test_large_logits_stable():
    n, C, heads, d = 6, 4, 1, 12
    x = _rand(n, C) * 30
    pos = np.zeros((n, 3, 2))
    pos[..., 1] = 1
    w = [_rand(C, d) for _ in range(3)] + [_rand(d, C)]
    y, _ = oracle.tile_forward(x, pos, None, *w, heads, d)
    yb, _ = _brute_forward(x, pos, None, *w, heads, d)
    assert np.all(np.isfinite(y))
    np.testing.assert_allclose(y, yb, rtol=1e-9, atol=1e-9)


def test_equal_positions_reduce_to_textbook_attention():
    """Equal positions rotate q and k alike, so q.k is unchanged: torch SDPA on the projections."""
    n, C, heads, d = 40, 16, 4, 64
    x = _rand(n, C)
    pos = np.tile(np.array([[3.0, 4.0], [7.0, 9.0], [2.0, 3.0]]), (n, 1, 1))
    w = [_rand(C, heads * d, scale=C ** -0.5) for _ in range(3)] + [_rand(heads * d, C)]
    y, _ = oracle.tile_forward(x, pos, None, *w, heads, d)
    X = torch.from_numpy(x)
    q, k, v = (X @ torch.from_numpy(wm) for wm in w[:3])
    sh = lambda t: t.view(n, heads, d).transpose(0, 1).contiguous()  # noqa: E731
    o = torch.nn.functional.scaled_dot_product_attention(sh(q), sh(k), sh(v))
    ref = o.transpose(0, 1).reshape(n, heads * d) @ torch.from_numpy(w[3])
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-10, atol=1e-11)


def test_zero_query_weights_give_uniform_attention():
    """Wq = 0: every logit is 0, so each output row is mean(V) Wo (closed form)."""
    n, C, heads, d, A = 23, 8, 3, 12, 4
    x, xa = _rand(n, C), _rand(A, C)
    pos = RNG.integers(0, 9, size=(n, 3, 1)).astype(float)
    pos = np.concatenate([pos, pos + 1], axis=2)
    wk, wv, wo = _rand(C, heads * d), _rand(C, heads * d), _rand(heads * d, C)
    y, ya = oracle.tile_forward(x, pos, xa, np.zeros((C, heads * d)), wk, wv, wo, heads, d)
    seq = np.concatenate([x, xa])
    want = (seq @ wv).mean(axis=0) @ wo
    np.testing.assert_allclose(y, np.broadcast_to(want, y.shape), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ya, np.broadcast_to(want, ya.shape), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("d", [64, 128])
def test_rope_matches_complex_rotation_and_keeps_norms(d):
    n = 50
    pos = RNG.uniform(-5, 40, size=(n, 3, 1))
    pos = np.concatenate([pos, pos + RNG.integers(1, 4, size=(n, 3, 1))], axis=2)
    ang = oracle.rope_angles(pos, d)
    x = _rand(n, d)
    y = oracle.apply_rope(x, ang)
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * ang)
    np.testing.assert_allclose(y[:, 0::2], z.real, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(y[:, 1::2], z.imag, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(np.hypot(y[:, 0::2], y[:, 1::2]), np.hypot(x[:, 0::2], x[:, 1::2]),
                               rtol=1e-13)


@pytest.mark.parametrize("d", [64, 128])
def test_rope_is_relative_and_axis_local(d):
    p = d // 6
    n = 30
    pos = RNG.integers(0, 20, size=(n, 3, 1)).astype(float)
    pos = np.concatenate([pos, pos + 1], axis=2)
    q, k = _rand(n, d), _rand(n, d)
    base = oracle.apply_rope(q, oracle.rope_angles(pos, d)) @ \
        oracle.apply_rope(k, oracle.rope_angles(pos, d)).T
    shift = np.array([7.0, -3.0, 11.0])[None, :, None]
    moved = oracle.apply_rope(q, oracle.rope_angles(pos + shift, d)) @ \
        oracle.apply_rope(k, oracle.rope_angles(pos + shift, d)).T
    np.testing.assert_allclose(moved, base, rtol=1e-10, atol=1e-10)
    # moving along one axis only touches that axis' block of pairs
    for axis in range(3):
        delta = np.zeros((1, 3, 1))
        delta[0, axis] = 5
        a0, a1 = oracle.rope_angles(pos, d), oracle.rope_angles(pos + delta, d)
        changed = np.any(a0 != a1, axis=0)
        assert np.all(changed[axis * p:(axis + 1) * p])
        assert not np.any(np.delete(changed, np.arange(axis * p, (axis + 1) * p)))
    # pairs beyond 3p are never rotated
    assert np.all(oracle.rope_angles(pos, d)[:, 3 * p:] == 0)


def test_normalization_does_not_change_attention():
    """RoPE is relative, so shifting a tile's positions leaves its attention output unchanged."""
    inp = ti.make_inputs("tiny_2x16x16")
    wl = inp.workload
    on = oracle.step(inp, normalize_positions=True)
    off = oracle.step(inp, normalize_positions=False)
    assert np.any(on.plan.tile_offset != 0)
    np.testing.assert_allclose(on.y_tiles, off.y_tiles, rtol=1e-9, atol=1e-11)


def test_single_tile_step_equals_untiled_layer():
    """A 1x1x1 tiling is the untiled layer: compare with torch attention + complex RoPE."""
    base = ti.make_inputs("tiny_2x16x16")
    wl = base.workload
    import dataclasses
    wl1 = dataclasses.replace(wl, tiling=((1, 0), (1, 0), (1, 0)), n_audio=4)
    inp = dataclasses.replace(base, workload=wl1, x_aud=_rand(1, 4, wl.channels))
    r = oracle.step(inp, normalize_positions=False)
    p = r.plan
    N = wl.n_gen
    kept = p.row_src[p.row_src >= N] - N
    # untiled sequence: all generated tokens, kept conditioning tokens, audio
    F, H, W = wl.grid
    f, h, w = np.meshgrid(np.arange(F), np.arange(H), np.arange(W), indexing="ij")
    cells = np.stack([f.ravel(), h.ravel(), w.ravel()], 1).astype(float)
    pos = np.concatenate([np.stack([cells, cells + 1], 2), inp.cond_pos[kept]])
    x = np.concatenate([inp.x_global[0, :N], inp.x_global[0, N + kept]]).astype(np.float64)
    xa = inp.x_aud[0]
    seq = torch.from_numpy(np.concatenate([x, xa]))
    d, heads = wl.head_dim, wl.heads
    ang = np.concatenate([oracle.rope_angles(pos, d), np.zeros((xa.shape[0], d // 2))])
    rot = torch.from_numpy(np.exp(1j * ang))

    def proj_rot(wm, rotate):
        t = (seq @ torch.from_numpy(wm.astype(np.float64))).view(-1, heads, d)
        if rotate:
            z = torch.view_as_complex(t.reshape(-1, heads, d // 2, 2).contiguous())
            t = torch.view_as_real(z * rot[:, None, :]).reshape(-1, heads, d)
        return t.transpose(0, 1).contiguous()

    o = torch.nn.functional.scaled_dot_product_attention(
        proj_rot(inp.wq, True), proj_rot(inp.wk, True), proj_rot(inp.wv, False))
    y = (o.transpose(0, 1).reshape(-1, heads * d) @ torch.from_numpy(inp.wo.astype(np.float64))).numpy()
    np.testing.assert_allclose(r.y_global[0, :N], y[:N], rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(r.y_global[0, N + kept], y[N:N + kept.size], rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(r.y_aud[0], y[N + kept.size:], rtol=1e-9, atol=1e-10)
