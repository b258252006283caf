"""Pins of the oracle's per-tile transformer block (CPU only).

Each function is tied to something other than its own formula: closed forms,
library special cases (erf GELU, the logistic function), explicit-loop brute
force on tiny inputs, and invariants (scaling, zero gates, a single text token,
a 1x1x1 tiling equal to the untiled model, position shift).
"""
import dataclasses
import math

import numpy as np
import pytest
from scipy import special

import oracle
import oracle.block as ob
import tdp_inputs as ti

RNG = np.random.default_rng(7)


def _rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


# --------------------------------------------------------------------------
# elementwise pieces
# --------------------------------------------------------------------------

def test_rms_norm_closed_forms():
    x = _rand(5, 64)
    y = ob.rms_norm(x)
    ms = np.mean(x * x, axis=1)
    # mean square of the output is ms / (ms + eps)
    assert np.allclose(np.mean(y * y, axis=1), ms / (ms + ob.RMS_EPS), rtol=1e-12)
    # a constant row c maps to c / sqrt(c^2 + eps)
    c = np.full((1, 32), -2.5)
    assert np.allclose(ob.rms_norm(c), -2.5 / math.sqrt(6.25 + ob.RMS_EPS), rtol=1e-14)
    # positive scaling invariance (eps aside)
    assert np.allclose(ob.rms_norm(1e3 * x), ob.rms_norm(x), rtol=1e-6)


def test_gelu_tanh_against_erf_gelu_and_odd_part():
    u = np.linspace(-8, 8, 4001)
    g = ob.gelu_tanh(u)
    exact = 0.5 * u * (1.0 + special.erf(u / math.sqrt(2.0)))
    # the tanh form is within 1e-3 of the erf form everywhere
    assert np.max(np.abs(g - exact)) < 1e-3
    # its odd part is exactly u/2: gelu(u) - gelu(-u) = u
    assert np.allclose(g - ob.gelu_tanh(-u), u, atol=1e-12)
    assert ob.gelu_tanh(np.array([0.0]))[0] == 0.0


def test_silu_is_u_times_logistic():
    u = np.linspace(-30, 30, 601)
    assert np.allclose(ob.silu(u), u * special.expit(u), rtol=1e-12, atol=1e-300)


def test_timestep_embedding_closed_forms():
    e0 = ob.timestep_embedding(0.0, 256)
    assert np.array_equal(e0, np.concatenate([np.ones(128), np.zeros(128)]))
    tau = 123.25
    e = ob.timestep_embedding(tau, 256)
    assert np.allclose(e[:128] ** 2 + e[128:] ** 2, 1.0, atol=1e-14)
    assert e[0] == pytest.approx(math.cos(tau)) and e[128] == pytest.approx(math.sin(tau))
    # lowest frequency 10000^(-127/128)
    w = 10000.0 ** (-127 / 128)
    assert e[127] == pytest.approx(math.cos(tau * w)) and e[255] == pytest.approx(math.sin(tau * w))


def test_modulation_is_table_when_projection_is_zero():
    D, T = 16, 32
    table = _rand(6, D)
    m = ob.modulation(5.0, _rand(T, D), np.zeros((D, 6 * D)), table)
    assert np.array_equal(m, table)
    # otherwise row r holds columns [r D, (r+1) D) of the projected embedding
    wt1, wt2 = _rand(T, D, scale=0.2), _rand(D, 6 * D, scale=0.2)
    m = ob.modulation(5.0, wt1, wt2, np.zeros((6, D)))
    e = ob.timestep_embedding(5.0, T) @ wt1
    e = (e * special.expit(e)) @ wt2
    for r in range(6):
        assert np.allclose(m[r], e[r * D:(r + 1) * D], rtol=1e-12)


# --------------------------------------------------------------------------
# cross-attention and FFN
# --------------------------------------------------------------------------

def _cross_brute(h, text, wq, wk, wv, wo, heads, d):
    q, k, v = h @ wq, text @ wk, text @ wv
    out = np.zeros((h.shape[0], heads * d))
    for i in range(h.shape[0]):
        for hd in range(heads):
            c = slice(hd * d, (hd + 1) * d)
            logits = [float(np.dot(q[i, c], k[j, c])) / math.sqrt(d) for j in range(text.shape[0])]
            m = max(logits)
            w = [math.exp(s - m) for s in logits]
            tot = sum(w)
            for j in range(text.shape[0]):
                out[i, c] += (w[j] / tot) * v[j, c]
    return out @ wo


def test_cross_attn_brute_force():
    heads, d, D = 2, 4, 8
    h, text = _rand(6, D), _rand(5, D)
    ws = [_rand(D, D, scale=0.4) for _ in range(4)]
    assert np.allclose(ob.cross_attn(h, text, *ws, heads, d), _cross_brute(h, text, *ws, heads, d),
                       rtol=1e-11, atol=1e-12)


def test_cross_attn_closed_forms():
    heads, d, D = 3, 4, 12
    h = _rand(7, D)
    wq, wk, wv, wo = (_rand(D, D, scale=0.3) for _ in range(4))
    # one text token: every query gets that token's value
    t1 = _rand(1, D)
    want = np.tile(t1 @ wv @ wo, (7, 1))
    assert np.allclose(ob.cross_attn(h, t1, wq, wk, wv, wo, heads, d), want, rtol=1e-12)
    # Wq = 0: uniform weights, the mean value
    text = _rand(9, D)
    want = np.tile((text @ wv).mean(axis=0) @ wo, (7, 1))
    assert np.allclose(ob.cross_attn(h, text, np.zeros((D, D)), wk, wv, wo, heads, d), want,
                       rtol=1e-12)


def test_ffn_brute_force_and_zero_output_weight():
    D, F = 4, 8
    h, w1, w2 = _rand(3, D), _rand(D, F), _rand(F, D)
    brute = np.zeros((3, D))
    for i in range(3):
        for f in range(F):
            u = sum(h[i, k] * w1[k, f] for k in range(D))
            g = 0.5 * u * (1 + math.tanh(math.sqrt(2 / math.pi) * (u + 0.044715 * u ** 3)))
            for j in range(D):
                brute[i, j] += g * w2[f, j]
    assert np.allclose(ob.ffn(h, w1, w2), brute, rtol=1e-12)
    assert np.array_equal(ob.ffn(h, w1, np.zeros((F, D))), np.zeros((3, D)))


# --------------------------------------------------------------------------
# the block and the per-tile transformer
# --------------------------------------------------------------------------

def _tiny_layer(D, scale=0.3):
    return ob.Layer(*(_rand(D, D, scale=scale) for _ in range(8)), _rand(D, 4 * D, scale=scale),
                    _rand(4 * D, D, scale=scale), _rand(6, D, scale=0.1))


def _pos(n):
    return np.stack([np.stack([np.full(n, 0.0), np.full(n, 1.0)], -1),
                     np.stack([np.arange(n, dtype=float), np.arange(n, dtype=float) + 1], -1),
                     np.stack([np.zeros(n), np.ones(n)], -1)], axis=1)


def test_block_with_closed_gates_is_identity():
    heads, d = 2, 64
    D = heads * d
    lay = dataclasses.replace(_tiny_layer(D), co=np.zeros((D, D)))
    mod = _rand(6, D)
    mod[2] = 0.0       # gate_a
    mod[5] = 0.0       # gate_f
    x = _rand(10, D)
    assert np.array_equal(ob.block_forward(x, _pos(10), _rand(4, D), mod, lay, heads, d), x)


def test_block_self_attention_branch_is_the_hot_path_layer():
    """shift = scale = 0, gate = 1: the branch is the hot path's layer on rms_norm(x)."""
    heads, d = 2, 64
    D = heads * d
    lay = dataclasses.replace(_tiny_layer(D), co=np.zeros((D, D)), w2=np.zeros((4 * D, D)))
    mod = np.zeros((6, D))
    mod[2] = 1.0
    x, pos = _rand(10, D), _pos(10)
    a, _ = oracle.tile_forward(ob.rms_norm(x), pos, None, lay.wq, lay.wk, lay.wv, lay.wo,
                               heads, d)
    assert np.allclose(ob.block_forward(x, pos, _rand(3, D), mod, lay, heads, d), x + a,
                       rtol=1e-12)


def test_block_scale_minus_one_feeds_the_shift():
    """scale = -1 turns every normalized row into the shift vector: all keys,
    queries and values of a head are then equal up to rotation, every softmax
    row averages one value, and the branches are closed forms."""
    heads, d = 2, 64
    D = heads * d
    lay = dataclasses.replace(_tiny_layer(D), co=np.zeros((D, D)))
    mod = _rand(6, D, scale=0.3)
    mod[1] = -1.0
    mod[4] = -1.0
    x, pos = _rand(10, D), _pos(10)
    attn = mod[0] @ lay.wv @ lay.wo
    ff = ob.gelu_tanh(mod[3] @ lay.w1) @ lay.w2
    want = x + mod[2] * attn + mod[5] * ff
    assert np.allclose(ob.block_forward(x, pos, _rand(3, D), mod, lay, heads, d), want,
                       rtol=1e-10, atol=1e-12)


def test_transformer_with_no_layers_is_norm_and_projections():
    C, D = 8, 16
    m = ob.Model(_rand(C, D), _rand(D, C), _rand(32, D), _rand(D, 6 * D), [], 2, 8)
    x = _rand(5, C)
    want = ob.rms_norm(x @ m.w_in) @ m.w_out
    assert np.allclose(ob.tile_transformer(x, _pos(5), _rand(2, D), 3.0, m), want, rtol=1e-12)


def test_single_tile_step_equals_untiled_model():
    """A 1x1x1 tiling: the TDP step is the model on the whole latent."""
    bw = dataclasses.replace(ti.BLOCK_WORKLOADS["block_tiny"], layers=1)
    binp = ti.make_block_inputs(bw)
    wl = binp.base.workload
    wl1 = dataclasses.replace(wl, tiling=((1, 0), (1, 0), (1, 0)))
    binp1 = dataclasses.replace(binp, base=dataclasses.replace(binp.base, workload=wl1))
    res = ob.block_step(binp1)
    p = res.plan
    model = ob.model_from_inputs(binp1)
    y = ob.tile_transformer(binp.base.x_global[0][p.row_src], p.row_pos, binp.text[0],
                            float(binp.tau[0]), model)
    got = res.y_global[0][p.row_src]
    assert np.allclose(got, y, rtol=1e-9, atol=1e-9)


def test_block_step_is_shift_invariant():
    """RoPE is relative, so normalizing positions leaves the output unchanged."""
    binp = ti.make_block_inputs("block_tiny")
    a = ob.block_step(binp, normalize_positions=True).y_global
    b = ob.block_step(binp, normalize_positions=False).y_global
    assert np.max(np.abs(a - b)) <= 1e-9 * np.max(np.abs(a))


def test_query_rows_match_full_evaluation():
    bw = dataclasses.replace(ti.BLOCK_WORKLOADS["block_tiny"], layers=1)
    binp = ti.make_block_inputs(bw)
    p = oracle.plan(binp.base.workload.grid, binp.base.workload.tiling, binp.base.cond_pos)
    x = oracle.gather_tiles(binp.base.x_global, p)[0]
    r0, r1 = int(p.tile_row_begin[1]), int(p.tile_row_begin[2])
    model = ob.model_from_inputs(binp)
    full = ob.tile_transformer(x[r0:r1], p.row_pos[r0:r1], binp.text[0], float(binp.tau[0]), model)
    rows = np.array([0, 3, 17, r1 - r0 - 1])
    part = ob.tile_transformer(x[r0:r1], p.row_pos[r0:r1], binp.text[0], float(binp.tau[0]), model,
                               query_rows=rows)
    assert np.allclose(part, full[rows], rtol=1e-12, atol=1e-12)
