"""Pins of the oracle's upscale loop (CPU only).

Each piece is tied to something other than its own formula:
  * the re-noise and Euler conventions together, by a velocity field whose
    exact flow is known: for a clean latent mu the straight path
    (1 - sigma) mu + sigma eps has velocity (x - mu) / sigma, and explicit
    Euler follows a straight path exactly for any step sizes;
  * the schedule by its closed form;
  * the seam spread by a two-tile closed form (weights 7/8 ... 1/8) and by an
    explicit-loop brute force that does not use the inverse map;
  * the loop with the identity denoiser by its product closed form;
  * one step of the loop with the transformer against the block step
    (pinned in test_oracle_block.py) at tau = 1000 sigma.
"""
import dataclasses
from collections import defaultdict

import numpy as np
import pytest

import oracle
import oracle.block as ob
import oracle.upscale as ou
import tdp_inputs as ti

RNG = np.random.default_rng(11)


def _straight_velocity(mu, n_gen, cond_value=7.0):
    """The exact velocity of the straight path towards mu; garbage on the
    conditioning rows, which the loop must ignore."""
    def velocity(x, sigma):
        v = np.full(x.shape, cond_value)
        v[:, :n_gen] = (x[:, :n_gen] - mu[:, :n_gen]) / sigma
        return v, None
    return velocity


def test_linear_sigmas_closed_forms():
    assert np.array_equal(ou.linear_sigmas(1.0, 4), np.array([1, .75, .5, .25, 0], np.float32))
    s = ou.linear_sigmas(0.3, 3)
    assert s.dtype == np.float32 and s.size == 4
    assert s[0] == np.float32(0.3) and s[-1] == 0.0
    assert np.all(np.diff(s) < 0)
    assert np.allclose(np.diff(s.astype(np.float64)), -0.1, rtol=1e-6)
    assert np.array_equal(ou.linear_sigmas(0.7, 0), np.array([0.7], np.float32))
    for bad in [(-0.1, 2), (1.5, 2), (0.5, -1)]:
        with pytest.raises(ValueError):
            ou.linear_sigmas(*bad)


@pytest.mark.parametrize("sigmas", [ou.linear_sigmas(0.5, 1), ou.linear_sigmas(0.8, 3),
                                    np.array([0.9, 0.6, 0.2, 0.05, 0.0], np.float32)])
def test_straight_path_is_followed_exactly(sigmas):
    B, N, M, C = 2, 10, 3, 4
    x1 = RNG.standard_normal((B, N + M, C))
    eps = RNG.standard_normal((B, N, C))
    res = ou.upscale_loop(x1, eps, sigmas, N, _straight_velocity(x1, N))
    assert len(res.states) == sigmas.size
    for st, s in zip(res.states, sigmas.astype(np.float64)):
        want = (1.0 - s) * x1[:, :N] + s * eps
        assert np.allclose(st[:, :N], want, rtol=1e-12, atol=1e-12)
        # conditioning rows are the clean stage-1 tokens throughout
        assert np.array_equal(st[:, N:], x1[:, N:])
    assert np.allclose(res.x[:, :N], x1[:, :N], rtol=1e-12, atol=1e-12)


def test_constant_velocity_telescopes():
    B, N, C = 1, 6, 3
    x1, eps = RNG.standard_normal((B, N, C)), RNG.standard_normal((B, N, C))
    c = RNG.standard_normal((B, N, C))
    sig = ou.linear_sigmas(0.6, 5)
    res = ou.upscale_loop(x1, eps, sig, N, lambda x, s: (c, None))
    s0 = np.float64(sig[0])
    assert np.allclose(res.x, (1 - s0) * x1 + s0 * eps - s0 * c, rtol=1e-12, atol=1e-12)


def test_zero_sigma_keeps_the_stage1_latent():
    x1, eps = RNG.standard_normal((1, 9, 2)), RNG.standard_normal((1, 7, 2))
    res = ou.upscale_loop(x1, eps, np.zeros(4, np.float32), 7,
                          lambda x, s: (RNG.standard_normal(x.shape), None))
    assert np.array_equal(res.x, x1)


def _two_tile_plan():
    return oracle.plan((1, 1, 16), ((1, 0), (1, 0), (2, 4)), np.zeros((0, 3, 2), np.float32))


def test_seam_spread_two_tile_closed_form():
    """Tile 0 predicts a everywhere, tile 1 predicts b: on the four overlap
    tokens the left weights are 7/8, 5/8, 3/8, 1/8, so S2 = |a - b|^2 *
    sum w (1 - w) = |a - b|^2 * 11/16 and S0 = sum |w a + (1 - w) b|^2."""
    p = _two_tile_plan()
    a, b = np.array([1.0, 2.0, -1.0]), np.array([3.0, -2.0, 0.5])
    y = np.zeros((1, p.n_rows, 3))
    y[0, p.tile_row_begin[0]:p.tile_row_begin[1]] = a
    y[0, p.tile_row_begin[1]:p.tile_row_begin[2]] = b
    s2, s0 = ou.seam_spread(y, p, 16)
    assert s2 == pytest.approx(np.sum((a - b) ** 2) * 11 / 16, rel=1e-14)
    want0 = sum(np.sum((w * a + (1 - w) * b) ** 2) for w in (7 / 8, 5 / 8, 3 / 8, 1 / 8))
    assert s0 == pytest.approx(want0, rel=1e-14)
    assert ou.relative_spread(s2, s0) == pytest.approx(np.sqrt(s2 / s0))


def _seam_brute(y, p, n_gen):
    groups = defaultdict(list)
    for r in range(p.n_rows):
        groups[int(p.row_src[r])].append(r)
    s2 = s0 = 0.0
    for n, rows in groups.items():
        if n >= n_gen or len(rows) < 2:
            continue
        for b in range(y.shape[0]):
            ybar = sum(float(p.row_weight[r]) * y[b, r] for r in rows)
            s0 += float(np.dot(ybar, ybar))
            for r in rows:
                d = y[b, r] - ybar
                s2 += float(p.row_weight[r]) * float(np.dot(d, d))
    return s2, s0


@pytest.mark.parametrize("name", ["tiny_2x16x16", "d64_8x32x32"])
def test_seam_spread_brute_force(name):
    inp = ti.make_inputs(name)
    wl = inp.workload
    p = oracle.plan(wl.grid, wl.tiling, inp.cond_pos)
    y = RNG.standard_normal((wl.batch, p.n_rows, 6))
    s2, s0 = ou.seam_spread(y, p, wl.n_gen)
    b2, b0 = _seam_brute(y, p, wl.n_gen)
    assert s2 == pytest.approx(b2, rel=1e-12) and s0 == pytest.approx(b0, rel=1e-12)
    # tiles that agree where they overlap have no spread (up to the rounding of w x)
    x = RNG.standard_normal((wl.batch, wl.n_gen + wl.n_cond, 6))
    z2, z0 = ou.seam_spread(oracle.gather_tiles(x, p), p, wl.n_gen)
    assert z2 <= 1e-28 * z0


def test_identity_denoiser_loop_closed_form():
    """With the identity tile denoiser the blend returns x itself on the
    generated rows, so each step multiplies them by 1 + sigma_{i+1} - sigma_i
    and the seam spread is zero."""
    inp = ti.make_inputs("tiny_2x16x16")
    wl = inp.workload
    p = oracle.plan(wl.grid, wl.tiling, inp.cond_pos)
    N = wl.n_gen

    def velocity(x, sigma):
        y = oracle.gather_tiles(x, p)
        return oracle.blend_tiles(y, p), ou.seam_spread(y, p, N)

    eps = RNG.standard_normal((wl.batch, N, wl.channels))
    sig = ou.linear_sigmas(0.4, 3).astype(np.float64)
    res = ou.upscale_loop(inp.x_global, eps, sig, N, velocity)
    factor = np.prod(1.0 + np.diff(sig))
    x0 = (1 - sig[0]) * inp.x_global[:, :N] + sig[0] * eps
    assert np.allclose(res.x[:, :N], factor * x0, rtol=1e-12, atol=1e-12)
    assert np.array_equal(res.x[:, N:], inp.x_global[:, N:])
    assert len(res.seam) == 3 and all(s2 <= 1e-28 * s0 for s2, s0 in res.seam)


def test_one_step_is_the_block_step():
    """One step from sigma_0 to 0 is x_0 - sigma_0 * (block step of x_0 at
    tau = 1000 sigma_0)."""
    up = ti.make_upscale_inputs(dataclasses.replace(ti.UPSCALE_WORKLOADS["upscale_tiny"],
                                                    n_steps=1))
    binp = up.block
    wl = binp.base.workload
    p = oracle.plan(wl.grid, wl.tiling, binp.base.cond_pos)
    N = wl.n_gen
    sig = ou.linear_sigmas(up.workload.sigma0, 1)
    res = ou.upscale_loop(binp.base.x_global, up.noise, sig, N, ou.tdp_velocity(binp, p))
    x0 = res.states[0]
    s0 = np.float64(sig[0])
    step_in = dataclasses.replace(
        binp, base=dataclasses.replace(binp.base, x_global=x0),
        tau=np.full(wl.batch, 1000.0 * s0))
    y = ob.block_step(step_in).y_global
    assert np.allclose(res.x[:, :N], x0[:, :N] - s0 * y[:, :N], rtol=1e-12, atol=1e-12)
    assert np.array_equal(res.x[:, N:], binp.base.x_global[:, N:])
    s2, s0_ = res.seam[0]
    assert s2 > 0 and s0_ > 0
