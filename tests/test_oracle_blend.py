"""Pins for the oracle's gather, blend and audio mean (CPU only).

With an identity denoiser the blend must give back the input latent, because
the masks sum to one and a token kept by k tiles is weighted 1/k (TDP page,
"What it is" and "Shared negative (reference) positions").  Splitting the
tiles over W ranks and summing their blends is the page's single all_reduce;
it must equal the one-rank blend.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import tdp_inputs as ti


def _cpu_sized(name):
    """The workload with fewer frames (same tiling structure) so the CPU suite stays quick."""
    wl = ti.workload(name)
    frames = {"audio_32x48x80": 8, "blend_32x96x160": 2}.get(name, wl.grid[0])
    return dataclasses.replace(wl, grid=(frames,) + wl.grid[1:])


@pytest.mark.parametrize("name", ["tiny_2x16x16", "d64_8x32x32", "audio_32x48x80", "blend_32x96x160"])
def test_identity_reconstructs_latent(name):
    wl = _cpu_sized(name)
    inp = ti.make_inputs(wl)
    p = oracle.plan(wl.grid, wl.tiling, inp.cond_pos)
    x_tiles = oracle.gather_tiles(inp.x_global, p)
    y = oracle.blend_tiles(x_tiles, p)
    kept = np.concatenate([np.ones(wl.n_gen, bool), p.cond_keep_count > 0])
    err = np.abs(y[:, kept] - inp.x_global[:, kept]).max()
    assert err <= 1e-5 * np.abs(inp.x_global).max()
    assert np.all(y[:, ~kept] == 0)
    # the generated part is exact: dyadic masks sum to exactly one
    assert np.all(y[:, :wl.n_gen] == inp.x_global[:, :wl.n_gen])


def test_identity_odd_overlap():
    wl = dataclasses.replace(ti.workload("tiny_2x16x16"), grid=(3, 17, 23),
                             tiling=((1, 0), (3, 5), (4, 5)), n_cond=12, n_cond_neg=3)
    inp = ti.make_inputs(wl)
    r = oracle.step(inp, identity=True)
    kept = np.concatenate([np.ones(wl.n_gen, bool), r.plan.cond_keep_count > 0])
    rel = np.abs(r.y_global[:, kept] - inp.x_global[:, kept]).max() / np.abs(inp.x_global).max()
    assert rel <= 1e-6


def test_gather_copies_rows():
    inp = ti.make_inputs("d64_8x32x32")
    wl = inp.workload
    p = oracle.plan(wl.grid, wl.tiling, inp.cond_pos)
    xt = oracle.gather_tiles(inp.x_global, p)
    F, H, W = wl.grid
    # row r of tile t is the token at the r-th box position (row-major), then kept cond tokens
    for t in range(p.tile_id.size):
        r0 = p.tile_row_begin[t]
        (af, bf), (ah, bh), (aw, bw) = p.tile_box[t]
        i = 0
        for f in range(af, bf):
            for h in range(ah, bh):
                for w in range(aw, bw):
                    assert np.array_equal(xt[0, r0 + i], inp.x_global[0, (f * H + h) * W + w])
                    i += 1
        assert i == p.tile_n_gen[t]


@pytest.mark.parametrize("W", [2, 3, 4])
def test_rank_sum_equals_single_rank(W):
    inp = ti.make_inputs(_cpu_sized("audio_32x48x80"))
    wl = inp.workload
    rng = np.random.default_rng(5)
    p1 = oracle.plan(wl.grid, wl.tiling, inp.cond_pos)
    # arbitrary per-tile outputs, keyed by (tile, source row) so ranks see the same values
    vals = {}
    y1 = np.zeros((wl.batch, p1.n_rows, 8))
    for t in range(p1.tile_id.size):
        r0, r1 = p1.tile_row_begin[t], p1.tile_row_begin[t + 1]
        y1[:, r0:r1] = rng.standard_normal((wl.batch, r1 - r0, 8))
        vals[int(p1.tile_id[t])] = y1[:, r0:r1]
    want = oracle.blend_tiles(y1, p1)
    acc = np.zeros_like(want)
    for r in range(W):
        p = oracle.plan(wl.grid, wl.tiling, inp.cond_pos, world_size=W, rank=r)
        yr = np.concatenate([vals[int(t)] for t in p.tile_id], axis=1)
        acc = oracle.blend_tiles(yr, p, y_global=acc)
    np.testing.assert_allclose(acc, want, rtol=1e-12, atol=1e-12)


def test_audio_mean_identity_and_ranks():
    inp = ti.make_inputs(_cpu_sized("audio_32x48x80"))
    wl = inp.workload
    T = wl.n_tiles
    y_aud_tiles = np.broadcast_to(inp.x_aud, (T,) + inp.x_aud.shape)
    np.testing.assert_allclose(oracle.audio_mean(y_aud_tiles, T), inp.x_aud, rtol=1e-12)
    rng = np.random.default_rng(9)
    y = rng.standard_normal((T, 1, 4, 3))
    parts = sum(oracle.audio_mean(y[r::4], T) for r in range(4))
    np.testing.assert_allclose(parts, y.mean(axis=0), rtol=1e-12)
