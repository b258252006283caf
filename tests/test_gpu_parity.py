"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: gather bit-exact; fp32 blend within 1e-5 (max abs error / max abs
reference, fed the GPU's own tile outputs); attention outputs within 2e-2 of
the float64 oracle by the same measure (bf16 operands on the GPU).  Full-size
workloads the oracle cannot finish quickly are checked on sampled query rows,
which the oracle evaluates one by one against all keys of their tile.
"""
import dataclasses
import sys

import numpy as np
import pytest

import oracle
import tdp_inputs as ti

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ATTN_TOL = 2e-2
BLEND_TOL = 1e-5


def say(*a):
    print("[gpu-parity]", *a, flush=True)
    sys.stdout.flush()


def rel_err(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    return float(np.abs(got - want).max() / max(np.abs(want).max(), 1e-30))


def _step(inp, **kw):
    from tiled_video_diffusion_amd.step import TdpStep
    return TdpStep(inp, **kw)


def _np(t):
    return t.detach().float().cpu().numpy()


# --------------------------------------------------------------------------
# gather / blend / identity
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny_2x16x16", "d64_8x32x32", "audio_32x48x80",
                                  "blend_32x96x160"])
def test_gather_bit_exact(name):
    say("gather", name)
    inp = ti.make_inputs(name)
    s = _step(inp, identity=True)
    s.gather()
    torch.cuda.synchronize()
    want = inp.x_global[:, s.plan.row_src, :]
    got = s.x_tiles.float().cpu().numpy()
    assert np.array_equal(got, want)


@pytest.mark.parametrize("name", ["tiny_2x16x16", "d64_8x32x32", "audio_32x48x80",
                                  "blend_32x96x160"])
def test_identity_step_reconstructs(name):
    """Identity denoiser: the blend gives back the latent (every kept row)."""
    say("identity", name)
    inp = ti.make_inputs(name)
    s = _step(inp, identity=True)
    s.run()
    torch.cuda.synchronize()
    y = _np(s.y_global)
    kept = np.concatenate([np.ones(inp.workload.n_gen, bool), s.plan.cond_keep_count > 0])
    assert rel_err(y[:, kept], inp.x_global[:, kept]) <= BLEND_TOL
    assert np.all(y[:, ~kept] == 0)


@pytest.mark.parametrize("name", ["tiny_2x16x16", "d64_8x32x32", "audio_32x48x80"])
def test_blend_matches_oracle_on_random_tile_outputs(name):
    """Blend of arbitrary tile outputs, overwrite then accumulate."""
    say("blend random", name)
    inp = ti.make_inputs(name)
    s = _step(inp, identity=True)
    rng = np.random.default_rng(11)
    y = rng.standard_normal(tuple(s.x_tiles.shape)).astype(np.float32)
    s.x_tiles.copy_(torch.from_numpy(y).to(s.x_tiles.dtype))
    yt = _np(s.x_tiles)
    s.blend(accumulate=False)
    torch.cuda.synchronize()
    p = oracle.plan(inp.workload.grid, inp.workload.tiling, inp.cond_pos)
    want = oracle.blend_tiles(yt, p)
    assert rel_err(_np(s.y_global), want) <= BLEND_TOL
    s.blend(accumulate=True)
    torch.cuda.synchronize()
    assert rel_err(_np(s.y_global), 2 * want) <= BLEND_TOL


# --------------------------------------------------------------------------
# attention end to end
# --------------------------------------------------------------------------

def _check_full(inp, s, normalize=True):
    """Whole-step parity against the oracle (all rows)."""
    r = oracle.step(inp, normalize_positions=normalize, p=None)
    torch.cuda.synchronize()
    yt = _np(s.y_tiles)
    e_tiles = rel_err(yt, r.y_tiles)
    e_glob = rel_err(_np(s.y_global), r.y_global)
    # blend bar: the oracle blend of the GPU's own tile outputs
    e_blend = rel_err(_np(s.y_global), oracle.blend_tiles(yt, r.plan))
    say(f"  y_tiles {e_tiles:.2e}  y_global {e_glob:.2e}  blend {e_blend:.2e}")
    assert e_tiles <= ATTN_TOL and e_glob <= ATTN_TOL and e_blend <= BLEND_TOL
    if r.y_aud is not None:
        e_at = rel_err(_np(s.y_audio_tiles), r.y_aud_tiles)
        e_a = rel_err(_np(s.y_audio), r.y_aud)
        say(f"  y_audio_tiles {e_at:.2e}  y_audio {e_a:.2e}")
        assert e_at <= ATTN_TOL and e_a <= ATTN_TOL
        e_am = rel_err(_np(s.y_audio), oracle.audio_mean(_np(s.y_audio_tiles), r.plan.n_tiles_total))
        assert e_am <= BLEND_TOL


@pytest.mark.parametrize("name", ["tiny_2x16x16", "d64_8x32x32"])
def test_attention_step_full(name):
    say("attention full", name)
    inp = ti.make_inputs(name)
    s = _step(inp)
    s.run()
    _check_full(inp, s)


def _variant(base, **kw):
    wl = dataclasses.replace(ti.workload(base), **kw)
    return ti.make_inputs(wl)


EDGE_CASES = {
    # odd overlaps, tiles not multiples of 64/128, audio not a multiple of 64, batch 2
    "odd_ragged_audio_d128": dict(base="tiny_2x16x16", grid=(3, 17, 23),
                                  tiling=((1, 0), (3, 5), (4, 5)), heads=2, head_dim=128,
                                  n_cond=12, n_cond_neg=3, n_audio=37, batch=2,
                                  latent_dtype="bf16"),
    # a single tile shorter than one key block, fp32 latent
    "one_small_tile": dict(base="tiny_2x16x16", grid=(1, 5, 7), tiling=((1, 0), (1, 0), (1, 0)),
                           n_cond=3, n_cond_neg=1),
    # tiles in all three dims, d=64, many heads, ragged rows
    "3d_tiles_d64": dict(base="d64_8x32x32", grid=(6, 13, 11), tiling=((2, 2), (2, 3), (3, 1)),
                         heads=6, n_cond=9, n_cond_neg=2, n_audio=65, batch=2),
    # a tile of more than one 128-row block plus a 1-row remainder
    "remainder_rows": dict(base="tiny_2x16x16", grid=(1, 129, 1), tiling=((1, 0), (1, 0), (1, 0)),
                           n_cond=0, n_cond_neg=0),
}


@pytest.mark.parametrize("case", list(EDGE_CASES))
def test_attention_edge_cases(case):
    kw = dict(EDGE_CASES[case])
    base = kw.pop("base")
    say("edge case", case)
    inp = _variant(base, **kw)
    s = _step(inp)
    s.run()
    _check_full(inp, s)


def test_normalize_off_matches_oracle():
    say("normalize off tiny")
    inp = ti.make_inputs("tiny_2x16x16")
    s = _step(inp, normalize_positions=False)
    s.run()
    _check_full(inp, s, normalize=False)


def test_stage_split_equals_fused_call():
    say("stage split d64")
    inp = ti.make_inputs("d64_8x32x32")
    s = _step(inp)
    s.gather()
    s.attention()
    torch.cuda.synchronize()
    fused = s.y_tiles.clone()
    s.y_tiles.zero_()
    s.attn_prepare()
    s.attn_qkv()
    s.attn_core()
    s.attn_out()
    torch.cuda.synchronize()
    assert torch.equal(fused, s.y_tiles)


# --------------------------------------------------------------------------
# key-split core: the keys of each query block in parts, combined after
# --------------------------------------------------------------------------

SPLIT_CASES = {
    # the unsplit kernel on a small launch (the automatic choice would split)
    "tiny_unsplit": ("tiny_2x16x16", {}, 1),
    "tiny_2": ("tiny_2x16x16", {}, 2),
    # more parts than key blocks: empty parts are skipped by the combine
    "tiny_8": ("tiny_2x16x16", {}, 8),
    "d64_3": ("d64_8x32x32", {}, 3),
    # two key segments (tile, then audio), audio queries, ragged lengths
    "odd_ragged_audio_3": ("tiny_2x16x16", EDGE_CASES["odd_ragged_audio_d128"], 3),
    "3d_tiles_d64_5": ("d64_8x32x32", EDGE_CASES["3d_tiles_d64"], 5),
    "remainder_rows_2": ("tiny_2x16x16", EDGE_CASES["remainder_rows"], 2),
}


@pytest.mark.parametrize("case", list(SPLIT_CASES))
def test_attention_key_split(case):
    base, kw, k = SPLIT_CASES[case]
    kw = {key: v for key, v in kw.items() if key != "base"}
    say("key split", case, "parts", k)
    inp = _variant(base, **kw) if kw else ti.make_inputs(base)
    s = _step(inp, kv_splits=k)
    s.run()
    _check_full(inp, s)


def _sample_rows(p, t, rng, k):
    r0, r1 = int(p.tile_row_begin[t]), int(p.tile_row_begin[t + 1])
    n = r1 - r0
    picks = {0, n - 1, int(p.tile_n_gen[t]) - 1, min(n - 1, 127), min(n - 1, 128)}
    picks |= set(rng.integers(0, n, size=k).tolist())
    return np.array(sorted(picks)), r0, r1


@pytest.mark.parametrize("name,kv_splits", [("t16_16x64x64", 0), ("audio_32x48x80", 0),
                                             ("t16_16x64x64", 2), ("audio_32x48x80", 3)])
def test_attention_full_size_sampled(name, kv_splits):
    """Full-size workloads in the benchmark's launch configuration (these
    launches fill the GPU, so the core runs unsplit), sampled rows; then the
    same with the key split forced."""
    say("attention sampled", name, "key parts", kv_splits)
    inp = ti.make_inputs(name)
    wl = inp.workload
    s = _step(inp, kv_splits=kv_splits)
    s.run()
    torch.cuda.synchronize()
    p = oracle.plan(wl.grid, wl.tiling, inp.cond_pos)
    yt = _np(s.y_tiles)
    # blend bar on every row: the oracle blend of the GPU's own tile outputs
    e_blend = rel_err(_np(s.y_global), oracle.blend_tiles(yt, p))
    say(f"  blend {e_blend:.2e}")
    assert e_blend <= BLEND_TOL
    rng = np.random.default_rng(3)
    tiles = sorted({0, p.tile_id.size - 1, int(np.argmax(np.diff(p.tile_row_begin)))} |
                   set(rng.integers(0, p.tile_id.size, size=1).tolist()))
    x_tiles = oracle.gather_tiles(inp.x_global, p)
    for t in tiles:
        rows, r0, r1 = _sample_rows(p, t, rng, 24)
        for b in range(wl.batch):
            xa = None if inp.x_aud is None else inp.x_aud[b]
            aq = None if xa is None else np.array([0, 5, xa.shape[0] - 1])
            y, ya = oracle.tile_forward(x_tiles[b, r0:r1], p.row_pos[r0:r1], xa, inp.wq, inp.wk,
                                        inp.wv, inp.wo, wl.heads, wl.head_dim,
                                        query_rows=rows, audio_query_rows=aq)
            e = rel_err(yt[b, r0 + rows], y)
            say(f"  tile {t} batch {b} rows {rows.size}: {e:.2e}")
            assert e <= ATTN_TOL
            if ya is not None:
                ea = rel_err(_np(s.y_audio_tiles)[t, b, aq], ya)
                say(f"  tile {t} batch {b} audio rows: {ea:.2e}")
                assert ea <= ATTN_TOL
    if s.y_audio is not None:
        e_am = rel_err(_np(s.y_audio), oracle.audio_mean(_np(s.y_audio_tiles), p.n_tiles_total))
        assert e_am <= BLEND_TOL


@pytest.mark.parametrize("assignment", ["round_robin", "longest_first"])
@pytest.mark.parametrize("W", [2, 4])
def test_multi_rank_sum_equals_single_rank(W, assignment):
    """The page's single all_reduce: summing the W ranks' blends equals one rank's
    (round-robin tiles as on the page, or longest first)."""
    say("multi-rank", W, assignment)
    inp = _variant("audio_32x48x80", grid=(8, 48, 80), heads=4)
    full = _step(inp)
    full.run()
    acc_g = torch.zeros_like(full.y_global)
    acc_a = torch.zeros_like(full.y_audio)
    for r in range(W):
        s = _step(inp, world_size=W, rank=r, assignment=assignment)
        s.y_global = acc_g
        s.y_audio = acc_a
        s.run(accumulate=True)
    torch.cuda.synchronize()
    assert rel_err(_np(acc_g), _np(full.y_global)) <= BLEND_TOL
    assert rel_err(_np(acc_a), _np(full.y_audio)) <= BLEND_TOL


DETERMINISM_CASES = {
    # head_dim 64: each block's S computed in its own step
    "d64": ("d64_8x32x32", {}),
    # head_dim 128 with audio: S(j+1) overlapped with block j, K staged two
    # blocks ahead (a missing barrier there once let a wave's K(2) load
    # overwrite K(0) while another wave still read it)
    "d128_audio": ("audio_32x48x80", dict(grid=(8, 48, 80), heads=4)),
}


@pytest.mark.parametrize("case", list(DETERMINISM_CASES))
def test_repeat_runs_are_deterministic(case):
    """Five runs of the same step give bit-identical outputs."""
    say("determinism", case)
    base, kw = DETERMINISM_CASES[case]
    inp = _variant(base, **kw) if kw else ti.make_inputs(base)
    s = _step(inp)
    s.run()
    torch.cuda.synchronize()
    a = s.y_global.clone()
    at = s.y_tiles.clone()
    for _ in range(4):
        s.run()
        torch.cuda.synchronize()
        assert torch.equal(at, s.y_tiles)
        assert torch.equal(a, s.y_global)


def test_claimed_tail_recomputed_on_every_launch():
    """A core launch of 16 rounds or more hands its last units to workgroups
    that claim them from a counter, which the launch's last claim puts back
    to zero.  A second launch without the prepare stage (which also zeroes
    it) must still compute every unit: new Q/K/V, core and projection again
    give bitwise what a launch after a fresh prepare gives."""
    inp = _variant("t16_16x64x64", heads=10)     # 4840 units of 256 rows >= 16 x 256 CUs
    say("claimed tail", inp.workload.name, "heads", inp.workload.heads)
    s = _step(inp)
    s.run()
    torch.cuda.synchronize()
    y1 = s.y_tiles.clone()
    s.x_global.neg_()
    s.gather()
    s.attn_qkv()
    s.attn_core()                                # no prepare: the counter reset by the last launch
    s.attn_out()
    torch.cuda.synchronize()
    y2 = s.y_tiles.clone()
    s.attn_prepare()
    s.attn_core()
    s.attn_out()
    torch.cuda.synchronize()
    assert not torch.equal(y1, y2)
    assert torch.equal(y2, s.y_tiles)
    # and a sample of rows against the oracle
    wl = inp.workload
    p = oracle.plan(wl.grid, wl.tiling, inp.cond_pos)
    x_tiles = oracle.gather_tiles(-inp.x_global, p)
    rng = np.random.default_rng(5)
    t = p.tile_id.size - 1                       # the last tile: its units are in the claimed tail
    rows, r0, r1 = _sample_rows(p, t, rng, 16)
    y, _ = oracle.tile_forward(x_tiles[0, r0:r1], p.row_pos[r0:r1], None, inp.wq, inp.wk,
                               inp.wv, inp.wo, wl.heads, wl.head_dim, query_rows=rows)
    e = rel_err(_np(y2)[0, r0 + rows], y)
    say(f"  last tile rows {rows.size}: {e:.2e}")
    assert e <= ATTN_TOL


@pytest.mark.parametrize("name,kw", [("d64_8x32x32", {}), ("t16_16x64x64", dict(heads=10))])
def test_two_launch_geometries_bitwise(name, kw):
    """The same step under two launch geometries of the core: every query
    block on a fixed workgroup (kv_splits 1), and the last ~1/12 of them
    claimed at run time by whichever workgroups reach them first (kv_splits
    0; these launches are two rounds or more).  A query block's result must
    not depend on where it runs, so the outputs are bitwise equal."""
    inp = _variant(name, **kw) if kw else ti.make_inputs(name)
    say("two launch geometries", name, kw)
    outs = []
    for k in (1, 0, 1):
        s = _step(inp, kv_splits=k)
        s.run()
        torch.cuda.synchronize()
        outs.append(s.y_tiles.clone())
        del s
    assert torch.equal(outs[0], outs[1])
    assert torch.equal(outs[0], outs[2])


def _fallback_inputs():
    """Inputs whose Cauchy-Schwarz bound |q| max|k| is far above every real
    score while the scores stay ordinary: each head's K is zero on the first
    half of its dims (RoPE rotates those pairs among themselves, so they stay
    zero) and Q is large there."""
    base = _variant("tiny_2x16x16", grid=(2, 8, 12), tiling=((1, 0), (1, 0), (2, 4)),
                    n_cond=3, n_cond_neg=1, n_audio=5)
    d, H = base.workload.head_dim, base.workload.heads
    wq, wk = base.wq.copy(), base.wk.copy()
    for h in range(H):
        wk[:, h * d:h * d + d // 2] = 0.0
        wq[:, h * d:h * d + d // 2] *= 32.0
    return dataclasses.replace(base, wq=wq, wk=wk)


def _score_bounds(inp):
    """Per tile (batch 0): the largest Cauchy-Schwarz bound |q| max|k| over
    its queries and the largest score, both in log2 units (scale log2(e)/sqrt(d)),
    max|k| over the tile's and the audio keys, as the kernel takes it."""
    wl = inp.workload
    d = wl.head_dim
    p = oracle.plan(wl.grid, wl.tiling, inp.cond_pos)
    sl2 = 1.4426950408889634 / np.sqrt(d)
    xa = inp.x_aud[0] if inp.x_aud is not None else np.zeros((0, wl.channels))
    out = []
    for t in range(p.tile_id.size):
        r0, r1 = int(p.tile_row_begin[t]), int(p.tile_row_begin[t + 1])
        seq = np.concatenate([inp.x_global[0, p.row_src[r0:r1]], xa]).astype(np.float64)
        ang = np.concatenate([oracle.rope_angles(p.row_pos[r0:r1], d),
                              np.zeros((len(xa), d // 2))])
        u_max, s_max = 0.0, -np.inf
        for h in range(wl.heads):
            q = oracle.apply_rope((seq @ inp.wq)[:, h * d:(h + 1) * d], ang)
            k = oracle.apply_rope((seq @ inp.wk)[:, h * d:(h + 1) * d], ang)
            u = np.linalg.norm(q, axis=1) * np.linalg.norm(k, axis=1).max() * sl2
            u_max = max(u_max, float(u.max()))
            s_max = max(s_max, float((q @ k.T).max() * sl2))
        out.append((u_max, s_max))
    return out


def test_exact_path_when_score_bound_is_large():
    """|q| max|k| is far above the shift-free range (and above every real
    score by > 150 in log2 units): the kernel must take the exact online
    softmax for the whole tile."""
    say("exact path, large bound")
    inp = _fallback_inputs()
    wl = inp.workload
    p = oracle.plan(wl.grid, wl.tiling, inp.cond_pos)
    r0, r1 = int(p.tile_row_begin[0]), int(p.tile_row_begin[1])
    seq = np.concatenate([inp.x_global[0, p.row_src[r0:r1]], inp.x_aud[0]]).astype(np.float64)
    d = wl.head_dim
    ang = np.concatenate([oracle.rope_angles(p.row_pos[r0:r1], d), np.zeros((5, d // 2))])
    q = oracle.apply_rope((seq @ inp.wq)[:, :d], ang)
    k = oracle.apply_rope((seq @ inp.wk)[:, :d], ang)
    sl2 = 1.4426950408889634 / np.sqrt(d)
    s_max = (q @ k.T).max(axis=1)
    gap = (np.linalg.norm(q, axis=1) * np.linalg.norm(k, axis=1).max() - s_max) * sl2
    assert gap.min() > 150 and np.abs(s_max * sl2).max() < 20
    for k in (0, 3):
        say("  key parts", k)
        s = _step(inp, kv_splits=k)
        s.run()
        _check_full(inp, s)


def test_shift_free_softmax_near_its_limit():
    """Wq = c Wk: each query's own key scores at its bound, so with the bound
    just under the shift-free limit (64 in log2 units) p reaches about 2^60."""
    say("shift-free near limit")
    base = _variant("tiny_2x16x16", grid=(2, 8, 12), tiling=((1, 0), (1, 0), (2, 4)),
                    n_cond=3, n_cond_neg=1, n_audio=5)
    u1 = max(u for u, _ in _score_bounds(dataclasses.replace(base, wq=base.wk.copy())))
    c = 60.0 / u1
    inp = dataclasses.replace(base, wq=ti.round_to_bf16(base.wk * c))
    bounds = _score_bounds(inp)
    say("  bounds", [(round(u, 1), round(sm, 1)) for u, sm in bounds])
    assert 55.0 < max(u for u, _ in bounds) < 62.0
    assert max(sm for _, sm in bounds) > 50.0
    for k in (0, 4):
        say("  key parts", k)
        s = _step(inp, kv_splits=k)
        s.run()
        _check_full(inp, s)


def test_shift_free_and_exact_workgroups_in_one_launch():
    """Rows only tile 0 holds are scaled up: tile 0's bound leaves the
    shift-free range (exact online softmax) while tile 1 stays inside it."""
    say("mixed shift-free / exact")
    base = _variant("tiny_2x16x16", grid=(2, 8, 12), tiling=((1, 0), (1, 0), (2, 4)),
                    n_cond=3, n_cond_neg=1, n_audio=5)
    F, H, W = base.workload.grid
    x = base.x_global.copy()
    n = np.arange(F * H * W)
    x[:, n[(n % W) < 4]] *= 2.5     # columns 0-3 lie in tile 0 only (boxes [0,8), [4,12))
    inp = dataclasses.replace(base, x_global=x)
    bounds = _score_bounds(inp)
    say("  bounds", [(round(u, 1), round(sm, 1)) for u, sm in bounds])
    assert bounds[0][0] > 80.0 and bounds[1][0] < 48.0
    for k in (0, 2):
        say("  key parts", k)
        s = _step(inp, kv_splits=k)
        s.run()
        _check_full(inp, s)


def _very_negative_inputs(head_dim, score_log2):
    """Inputs where a few query rows score about -score_log2 (log2 units, the
    kernel's scale log2(e)/sqrt(d)) against every real key of their tile and
    every audio key, far below the score 0 of a key padding a block.  Tile
    rows (129-131) and audio rows (5) are not multiples of any key block.

    Construction: channel 0 holds a constant a on every token (tile rows,
    conditioning rows and audio), channel 1 is -1 on the chosen query tokens
    and 0 elsewhere.  In each head the last feature, which RoPE leaves
    unrotated, is fed only by channel 0 for K (= a) and by channel 1 for Q
    (= -Bq), so those queries score -a Bq against every key.  All other
    weights are the workload's, scaled by 0.1, so the rest of the scores are
    small and the Cauchy-Schwarz bound of the chosen rows stays near
    a Bq log2(e)/sqrt(d)."""
    base = _variant("tiny_2x16x16", grid=(2, 8, 12), tiling=((1, 0), (1, 0), (2, 4)),
                    n_cond=3, n_cond_neg=1, n_audio=5, head_dim=head_dim, heads=2)
    wl = base.workload
    F, H, W = wl.grid
    d = wl.head_dim
    a = 8.0
    bq = score_log2 / (a * 1.4426950408889634 / np.sqrt(d))
    x = base.x_global.copy()
    xa = base.x_aud.copy()
    x[:, :, 0] = a
    x[:, :, 1] = 0.0
    xa[:, :, 0] = a
    xa[:, :, 1] = 0.0
    # (f, h, w): in both tiles (w in [4, 8)), tile 0 only, tile 1 only
    targets = [(1 * H + 3) * W + 5, (0 * H + 2) * W + 1, (1 * H + 7) * W + 10]
    x[:, targets, 1] = -1.0
    wq = ti.round_to_bf16(base.wq * 0.1)
    wk = ti.round_to_bf16(base.wk * 0.1)
    wq[0, :] = 0.0
    wk[1, :] = 0.0
    for h in range(wl.heads):
        u = h * d + d - 1
        wq[:, u] = 0.0
        wk[:, u] = 0.0
        wq[1, u] = ti.round_to_bf16(np.array([bq], np.float32))[0]
        wk[0, u] = 1.0
    return dataclasses.replace(base, x_global=x, x_aud=xa, wq=wq, wk=wk), targets


def _target_scores(inp, targets):
    """Largest score (log2 units) of each target token's query against the
    real keys of every tile holding it (tile rows and audio rows), batch 0."""
    wl = inp.workload
    d = wl.head_dim
    p = oracle.plan(wl.grid, wl.tiling, inp.cond_pos)
    sl2 = 1.4426950408889634 / np.sqrt(d)
    worst = -np.inf
    for t in range(p.tile_id.size):
        r0, r1 = int(p.tile_row_begin[t]), int(p.tile_row_begin[t + 1])
        src = p.row_src[r0:r1]
        seq = np.concatenate([inp.x_global[0, src], inp.x_aud[0]]).astype(np.float64)
        ang = np.concatenate([oracle.rope_angles(p.row_pos[r0:r1], d),
                              np.zeros((inp.x_aud.shape[1], d // 2))])
        rows = [i for i, n in enumerate(src) if n in targets]
        for h in range(wl.heads):
            q = oracle.apply_rope((seq @ inp.wq)[:, h * d:(h + 1) * d], ang)
            k = oracle.apply_rope((seq @ inp.wk)[:, h * d:(h + 1) * d], ang)
            worst = max(worst, float((q[rows] @ k.T).max() * sl2))
    return worst


@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("score_log2,regime", [(45.0, "shift-free"), (100.0, "exact")])
def test_queries_far_below_padded_key_scores(head_dim, score_log2, regime):
    """Every real score of some queries lies near -45 (bound under the
    shift-free limit 64) or -100 (bound above it: exact online softmax), far
    below the 0 that a padded key would score.  Padded keys must weigh
    nothing on either path, unsplit and with the keys split in parts."""
    say("queries far below padding", head_dim, regime)
    inp, targets = _very_negative_inputs(head_dim, score_log2)
    worst = _target_scores(inp, targets)
    bound = max(u for u, _ in _score_bounds(inp))
    say(f"  largest target score {worst:.1f}, largest bound {bound:.1f}")
    assert worst < -30.0
    assert (bound < 64.0) if regime == "shift-free" else (bound > 64.0)
    wl = inp.workload
    p = oracle.plan(wl.grid, wl.tiling, inp.cond_pos)
    rows = np.nonzero(np.isin(p.row_src, targets))[0]
    for k in (1, 3):
        say("  key parts", k)
        s = _step(inp, kv_splits=k)
        s.run()
        _check_full(inp, s)
        r = oracle.step(inp)
        yt = _np(s.y_tiles)
        for b in range(wl.batch):
            for i in rows:
                e = rel_err(yt[b, i], r.y_tiles[b, i])
                assert np.all(np.isfinite(yt[b, i])) and e <= ATTN_TOL, (b, i, e)
