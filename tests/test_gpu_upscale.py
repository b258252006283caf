"""GPU parity of the upscale loop (tdp_renoise, tdp_blend_euler,
tdp_upscale_loop) against the float64 oracle (oracle/upscale.py).

Bars (max abs error / max abs reference per tensor, as elsewhere):
  * re-noise 1e-6 (one float32 multiply-add per element); conditioning rows
    bit-exact;
  * blend_euler 1e-5 on the updated latent, on the velocity it applied and on
    the seam sums (float32 blend, as the blend's own bar); untouched rows
    bit-exact;
  * the loop 2e-2 on the result and on its displacement from the re-noised
    latent, 3e-2 on each step's seam sums (bf16 operands in the transformer,
    as the block's 2e-2; the seam sums are differences of tile outputs, so
    they get a little more); conditioning rows bit-exact.
The 16-tile workload at width 4096 runs one step and is checked three ways:
against the composition of the separately checked entry points (bit for
bit), the oracle's seam spread of those tile outputs (1e-5), and sampled
velocities of a corner tile and its seam with the next tile against the
oracle's transformer (2e-2).
"""
import dataclasses
import sys

import numpy as np
import pytest

import oracle
import oracle.block as ob
import oracle.upscale as ou
import tdp_inputs as ti

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

RENOISE_TOL = 1e-6
BLEND_TOL = 1e-5
TOL = 2e-2
SEAM_TOL = TOL         # seam sums: the bf16 value bar (measured 1.2e-2)


def say(*a):
    print("[gpu-upscale]", *a, flush=True)
    sys.stdout.flush()


def rel_err(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    return float(np.abs(got - want).max() / max(np.abs(want).max(), 1e-30))


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda:0")


@pytest.mark.parametrize("name", ["upscale_tiny", "upscale_d128"])
def test_renoise_matches_oracle(name):
    from tiled_video_diffusion_amd import tdp
    say("renoise", name)
    up = ti.make_upscale_inputs(name)
    wl = up.block.base.workload
    N, n_dst = wl.n_gen, wl.n_gen + wl.n_cond
    x1 = np.asarray(up.block.base.x_global, np.float32)
    s0 = np.float32(up.workload.sigma0)
    x1_d, eps_d = _dev(x1), _dev(up.noise)
    x = torch.empty_like(x1_d)
    tdp.tdp_renoise(x1_d, eps_d, wl.batch, N, n_dst, wl.channels, s0, x)
    torch.cuda.synchronize()
    got = x.double().cpu().numpy()
    want = ou.renoise(x1, up.noise, s0, N)
    e = rel_err(got[:, :N], want[:, :N])
    say(f"  generated rows {e:.2e}")
    assert e <= RENOISE_TOL
    assert np.array_equal(got[:, N:], x1[:, N:])
    tdp.tdp_renoise(x1_d, eps_d, wl.batch, N, n_dst, wl.channels, s0, x1_d)   # in place
    torch.cuda.synchronize()
    assert torch.equal(x1_d, x)


BLEND_CASES = {
    "tiny": ("tiny_2x16x16", None),            # 2D overlaps, conditioning rows
    "d64": ("d64_8x32x32", None),
    "3d": ("audio_32x48x80", (8, 48, 80)),     # batch 2, 3D overlaps (up to 8 rows a token)
    "t16": ("t16_16x64x64", None),             # the 16-tile step's plan
}


@pytest.mark.parametrize("ydtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", list(BLEND_CASES))
def test_blend_euler_matches_oracle(case, ydtype):
    from tiled_video_diffusion_amd import tdp
    name, grid = BLEND_CASES[case]
    say("blend_euler", case, ydtype)
    inp = ti.make_inputs(name)
    wl = inp.workload if grid is None else dataclasses.replace(inp.workload, grid=grid)
    p = tdp.tdp_plan(wl.grid, wl.tiling, inp.cond_pos)
    po = oracle.plan(wl.grid, wl.tiling, inp.cond_pos)
    N = int(np.prod(wl.grid))
    n_dst, B, C = p.n_dst_rows, wl.batch, wl.channels
    rng = np.random.default_rng(3)
    y = rng.standard_normal((B, p.n_rows, C), dtype=np.float32)
    if ydtype == "bf16":
        y = ti.round_to_bf16(y)
    x = rng.standard_normal((B, n_dst, C), dtype=np.float32)
    sig, sig_next = np.float32(0.6), np.float32(0.45)
    y_d = _dev(y, torch.bfloat16 if ydtype == "bf16" else torch.float32)
    code = tdp.TDP_BF16 if ydtype == "bf16" else tdp.TDP_F32
    x_d = _dev(x)
    drb, dr, rw = _dev(p.dst_row_begin), _dev(p.dst_rows), _dev(p.row_weight)
    ws_bytes = tdp.tdp_blend_euler_workspace(B, N, C)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda:0")
    seam = torch.zeros(3, dtype=torch.float64, device="cuda:0")
    x_plain = x_d.clone()
    tdp.tdp_blend_euler(y_d, code, B, p.n_rows, C, drb, dr, rw, N, x_d, n_dst, sig, sig_next,
                        seam, ws, ws_bytes)
    tdp.tdp_blend_euler(y_d, code, B, p.n_rows, C, drb, dr, rw, N, x_plain, n_dst, sig, sig_next,
                        None, None, 0)
    torch.cuda.synchronize()
    got = x_d.double().cpu().numpy()
    v = oracle.blend_tiles(y, po)
    want = ou.euler_step(x, v, sig, sig_next, N)
    e_x = rel_err(got[:, :N], want[:, :N])
    dsig = np.float64(sig_next) - np.float64(sig)
    e_v = rel_err((got[:, :N] - x[:, :N]) / dsig, v[:, :N])
    s = seam.cpu().numpy()
    s2, s0 = ou.seam_spread(y, po, N)
    e_s2, e_s0 = abs(s[0] - s2) / s2, abs(s[1] - s0) / s0
    say(f"  x {e_x:.2e}  v {e_v:.2e}  S2 {e_s2:.2e}  S0 {e_s0:.2e}  spread {s[2]:.4f}")
    assert e_x <= BLEND_TOL and e_v <= BLEND_TOL
    assert e_s2 <= BLEND_TOL and e_s0 <= BLEND_TOL
    assert s[2] == pytest.approx(np.sqrt(s[0] / s[1]), rel=1e-12)
    assert np.array_equal(got[:, N:], x[:, N:])          # conditioning rows untouched
    assert torch.equal(x_plain, x_d)                     # the seam does not change the update


def test_blend_euler_agreeing_tiles_have_no_spread():
    """Tile outputs that are the gathered latent agree on every overlap."""
    from tiled_video_diffusion_amd import tdp
    inp = ti.make_inputs("tiny_2x16x16")
    wl = inp.workload
    p = tdp.tdp_plan(wl.grid, wl.tiling, inp.cond_pos)
    N = wl.n_gen
    x = np.asarray(inp.x_global, np.float32)
    y = np.ascontiguousarray(x[:, p.row_src])
    ws_bytes = tdp.tdp_blend_euler_workspace(wl.batch, N, wl.channels)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda:0")
    seam = torch.full((3,), -1.0, dtype=torch.float64, device="cuda:0")
    x_d = _dev(x)
    tdp.tdp_blend_euler(_dev(y), tdp.TDP_F32, wl.batch, p.n_rows, wl.channels,
                        _dev(p.dst_row_begin), _dev(p.dst_rows), _dev(p.row_weight), N, x_d,
                        p.n_dst_rows, 0.5, 0.25, seam, ws, ws_bytes)
    torch.cuda.synchronize()
    s = seam.cpu().numpy()
    say(f"agreeing tiles: S2 {s[0]:.3e} S0 {s[1]:.3e}")
    assert s[1] > 0 and s[0] <= 1e-10 * s[1]
    got = x_d.double().cpu().numpy()
    assert rel_err(got[:, :N], 0.75 * x[:, :N].astype(np.float64)) <= BLEND_TOL


def _loop(up, sigmas=None):
    from tiled_video_diffusion_amd.step import UpscaleLoop
    L = UpscaleLoop(up, sigmas=sigmas)
    L.renoise()
    x0 = L.x.clone()
    L.loop()
    torch.cuda.synchronize()
    return L, x0


@pytest.mark.parametrize("name", ["upscale_tiny", "upscale_d128"])
def test_upscale_loop_matches_oracle(name):
    say("loop", name)
    up = ti.make_upscale_inputs(name)
    L, x0 = _loop(up)
    binp = up.block
    wl = binp.base.workload
    N = wl.n_gen
    po = oracle.plan(wl.grid, wl.tiling, binp.base.cond_pos)
    ref = ou.upscale_loop(binp.base.x_global, up.noise, L.sigmas, N, ou.tdp_velocity(binp, po))
    got = L.x.double().cpu().numpy()
    x0 = x0.double().cpu().numpy()
    e_x = rel_err(got[:, :N], ref.x[:, :N])
    e_d = rel_err(got[:, :N] - x0[:, :N], ref.x[:, :N] - ref.states[0][:, :N])
    say(f"  x {e_x:.2e}  displacement {e_d:.2e}")
    assert e_x <= TOL and e_d <= TOL
    assert np.array_equal(got[:, N:], np.asarray(binp.base.x_global, np.float32)[:, N:])
    seam = L.seam.cpu().numpy()
    assert len(ref.seam) == L.n_steps
    for i, (s2, s0) in enumerate(ref.seam):
        e2, e0 = abs(seam[i, 0] - s2) / s2, abs(seam[i, 1] - s0) / s0
        say(f"  step {i}: spread {seam[i, 2]:.4f} (oracle {ou.relative_spread(s2, s0):.4f})"
            f"  S2 {e2:.2e}  S0 {e0:.2e}")
        assert e2 <= SEAM_TOL and e0 <= SEAM_TOL


@pytest.mark.parametrize("sigma0", [0.1, 0.9])
def test_upscale_loop_first_sigma_sweep(sigma0):
    """Drift is tied to the first sigma: from other first sigmas than the
    workload's, the same number of linear steps still matches the oracle in
    the latent and in every step's seam sums."""
    say("loop upscale_tiny sigma0", sigma0)
    up = ti.make_upscale_inputs("upscale_tiny")
    n = up.workload.n_steps
    from tiled_video_diffusion_amd import tdp
    sig = tdp.tdp_linear_sigmas(sigma0, n)
    assert np.array_equal(sig, ou.linear_sigmas(sigma0, n))
    L, x0 = _loop(up, sigmas=sig)
    binp = up.block
    wl = binp.base.workload
    N = wl.n_gen
    po = oracle.plan(wl.grid, wl.tiling, binp.base.cond_pos)
    ref = ou.upscale_loop(binp.base.x_global, up.noise, L.sigmas, N, ou.tdp_velocity(binp, po))
    got = L.x.double().cpu().numpy()
    e_x = rel_err(got[:, :N], ref.x[:, :N])
    e_d = rel_err(got[:, :N] - x0.double().cpu().numpy()[:, :N], ref.x[:, :N] - ref.states[0][:, :N])
    say(f"  x {e_x:.2e}  displacement {e_d:.2e}")
    assert e_x <= TOL and e_d <= TOL
    seam = L.seam.cpu().numpy()
    assert len(ref.seam) == n
    for i, (s2, s0) in enumerate(ref.seam):
        e2, e0 = abs(seam[i, 0] - s2) / s2, abs(seam[i, 1] - s0) / s0
        say(f"  step {i}: spread {seam[i, 2]:.4f} (oracle {ou.relative_spread(s2, s0):.4f})"
            f"  S2 {e2:.2e}  S0 {e0:.2e}")
        assert e2 <= SEAM_TOL and e0 <= SEAM_TOL


def test_upscale_loop_edge_schedules():
    """No steps leaves the re-noised latent; sigma 0 throughout leaves the
    stage-1 latent; a non-uniform schedule matches the oracle."""
    up = ti.make_upscale_inputs("upscale_tiny")
    binp = up.block
    wl = binp.base.workload
    N = wl.n_gen
    x1 = np.asarray(binp.base.x_global, np.float32)
    L, x0 = _loop(up, sigmas=np.array([0.4], np.float32))
    assert torch.equal(L.x, x0)
    L, _ = _loop(up, sigmas=np.zeros(3, np.float32))
    assert np.array_equal(L.x.cpu().numpy(), x1)
    sig = np.array([0.7, 0.3, 0.05], np.float32)
    L, _ = _loop(up, sigmas=sig)
    po = oracle.plan(wl.grid, wl.tiling, binp.base.cond_pos)
    ref = ou.upscale_loop(binp.base.x_global, up.noise, sig, N, ou.tdp_velocity(binp, po))
    e = rel_err(L.x.double().cpu().numpy()[:, :N], ref.x[:, :N])
    say(f"non-uniform schedule: x {e:.2e}")
    assert e <= TOL


def test_upscale_loop_is_deterministic():
    up = ti.make_upscale_inputs("upscale_tiny")
    L, _ = _loop(up)
    x, seam = L.x.clone(), L.seam.clone()
    for _ in range(2):
        L.run()
        torch.cuda.synchronize()
        assert torch.equal(L.x, x) and torch.equal(L.seam, seam)


def test_upscale_loop_full_width_one_step():
    from tiled_video_diffusion_amd import tdp
    say("loop t16, one step")
    uw = dataclasses.replace(ti.UPSCALE_WORKLOADS["upscale_t16"], n_steps=1)
    up = ti.make_upscale_inputs(uw)
    L, x0 = _loop(up)
    bs, s, p = L.bs, L.bs.s, L.bs.plan
    wl = up.block.base.workload
    B, C, N, R = wl.batch, wl.channels, wl.n_gen, p.n_rows
    sig = L.sigmas
    # (a) the composition of gather, block forward and blend_euler, bit for bit
    xt = torch.empty((B, R, C), dtype=torch.float32, device="cuda:0")
    yt = torch.empty_like(xt)
    tdp.tdp_gather_tiles(x0, tdp.TDP_F32, B, L.n_dst, C, s.row_src, R, xt)
    wsb_bytes = tdp.tdp_block_workspace(L.desc, p.n_tiles_local, R)
    wsb = torch.empty(wsb_bytes, dtype=torch.uint8, device="cuda:0")
    tau = torch.full((B,), float(np.float32(1000.0) * sig[0]), dtype=torch.float32,
                     device="cuda:0")
    tdp.tdp_block_forward(L.desc, p.n_tiles_local, s.tile_row_begin, p.max_tile_rows, R, xt,
                          s.row_pos, bs.text, tau, bs.weights, yt, wsb, wsb_bytes)
    wsb = None
    x_c = x0.clone()
    seam_c = torch.zeros(3, dtype=torch.float64, device="cuda:0")
    wse_bytes = tdp.tdp_blend_euler_workspace(B, N, C)
    wse = torch.empty(wse_bytes, dtype=torch.uint8, device="cuda:0")
    tdp.tdp_blend_euler(yt, tdp.TDP_F32, B, R, C, s.dst_row_begin, s.dst_rows, s.row_weight, N,
                        x_c, L.n_dst, sig[0], sig[1], seam_c, wse, wse_bytes)
    torch.cuda.synchronize()
    assert torch.equal(x_c, L.x) and torch.equal(seam_c, L.seam[0])
    # (b) the seam spread of those tile outputs
    po = oracle.plan(wl.grid, wl.tiling, up.block.base.cond_pos)
    s2, s0 = ou.seam_spread(yt.double().cpu().numpy(), po, N)
    seam = L.seam[0].cpu().numpy()
    e2, e0 = abs(seam[0] - s2) / s2, abs(seam[1] - s0) / s0
    say(f"  seam spread {seam[2]:.4f}  S2 {e2:.2e}  S0 {e0:.2e}")
    assert e2 <= BLEND_TOL and e0 <= BLEND_TOL
    # (c) sampled velocities: tokens of the corner tile 0 alone and on its seam with tile 1
    x0_ref = ou.renoise(up.block.base.x_global, up.noise, sig[0], N)
    v_gpu = (x0.double().cpu().numpy()[0] - L.x.double().cpu().numpy()[0]) / np.float64(sig[0])
    tb = po.tile_row_begin
    cnt = np.diff(po.dst_row_begin)
    tok0 = po.row_src[tb[0]:tb[1]]
    tok1 = set(po.row_src[tb[1]:tb[2]].tolist())
    rng = np.random.default_rng(13)
    alone = rng.choice(tok0[cnt[tok0] == 1], 6, replace=False)
    shared = rng.choice(np.array([n for n in tok0 if cnt[n] == 2 and n in tok1]), 6,
                        replace=False)
    toks = np.concatenate([alone, shared])
    model = ob.model_from_inputs(up.block)
    tau_ref = 1000.0 * np.float64(sig[0])
    v_ref = np.zeros((toks.size, C))
    x_tiles = oracle.gather_tiles(x0_ref, po)[0]
    for t in (0, 1):
        r0, r1 = int(tb[t]), int(tb[t + 1])
        local = {int(n): i for i, n in enumerate(po.row_src[r0:r1])}
        pick = [(k, local[int(n)]) for k, n in enumerate(toks) if int(n) in local]
        rows = np.array(sorted({q for _, q in pick}))
        y = ob.tile_transformer(x_tiles[r0:r1], po.row_pos[r0:r1], up.block.text[0], tau_ref,
                                model, query_rows=rows)
        at = {q: i for i, q in enumerate(rows)}
        for k, q in pick:
            v_ref[k] += np.float64(po.row_weight[r0 + q]) * y[at[q]]
    e = rel_err(v_gpu[toks], v_ref)
    say(f"  sampled velocities ({toks.size} tokens): {e:.2e}")
    assert e <= TOL


def test_edge_cases():
    """renoise at sigma 0 and 1 (closed forms), blend_euler with no generated
    tokens (x untouched, seam sums zero)."""
    from tiled_video_diffusion_amd import tdp
    rng = np.random.default_rng(9)
    x1 = rng.standard_normal((2, 7, 8)).astype(np.float32)
    eps = rng.standard_normal((2, 5, 8)).astype(np.float32)
    x1_d, eps_d = _dev(x1), _dev(eps)
    x = torch.empty_like(x1_d)
    tdp.tdp_renoise(x1_d, eps_d, 2, 5, 7, 8, 0.0, x)
    torch.cuda.synchronize()
    assert np.array_equal(x.cpu().numpy(), x1)
    tdp.tdp_renoise(x1_d, eps_d, 2, 5, 7, 8, 1.0, x)
    torch.cuda.synchronize()
    got = x.cpu().numpy()
    assert np.array_equal(got[:, :5], eps) and np.array_equal(got[:, 5:], x1[:, 5:])
    # no generated tokens: only conditioning rows, nothing updated
    ws_bytes = max(tdp.tdp_blend_euler_workspace(1, 0, 128), 256)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda:0")
    seam = torch.full((3,), -1.0, dtype=torch.float64, device="cuda:0")
    xc = _dev(rng.standard_normal((1, 4, 128)).astype(np.float32))
    before = xc.clone()
    drb = torch.zeros(5, dtype=torch.int64, device="cuda:0")
    tdp.tdp_blend_euler(None, tdp.TDP_F32, 1, 0, 128, drb, None, None, 0, xc, 4, 0.5, 0.25, seam,
                        ws, ws_bytes)
    torch.cuda.synchronize()
    assert torch.equal(xc, before)
    assert seam.cpu().tolist() == [0.0, 0.0, 0.0]
