"""GPU parity of the per-tile transformer block (tdp_block_forward) against the
float64 oracle (oracle/block.py).

Bar: 2e-2, max abs error / max abs reference per output tensor, as for the
attention layer (bf16 operands, one more bf16 rounding of Q/K/V between the
projection and the attention core, float32 residual stream).  The 16-tile
workload at width 4096 is checked on sampled rows of two tiles.
"""
import dataclasses
import sys

import numpy as np
import pytest

import oracle
import oracle.block as ob
import tdp_inputs as ti

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-2
BLEND_TOL = 1e-5


def say(*a):
    print("[gpu-block]", *a, flush=True)
    sys.stdout.flush()


def rel_err(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    return float(np.abs(got - want).max() / max(np.abs(want).max(), 1e-30))


def _run(binp, **kw):
    from tiled_video_diffusion_amd.step import BlockStep
    s = BlockStep(binp, **kw)
    s.run()
    torch.cuda.synchronize()
    return s


@pytest.mark.parametrize("name", ["block_tiny", "block_d128"])
def test_block_step_full(name):
    say("block step", name)
    binp = ti.make_block_inputs(name)
    s = _run(binp)
    ref = ob.block_step(binp)
    yt = s.y_tiles.double().cpu().numpy()
    e_t = rel_err(yt, ref.y_tiles)
    e_g = rel_err(s.y_global.double().cpu().numpy(), ref.y_global)
    e_b = rel_err(s.y_global.double().cpu().numpy(), oracle.blend_tiles(yt, ref.plan))
    say(f"  y_tiles {e_t:.2e}  y_global {e_g:.2e}  blend {e_b:.2e}")
    assert e_t <= TOL and e_g <= TOL and e_b <= BLEND_TOL


def test_block_no_layers_and_three_layers():
    for layers in (0, 3):
        bw = dataclasses.replace(ti.BLOCK_WORKLOADS["block_tiny"], layers=layers)
        say("block layers", layers)
        binp = ti.make_block_inputs(bw)
        s = _run(binp)
        ref = ob.block_step(binp)
        e = rel_err(s.y_tiles.double().cpu().numpy(), ref.y_tiles)
        say(f"  y_tiles {e:.2e}")
        assert e <= TOL


def test_block_batch2_ragged_text():
    """Batch 2 (per-entry timestep and text), 37 text tokens, bf16 latent, head_dim 64."""
    bw = ti.BlockWorkload("block_b2", base="d64_8x32x32", layers=1, n_text=37, heads=4)
    base = dataclasses.replace(bw.base_workload(), batch=2, grid=(2, 24, 20),
                               tiling=((1, 0), (2, 6), (2, 4)))
    say("block batch 2")
    binp = ti.make_block_inputs(bw)
    binp = dataclasses.replace(binp, base=ti.make_inputs(base))
    rng = np.random.default_rng(5)
    binp.text = ti.round_to_bf16(rng.standard_normal((2, 37, base.hidden), dtype=np.float32))
    binp.tau = np.array([3.5, 870.0], dtype=np.float32)
    s = _run(binp)
    ref = ob.block_step(binp)
    e = rel_err(s.y_tiles.double().cpu().numpy(), ref.y_tiles)
    say(f"  y_tiles {e:.2e}")
    assert e <= TOL


def test_block_runs_are_deterministic():
    binp = ti.make_block_inputs("block_d128")
    s = _run(binp)
    first = s.y_global.clone()
    for _ in range(3):
        s.run()
        torch.cuda.synchronize()
        assert torch.equal(first, s.y_global)


def test_block_full_width_sampled():
    """The 16-tile step at width 4096 (one block): sampled rows of two corner
    tiles and an interior tile against the oracle (every row gives keys and
    values).  The last tile's rows are in the large GEMMs' claimed tail of
    tiles (the last ~1/12 of the tile order), which each of the block's GEMM
    launches takes through one shared counter."""
    say("block t16 sampled")
    binp = ti.make_block_inputs("block_t16")
    s = _run(binp)
    wl = binp.base.workload
    p = oracle.plan(wl.grid, wl.tiling, binp.base.cond_pos)
    x = oracle.gather_tiles(binp.base.x_global, p)[0]
    yt = s.y_tiles.double().cpu().numpy()[0]
    model = ob.model_from_inputs(binp)
    rng = np.random.default_rng(11)
    for t in (0, 5, p.tile_id.size - 1):
        r0, r1 = int(p.tile_row_begin[t]), int(p.tile_row_begin[t + 1])
        rows = np.array(sorted({0, r1 - r0 - 1, 127, 128} |
                               set(rng.integers(0, r1 - r0, size=12).tolist())))
        want = ob.tile_transformer(x[r0:r1], p.row_pos[r0:r1], binp.text[0], float(binp.tau[0]),
                                   model, query_rows=rows)
        e = rel_err(yt[r0 + rows], want)
        say(f"  tile {t} rows {rows.size}: {e:.2e}")
        assert e <= TOL
    e_b = rel_err(s.y_global.double().cpu().numpy(), oracle.blend_tiles(
        s.y_tiles.double().cpu().numpy(), p))
    assert e_b <= BLEND_TOL
