"""The C ABI on the CPU: exported symbols, host plan bit-parity with the oracle,
status codes for invalid arguments.  No GPU work is launched: device entry
points are only called with arguments that fail validation on the host.
"""
import ctypes
import dataclasses

import numpy as np
import pytest

import oracle
import tdp_inputs as ti
from tiled_video_diffusion_amd import tdp

PLAN_FIELDS = ["tile_id", "tile_box", "tile_offset", "tile_row_begin", "tile_n_gen", "row_src",
               "row_weight", "row_pos", "cond_keep_count", "dst_row_begin", "dst_rows"]


def test_library_exports_every_declared_symbol():
    names = tdp.declared_symbols()
    assert len(names) >= 12
    L = tdp.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(tdp._SIGS)


def test_status_strings():
    for code in range(-7, 1):
        assert tdp.status_string(code) and tdp.status_string(code) != "unknown status"
    assert tdp.status_string(-99) == "unknown status"


def _assert_same_plan(pc, po):
    for f in PLAN_FIELDS:
        a, b = getattr(pc, f), getattr(po, f)
        assert a.dtype == b.dtype, f
        assert a.shape == b.shape, (f, a.shape, b.shape)
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f   # bit-exact
    assert pc.n_rows == po.n_rows and pc.max_tile_rows == po.max_tile_rows


@pytest.mark.parametrize("name", [n for n in ti.WORKLOADS if n != "blend_32x96x160"])
@pytest.mark.parametrize("normalize", [True, False])
def test_plan_bit_exact_vs_oracle(name, normalize):
    inp = ti.make_inputs(name)
    wl = inp.workload
    pc = tdp.tdp_plan(wl.grid, wl.tiling, inp.cond_pos, normalize)
    po = oracle.plan(wl.grid, wl.tiling, inp.cond_pos, normalize)
    _assert_same_plan(pc, po)
    assert pc.n_tiles_total == po.n_tiles_total


def test_plan_bit_exact_blend_workload():
    wl = ti.workload("blend_32x96x160")
    wl = dataclasses.replace(wl, grid=(4,) + wl.grid[1:])       # same tiling, fewer frames
    pc = tdp.tdp_plan(wl.grid, wl.tiling)
    po = oracle.plan(wl.grid, wl.tiling)
    _assert_same_plan(pc, po)


@pytest.mark.parametrize("assignment", ["round_robin", "longest_first"])
@pytest.mark.parametrize("W", [2, 3, 4, 7])
def test_plan_bit_exact_multi_rank(W, assignment):
    inp = ti.make_inputs("audio_32x48x80")
    wl = dataclasses.replace(inp.workload, grid=(8, 48, 80))
    for r in range(W):
        pc = tdp.tdp_plan(wl.grid, wl.tiling, inp.cond_pos, True, W, r, assignment)
        po = oracle.plan(wl.grid, wl.tiling, inp.cond_pos, True, W, r, assignment)
        _assert_same_plan(pc, po)


@pytest.mark.parametrize("W", [3, 4, 5])
def test_plan_bit_exact_longest_first_t16(W):
    inp = ti.make_inputs("t16_16x64x64")
    wl = inp.workload
    for r in range(W):
        pc = tdp.tdp_plan(wl.grid, wl.tiling, None, True, W, r, "longest_first")
        po = oracle.plan(wl.grid, wl.tiling, None, True, W, r, "longest_first")
        _assert_same_plan(pc, po)


def _random_case(rng):
    grid = [int(rng.integers(1, 13)) for _ in range(3)]
    tiling = []
    for L in grid:
        n = int(rng.integers(1, min(L, 4) + 1))
        core = L // n
        o = int(rng.integers(0, core + 1)) if n > 1 else int(rng.integers(0, 3))
        tiling.append((n, o))
    M = int(rng.integers(0, 7))
    cond = np.zeros((M, 3, 2), np.float32)
    for j in range(M):
        for d in range(3):
            s = float(rng.integers(-3, grid[d] + 2))
            cond[j, d] = (s, s + float(rng.integers(0, 4)))
    return grid, tiling, cond


def test_plan_bit_exact_random_descriptors():
    rng = np.random.default_rng(77)
    for _ in range(150):
        grid, tiling, cond = _random_case(rng)
        W = int(rng.integers(1, 4))
        r = int(rng.integers(0, W))
        norm = bool(rng.integers(0, 2))
        asg = "longest_first" if rng.integers(0, 2) else "round_robin"
        pc = tdp.tdp_plan(grid, tiling, cond, norm, W, r, asg)
        po = oracle.plan(grid, tiling, cond, norm, W, r, asg)
        _assert_same_plan(pc, po)


def test_plan_fractional_cond_positions():
    cond = np.array([[[0.5, 1.25], [3.5, 7.75], [-0.5, 2.0]],
                     [[-0.25, 0.5], [10.0, 10.0], [0.0, 0.5]]], np.float32)
    grid, tiling = (3, 12, 10), ((1, 0), (2, 3), (2, 5))
    _assert_same_plan(tdp.tdp_plan(grid, tiling, cond), oracle.plan(grid, tiling, cond))


@pytest.mark.parametrize("grid,tiling,cond,world,rank,code", [
    ((0, 4, 4), ((1, 0), (1, 0), (1, 0)), None, 1, 0, -2),
    ((2, 4, 4), ((1, 0), (5, 0), (1, 0)), None, 1, 0, -2),
    ((2, 4, 4), ((1, 0), (0, 0), (1, 0)), None, 1, 0, -2),
    ((2, 8, 8), ((1, 0), (2, 5), (1, 0)), None, 1, 0, -2),
    ((2, 8, 8), ((1, 0), (2, -1), (1, 0)), None, 1, 0, -2),
    ((2, 8, 8), ((1, 0), (2, 2), (1, 0)), None, 0, 0, -2),
    ((2, 8, 8), ((1, 0), (2, 2), (1, 0)), None, 2, 2, -2),
    ((2, 8, 8), ((1, 0), (2, 2), (1, 0)), [[[0, np.nan], [0, 1], [0, 1]]], 1, 0, -2),
    ((2, 8, 8), ((1, 0), (2, 2), (1, 0)), [[[2, 1], [0, 1], [0, 1]]], 1, 0, -2),
])
def test_plan_rejects_invalid(grid, tiling, cond, world, rank, code):
    cond = None if cond is None else np.array(cond, np.float32)
    with pytest.raises(tdp.TdpError) as e:
        tdp.tdp_plan_query(grid, tiling, cond, True, world, rank)
    assert e.value.status == code
    with pytest.raises(oracle.PlanError):
        oracle.plan(grid, tiling, cond, True, world, rank)


def test_plan_rejects_unknown_assignment():
    d, _ = tdp._desc((2, 8, 8), ((1, 0), (2, 2), (1, 0)), None, True, 2, 0)
    d.assignment = 2
    s = tdp.PlanSizes()
    assert tdp.lib().tdp_plan_query(ctypes.byref(d), ctypes.byref(s)) == -2


def test_plan_null_and_shape_errors():
    L = tdp.lib()
    s = tdp.PlanSizes()
    assert L.tdp_plan_query(None, ctypes.byref(s)) == -1
    d, _ = tdp._desc((2, 8, 8), ((1, 0), (2, 2), (1, 0)), None, True, 1, 0)
    assert L.tdp_plan_query(ctypes.byref(d), None) == -1
    d.n_cond = 3                                          # M > 0 with NULL positions
    assert L.tdp_plan_query(ctypes.byref(d), ctypes.byref(s)) == -1
    d.n_cond = 0
    assert L.tdp_plan_query(ctypes.byref(d), ctypes.byref(s)) == 0
    out = tdp.PlanOut()
    assert L.tdp_plan(ctypes.byref(d), ctypes.byref(s), ctypes.byref(out)) == -1
    s.n_rows += 1                                         # sizes that disagree with desc
    assert L.tdp_plan(ctypes.byref(d), ctypes.byref(s), ctypes.byref(out)) == -3


# --- device entry points: host-side validation only (nothing is launched) ---

FAKE = 1 << 20          # a non-null, 16-byte aligned value that is never dereferenced


def test_gather_validation():
    L = tdp.lib()
    assert L.tdp_gather_tiles(FAKE, 5, 1, 10, 128, FAKE, 4, FAKE, None) == -4   # dtype
    assert L.tdp_gather_tiles(FAKE, 0, 0, 10, 128, FAKE, 4, FAKE, None) == -2   # batch
    assert L.tdp_gather_tiles(FAKE, 0, 1, 10, 12, FAKE, 4, FAKE, None) == -2    # C % 8
    assert L.tdp_gather_tiles(None, 0, 1, 10, 128, FAKE, 4, FAKE, None) == -1
    assert L.tdp_gather_tiles(FAKE + 4, 0, 1, 10, 128, FAKE, 4, FAKE, None) == -7
    assert L.tdp_gather_tiles(None, 0, 1, 10, 128, None, 0, None, None) == 0     # empty: no-op


def test_blend_validation():
    L = tdp.lib()
    assert L.tdp_blend_accumulate(FAKE, 0, 1, 4, 128, FAKE, FAKE, FAKE, 4, FAKE, 2, None) == -2
    assert L.tdp_blend_accumulate(FAKE, 3, 1, 4, 128, FAKE, FAKE, FAKE, 4, FAKE, 0, None) == -4
    assert L.tdp_blend_accumulate(FAKE, 0, 1, 4, 128, None, FAKE, FAKE, 4, FAKE, 0, None) == -1
    assert L.tdp_blend_accumulate(FAKE, 0, 1, 4, 128, FAKE, FAKE, FAKE, 4, FAKE + 8, 0, None) == -7
    assert L.tdp_blend_accumulate(None, 0, 1, 0, 128, None, None, None, 0, None, 0, None) == 0
    assert L.tdp_audio_accumulate(FAKE, 3, 2, 1, 4, 128, FAKE, 0, None) == -2   # local > total
    assert L.tdp_audio_accumulate(None, 2, 2, 1, 4, 128, FAKE, 0, None) == -1
    assert L.tdp_audio_accumulate(None, 0, 2, 1, 0, 128, None, 0, None) == 0


def test_attention_validation():
    L = tdp.lib()
    good = tdp.attn_desc(1, 128, 2, 64, 0, 0, 0)
    n = ctypes.c_size_t()
    assert L.tdp_tile_attention_workspace(ctypes.byref(good), 4, 800, ctypes.byref(n)) == 0
    ws = n.value
    assert ws > 0
    for field, val, code in [("C", 64, -4), ("head_dim", 96, -4), ("heads", 0, -2),
                             ("batch", 0, -2), ("x_dtype", 7, -4), ("n_audio", -1, -2),
                             ("rope_base", 0.0, -2)]:
        d = tdp.attn_desc(1, 128, 2, 64, 0, 0, 0)
        setattr(d, field, val)
        assert L.tdp_tile_attention_workspace(ctypes.byref(d), 4, 800, ctypes.byref(n)) == code
    args = lambda **k: dict(dict(desc=ctypes.byref(good), T=4, trb=FAKE, maxr=200, rows=800,  # noqa
                                 x=FAKE, pos=FAKE, wq=FAKE, wk=FAKE, wv=FAKE, wo=FAKE, xa=None,
                                 y=FAKE, ya=None, ws=FAKE, wsb=ws, s=None), **k)

    def call(**k):
        a = args(**k)
        return L.tdp_tile_attention(*a.values())
    assert call(wsb=ws - 1) == -5
    assert call(wq=None) == -1
    assert call(trb=None) == -1
    assert call(maxr=0) == -2
    assert call(maxr=801) == -2
    assert call(ws=FAKE + 2) == -7
    assert call(T=0) == -2
    audio = tdp.attn_desc(1, 128, 2, 64, 16, 0, 0)
    assert L.tdp_tile_attention_workspace(ctypes.byref(audio), 4, 800, ctypes.byref(n)) == 0
    assert call(desc=ctypes.byref(audio), wsb=n.value) == -1       # audio without buffers
    assert L.tdp_attn_core(ctypes.byref(good), 4, FAKE, 200, 800, None, ws, None) == -1
    assert L.tdp_attn_out_proj(ctypes.byref(good), 4, FAKE, 200, 800, None, None, FAKE, ws,
                               None) == -1


def test_attention_kv_splits_field():
    """kv_splits: 0..8 accepted, others rejected; forced parts add their fp32
    partial results to the workspace; the automatic choice never splits a
    launch that already fills the GPU and splits the sequence-parallel share
    (one 6144-row tile, 4 heads of 128: 96 query blocks) into 2 parts."""
    L = tdp.lib()
    n = ctypes.c_size_t()

    def ws(heads, hd, T, R, k):
        d = tdp.attn_desc(1, 128, heads, hd, 0, 0, 0, 10000.0, k)
        st = L.tdp_tile_attention_workspace(ctypes.byref(d), T, R, ctypes.byref(n))
        return st if st else n.value
    for bad in (-1, 9, 100):
        assert ws(2, 64, 4, 800, bad) == -2
    one = ws(4, 128, 1, 6144, 1)
    eight = ws(4, 128, 1, 6144, 8)
    parts = 96 * 8 * 256                               # slots x parts x rows
    assert eight - one >= parts * (128 * 4 + 8)
    assert eight - one < parts * (128 * 4 + 8) + 1024
    two = ws(4, 128, 1, 6144, 2)
    assert two - one >= 96 * 2 * 256 * (128 * 4 + 8)
    assert ws(4, 128, 1, 6144, 0) == two               # automatic: 2 parts
    # the other measured shares: 2 heads (48 query blocks) take 5 parts,
    # 8 heads (192 query blocks) none
    assert ws(2, 128, 1, 6144, 0) == ws(2, 128, 1, 6144, 5)
    assert ws(8, 128, 1, 6144, 0) == ws(8, 128, 1, 6144, 1)
    big = dict(heads=32, hd=128, T=16, R=16 * 4096)    # 16 tiles of 4096 rows, 32 heads
    assert ws(k=0, **big) == ws(k=1, **big)            # automatic: unsplit


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(tdp, "_lib", None)
    monkeypatch.setattr(tdp, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError):
        tdp.tdp_plan_query((2, 4, 4), ((1, 0), (1, 0), (1, 0)))


def test_balanced_split_matches_oracle():
    for n in range(1, 5001):
        assert tdp.tdp_balanced_tile_split(n) == oracle.balanced_tile_split(n), n
    L = tdp.lib()
    h, w = ctypes.c_int32(), ctypes.c_int32()
    for n in [0, -1, -100]:
        assert L.tdp_balanced_tile_split(n, ctypes.byref(h), ctypes.byref(w)) == -2   # TDP_ERR_ARG
    assert L.tdp_balanced_tile_split(4, None, ctypes.byref(w)) == -1                  # TDP_ERR_NULL
    assert L.tdp_balanced_tile_split(4, ctypes.byref(h), None) == -1


def test_block_validation():
    ok = dict(batch=1, C_=128, heads=2, head_dim=64, n_text=16, layers=2,
              x_dtype=tdp.TDP_F32, y_dtype=tdp.TDP_F32)
    assert tdp.tdp_block_workspace(tdp.block_desc(**ok), 4, 520) > 0
    bad = [(dict(C_=64), -4), (dict(head_dim=96), -4), (dict(heads=3), -4),   # D = 192
           (dict(n_text=0), -2), (dict(layers=-1), -2), (dict(batch=0), -2),
           (dict(x_dtype=7), -4)]
    L = tdp.lib()
    n = ctypes.c_size_t()
    for kw, code in bad:
        d = tdp.block_desc(**{**ok, **kw})
        assert L.tdp_block_workspace(ctypes.byref(d), 4, 520, ctypes.byref(n)) == code, kw
    d = tdp.block_desc(**ok, time_dim=100)
    assert L.tdp_block_workspace(ctypes.byref(d), 4, 520, ctypes.byref(n)) == -2
    # missing pointers fail before any launch
    w = tdp.BlockWeights()
    d = tdp.block_desc(**ok)
    assert L.tdp_block_forward(ctypes.byref(d), 4, None, 130, 520, None, None, None, None,
                               ctypes.byref(w), None, None, 0, None) == -1


@pytest.mark.parametrize("sigma0,n_steps", [(0.3, 3), (1.0, 4), (0.5, 1), (0.7, 0), (0.123, 7),
                                            (0.0, 2)])
def test_linear_sigmas_match_oracle_bitwise(sigma0, n_steps):
    import oracle.upscale as ou
    assert np.array_equal(tdp.tdp_linear_sigmas(sigma0, n_steps), ou.linear_sigmas(sigma0, n_steps))


def test_upscale_validation():
    L = tdp.lib()
    n = ctypes.c_size_t()
    out = (ctypes.c_float * 4)()
    assert L.tdp_linear_sigmas(1.5, 3, out) == -2
    assert L.tdp_linear_sigmas(0.5, -1, out) == -2
    assert L.tdp_linear_sigmas(float("nan"), 3, out) == -2
    assert L.tdp_linear_sigmas(0.5, 3, None) == -1
    # re-noise: sigma outside [0, 1], missing buffers, C not a multiple of 4
    assert L.tdp_renoise(None, None, 1, 8, 10, 128, 1.5, None, None) == -2
    assert L.tdp_renoise(None, None, 1, 8, 10, 128, 0.5, None, None) == -1
    assert L.tdp_renoise(None, None, 1, 8, 10, 126, 0.5, None, None) == -2
    assert L.tdp_renoise(None, None, 1, 11, 10, 128, 0.5, None, None) == -2   # n_gen > n_dst
    # blend_euler: workspace sizes and argument checks
    assert tdp.tdp_blend_euler_workspace(1, 512, 128) >= 64 * 8
    assert L.tdp_blend_euler_workspace(0, 512, 128, ctypes.byref(n)) == -2
    assert L.tdp_blend_euler(None, 5, 1, 10, 128, None, None, None, 8, None, 10, 0.5, 0.25, None,
                             None, 0, None) == -4
    assert L.tdp_blend_euler(None, 0, 1, 10, 128, None, None, None, 11, None, 10, 0.5, 0.25,
                             None, None, 0, None) == -2
    assert L.tdp_blend_euler(None, 0, 1, 10, 128, None, None, None, 8, None, 10, 0.5, 0.25,
                             None, None, 0, None) == -1
    # the loop: float32 state only, plan sizes checked before any launch
    d = tdp.block_desc(1, 128, 2, 64, 16, 2, tdp.TDP_F32, tdp.TDP_F32)
    p = tdp.plan_dev(4, 130, 520, 512, 520, None, None, None, None, None, None)
    assert tdp.tdp_upscale_workspace(d, p) > tdp.tdp_block_workspace(d, 4, 520)
    d_bf = tdp.block_desc(1, 128, 2, 64, 16, 2, tdp.TDP_BF16, tdp.TDP_F32)
    assert L.tdp_upscale_workspace(ctypes.byref(d_bf), ctypes.byref(p), ctypes.byref(n)) == -4
    for bad in [dict(n_gen=0), dict(n_dst_rows=500), dict(max_tile_rows=600), dict(n_tiles=0)]:
        q = tdp.plan_dev(**{**dict(n_tiles=4, max_tile_rows=130, n_rows=520, n_gen=512,
                                   n_dst_rows=520, tile_row_begin=None, row_src=None,
                                   row_weight=None, row_pos=None, dst_row_begin=None,
                                   dst_rows=None), **bad})
        assert L.tdp_upscale_workspace(ctypes.byref(d), ctypes.byref(q), ctypes.byref(n)) == -2, bad
    w = tdp.BlockWeights()
    sig = (ctypes.c_float * 4)(0.5, 0.3, 0.1, 0.0)
    assert L.tdp_upscale_loop(ctypes.byref(d), ctypes.byref(p), ctypes.byref(w), None, sig, 3,
                              None, None, None, 0, None) == -1


def test_sp_exchange_validation():
    L = tdp.lib()
    arr = (ctypes.c_void_p * 4)(FAKE, FAKE, FAKE, FAKE)
    P = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    assert L.tdp_sp_send_heads(FAKE, 1, 16, 32, 128, 4, 4, P, None) == -2      # rank >= world
    assert L.tdp_sp_send_heads(FAKE, 1, 16, 30, 128, 4, 0, P, None) == -4      # heads % world
    assert L.tdp_sp_send_heads(FAKE, 1, 16, 32, 128, 17, 0, P, None) == -4     # world > 16
    assert L.tdp_sp_send_heads(FAKE, 1, 16, 4, 4, 4, 0, P, None) == -4         # 2-byte segments
    assert L.tdp_sp_send_heads(FAKE, 7, 16, 32, 128, 4, 0, P, None) == -4      # dtype
    assert L.tdp_sp_send_heads(None, 1, 16, 32, 128, 4, 0, P, None) == -1
    assert L.tdp_sp_send_heads(FAKE + 8, 1, 16, 32, 128, 4, 0, P, None) == -7
    bad = (ctypes.c_void_p * 4)(FAKE, None, FAKE, FAKE)
    assert L.tdp_sp_send_heads(FAKE, 1, 16, 32, 128, 4, 0,
                               ctypes.cast(bad, ctypes.POINTER(ctypes.c_void_p)), None) == -1
    assert L.tdp_sp_gather_heads(P, 1, 16, 32, 128, 4, 0, None, None) == -1
    assert L.tdp_sp_gather_heads(P, 1, 0, 32, 128, 4, 0, None, None) == 0      # empty slice


def _declared_arg_counts():
    """Argument count of every function declared in include/tdp.h."""
    import re
    text = open(tdp.HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    out = {}
    for m in re.finditer(r"\b(tdp_[a-z_0-9]+)\s*\(([^;{]*?)\)\s*;", text):
        args = m.group(2).strip()
        out[m.group(1)] = 0 if args in ("", "void") else args.count(",") + 1
    return out


# The calls of the boundary the hot path's design fixes (the plan, gather,
# attention and blend of one step), with their argument counts as declared.
# Two depart from that design, on purpose: tdp_tile_attention takes n_rows
# (the device CSR's last entry, needed by the host to size launches without
# a device read), and the audio mean is its own call rather than the blend
# over a second plan.
BOUNDARY_ARGS = {
    "tdp_status_string": 1,
    "tdp_plan_query": 2,
    "tdp_plan": 3,
    "tdp_gather_tiles": 9,
    "tdp_tile_attention_workspace": 4,
    "tdp_tile_attention": 17,
    "tdp_blend_accumulate": 12,
    "tdp_audio_accumulate": 9,
    "tdp_balanced_tile_split": 3,
}


def test_boundary_calls_and_argument_counts():
    declared = _declared_arg_counts()
    for name, n in BOUNDARY_ARGS.items():
        assert name in declared, name
        assert declared[name] == n, (name, declared[name], n)
    # the binding marshals exactly the declared arguments of every call
    for name, n in declared.items():
        assert len(tdp._SIGS[name][1]) == n, (name, len(tdp._SIGS[name][1]), n)
    # the descriptor fields the departures add
    assert [f for f, _ in tdp.AttnDesc._fields_][-1] == "kv_splits"
    assert "assignment" in [f for f, _ in tdp.PlanDesc._fields_]
    assert "n_gen_total" in [f for f, _ in tdp.PlanSizes._fields_]
