#!/usr/bin/env python3
"""Benchmark of one TDP upscale step on one MI355X (gfx950).

A step is one pass of the device hot path over one batch of synthetic input:
gather of tile rows -> per-tile attention (QKV + 3D RoPE, flash attention,
output projection) -> blend into the global latent -> audio average.  The host
plan (tiles, masks, positions, keep rule) is computed once per shape, outside
the timed region, and reported as ``plan_ms``.

Default workload: the 16-tile step (latent 16x64x64, 128 channels, 4x4 tiles
with overlap 8, 32 heads x 128, bf16).  Prints ONE JSON line.

  value        latent tokens/s = B*N / (wall time per step)
  roofline     the attention core kernel (dominant): algorithmic flops
               sum over (tile, batch, head) of 4*d*n_t^2, divided by its mean
               launch time from HIP events on the launch stream, against the
               dense bf16 MFMA peak
  blend_stress gather and blend alone on the 32x96x160 fp32 latent
               (6x10 tiles, overlap 16, identity denoiser), algorithmic bytes
               per launch over mean launch time, against 8 TB/s
  cpu_baseline the CPU oracle (float64 NumPy) on a bounded sample of the same
               step, scaled to a whole step by attention flops
  shares       (--shares W) how the step would split over W GPUs: each rank's
               round-robin share (its real shape) timed alone on this GPU, the
               critical path (slowest rank), and each tile timed alone, from
               which the longest-processing-time assignment's critical path
               follows; the exchange between ranks is not modeled
  block        (--block NAME) the step with the per-tile transformer block as
               the tile denoiser (a block workload of tdp_inputs): wall time per
               step, algorithmic flops (GEMMs, self- and cross-attention) per
               step over that time, against the dense bf16 MFMA peak
  loop         (--loop NAME) the upscale loop (an upscale workload of
               tdp_inputs): re-noise, then per step gather -> transformer ->
               blend fused with the Euler update; wall time per step, each
               step's seam spread, and the fused blend/Euler kernel alone on the
               workload's plan against 8 TB/s (algorithmic bytes: tile rows,
               the latent read and written, the inverse map)
  sp           (--sp W) sequence parallelism for the first stage on the
               6144-token latent (16x16x24, 32 heads x 128): one rank's share
               (all tokens, H/W heads) timed on this GPU with its attention
               core against the bf16 peak, and the head exchange (send of Q, K
               and V, gather of the output) with every rank's buffer in this
               GPU's memory, against 8 TB/s
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
CSRC = os.path.join(ROOT, "tiled_video_diffusion_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_core_t16_16x64x64_traffic.json")


def core_source_digest() -> str:
    """Digest of the sources the attention core is compiled from."""
    h = hashlib.sha256()
    for f in ("tdp_attention.hip", "tdp_common.h"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def core_traffic(workload: str):
    """HBM bytes per attention-core launch from the committed counter runs.

    None unless the counters were taken on this workload from the same kernel
    source (a changed kernel makes them stale).
    """
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("workload") != workload or rec.get("source_digest") != core_source_digest():
        return None
    return rec.get("attn_core_bytes_per_launch")


def calibrate_copy(mib: int) -> None:
    """Known-size kernels for scaling FETCH_SIZE / WRITE_SIZE: a fill (writes
    `mib` MiB) and an elementwise negation (reads and writes `mib` MiB)."""
    import torch
    n = (mib << 20) // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1.0)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def attn_flops(plan, wl) -> float:
    import numpy as np
    n = np.diff(plan.tile_row_begin).astype(np.float64) + wl.n_audio
    return float(4.0 * wl.head_dim * wl.heads * wl.batch * np.sum(n * n))


def gather_bytes(plan, wl) -> float:
    es = 2 if wl.latent_dtype == "bf16" else 4
    return 2.0 * wl.batch * plan.n_rows * wl.channels * es + 4.0 * plan.n_rows


def blend_bytes(plan, wl) -> float:
    es = 2 if wl.latent_dtype == "bf16" else 4
    rows = plan.n_rows
    return (wl.batch * rows * wl.channels * es          # y_tiles read
            + wl.batch * plan.n_dst_rows * wl.channels * 4  # y_global written
            + 4.0 * rows + 4.0 * rows                    # dst_rows, row_weight
            + 8.0 * (plan.n_dst_rows + 1))               # dst_row_begin


def cpu_baseline(inp, plan, budget_s: float = 15.0) -> dict:
    """Time the oracle on whole tiles until the budget is spent; scale by flops."""
    import numpy as np
    import oracle
    wl = inp.workload
    threads = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        if info:
            threads = max(int(i.get("num_threads", 0)) for i in info)
    except Exception:
        pass
    t0 = time.perf_counter()
    p = oracle.plan(wl.grid, wl.tiling, inp.cond_pos)
    x_tiles = oracle.gather_tiles(inp.x_global, p)
    t_plan_gather = time.perf_counter() - t0
    order = np.argsort(np.diff(p.tile_row_begin))           # smallest tiles first
    done_flops, t_tiles, n_tiles = 0.0, 0.0, 0
    y_tiles = np.zeros(x_tiles.shape, dtype=np.float64)
    for t in order:
        r0, r1 = int(p.tile_row_begin[t]), int(p.tile_row_begin[t + 1])
        t1 = time.perf_counter()
        for b in range(wl.batch):
            xa = None if inp.x_aud is None else inp.x_aud[b]
            y, _ = oracle.tile_forward(x_tiles[b, r0:r1], p.row_pos[r0:r1], xa, inp.wq, inp.wk,
                                       inp.wv, inp.wo, wl.heads, wl.head_dim)
            y_tiles[b, r0:r1] = y
        t_tiles += time.perf_counter() - t1
        n = (r1 - r0) + wl.n_audio
        done_flops += 4.0 * wl.head_dim * wl.heads * wl.batch * n * n
        n_tiles += 1
        if t_tiles >= budget_s:
            break
    t1 = time.perf_counter()
    oracle.blend_tiles(y_tiles, p)
    t_blend = time.perf_counter() - t1
    total_flops = attn_flops(plan, wl)
    est = t_plan_gather + t_blend + t_tiles * total_flops / done_flops
    tokens = wl.batch * wl.n_gen
    return {"value": tokens / est, "unit": "latent tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"float64 NumPy oracle: plan + gather + blend of the whole step, "
                       f"denoiser on {n_tiles} of {p.tile_id.size} tiles "
                       f"({t_tiles:.1f} s), scaled to the step by attention flops; "
                       f"estimated {est:.1f} s per step")}


def shares(inp, world_size: int, reps: int = 5) -> dict:
    """Round-robin shares of `world_size` ranks, each timed alone on this GPU."""
    import numpy as np
    import torch
    from tiled_video_diffusion_amd.step import TdpStep

    stream = torch.cuda.current_stream()

    def time_share(world, rank, assignment="round_robin"):
        st = TdpStep(inp, world_size=world, rank=rank, assignment=assignment)
        for _ in range(2):
            st.run()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            st.run()
            b.record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        tiles = [int(t) for t in st.plan.tile_id]
        n_total = st.plan.n_tiles_total
        del st
        torch.cuda.empty_cache()
        return ms, tiles, n_total

    rr = [time_share(world_size, r) for r in range(world_size)]
    lf = [time_share(world_size, r, "longest_first") for r in range(world_size)]
    n_tiles = rr[0][2]
    per_tile = [time_share(n_tiles, t)[0] for t in range(n_tiles)]
    # longest processing time first: each tile to the least loaded rank
    loads = [0.0] * world_size
    for t in sorted(range(n_tiles), key=lambda t: -per_tile[t]):
        r = int(np.argmin(loads))
        loads[r] += per_tile[t]
    rr_from_tiles = [sum(per_tile[t] for t in tiles) for _, tiles, _ in rr]
    return {"world_size": world_size, "assignment": "round robin (tile t -> rank t mod W)",
            "ms_per_rank": [m for m, _, _ in rr], "tiles_per_rank": [t for _, t, _ in rr],
            "critical_ms": max(m for m, _, _ in rr),
            "longest_first": {"ms_per_rank": [m for m, _, _ in lf],
                              "tiles_per_rank": [t for _, t, _ in lf],
                              "critical_ms": max(m for m, _, _ in lf),
                              "assignment": "tiles by rows^2, largest first, each to the "
                                            "least loaded rank (tdp_plan_desc.assignment = 1)"},
            "per_tile_ms": per_tile,
            "critical_ms_from_tile_times": {"round_robin": max(rr_from_tiles),
                                            "longest_first": max(loads)},
            "note": "shares run one after another on one GPU; the all_reduce (or halo "
                    "exchange) between ranks is not included"}


def block_flops(plan, bw, wl) -> dict:
    """Algorithmic flops of one block step (multiply-add = 2 flops)."""
    import numpy as np
    D, B, C = wl.hidden, wl.batch, wl.channels
    M = B * plan.n_rows
    nt = np.diff(plan.tile_row_begin).astype(np.float64)
    L = bw.layers
    gemm = (2.0 * M * C * D * 2                                       # proj_in, proj_out
            + 2.0 * B * (bw.time_dim * D + 6.0 * D * D)               # timestep MLP
            + L * (28.0 * M * D * D + 4.0 * B * bw.n_text * D * D))   # QKV, O, cross Q/KV/O, FFN
    self_attn = L * 4.0 * D * B * float(np.sum(nt * nt))
    cross_attn = L * 4.0 * D * M * bw.n_text
    return {"gemm": gemm, "self_attention": self_attn, "cross_attention": cross_attn,
            "total": gemm + self_attn + cross_attn}


def block_bench(name: str, steps: int, warmup: int) -> dict:
    """The step with the per-tile transformer block as tile denoiser."""
    import numpy as np
    import torch

    import tdp_inputs as ti
    from tiled_video_diffusion_amd.step import BlockStep

    binp = ti.make_block_inputs(name)
    bw, wl = binp.workload, binp.base.workload
    st = BlockStep(binp)
    for _ in range(warmup):
        st.run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        st.gather()
        a.record(stream)
        st.block()
        b.record(stream)
        st.blend()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    ms_block = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    fl = block_flops(st.plan, bw, wl)
    ach = fl["total"] / (ms_block * 1e-3) / 1e12
    return {"workload": name, "layers": bw.layers, "width": wl.hidden, "n_text": bw.n_text,
            "tiles": st.plan.n_tiles_total, "rows": st.plan.n_rows,
            "ms_per_step": ms_step, "block_ms": ms_block,
            "latent_tokens_per_s": wl.batch * wl.n_gen / (ms_step * 1e-3),
            "flops_per_step": fl, "achieved_tflops": ach, "peak_tflops": PEAK_BF16_TFLOPS,
            "frac": ach / PEAK_BF16_TFLOPS}


def blend_euler_bytes(plan, n_gen, batch, C) -> int:
    """Algorithmic bytes of one tdp_blend_euler launch (float32 tile rows)."""
    return (batch * plan.n_rows * C * 4 + 2 * batch * n_gen * C * 4
            + plan.n_rows * (4 + 4) + (n_gen + 1) * 8)


def loop_bench(name: str, reps: int, warmup: int) -> dict:
    """The upscale loop, and its fused blend/Euler kernel alone."""
    import numpy as np
    import torch

    import tdp_inputs as ti
    from tiled_video_diffusion_amd.step import TdpStep, UpscaleLoop

    up = ti.make_upscale_inputs(name)
    wl = up.block.base.workload
    lp = UpscaleLoop(up)
    for _ in range(warmup):
        lp.run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        lp.run()
        b.record(stream)
    torch.cuda.synchronize()
    ms_loop = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    seam = lp.seam.cpu().numpy()
    n_steps = lp.n_steps
    # the fused blend/Euler kernel alone (float32 tile rows) on this plan and on
    # the 32x96x160 latent's plan, with and without the seam sums
    B = wl.batch
    kern = {"workload_plan": _time_blend_euler(lp.bs.s, B, wl.channels, wl.n_gen, lp.n_dst)}
    lp = None
    torch.cuda.empty_cache()
    big = ti.make_inputs("blend_32x96x160")
    bst = TdpStep(big, identity=True)
    kern["blend_32x96x160_plan"] = _time_blend_euler(bst, big.workload.batch,
                                                     big.workload.channels, big.workload.n_gen,
                                                     bst.plan.n_dst_rows)
    return {"workload": name, "block": up.workload.block, "sigma0": up.workload.sigma0,
            "n_steps": n_steps, "ms_per_loop": ms_loop,
            "ms_per_step": ms_loop / max(n_steps, 1),
            "latent_tokens_per_s_per_step": B * wl.n_gen / (ms_loop / max(n_steps, 1) * 1e-3),
            "seam_relative_spread": [float(v) for v in seam[:n_steps, 2]],
            "seam_note": "synthetic weights: the spread shows the metric, not a quality",
            "blend_euler": kern}


def _time_blend_euler(s, B, C, N, n_dst, n_launch=50) -> dict:
    """Mean launch time of tdp_blend_euler on TdpStep ``s``'s plan with random
    float32 tile rows, with and without the seam sums (HIP events on the
    launch stream)."""
    import numpy as np
    import torch

    from tiled_video_diffusion_amd import tdp

    p = s.plan
    stream = torch.cuda.current_stream()
    g = torch.Generator(device="cuda:0").manual_seed(0)
    y = torch.randn((B, p.n_rows, C), generator=g, device="cuda:0", dtype=torch.float32)
    x = torch.randn((B, n_dst, C), generator=g, device="cuda:0", dtype=torch.float32)
    ws_bytes = tdp.tdp_blend_euler_workspace(B, N, C)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda:0")
    seam = torch.zeros(3, dtype=torch.float64, device="cuda:0")
    out = {"bytes_per_launch": blend_euler_bytes(p, N, B, C), "unit": "GB/s",
           "peak": PEAK_HBM_GBS}
    for key, sm in (("with_seam", seam), ("no_seam", None)):
        def launch():
            tdp.tdp_blend_euler(y, tdp.TDP_F32, B, p.n_rows, C, s.dst_row_begin, s.dst_rows,
                                s.row_weight, N, x, n_dst, 0.3, 0.2999, sm, ws, ws_bytes, stream)
        for _ in range(3):
            launch()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n_launch)]
        for a, b in ev:
            a.record(stream)
            launch()
            b.record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        gbs = out["bytes_per_launch"] / (ms * 1e-3) / 1e9
        out[key] = {"ms_per_launch": ms, "achieved": gbs, "frac": gbs / PEAK_HBM_GBS}
    return out


def sp_bench(world: int, reps: int = 20) -> dict:
    """One rank's share of the first stage's attention layer, and the head
    exchange, on this GPU."""
    import dataclasses as dc

    import numpy as np
    import torch

    import tdp_inputs as ti
    from tiled_video_diffusion_amd import tdp
    from tiled_video_diffusion_amd.step import TdpStep

    inp = ti.make_inputs("sp_16x16x24")
    wl = inp.workload
    H, d, C = wl.heads, wl.head_dim, wl.channels
    if H % world:
        raise SystemExit(f"--sp {world}: {H} heads do not divide by the world size")
    hw = H // world
    cols = slice(0, hw * d)                    # rank 0's heads
    share = dc.replace(inp, workload=dc.replace(wl, heads=hw),
                       wq=np.ascontiguousarray(inp.wq[:, cols]),
                       wk=np.ascontiguousarray(inp.wk[:, cols]),
                       wv=np.ascontiguousarray(inp.wv[:, cols]),
                       wo=np.ascontiguousarray(inp.wo[cols]))
    stream = torch.cuda.current_stream()
    T = wl.n_gen
    flops = 4.0 * d * hw * T * T

    def share_ms(kv_splits):
        st = TdpStep(share, kv_splits=kv_splits)
        st.gather()
        st.attn_prepare()
        for _ in range(3):
            st.attn_qkv()
            st.attn_core()
            st.attn_out()
        torch.cuda.synchronize()
        ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(reps)] for n in ("qkv", "core", "out")}
        for i in range(reps):
            for n, fn in (("qkv", st.attn_qkv), ("core", st.attn_core), ("out", st.attn_out)):
                ev[n][i][0].record(stream)
                fn()
                ev[n][i][1].record(stream)
        torch.cuda.synchronize()
        return {n: float(np.mean([a.elapsed_time(b) for a, b in v])) for n, v in ev.items()}

    # the automatic choice splits the keys of this launch (few query blocks);
    # the unsplit core is timed beside it
    ms = share_ms(0)
    ms_unsplit = share_ms(1)
    core_tf = flops / (ms["core"] * 1e-3) / 1e12
    core_tf1 = flops / (ms_unsplit["core"] * 1e-3) / 1e12
    # the exchange: this rank's slice of Q, K, V (all heads) to every rank's
    # buffer, and the output back; every buffer in this GPU's memory
    t_loc = T // world
    g = torch.Generator(device="cuda:0").manual_seed(0)
    src = torch.randn((t_loc, H, d), generator=g, device="cuda:0").to(torch.bfloat16)
    bufs = [torch.empty((world * t_loc, hw, d), dtype=torch.bfloat16, device="cuda:0")
            for _ in range(world)]
    back = torch.empty_like(src)
    nbytes = 2 * t_loc * H * d * 2             # read + write of one slice

    def timed(fn, n=50):
        for _ in range(3):
            fn()
        e = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(n)]
        for a, b in e:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in e]))

    send_ms = timed(lambda: tdp.tdp_sp_send_heads(src, tdp.TDP_BF16, t_loc, H, d, world, 0, bufs,
                                                  stream))
    gather_ms = timed(lambda: tdp.tdp_sp_gather_heads(bufs, tdp.TDP_BF16, t_loc, H, d, world, 0,
                                                      back, stream))
    return {"workload": wl.name, "tokens": T, "world": world, "heads_per_rank": hw,
            "share_ms": {k: v for k, v in ms.items()},
            "share_core": {"achieved": core_tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": core_tf / PEAK_BF16_TFLOPS, "flops_per_launch": flops,
                           "kv_splits": "automatic (key parts + combine)"},
            "share_core_unsplit": {"ms": ms_unsplit["core"], "achieved": core_tf1,
                                   "frac": core_tf1 / PEAK_BF16_TFLOPS},
            "exchange": {"bytes_per_launch": nbytes, "send_ms": send_ms,
                         "gather_ms": gather_ms,
                         "send_gbs": nbytes / (send_ms * 1e-3) / 1e9,
                         "gather_gbs": nbytes / (gather_ms * 1e-3) / 1e9,
                         "per_step": "3 sends (Q, K, V) and 1 gather per attention layer",
                         "note": "every rank's buffer in this GPU's memory; with peer "
                                 "pointers the same copies go over the GPU links"}}


def run(args) -> dict:
    import numpy as np
    import torch

    import tdp_inputs as ti
    from tiled_video_diffusion_amd import tdp
    from tiled_video_diffusion_amd.step import TdpStep

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    inp = ti.make_inputs(args.workload)
    wl = inp.workload
    t0 = time.perf_counter()
    tdp.tdp_plan(wl.grid, wl.tiling, inp.cond_pos)
    plan_ms = (time.perf_counter() - t0) * 1e3
    step = TdpStep(inp)
    p = step.plan
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()

    names = ["gather", "prepare", "qkv", "core", "out", "blend", "audio"]
    ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)] for n in names}

    def stage(i, name, fn):
        ev[name][i][0].record(stream)
        fn()
        ev[name][i][1].record(stream)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        stage(i, "gather", step.gather)
        if not step.identity:
            stage(i, "prepare", step.attn_prepare)
            stage(i, "qkv", step.attn_qkv)
            stage(i, "core", step.attn_core)
            stage(i, "out", step.attn_out)
        stage(i, "blend", step.blend)
        if step.n_audio:
            stage(i, "audio", step.audio)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    def mean_ms(name):
        vals = [a.elapsed_time(b) for a, b in ev[name]]
        return float(np.mean(vals))

    used = ["gather", "blend"] + ([] if step.identity else ["prepare", "qkv", "core", "out"]) + \
        (["audio"] if step.n_audio else [])
    stage_ms = {n: mean_ms(n) for n in used}
    tokens = wl.batch * wl.n_gen
    value = tokens / (ms_per_step * 1e-3)

    flops = attn_flops(p, wl)
    core_ms = stage_ms.get("core", float("nan"))
    achieved = flops / (core_ms * 1e-3) / 1e12
    roofline = {"kernel": "attn_core_kernel", "bound": "mfma", "achieved": achieved,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": core_traffic(wl.name), "flops_per_launch": flops,
                "ms_per_launch": core_ms}

    # gather + blend stress, alone
    bs = None
    if not args.skip_blend_stress:
        binp = ti.make_inputs("blend_32x96x160")
        bstep = TdpStep(binp)
        bwl = binp.workload
        for _ in range(3):
            bstep.run()
        torch.cuda.synchronize()
        nrep = 20
        ge = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nrep)]
        be = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nrep)]
        for i in range(nrep):
            ge[i][0].record(stream); bstep.gather(); ge[i][1].record(stream)
            be[i][0].record(stream); bstep.blend(); be[i][1].record(stream)
        torch.cuda.synchronize()
        g_ms = float(np.mean([a.elapsed_time(b) for a, b in ge]))
        b_ms = float(np.mean([a.elapsed_time(b) for a, b in be]))
        gb = gather_bytes(bstep.plan, bwl) / (g_ms * 1e-3) / 1e9
        bb = blend_bytes(bstep.plan, bwl) / (b_ms * 1e-3) / 1e9
        bs = {"workload": "blend_32x96x160", "unit": "GB/s", "peak": PEAK_HBM_GBS,
              "gather": {"achieved": gb, "frac": gb / PEAK_HBM_GBS, "ms_per_launch": g_ms,
                         "bytes_per_launch": gather_bytes(bstep.plan, bwl)},
              "blend": {"achieved": bb, "frac": bb / PEAK_HBM_GBS, "ms_per_launch": b_ms,
                        "bytes_per_launch": blend_bytes(bstep.plan, bwl)}}
        del bstep

    out = {
        "metric": "latent tokens/s per TDP step (1 GPU); attn MFMA %; blend HBM GB/s",
        "value": value, "unit": "latent tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if wl.latent_dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "grid": list(wl.grid),
                   "tiling": [list(t) for t in wl.tiling], "tiles": p.n_tiles_total,
                   "batch": wl.batch, "channels": wl.channels, "heads": wl.heads,
                   "head_dim": wl.head_dim, "n_cond": wl.n_cond, "n_audio": wl.n_audio,
                   "rows": p.n_rows, "parallelism": "all tiles on one GPU"},
        "roofline": roofline,
        "stage_ms": stage_ms, "plan_ms": plan_ms,
        "attn_mfma_frac_whole_attention": flops / (sum(stage_ms.get(n, 0.0) for n in
                                                       ("prepare", "qkv", "core", "out")) * 1e-3)
        / (PEAK_BF16_TFLOPS * 1e12) if not step.identity else None,
        "blend_stress": bs,
    }
    if args.calibrate_copy_mib:
        step = None
        torch.cuda.empty_cache()
        calibrate_copy(args.calibrate_copy_mib)
        out["calibrate_copy_mib"] = args.calibrate_copy_mib
    if args.block:
        step = None
        torch.cuda.empty_cache()
        out["block"] = block_bench(args.block, max(2, args.steps // 4), 1)
    if args.loop:
        step = None
        torch.cuda.empty_cache()
        out["loop"] = loop_bench(args.loop, max(2, args.steps // 8), 1)
    if args.sp:
        step = None
        torch.cuda.empty_cache()
        out["sp"] = sp_bench(args.sp)
    if args.shares:
        step = None
        torch.cuda.empty_cache()
        out["shares"] = shares(inp, args.shares)
    if not args.skip_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, p, args.cpu_budget)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="t16_16x64x64")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle denoiser work in the CPU baseline sample")
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--skip-blend-stress", action="store_true")
    ap.add_argument("--block", default="",
                    help="also time the step with the per-tile transformer block (a block "
                         "workload name, e.g. block_t16)")
    ap.add_argument("--loop", default="",
                    help="also time the upscale loop (an upscale workload name, e.g. "
                         "upscale_t16)")
    ap.add_argument("--sp", type=int, default=0,
                    help="also time one rank's share of sequence parallelism on the "
                         "first-stage latent for this many ranks")
    ap.add_argument("--shares", type=int, default=0,
                    help="also time each rank's round-robin share for this many ranks "
                         "(one after another on this GPU)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after the run, a fill and a negation of this many MiB (for scaling "
                         "HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the multi-GPU path of this build is design only", file=sys.stderr)
        sys.exit(2)
    print(json.dumps(run(args)), flush=True)


if __name__ == "__main__":
    main()
