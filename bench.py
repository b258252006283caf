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
  legs         the same step timed on the 8x32x32 latent (4 tiles, 32 heads x
               64) and on the audio workload (32x48x80, 2x3x4 tiles, batch 2,
               256 audio tokens, 16 heads x 128): wall time per step, latent
               tokens/s, per-stage times and the attention core's roofline
  gpu_clock    the shader clock sampled (sysfs, else amd-smi / rocm-smi) while
               the 16-tile core repeats for a few seconds after the timed
               region, with the ROCm and HIP versions
  cpu_baseline the CPU oracle (float64 NumPy, untuned) on a stated sample of
               the same step: plan, gather and blend of the whole step, and the
               denoiser on one whole tile of each distinct size (all heads and
               batch entries) as (tile, batch, head) work items in a pool of
               one process per host core (at most 16); the measured wall times
               are reported, and the step's value scales the denoiser sample to
               all tiles by attention flops
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
import csv
import glob
import hashlib
import json
import os
import re
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
CSRC = os.path.join(ROOT, "tiled_video_diffusion_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")

# Source files each kernel family is compiled from (a change in any of them
# makes that family's recorded counters stale).
KERNEL_SOURCES = {
    "attn_core_kernel": ("tdp_attention.hip", "tdp_common.h"),
    "attn_core2_kernel": ("tdp_attention.hip", "tdp_common.h"),
    "attn_combine_kernel": ("tdp_attention.hip", "tdp_common.h"),
    "qkv_rope_kernel": ("tdp_attention.hip", "tdp_common.h"),
    "gemm_kernel": ("tdp_gemm.hip", "tdp_common.h", "tdp_internal.h"),
    "gather_rows_kernel": ("tdp_gather_blend.hip", "tdp_common.h"),
    "blend_rows_kernel": ("tdp_gather_blend.hip", "tdp_common.h"),
    "audio_mean_kernel": ("tdp_gather_blend.hip", "tdp_common.h"),
}


def source_digest(kernel: str) -> str:
    """Digest of the sources a kernel is compiled from."""
    family = kernel.split("<")[0]
    files = KERNEL_SOURCES.get(family, ("tdp_attention.hip", "tdp_gemm.hip",
                                        "tdp_gather_blend.hip", "tdp_common.h"))
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, kernel: str):
    """HBM bytes (read, write) per launch of `kernel` on `workload` from the
    committed counter runs (profiles/hbm_traffic.json); None unless they were
    taken from the kernel's current sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    for e in rec.get("entries", []):
        if e.get("workload") == workload and e.get("kernel") == kernel:
            if e.get("source_digest") != source_digest(kernel):
                return None
            return e["read_bytes"], e["write_bytes"]
    return None


def _unmangle(n: str) -> str:
    """The kernel name and template arguments of an Itanium-mangled
    `tdp::(anonymous namespace)::k<...>` symbol, which rocprofv3 leaves mangled
    when a template argument is bfloat16 (`DF16b`), e.g.
    '_ZN3tdp12_GLOBAL__N_115qkv_rope_kernelIDF16bLi128ELb0EEEv...' ->
    'qkv_rope_kernel<__bf16, 128, false>'.  Other forms come back unchanged."""
    m = re.match(r"_ZN(?:3tdp)?(?:12_GLOBAL__N_1)?(\d+)", n)
    if not m:
        return n
    ln = int(m.group(1))
    name = n[m.end():m.end() + ln]
    rest = n[m.end() + ln:]
    if not rest.startswith("I"):
        return name
    args, i = [], 1
    types = {"DF16b": "__bf16", "f": "float", "d": "double", "i": "int", "l": "long"}
    while i < len(rest) and rest[i] != "E":
        lit = re.match(r"L(b|i|l)(n?\d+)E", rest[i:])
        if lit:
            v = lit.group(2).replace("n", "-")
            args.append({"0": "false", "1": "true"}[v] if lit.group(1) == "b" else v)
            i += lit.end()
            continue
        for code, ty in types.items():
            if rest.startswith(code, i):
                args.append(ty)
                i += len(code)
                break
        else:
            return n
    return f"{name}<{', '.join(args)}>"


def short_kernel_name(name: str) -> str:
    """'void tdp::(anonymous namespace)::k<128, false>(tdp::...)' -> 'k<128, false>'."""
    n = name.strip()
    if n.startswith("_Z"):
        return _unmangle(n)
    if n.startswith("void "):
        n = n[5:]
    depth = 0
    for i, ch in enumerate(n):                 # cut the argument list at depth 0
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and not n[:i].endswith("anonymous namespace"):
            if n[i:].startswith("(anonymous"):
                continue
            n = n[:i]
            break
    return n.replace("tdp::(anonymous namespace)::", "").replace("tdp::", "").strip()


def counters_to_json(workload: str, fetch_dir: str, write_dir: str) -> dict:
    """Fold two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per
    dispatch) of one bench.py run with --calibrate-copy-mib 2048 into
    profiles/hbm_traffic.json: per kernel, the mean over its dispatches, scaled
    by what each counter reads for the run's 2 GiB fill (writes only) and 2 GiB
    float32 negation (reads and writes)."""
    def per_kernel(d, counter):
        out = {}
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        for f in files:
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if r["Counter_Name"] == counter:
                        out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return out

    f = per_kernel(fetch_dir, "FETCH_SIZE")
    w = per_kernel(write_dir, "WRITE_SIZE")
    mean = {k: sum(v) / len(v) for k, v in f.items()}
    wmean = {k: sum(v) / len(v) for k, v in w.items()}
    fill = [k for k in f if "FillFunctor" in k]
    neg = [k for k in f if "neg" in k.lower()]
    if len(fill) != 1 or len(neg) != 1:
        raise SystemExit(f"calibration kernels not found (fill {fill}, negation {neg})")
    fs = 2097152.0 / mean[neg[0]]
    ws = 2097152.0 / wmean[fill[0]]
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        rec = {"entries": []}
    rec["note"] = ("HBM bytes per launch: rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per "
                   "dispatch, mean over the run's dispatches of each kernel) times 1024 "
                   "times the scale each counter needs to read a 2 GiB float32 negation "
                   "(FETCH_SIZE) and a 2 GiB fill (WRITE_SIZE) as their true sizes")
    keep = [e for e in rec.get("entries", []) if e.get("workload") != workload]
    for k in sorted(mean):
        if k in fill or k in neg or k not in wmean or k.startswith("__amd"):
            continue
        kern = short_kernel_name(k)
        keep.append({"workload": workload, "kernel": kern, "source_digest": source_digest(kern),
                     "dispatches": len(f[k]), "fetch_kib_raw": round(mean[k], 1),
                     "write_kib_raw": round(wmean[k], 1), "fetch_scale": round(fs, 5),
                     "write_scale": round(ws, 5),
                     "read_bytes": int(round(mean[k] * 1024 * fs)),
                     "write_bytes": int(round(wmean[k] * 1024 * ws))})
    rec["entries"] = keep
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    return rec


def versions() -> dict:
    """ROCm, HIP (torch build) and amdgpu driver versions of this machine."""
    out = {}
    try:
        with open("/opt/rocm/.info/version") as fh:
            out["rocm"] = fh.read().strip()
    except OSError:
        out["rocm"] = None
    try:
        import torch
        out["torch"] = torch.__version__
        out["torch_hip"] = torch.version.hip
    except Exception:
        pass
    try:
        with open("/sys/module/amdgpu/version") as fh:
            out["amdgpu_driver"] = fh.read().strip()
    except OSError:
        out["amdgpu_driver"] = None
    return out


class ClockSampler:
    """Samples the shader (gfx) clock of the GPU at PCI address `bdf` in a
    thread: sysfs (hwmon freq1 'sclk', else the current pp_dpm_sclk level),
    else amd-smi / rocm-smi.  Values in MHz."""

    def __init__(self, bdf: str):
        self.bdf = bdf
        self.samples = []
        self.source = None
        self.errors = []
        self._stop = threading.Event()
        self._thread = None
        dev = os.path.join("/sys/bus/pci/devices", bdf)
        self._hwmon = None
        for h in sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*"))):
            try:
                with open(os.path.join(h, "freq1_label")) as fh:
                    if fh.read().strip() == "sclk":
                        self._hwmon = os.path.join(h, "freq1_input")
            except OSError:
                pass
        self._dpm = os.path.join(dev, "pp_dpm_sclk")

    def _sysfs(self):
        if self._hwmon:
            try:
                with open(self._hwmon) as fh:
                    return float(fh.read().strip()) / 1e6, "sysfs hwmon freq1_input (sclk)"
            except (OSError, ValueError) as e:
                self.errors.append(f"hwmon: {e}")
                self._hwmon = None
        try:
            with open(self._dpm) as fh:
                for line in fh:
                    if line.rstrip().endswith("*"):
                        m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                        if m:
                            return float(m.group(1)), "sysfs pp_dpm_sclk (current level)"
        except OSError:
            pass
        return None, None

    def _smi(self):
        cmds = (["amd-smi", "metric", "--clock", "--json"],
                ["rocm-smi", "--showclocks", "--json"])
        for cmd in cmds:
            try:
                r = subprocess.run(cmd, capture_output=True, text=True, timeout=20)
            except (OSError, subprocess.TimeoutExpired) as e:
                self.errors.append(f"{cmd[0]}: {e}")
                continue
            if r.returncode != 0:
                self.errors.append(f"{cmd[0]}: rc {r.returncode}")
                continue
            vals = self._parse_smi(r.stdout)
            if vals:
                return vals, " ".join(cmd) + " (median over the GPU's gfx clocks)"
        return None, None

    def _parse_smi(self, text):
        """MHz values of the gfx clocks of this GPU in amd-smi / rocm-smi JSON."""
        try:
            data = json.loads(text)
        except ValueError:
            return None
        found = []

        def num(v):
            if isinstance(v, dict):
                v = v.get("value", v.get("clk"))
                if isinstance(v, dict):
                    v = v.get("value")
            if isinstance(v, (int, float)):
                return float(v)
            if isinstance(v, str):
                m = re.search(r"(\d+(?:\.\d+)?)\s*[Mm][Hh]z", v)
                return float(m.group(1)) if m else None
            return None

        def walk(o, want):
            if isinstance(o, dict):
                for k, v in o.items():
                    kl = str(k).lower()
                    if kl.startswith("gfx") and isinstance(v, dict) and "clk" in v:
                        x = num(v["clk"])
                        if x:
                            found.append(x)
                    elif "sclk clock speed" in kl:
                        x = num(v)
                        if x:
                            found.append(x)
                    else:
                        walk(v, want)
            elif isinstance(o, list):
                for v in o:
                    walk(v, want)

        gpus = data if isinstance(data, list) else [data]
        # amd-smi lists every GPU; keep the one whose bus id matches, when given
        chosen = [g for g in gpus if isinstance(g, dict) and
                  self.bdf.lower() in json.dumps(g).lower()] or gpus[:1]
        walk(chosen, None)
        if not found:
            return None
        found.sort()
        return found[len(found) // 2]

    def _run(self):
        while not self._stop.is_set():
            v, src = self._sysfs()
            if v is None:
                v, src = self._smi()
            if v is None:
                return
            self.source = src
            self.samples.append(v)
            self._stop.wait(0.02)

    def __enter__(self):
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join(timeout=30)

    def summary(self, what: str) -> dict:
        if not self.samples:
            return {"mhz_median": None, "source": None, "window": what,
                    "errors": self.errors[:4] or ["no clock source answered"]}
        v = sorted(self.samples)
        return {"mhz_median": v[len(v) // 2], "mhz_min": v[0], "mhz_max": v[-1],
                "n_samples": len(v), "source": self.source, "window": what}


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


_CPU = {}


def _cpu_init(shared: dict) -> None:
    """Pool worker set-up: one BLAS thread per process, the sample's arrays."""
    try:
        from threadpoolctl import threadpool_limits
        _CPU["limit"] = threadpool_limits(1)
    except Exception:
        pass
    _CPU.update(shared)


def _cpu_item(item):
    """One (tile, batch, head) work item: the oracle's tile forward restricted
    to head h (its columns of Wq/Wk/Wv and rows of Wo), whose output is head
    h's share of the tile's y (the output projection is a sum over heads)."""
    import oracle
    t, b, h = item
    d = _CPU["head_dim"]
    cols = slice(h * d, (h + 1) * d)
    xa = None if _CPU["x_aud"] is None else _CPU["x_aud"][b]
    y, ya = oracle.tile_forward(_CPU["x"][t][b], _CPU["pos"][t], xa, _CPU["wq"][:, cols],
                                _CPU["wk"][:, cols], _CPU["wv"][:, cols], _CPU["wo"][cols],
                                1, d)
    return t, b, h, y, ya


def _cpu_nop(_):
    return os.getpid()


def cpu_baseline(inp, plan, max_workers: int = 16, full: bool = False,
                 full_budget_s: float = 45.0) -> dict:
    """The oracle, untuned, on this host's cores: plan + gather + blend of the
    whole step, and the denoiser as (tile, batch, head) items in a process
    pool.  The denoiser first runs on one whole tile of each distinct row
    count (all heads and batch entries); when the rest of the step would take
    at most ``full_budget_s`` at that rate (or with ``full``), it then runs on
    every tile of the step and that whole-step wall time is the result, with
    no scaling; otherwise the sample is scaled to the step by attention flops."""
    import concurrent.futures as cf
    import multiprocessing as mp

    import numpy as np

    import oracle
    wl = inp.workload
    workers = max(1, min(max_workers, len(os.sched_getaffinity(0))))
    t0 = time.perf_counter()
    p = oracle.plan(wl.grid, wl.tiling, inp.cond_pos)
    t_plan = time.perf_counter() - t0
    t0 = time.perf_counter()
    x_tiles = oracle.gather_tiles(inp.x_global, p)
    t_gather = time.perf_counter() - t0
    rows = np.diff(p.tile_row_begin)
    all_tiles = list(range(rows.size))
    sample = sorted({int(np.nonzero(rows == r)[0][0]) for r in np.unique(rows)})
    n = rows.astype(np.float64) + wl.n_audio
    per_tile = 4.0 * wl.head_dim * wl.heads * wl.batch * n * n
    f_total = float(per_tile.sum())
    shared = {"head_dim": wl.head_dim, "wq": inp.wq, "wk": inp.wk, "wv": inp.wv, "wo": inp.wo,
              "x_aud": inp.x_aud,
              "x": {t: x_tiles[:, p.tile_row_begin[t]:p.tile_row_begin[t + 1]] for t in all_tiles},
              "pos": {t: p.row_pos[p.tile_row_begin[t]:p.tile_row_begin[t + 1]]
                      for t in all_tiles}}

    def denoise(pool, tiles):
        items = [(t, b, h) for t in tiles for b in range(wl.batch) for h in range(wl.heads)]
        y_tiles = np.zeros(x_tiles.shape, dtype=np.float64)
        t0 = time.perf_counter()
        for t, b, h, y, ya in pool.map(_cpu_item, items):
            r0 = p.tile_row_begin[t]
            y_tiles[b, r0:r0 + y.shape[0]] += y
        return time.perf_counter() - t0, y_tiles, len(items)

    # spawned workers (fresh interpreters: this process has initialised the
    # GPU); a worker that dies raises BrokenProcessPool instead of hanging
    with cf.ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn"),
                                initializer=_cpu_init, initargs=(shared,)) as pool:
        list(pool.map(_cpu_nop, range(4 * workers)))     # workers up before the clock
        t_sample, y_tiles, n_items = denoise(pool, sample)
        f_sample = float(per_tile[sample].sum())
        whole = full or t_sample * (f_total - f_sample) / f_sample <= full_budget_s
        if whole:
            t_denoise, y_tiles, n_items = denoise(pool, all_tiles)
    t0 = time.perf_counter()
    oracle.blend_tiles(y_tiles, p)
    t_blend = time.perf_counter() - t0
    tokens = wl.batch * wl.n_gen
    head = (f"float64 NumPy oracle, {workers} processes x 1 BLAS thread: plan {t_plan:.2f} s "
            f"+ gather {t_gather:.2f} s + blend {t_blend:.2f} s of the whole step")
    measured = {"plan_s": t_plan, "gather_s": t_gather, "blend_s": t_blend,
                "sample_tiles": sample, "sample_tile_rows": [int(rows[t]) for t in sample],
                "sample_denoiser_wall_s": t_sample}
    if whole:
        step_s = t_plan + t_gather + t_denoise + t_blend
        measured.update({"denoiser_wall_s": t_denoise, "tiles": rows.size,
                         "work_items": n_items})
        sample_txt = (f"{head}, and the denoiser on all {rows.size} tiles x {wl.heads} heads x "
                      f"{wl.batch} batch entries = {n_items} (tile, batch, head) items: "
                      f"{t_denoise:.1f} s; the whole step measured, {step_s:.1f} s, no scaling")
    else:
        step_s = t_plan + t_gather + t_blend + t_sample * f_total / f_sample
        measured.update({"denoiser_wall_s": t_sample, "tiles": sample, "work_items": n_items})
        sample_txt = (f"{head}, and the denoiser on tiles {sample} (one of each distinct row "
                      f"count, {[int(rows[t]) for t in sample]}) x {wl.heads} heads x "
                      f"{wl.batch} batch entries = {n_items} items: {t_sample:.1f} s measured; "
                      f"scaled to the step's {rows.size} tiles by attention flops "
                      f"({f_total / f_sample:.2f}x): {step_s:.1f} s per step")
    return {"value": tokens / step_s, "unit": "latent tokens/s", "cores": workers,
            "kind": "oracle", "sample": sample_txt, "whole_step_measured": whole,
            "measured": measured, "step_s": step_s, "attn_flops_step": f_total}


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


def drift_sweep(name: str, sigma0s=(0.1, 0.3, 0.5, 0.7, 0.9)) -> dict:
    """The upscale loop of workload `name` from several first sigmas, the same
    number of linearly spaced steps each: every step's seam spread
    sqrt(S2/S0) (the tiles' disagreement where they overlap) and how far the
    loop moved the generated tokens from the stage-1 latent."""
    import torch

    import tdp_inputs as ti
    from tiled_video_diffusion_amd import tdp
    from tiled_video_diffusion_amd.step import UpscaleLoop

    up = ti.make_upscale_inputs(name)
    uw = up.workload
    out = {"workload": name, "block": uw.block, "n_steps": uw.n_steps, "by_sigma0": {},
           "note": ("synthetic weights: the spread shows the metric across first sigmas, "
                    "not a quality; the page ties drift to the first sigma")}
    for s0 in sigma0s:
        lp = UpscaleLoop(up, sigmas=tdp.tdp_linear_sigmas(float(s0), uw.n_steps))
        lp.renoise()
        lp.loop()
        torch.cuda.synchronize()
        n = lp.n_gen
        x1 = lp.x_stage1[:, :n].double()
        moved = float((lp.x[:, :n].double() - x1).norm() / x1.norm())
        seam = lp.seam.cpu().numpy()
        out["by_sigma0"][f"{s0:g}"] = {"seam_relative_spread": [float(v) for v in seam[:lp.n_steps, 2]],
                                       "displacement_from_stage1": moved}
        lp = None
        torch.cuda.empty_cache()
    return out


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


def time_step(step, steps: int, warmup: int, stream) -> tuple:
    """W untimed steps, then K timed ones: wall ms per step (synchronized on
    both sides) and the mean ms of every stage from HIP events recorded on the
    launch stream around each stage."""
    import numpy as np
    import torch

    for _ in range(warmup):
        step.run()
    torch.cuda.synchronize()
    names = ["gather", "prepare", "qkv", "core", "out", "blend", "audio"]
    ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)] for n in names}

    def stage(i, name, fn):
        ev[name][i][0].record(stream)
        fn()
        ev[name][i][1].record(stream)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
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
    ms_per_step = (time.perf_counter() - t0) * 1e3 / steps
    used = ["gather", "blend"] + ([] if step.identity else ["prepare", "qkv", "core", "out"]) + \
        (["audio"] if step.n_audio else [])
    stage_ms = {n: float(np.mean([a.elapsed_time(b) for a, b in ev[n]])) for n in used}
    return ms_per_step, stage_ms


def core_roofline(wl, plan, core_ms: float) -> dict:
    flops = attn_flops(plan, wl)
    achieved = flops / (core_ms * 1e-3) / 1e12
    # Unsplit launches run the two-query-group kernel at either head dim;
    # none of the timed workloads splits its keys (the rocprofv3 traces of
    # each workload show the kernel launched).
    kern = f"attn_core2_kernel<{wl.head_dim}>"
    tr = recorded_traffic(wl.name, kern)
    return {"kernel": kern, "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": None if tr is None else tr[0] + tr[1],
            "flops_per_launch": flops, "ms_per_launch": core_ms}


LEG_WARM_S = 0.5    # a leg's warm-up lasts at least this long (after its own setup)
LEG_TIMED_S = 0.3   # and its timed region at least this long


def leg(name: str, steps: int, warmup: int) -> dict:
    """The whole step on another workload: throughput and the core's roofline.

    A leg follows seconds of host-side setup with the GPU idle, and its
    shader clock takes a while to come back up: W warm-up steps of the
    half-millisecond head-dim-64 step are 1.5 ms, and its core measured
    8-9% slower that way than in steady state.  So a leg warms up for at
    least LEG_WARM_S and times at least LEG_TIMED_S of steps (more than K
    steps when the step is short); the counts used are reported."""
    import torch

    import tdp_inputs as ti
    from tiled_video_diffusion_amd.step import TdpStep

    inp = ti.make_inputs(name)
    wl = inp.workload
    step = TdpStep(inp)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < LEG_WARM_S:
        step.run()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    per_step = (time.perf_counter() - t0) / n
    warmup = n
    steps = max(steps, int(LEG_TIMED_S / max(per_step, 1e-6)) + 1)
    ms, stage_ms = time_step(step, steps, 0, torch.cuda.current_stream())
    p = step.plan
    out = {"workload": name, "batch": wl.batch, "grid": list(wl.grid), "tiles": p.n_tiles_total,
           "rows": p.n_rows, "heads": wl.heads, "head_dim": wl.head_dim, "n_cond": wl.n_cond,
           "n_audio": wl.n_audio, "steps": steps, "warmup": warmup, "ms_per_step": ms,
           "latent_tokens_per_s": wl.batch * wl.n_gen / (ms * 1e-3), "stage_ms": stage_ms,
           "core": core_roofline(wl, p, stage_ms["core"])}
    del step
    torch.cuda.empty_cache()
    return out


def clock_window(step, seconds: float) -> dict:
    """The core of `step` repeated for about `seconds` while a thread samples
    the shader clock of this GPU."""
    import torch

    props = torch.cuda.get_device_properties(0)
    bdf = "{:04x}:{:02x}:{:02x}.0".format(getattr(props, "pci_domain_id", 0),
                                          getattr(props, "pci_bus_id", 0),
                                          getattr(props, "pci_device_id", 0))
    step.attn_core()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step.attn_core()
    torch.cuda.synchronize()
    one = max(time.perf_counter() - t0, 1e-4)
    n = max(1, int(seconds / one))
    with ClockSampler(bdf) as cs:
        for i in range(n):
            step.attn_core()
            if i % 16 == 15:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
    out = cs.summary(f"{n} back-to-back launches of the attention core ({n * one:.1f} s) "
                     "after the timed region")
    out["pci_bdf"] = bdf
    return out


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
    ms_per_step, stage_ms = time_step(step, args.steps, args.warmup, stream)
    tokens = wl.batch * wl.n_gen
    value = tokens / (ms_per_step * 1e-3)
    roofline = (core_roofline(wl, p, stage_ms["core"]) if not step.identity else None)

    gpu_clock = None
    if args.clock_s > 0 and not step.identity:
        gpu_clock = clock_window(step, args.clock_s)
    gpu_clock = {**(gpu_clock or {}), "versions": versions()}

    # gather + blend stress, alone
    bs = None
    if not args.skip_blend_stress:
        if args.workload != "blend_32x96x160":
            step = None
            torch.cuda.empty_cache()
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
        # HBM bytes the counters saw (overlap rows the gather reads twice hit
        # in cache, so its counter bytes are below the algorithmic ones)
        for key, kern, ms in (("gather", "gather_rows_kernel<true>", g_ms),
                              ("blend", "blend_rows_kernel<float, true>", b_ms)):
            tr = recorded_traffic("blend_32x96x160", kern)
            if tr is not None:
                cb = (tr[0] + tr[1]) / (ms * 1e-3) / 1e9
                bs[key]["counter_bytes_per_launch"] = tr[0] + tr[1]
                bs[key]["counter_achieved"] = cb
                bs[key]["counter_frac"] = cb / PEAK_HBM_GBS
            else:
                bs[key]["counter_bytes_per_launch"] = None
        del bstep
        torch.cuda.empty_cache()

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
        "attn_mfma_frac_whole_attention": attn_flops(p, wl) / (sum(stage_ms.get(n, 0.0) for n in
                                                                   ("prepare", "qkv", "core", "out")) * 1e-3)
        / (PEAK_BF16_TFLOPS * 1e12) if roofline else None,
        "gpu_clock": gpu_clock,
        "blend_stress": bs,
    }
    step = None
    torch.cuda.empty_cache()
    if not args.skip_legs:
        out["legs"] = {n: leg(n, args.steps, args.warmup) for n in args.legs.split(",") if n}
    if args.calibrate_copy_mib:
        torch.cuda.empty_cache()
        calibrate_copy(args.calibrate_copy_mib)
        out["calibrate_copy_mib"] = args.calibrate_copy_mib
    if args.block:
        torch.cuda.empty_cache()
        out["block"] = block_bench(args.block, max(2, args.steps // 4), 1)
    if args.loop:
        torch.cuda.empty_cache()
        out["loop"] = loop_bench(args.loop, max(2, args.steps // 8), 1)
    if args.drift:
        torch.cuda.empty_cache()
        out["drift"] = drift_sweep(args.drift)
    if args.sp:
        torch.cuda.empty_cache()
        out["sp"] = sp_bench(args.sp)
    if args.shares:
        torch.cuda.empty_cache()
        out["shares"] = shares(inp, args.shares)
    if not args.skip_cpu_baseline and not wl.identity:
        try:
            out["cpu_baseline"] = cpu_baseline(inp, p, full=args.cpu_full)
        except Exception as e:        # report, keep the GPU figures
            out["cpu_baseline"] = {"value": None, "error": f"{type(e).__name__}: {e}"}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="t16_16x64x64")
    ap.add_argument("--cpu-full", action="store_true",
                    help="CPU baseline on every tile of the step (no scaling; minutes)")
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--skip-blend-stress", action="store_true")
    ap.add_argument("--legs", default="d64_8x32x32,audio_32x48x80",
                    help="other workloads whose whole step is also timed (comma list)")
    ap.add_argument("--skip-legs", action="store_true")
    ap.add_argument("--clock-s", type=float, default=2.0,
                    help="seconds of repeated core launches while the shader clock is "
                         "sampled (0: no clock window)")
    ap.add_argument("--counters-to-json", nargs=3, metavar=("WORKLOAD", "FETCH_DIR", "WRITE_DIR"),
                    help="fold two rocprofv3 --pmc output directories (FETCH_SIZE, "
                         "WRITE_SIZE) of a bench.py run on WORKLOAD into "
                         "profiles/hbm_traffic.json, then exit (no GPU needed)")
    ap.add_argument("--block", default="",
                    help="also time the step with the per-tile transformer block (a block "
                         "workload name, e.g. block_t16)")
    ap.add_argument("--loop", default="",
                    help="also time the upscale loop (an upscale workload name, e.g. "
                         "upscale_t16)")
    ap.add_argument("--drift", default="",
                    help="also run the upscale loop of this upscale workload from several first "
                         "sigmas and report its seam spread per step (e.g. upscale_d128)")
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
    if args.counters_to_json:
        rec = counters_to_json(*args.counters_to_json)
        print(json.dumps(rec, indent=1))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the multi-GPU path of this build is design only", file=sys.stderr)
        sys.exit(2)
    print(json.dumps(run(args)), flush=True)


if __name__ == "__main__":
    main()
