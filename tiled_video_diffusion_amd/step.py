"""One TDP step on the GPU through the C ABI, with device-resident buffers.

Uploads a workload's plan and inputs once, then runs gather -> per-tile
attention (or the identity denoiser) -> blend -> audio average, every stage in
libtdp.so.  Used by the tests, the smoke check and the benchmark.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import tdp


def _dev(a: np.ndarray, device, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


class TdpStep:
    """Device state of one rank's share of a TDP step."""

    def __init__(self, inputs, normalize_positions: bool = True, world_size: int = 1,
                 rank: int = 0, device: str = "cuda:0", identity: Optional[bool] = None,
                 rope_base: float = 10000.0, assignment: str = "round_robin",
                 kv_splits: int = 0):
        wl = inputs.workload
        self.wl = wl
        self.device = torch.device(device)
        self.identity = wl.identity if identity is None else identity
        self.plan = tdp.tdp_plan(wl.grid, wl.tiling, inputs.cond_pos, normalize_positions,
                                 world_size, rank, assignment)
        p = self.plan
        dev = self.device
        self.latent_dtype = torch.bfloat16 if wl.latent_dtype == "bf16" else torch.float32
        self.code = tdp.TDP_BF16 if wl.latent_dtype == "bf16" else tdp.TDP_F32
        B, C = wl.batch, wl.channels
        self.B, self.C = B, C
        self.n_src = wl.n_gen + wl.n_cond
        # plan arrays on the device
        self.row_src = _dev(p.row_src, dev)
        self.row_weight = _dev(p.row_weight, dev)
        self.row_pos = _dev(p.row_pos, dev)
        self.tile_row_begin = _dev(p.tile_row_begin, dev)
        self.dst_row_begin = _dev(p.dst_row_begin, dev)
        self.dst_rows = _dev(p.dst_rows, dev)
        # data
        self.x_global = _dev(inputs.x_global, dev, self.latent_dtype)
        R = max(p.n_rows, 1)
        self.x_tiles = torch.empty((B, R, C), dtype=self.latent_dtype, device=dev)
        self.y_global = torch.empty((B, p.n_dst_rows, C), dtype=torch.float32, device=dev)
        self.n_audio = 0 if inputs.x_aud is None else inputs.x_aud.shape[1]
        self.y_audio = None
        self.y_audio_tiles = None
        self.x_audio = None
        if self.identity:
            self.y_tiles = self.x_tiles
            self.workspace = None
            self.ws_bytes = 0
        else:
            self.y_tiles = torch.empty((B, R, C), dtype=self.latent_dtype, device=dev)
            self.wq = _dev(inputs.wq, dev, torch.bfloat16)
            self.wk = _dev(inputs.wk, dev, torch.bfloat16)
            self.wv = _dev(inputs.wv, dev, torch.bfloat16)
            self.wo = _dev(inputs.wo, dev, torch.bfloat16)
            self.desc = tdp.attn_desc(B, C, wl.heads, wl.head_dim, self.n_audio, self.code,
                                      self.code, rope_base, kv_splits)
            if self.n_audio:
                self.x_audio = _dev(inputs.x_aud, dev, self.latent_dtype)
                self.y_audio_tiles = torch.empty((p.n_tiles_local, B, self.n_audio, C),
                                                 dtype=torch.float32, device=dev)
                self.y_audio = torch.empty((B, self.n_audio, C), dtype=torch.float32, device=dev)
            self.ws_bytes = tdp.tdp_tile_attention_workspace(self.desc, p.n_tiles_local, p.n_rows)
            self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)

    # -- stages ------------------------------------------------------------
    def gather(self, stream=None):
        p = self.plan
        tdp.tdp_gather_tiles(self.x_global, self.code, self.B, self.n_src, self.C, self.row_src,
                             p.n_rows, self.x_tiles, stream)

    def _attn_args(self):
        p = self.plan
        return (self.desc, p.n_tiles_local, self.tile_row_begin, p.max_tile_rows, p.n_rows)

    def attn_prepare(self, stream=None):
        tdp.tdp_attn_prepare(*self._attn_args(), self.wq, self.wk, self.wv, self.wo,
                             self.workspace, self.ws_bytes, stream)

    def attn_qkv(self, stream=None):
        tdp.tdp_attn_qkv_rope(*self._attn_args(), self.x_tiles, self.row_pos, self.x_audio,
                              self.workspace, self.ws_bytes, stream)

    def attn_core(self, stream=None):
        tdp.tdp_attn_core(*self._attn_args(), self.workspace, self.ws_bytes, stream)

    def attn_out(self, stream=None):
        tdp.tdp_attn_out_proj(*self._attn_args(), self.y_tiles, self.y_audio_tiles,
                              self.workspace, self.ws_bytes, stream)

    def attention(self, stream=None):
        tdp.tdp_tile_attention(*self._attn_args(), self.x_tiles, self.row_pos, self.wq, self.wk,
                               self.wv, self.wo, self.x_audio, self.y_tiles, self.y_audio_tiles,
                               self.workspace, self.ws_bytes, stream)

    def blend(self, accumulate: bool = False, stream=None):
        p = self.plan
        tdp.tdp_blend_accumulate(self.y_tiles, self.code, self.B, p.n_rows, self.C,
                                 self.dst_row_begin, self.dst_rows, self.row_weight,
                                 p.n_dst_rows, self.y_global, accumulate, stream)

    def audio(self, accumulate: bool = False, stream=None):
        if self.n_audio and not self.identity:
            p = self.plan
            tdp.tdp_audio_accumulate(self.y_audio_tiles, p.n_tiles_local, p.n_tiles_total,
                                     self.B, self.n_audio, self.C, self.y_audio, accumulate,
                                     stream)

    def run(self, accumulate: bool = False, stream=None):
        """One whole step: gather, denoiser, blend, audio average."""
        self.gather(stream)
        if not self.identity:
            self.attention(stream)
        self.blend(accumulate, stream)
        self.audio(accumulate, stream)


class BlockStep:
    """One rank's share of a TDP step whose tile denoiser is the per-tile
    transformer block (``tdp_block_forward``); gather and blend as in TdpStep."""

    def __init__(self, binputs, normalize_positions: bool = True, world_size: int = 1,
                 rank: int = 0, device: str = "cuda:0", workspace: bool = True):
        inp = binputs.base
        wl = inp.workload
        bw = binputs.workload
        self.s = TdpStep(inp, normalize_positions, world_size, rank, device, identity=True)
        s = self.s
        dev = s.device
        p = s.plan
        self.plan = p
        s.y_tiles = torch.empty_like(s.x_tiles)
        bf = torch.bfloat16

        def t(a):             # [in][out] -> the library's [out][in]
            return _dev(np.ascontiguousarray(np.asarray(a).T), dev, bf)

        self.w_in, self.w_out = t(binputs.w_in), t(binputs.w_out)
        self.wt1, self.wt2 = t(binputs.wt1), t(binputs.wt2)
        self.layers = []
        for lay in binputs.layers:
            self.layers.append({
                "wqkv": _dev(np.concatenate([np.asarray(lay[k]).T for k in ("wq", "wk", "wv")]),
                             dev, bf),
                "wo": t(lay["wo"]), "cq": t(lay["cq"]),
                "ckv": _dev(np.concatenate([np.asarray(lay[k]).T for k in ("ck", "cv")]), dev, bf),
                "co": t(lay["co"]), "w1": t(lay["w1"]), "w2": t(lay["w2"]),
                "table": _dev(lay["table"], dev, torch.float32)})
        self.weights = tdp.block_weights(self.w_in, self.w_out, self.wt1, self.wt2, self.layers)
        self.text = _dev(binputs.text, dev, bf)
        self.tau = _dev(binputs.tau, dev, torch.float32)
        self.desc = tdp.block_desc(wl.batch, wl.channels, wl.heads, wl.head_dim, bw.n_text,
                                   bw.layers, s.code, s.code, bw.time_dim)
        self.ws_bytes = tdp.tdp_block_workspace(self.desc, p.n_tiles_local, p.n_rows)
        self.workspace = (torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
                          if workspace else None)

    @property
    def y_tiles(self):
        return self.s.y_tiles

    @property
    def y_global(self):
        return self.s.y_global

    def gather(self, stream=None):
        self.s.gather(stream)

    def block(self, stream=None):
        p = self.plan
        tdp.tdp_block_forward(self.desc, p.n_tiles_local, self.s.tile_row_begin, p.max_tile_rows,
                              p.n_rows, self.s.x_tiles, self.s.row_pos, self.text, self.tau,
                              self.weights, self.s.y_tiles, self.workspace, self.ws_bytes, stream)

    def blend(self, accumulate: bool = False, stream=None):
        self.s.blend(accumulate, stream)

    def run(self, accumulate: bool = False, stream=None):
        self.gather(stream)
        self.block(stream)
        self.blend(accumulate, stream)


class UpscaleLoop:
    """The TDP upscale loop on the GPU: re-noise the stage-1 latent to the
    first sigma (``tdp_renoise``), then ``n_steps`` steps of gather -> per-tile
    transformer -> blend fused with the Euler update (``tdp_upscale_loop``).
    The state ``x`` is the float32 global latent ``[B][N+M][C]``; ``seam``
    receives each step's {S2, S0, sqrt(S2/S0)}.  Weights, text and the plan come
    from a ``BlockStep`` on the same inputs."""

    def __init__(self, uinputs, device: str = "cuda:0", sigmas=None):
        binp = uinputs.block
        self.bs = BlockStep(binp, device=device, workspace=False)
        bs, s, p = self.bs, self.bs.s, self.bs.plan
        wl, bw, uw = binp.base.workload, binp.workload, uinputs.workload
        self.wl = wl
        self.sigmas = (tdp.tdp_linear_sigmas(uw.sigma0, uw.n_steps) if sigmas is None
                       else np.ascontiguousarray(sigmas, np.float32))
        self.n_steps = self.sigmas.size - 1
        dev = s.device
        self.n_gen = wl.n_gen
        self.n_dst = p.n_dst_rows
        self.x_stage1 = _dev(binp.base.x_global, dev, torch.float32)
        self.noise = _dev(uinputs.noise, dev, torch.float32)
        self.x = torch.empty_like(self.x_stage1)
        self.seam = torch.zeros((max(self.n_steps, 1), 3), dtype=torch.float64, device=dev)
        self.desc = tdp.block_desc(wl.batch, wl.channels, wl.heads, wl.head_dim, bw.n_text,
                                   bw.layers, tdp.TDP_F32, tdp.TDP_F32, bw.time_dim)
        self.plan_dev = tdp.plan_dev(p.n_tiles_local, p.max_tile_rows, p.n_rows, self.n_gen,
                                     self.n_dst, s.tile_row_begin, s.row_src, s.row_weight,
                                     s.row_pos, s.dst_row_begin, s.dst_rows)
        self.ws_bytes = tdp.tdp_upscale_workspace(self.desc, self.plan_dev)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)

    def renoise(self, stream=None):
        tdp.tdp_renoise(self.x_stage1, self.noise, self.wl.batch, self.n_gen, self.n_dst,
                        self.wl.channels, float(self.sigmas[0]), self.x, stream)

    def loop(self, stream=None):
        tdp.tdp_upscale_loop(self.desc, self.plan_dev, self.bs.weights, self.bs.text, self.sigmas,
                             self.n_steps, self.x, self.seam, self.workspace, self.ws_bytes,
                             stream)

    def run(self, stream=None):
        self.renoise(stream)
        self.loop(stream)
