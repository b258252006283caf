"""ctypes binding of libtdp.so, one Python function per C entry point.

Argument marshalling only: every step of the path runs in the library.  Device
buffers are torch tensors on the GPU (their ``data_ptr()`` is passed); the
stream is torch's current stream unless one is given.  A non-zero status from
the library raises ``TdpError``.  If the library has not been built the first
call raises ``RuntimeError``: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import dataclasses
import os
import re
from typing import Optional

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtdp.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "tdp.h")

TDP_F32, TDP_BF16 = 0, 1
STATUS = {0: "TDP_OK", -1: "TDP_ERR_NULL", -2: "TDP_ERR_ARG", -3: "TDP_ERR_SHAPE",
          -4: "TDP_ERR_UNSUPPORTED", -5: "TDP_ERR_BUFFER", -6: "TDP_ERR_HIP",
          -7: "TDP_ERR_ALIGN"}


class TdpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_string(status)})")


class DimTiling(C.Structure):
    _fields_ = [("num_tiles", C.c_int32), ("overlap", C.c_int32)]


class PlanDesc(C.Structure):
    _fields_ = [("grid", C.c_int32 * 3), ("tiling", DimTiling * 3), ("n_cond", C.c_int32),
                ("cond_pos", C.POINTER(C.c_float)), ("normalize_positions", C.c_int32),
                ("world_size", C.c_int32), ("rank", C.c_int32), ("assignment", C.c_int32)]


ASSIGNMENTS = {"round_robin": 0, "longest_first": 1}


class PlanSizes(C.Structure):
    _fields_ = [("n_tiles_total", C.c_int32), ("n_tiles_local", C.c_int32),
                ("max_tile_rows", C.c_int32), ("n_gen_total", C.c_int32),
                ("n_rows", C.c_int64), ("n_dst_rows", C.c_int64)]


class PlanOut(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "tile_id", "tile_box", "tile_offset", "tile_row_begin", "tile_n_gen", "row_src",
        "row_weight", "row_pos", "cond_keep_count", "dst_row_begin", "dst_rows")]


class AttnDesc(C.Structure):
    _fields_ = [("batch", C.c_int32), ("C", C.c_int32), ("heads", C.c_int32),
                ("head_dim", C.c_int32), ("n_audio", C.c_int32), ("x_dtype", C.c_int32),
                ("y_dtype", C.c_int32), ("rope_base", C.c_float), ("kv_splits", C.c_int32)]


class BlockDesc(C.Structure):
    _fields_ = [("batch", C.c_int32), ("C", C.c_int32), ("heads", C.c_int32),
                ("head_dim", C.c_int32), ("n_text", C.c_int32), ("layers", C.c_int32),
                ("time_dim", C.c_int32), ("x_dtype", C.c_int32), ("y_dtype", C.c_int32),
                ("rope_base", C.c_float)]


class BlockLayer(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("wqkv", "wo", "cq", "ckv", "co", "w1", "w2", "table")]


class BlockWeights(C.Structure):
    _fields_ = [("w_in", C.c_void_p), ("w_out", C.c_void_p), ("wt1", C.c_void_p),
                ("wt2", C.c_void_p), ("layers", C.POINTER(BlockLayer))]


class PlanDev(C.Structure):
    _fields_ = [("n_tiles", C.c_int32), ("max_tile_rows", C.c_int32), ("n_rows", C.c_int64),
                ("n_gen", C.c_int64), ("n_dst_rows", C.c_int64)] + [
        (n, C.c_void_p) for n in ("tile_row_begin", "row_src", "row_weight", "row_pos",
                                  "dst_row_begin", "dst_rows")]


_P, _I32, _I64, _SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
_SIGS = {
    "tdp_status_string": (C.c_char_p, [_I32]),
    "tdp_plan_query": (_I32, [C.POINTER(PlanDesc), C.POINTER(PlanSizes)]),
    "tdp_plan": (_I32, [C.POINTER(PlanDesc), C.POINTER(PlanSizes), C.POINTER(PlanOut)]),
    "tdp_balanced_tile_split": (_I32, [_I32, C.POINTER(_I32), C.POINTER(_I32)]),
    "tdp_gather_tiles": (_I32, [_P, _I32, _I32, _I64, _I32, _P, _I64, _P, _P]),
    "tdp_tile_attention_workspace": (_I32, [C.POINTER(AttnDesc), _I32, _I64, C.POINTER(_SZ)]),
    "tdp_tile_attention": (_I32, [C.POINTER(AttnDesc), _I32, _P, _I32, _I64, _P, _P, _P, _P, _P,
                                  _P, _P, _P, _P, _P, _SZ, _P]),
    "tdp_tile_attention_noalloc": (_I32, [C.POINTER(AttnDesc), _I32, _P, _I32, _I64, _P, _P, _P,
                                          _P, _P, _P, _P, _P, _P, _P]),
    "tdp_attn_prepare": (_I32, [C.POINTER(AttnDesc), _I32, _P, _I32, _I64, _P, _P, _P, _P, _P,
                                _SZ, _P]),
    "tdp_attn_qkv_rope": (_I32, [C.POINTER(AttnDesc), _I32, _P, _I32, _I64, _P, _P, _P, _P, _SZ,
                                 _P]),
    "tdp_attn_core": (_I32, [C.POINTER(AttnDesc), _I32, _P, _I32, _I64, _P, _SZ, _P]),
    "tdp_attn_out_proj": (_I32, [C.POINTER(AttnDesc), _I32, _P, _I32, _I64, _P, _P, _P, _SZ,
                                 _P]),
    "tdp_blend_accumulate": (_I32, [_P, _I32, _I32, _I64, _I32, _P, _P, _P, _I64, _P, _I32, _P]),
    "tdp_audio_accumulate": (_I32, [_P, _I32, _I32, _I32, _I32, _I32, _P, _I32, _P]),
    "tdp_block_workspace": (_I32, [C.POINTER(BlockDesc), _I32, _I64, C.POINTER(_SZ)]),
    "tdp_block_forward": (_I32, [C.POINTER(BlockDesc), _I32, _P, _I32, _I64, _P, _P, _P, _P,
                                 C.POINTER(BlockWeights), _P, _P, _SZ, _P]),
    "tdp_linear_sigmas": (_I32, [C.c_float, _I32, C.POINTER(C.c_float)]),
    "tdp_renoise": (_I32, [_P, _P, _I32, _I64, _I64, _I32, C.c_float, _P, _P]),
    "tdp_blend_euler_workspace": (_I32, [_I32, _I64, _I32, C.POINTER(_SZ)]),
    "tdp_blend_euler": (_I32, [_P, _I32, _I32, _I64, _I32, _P, _P, _P, _I64, _P, _I64, C.c_float,
                               C.c_float, _P, _P, _SZ, _P]),
    "tdp_upscale_workspace": (_I32, [C.POINTER(BlockDesc), C.POINTER(PlanDev), C.POINTER(_SZ)]),
    "tdp_upscale_loop": (_I32, [C.POINTER(BlockDesc), C.POINTER(PlanDev), C.POINTER(BlockWeights),
                                _P, C.POINTER(C.c_float), _I32, _P, _P, _P, _SZ, _P]),
    "tdp_sp_send_heads": (_I32, [_P, _I32, _I64, _I32, _I32, _I32, _I32, C.POINTER(_P), _P]),
    "tdp_sp_gather_heads": (_I32, [C.POINTER(_P), _I32, _I64, _I32, _I32, _I32, _I32, _P, _P]),
}

_lib = None


def lib() -> C.CDLL:
    """The loaded library (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def declared_symbols() -> list:
    """Function names declared in include/tdp.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tdp_[a-z_0-9]+)\s*\(", text)))


def status_string(status: int) -> str:
    return lib().tdp_status_string(int(status)).decode()


def tdp_status_string(status: int) -> str:
    return status_string(status)


def _check(status: int, where: str) -> None:
    if status != 0:
        raise TdpError(status, where)


# ---------------------------------------------------------------------------
# plan (host)
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Plan:
    sizes: dict
    tile_id: np.ndarray
    tile_box: np.ndarray
    tile_offset: np.ndarray
    tile_row_begin: np.ndarray
    tile_n_gen: np.ndarray
    row_src: np.ndarray
    row_weight: np.ndarray
    row_pos: np.ndarray
    cond_keep_count: np.ndarray
    dst_row_begin: np.ndarray
    dst_rows: np.ndarray

    @property
    def n_rows(self) -> int:
        return int(self.sizes["n_rows"])

    @property
    def n_tiles_local(self) -> int:
        return int(self.sizes["n_tiles_local"])

    @property
    def n_tiles_total(self) -> int:
        return int(self.sizes["n_tiles_total"])

    @property
    def max_tile_rows(self) -> int:
        return int(self.sizes["max_tile_rows"])

    @property
    def n_dst_rows(self) -> int:
        return int(self.sizes["n_dst_rows"])


def _desc(grid, tiling, cond_pos, normalize_positions, world_size, rank,
          assignment="round_robin"):
    d = PlanDesc()
    d.assignment = ASSIGNMENTS[assignment]
    for i in range(3):
        d.grid[i] = int(grid[i])
        d.tiling[i].num_tiles = int(tiling[i][0])
        d.tiling[i].overlap = int(tiling[i][1])
    keep = None
    if cond_pos is not None and len(cond_pos) > 0:
        keep = np.ascontiguousarray(cond_pos, dtype=np.float32).reshape(-1, 3, 2)
        d.n_cond = keep.shape[0]
        d.cond_pos = keep.ctypes.data_as(C.POINTER(C.c_float))
    d.normalize_positions = int(bool(normalize_positions))
    d.world_size = int(world_size)
    d.rank = int(rank)
    return d, keep


def tdp_balanced_tile_split(n):
    """(h_tiles, w_tiles) of a balanced 2D grid of ``n`` tiles."""
    h, w = _I32(), _I32()
    _check(lib().tdp_balanced_tile_split(int(n), C.byref(h), C.byref(w)), "tdp_balanced_tile_split")
    return h.value, w.value


def tdp_plan_query(grid, tiling, cond_pos=None, normalize_positions=True, world_size=1,
                   rank=0, assignment="round_robin") -> dict:
    d, _keep = _desc(grid, tiling, cond_pos, normalize_positions, world_size, rank, assignment)
    s = PlanSizes()
    _check(lib().tdp_plan_query(C.byref(d), C.byref(s)), "tdp_plan_query")
    return {f: getattr(s, f) for f, _ in PlanSizes._fields_}


def tdp_plan(grid, tiling, cond_pos=None, normalize_positions=True, world_size=1,
             rank=0, assignment="round_robin") -> Plan:
    """Query sizes, allocate the host arrays and fill them (host only)."""
    d, _keep = _desc(grid, tiling, cond_pos, normalize_positions, world_size, rank, assignment)
    s = PlanSizes()
    _check(lib().tdp_plan_query(C.byref(d), C.byref(s)), "tdp_plan_query")
    T, R, M = s.n_tiles_local, s.n_rows, d.n_cond
    arrs = dict(
        tile_id=np.zeros(T, np.int32), tile_box=np.zeros((T, 3, 2), np.int32),
        tile_offset=np.zeros((T, 3), np.float32), tile_row_begin=np.zeros(T + 1, np.int64),
        tile_n_gen=np.zeros(T, np.int32), row_src=np.zeros(R, np.int32),
        row_weight=np.zeros(R, np.float32), row_pos=np.zeros((R, 3, 2), np.float32),
        cond_keep_count=np.zeros(max(M, 1), np.int32),
        dst_row_begin=np.zeros(s.n_dst_rows + 1, np.int64), dst_rows=np.zeros(max(R, 1), np.int32))
    out = PlanOut(**{k: v.ctypes.data for k, v in arrs.items()})
    _check(lib().tdp_plan(C.byref(d), C.byref(s), C.byref(out)), "tdp_plan")
    arrs["cond_keep_count"] = arrs["cond_keep_count"][:M]
    arrs["dst_rows"] = arrs["dst_rows"][:R]
    return Plan(sizes={f: getattr(s, f) for f, _ in PlanSizes._fields_}, **arrs)


# ---------------------------------------------------------------------------
# device calls
# ---------------------------------------------------------------------------

def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return TDP_F32
    if t.dtype == torch.bfloat16:
        return TDP_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def tdp_gather_tiles(x_global, dtype, batch, n_src_rows, C_, row_src, n_rows, x_tiles,
                     stream=None) -> None:
    _check(lib().tdp_gather_tiles(_ptr(x_global), dtype, batch, n_src_rows, C_, _ptr(row_src),
                                  n_rows, _ptr(x_tiles), _stream(stream)), "tdp_gather_tiles")


def attn_desc(batch, C_, heads, head_dim, n_audio, x_dtype, y_dtype, rope_base=10000.0,
              kv_splits=0):
    return AttnDesc(batch, C_, heads, head_dim, n_audio, x_dtype, y_dtype, rope_base, kv_splits)


def tdp_tile_attention_workspace(desc: AttnDesc, n_tiles, n_rows) -> int:
    n = C.c_size_t()
    _check(lib().tdp_tile_attention_workspace(C.byref(desc), n_tiles, n_rows, C.byref(n)),
           "tdp_tile_attention_workspace")
    return n.value


def tdp_tile_attention(desc, n_tiles, tile_row_begin, max_tile_rows, n_rows, x_tiles, row_pos,
                       wq, wk, wv, wo, x_audio, y_tiles, y_audio_tiles, workspace,
                       workspace_bytes, stream=None) -> None:
    _check(lib().tdp_tile_attention(
        C.byref(desc), n_tiles, _ptr(tile_row_begin), max_tile_rows, n_rows, _ptr(x_tiles),
        _ptr(row_pos), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo), _ptr(x_audio), _ptr(y_tiles),
        _ptr(y_audio_tiles), _ptr(workspace), workspace_bytes, _stream(stream)),
        "tdp_tile_attention")


def tdp_tile_attention_noalloc(desc, n_tiles, tile_row_begin, max_tile_rows, n_rows, x_tiles,
                               row_pos, wq, wk, wv, wo, x_audio, y_tiles, y_audio_tiles,
                               stream=None) -> None:
    _check(lib().tdp_tile_attention_noalloc(
        C.byref(desc), n_tiles, _ptr(tile_row_begin), max_tile_rows, n_rows, _ptr(x_tiles),
        _ptr(row_pos), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo), _ptr(x_audio), _ptr(y_tiles),
        _ptr(y_audio_tiles), _stream(stream)),
        "tdp_tile_attention_noalloc")


def tdp_attn_prepare(desc, n_tiles, tile_row_begin, max_tile_rows, n_rows, wq, wk, wv, wo,
                     workspace, workspace_bytes, stream=None) -> None:
    _check(lib().tdp_attn_prepare(C.byref(desc), n_tiles, _ptr(tile_row_begin), max_tile_rows,
                                  n_rows, _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo),
                                  _ptr(workspace), workspace_bytes, _stream(stream)),
           "tdp_attn_prepare")


def tdp_attn_qkv_rope(desc, n_tiles, tile_row_begin, max_tile_rows, n_rows, x_tiles, row_pos,
                      x_audio, workspace, workspace_bytes, stream=None) -> None:
    _check(lib().tdp_attn_qkv_rope(C.byref(desc), n_tiles, _ptr(tile_row_begin), max_tile_rows,
                                   n_rows, _ptr(x_tiles), _ptr(row_pos), _ptr(x_audio),
                                   _ptr(workspace), workspace_bytes, _stream(stream)),
           "tdp_attn_qkv_rope")


def tdp_attn_core(desc, n_tiles, tile_row_begin, max_tile_rows, n_rows, workspace,
                  workspace_bytes, stream=None) -> None:
    _check(lib().tdp_attn_core(C.byref(desc), n_tiles, _ptr(tile_row_begin), max_tile_rows,
                               n_rows, _ptr(workspace), workspace_bytes, _stream(stream)),
           "tdp_attn_core")


def tdp_attn_out_proj(desc, n_tiles, tile_row_begin, max_tile_rows, n_rows, y_tiles,
                      y_audio_tiles, workspace, workspace_bytes, stream=None) -> None:
    _check(lib().tdp_attn_out_proj(C.byref(desc), n_tiles, _ptr(tile_row_begin), max_tile_rows,
                                   n_rows, _ptr(y_tiles), _ptr(y_audio_tiles), _ptr(workspace),
                                   workspace_bytes, _stream(stream)), "tdp_attn_out_proj")


def tdp_blend_accumulate(y_tiles, dtype, batch, n_rows, C_, dst_row_begin, dst_rows, row_weight,
                         n_dst_rows, y_global, accumulate, stream=None) -> None:
    _check(lib().tdp_blend_accumulate(_ptr(y_tiles), dtype, batch, n_rows, C_,
                                      _ptr(dst_row_begin), _ptr(dst_rows), _ptr(row_weight),
                                      n_dst_rows, _ptr(y_global), int(accumulate),
                                      _stream(stream)), "tdp_blend_accumulate")


def tdp_audio_accumulate(y_audio_tiles, n_tiles_local, n_tiles_total, batch, n_audio, C_,
                         y_audio, accumulate, stream=None) -> None:
    _check(lib().tdp_audio_accumulate(_ptr(y_audio_tiles), n_tiles_local, n_tiles_total, batch,
                                      n_audio, C_, _ptr(y_audio), int(accumulate),
                                      _stream(stream)), "tdp_audio_accumulate")


def block_desc(batch, C_, heads, head_dim, n_text, layers, x_dtype, y_dtype, time_dim=256,
               rope_base=10000.0) -> BlockDesc:
    return BlockDesc(batch, C_, heads, head_dim, n_text, layers, time_dim, x_dtype, y_dtype,
                     rope_base)


def block_weights(w_in, w_out, wt1, wt2, layers) -> BlockWeights:
    """``layers``: list of dicts of device tensors keyed like tdp_block_layer."""
    arr = (BlockLayer * max(1, len(layers)))()
    for i, lay in enumerate(layers):
        arr[i] = BlockLayer(*(_ptr(lay[k]) for k in ("wqkv", "wo", "cq", "ckv", "co", "w1", "w2",
                                                      "table")))
    w = BlockWeights(_ptr(w_in), _ptr(w_out), _ptr(wt1), _ptr(wt2),
                     C.cast(arr, C.POINTER(BlockLayer)))
    w._keep = arr          # the host array must outlive the call
    return w


def tdp_block_workspace(desc: BlockDesc, n_tiles, n_rows) -> int:
    n = C.c_size_t()
    _check(lib().tdp_block_workspace(C.byref(desc), n_tiles, n_rows, C.byref(n)),
           "tdp_block_workspace")
    return n.value


def tdp_block_forward(desc, n_tiles, tile_row_begin, max_tile_rows, n_rows, x_tiles, row_pos,
                      text, tau, weights: BlockWeights, y_tiles, workspace, workspace_bytes,
                      stream=None) -> None:
    _check(lib().tdp_block_forward(
        C.byref(desc), n_tiles, _ptr(tile_row_begin), max_tile_rows, n_rows, _ptr(x_tiles),
        _ptr(row_pos), _ptr(text), _ptr(tau), C.byref(weights), _ptr(y_tiles), _ptr(workspace),
        workspace_bytes, _stream(stream)), "tdp_block_forward")


# ---------------------------------------------------------------------------
# upscale loop
# ---------------------------------------------------------------------------

def tdp_linear_sigmas(sigma0, n_steps) -> np.ndarray:
    """The linear schedule, float32 ``[n_steps + 1]`` (host)."""
    out = np.zeros(max(int(n_steps), 0) + 1, np.float32)
    _check(lib().tdp_linear_sigmas(float(sigma0), int(n_steps),
                                   out.ctypes.data_as(C.POINTER(C.c_float))), "tdp_linear_sigmas")
    return out


def tdp_renoise(x_stage1, noise, batch, n_gen, n_dst_rows, C_, sigma0, x, stream=None) -> None:
    _check(lib().tdp_renoise(_ptr(x_stage1), _ptr(noise), batch, n_gen, n_dst_rows, C_,
                             float(sigma0), _ptr(x), _stream(stream)), "tdp_renoise")


def tdp_blend_euler_workspace(batch, n_gen, C_) -> int:
    n = C.c_size_t()
    _check(lib().tdp_blend_euler_workspace(batch, n_gen, C_, C.byref(n)),
           "tdp_blend_euler_workspace")
    return n.value


def tdp_blend_euler(y_tiles, dtype, batch, n_rows, C_, dst_row_begin, dst_rows, row_weight,
                    n_gen, x, n_dst_rows, sigma, sigma_next, seam, workspace, workspace_bytes,
                    stream=None) -> None:
    _check(lib().tdp_blend_euler(_ptr(y_tiles), dtype, batch, n_rows, C_, _ptr(dst_row_begin),
                                 _ptr(dst_rows), _ptr(row_weight), n_gen, _ptr(x), n_dst_rows,
                                 float(sigma), float(sigma_next), _ptr(seam), _ptr(workspace),
                                 workspace_bytes, _stream(stream)), "tdp_blend_euler")


def plan_dev(n_tiles, max_tile_rows, n_rows, n_gen, n_dst_rows, tile_row_begin, row_src,
             row_weight, row_pos, dst_row_begin, dst_rows) -> PlanDev:
    return PlanDev(n_tiles, max_tile_rows, n_rows, n_gen, n_dst_rows, _ptr(tile_row_begin),
                   _ptr(row_src), _ptr(row_weight), _ptr(row_pos), _ptr(dst_row_begin),
                   _ptr(dst_rows))


def tdp_upscale_workspace(desc: BlockDesc, plan: PlanDev) -> int:
    n = C.c_size_t()
    _check(lib().tdp_upscale_workspace(C.byref(desc), C.byref(plan), C.byref(n)),
           "tdp_upscale_workspace")
    return n.value


def tdp_upscale_loop(desc, plan: PlanDev, weights: BlockWeights, text, sigmas, n_steps, x, seam,
                     workspace, workspace_bytes, stream=None) -> None:
    sig = np.ascontiguousarray(sigmas, dtype=np.float32)
    if sig.size < int(n_steps) + 1:
        raise ValueError("sigmas needs n_steps + 1 entries")
    _check(lib().tdp_upscale_loop(C.byref(desc), C.byref(plan), C.byref(weights), _ptr(text),
                                  sig.ctypes.data_as(C.POINTER(C.c_float)), int(n_steps), _ptr(x),
                                  _ptr(seam), _ptr(workspace), workspace_bytes, _stream(stream)),
           "tdp_upscale_loop")


# ---------------------------------------------------------------------------
# sequence parallelism: the head exchange
# ---------------------------------------------------------------------------

def _ptr_array(bufs):
    return (C.c_void_p * len(bufs))(*[_ptr(b) for b in bufs])


def tdp_sp_send_heads(src, dtype, t_loc, heads, head_dim, world, rank, dst_bufs,
                      stream=None) -> None:
    arr = _ptr_array(dst_bufs)
    _check(lib().tdp_sp_send_heads(_ptr(src), dtype, t_loc, heads, head_dim, world, rank,
                                   C.cast(arr, C.POINTER(C.c_void_p)), _stream(stream)),
           "tdp_sp_send_heads")


def tdp_sp_gather_heads(src_bufs, dtype, t_loc, heads, head_dim, world, rank, dst,
                        stream=None) -> None:
    arr = _ptr_array(src_bufs)
    _check(lib().tdp_sp_gather_heads(C.cast(arr, C.POINTER(C.c_void_p)), dtype, t_loc, heads,
                                     head_dim, world, rank, _ptr(dst), _stream(stream)),
           "tdp_sp_gather_heads")
