"""The attention layer without a caller workspace (tdp_tile_attention_noalloc,
for callers that cannot allocate device memory) against tdp_tile_attention
with a workspace: the same kernels, so the outputs must be identical bit for
bit.  Two calls in a row, the second on a smaller input (the scratch keeps
the first call's contents).  Sizes beyond the library's scratch are refused
before any device work."""
import dataclasses
import sys

import numpy as np
import pytest

import tdp_inputs as ti

torch = pytest.importorskip("torch")

SCRATCH_BYTES = 64 << 20          # TDP_NOALLOC_SCRATCH_BYTES in include/tdp.h


def say(*a):
    print("[no-alloc]", *a, flush=True)
    sys.stdout.flush()


def _variant(base, **kw):
    return ti.make_inputs(dataclasses.replace(ti.workload(base), **kw))


# the first input is the larger: head dim 128, batch 2, audio, ragged tiles;
# the second is the 2x16x16 latent at head dim 64 with no audio
CASES = [
    ("ragged_audio_d128", lambda: _variant("tiny_2x16x16", grid=(3, 17, 23),
                                           tiling=((1, 0), (3, 5), (4, 5)), heads=4,
                                           head_dim=128, n_cond=12, n_cond_neg=3, n_audio=37,
                                           batch=2, latent_dtype="bf16")),
    ("tiny_2x16x16", lambda: ti.make_inputs("tiny_2x16x16")),
]


@pytest.mark.gpu
def test_noalloc_equals_workspace_entry_point():
    from tiled_video_diffusion_amd import tdp
    from tiled_video_diffusion_amd.step import TdpStep

    sizes = []
    for name, make in CASES:
        inp = make()
        s = TdpStep(inp)
        p = s.plan
        say(name, "rows", p.n_rows, "workspace bytes", s.ws_bytes)
        assert s.ws_bytes <= SCRATCH_BYTES
        sizes.append(s.ws_bytes)
        s.gather()
        s.attention()
        torch.cuda.synchronize()
        want = s.y_tiles.clone()
        want_a = None if s.y_audio_tiles is None else s.y_audio_tiles.clone()
        y = torch.full_like(s.y_tiles, float("nan"))
        ya = None if want_a is None else torch.full_like(want_a, float("nan"))
        tdp.tdp_tile_attention_noalloc(s.desc, p.n_tiles_local, s.tile_row_begin,
                                       p.max_tile_rows, p.n_rows, s.x_tiles, s.row_pos, s.wq,
                                       s.wk, s.wv, s.wo, s.x_audio, y, ya)
        torch.cuda.synchronize()
        assert torch.equal(y, want), name
        if want_a is not None:
            assert torch.equal(ya, want_a), name
        del s
    assert sizes[1] < sizes[0]


def test_noalloc_refuses_sizes_beyond_its_scratch():
    """The 16-tile step needs gigabytes of workspace: refused with
    TDP_ERR_BUFFER before anything reaches the device (runs without a GPU)."""
    from tiled_video_diffusion_amd import tdp

    wl = ti.workload("t16_16x64x64")
    desc = tdp.attn_desc(1, 128, wl.heads, wl.head_dim, 0, tdp.TDP_BF16, tdp.TDP_BF16)
    n_rows, n_tiles, max_rows = 123904, 16, 9216
    assert tdp.tdp_tile_attention_workspace(desc, n_tiles, n_rows) > SCRATCH_BYTES
    fake = 1 << 20                           # never dereferenced: the size check comes first
    with pytest.raises(tdp.TdpError) as e:
        tdp.tdp_tile_attention_noalloc(desc, n_tiles, fake, max_rows, n_rows, fake, fake, fake,
                                       fake, fake, fake, None, fake, None, 0)
    assert e.value.status == -5              # TDP_ERR_BUFFER
