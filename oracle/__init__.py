"""CPU oracle for one Tiled Data Parallelism (TDP) upscale step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The GPU library never imports,
links or calls it, and it shares no code with the GPU library: the only module
both sides use is ``tdp_inputs``, which draws seeded inputs and holds none of
the method's arithmetic.

The oracle follows the TDP design page ("Tiled Data Parallelism (TDP)") step by
step, in plain NumPy:

  tile_plan.py  tiles, round-robin share, generated rows and trapezoid masks,
              position normalization, conditioning keep rule and 1/k weights,
              and the inverse (destination -> rows) map
  denoise.py    the per-tile denoiser: QKV projection, 3D RoPE, multi-head
              softmax attention, output projection (float64)
  blend.py      gather of tile rows and the weighted blend into the global
              latent that stands in for the multi-GPU all_reduce (float64)
  tdp_step.py   one whole step built from the three
  block.py      the per-tile transformer block (norms, timestep modulation,
              self- and cross-attention, FFN) and a step that uses it
  upscale.py    the upscale loop: re-noise, TDP velocity and Euler update per
              step, seam spread of the tiles
  sp.py         sequence parallelism for the first stage: token partition,
              head exchange and its inverse, the layer computed the SP way

Where the pages are silent, the readings used are stated in each function's
docstring.  Pins (tests that tie each function to something other than
itself) live in ``tests/test_oracle_*.py``.  Parity unpinned: the specific
constants of the trapezoid ramp, the tile-geometry rule, the RoPE frequency
split and the audio joint-attention reading are fixed by the readings stated
here and checked only through invariants (masks sum to one, shift invariance,
brute force), because the pages print no worked example.
"""
from .tile_plan import (Plan, plan, dim_boxes, dim_weights, PlanError,  # noqa: F401
                        balanced_tile_split, assign_tiles)
from .denoise import rope_angles, apply_rope, tile_forward  # noqa: F401
from .blend import gather_tiles, blend_tiles, audio_mean  # noqa: F401
from .tdp_step import step  # noqa: F401
from .upscale import (linear_sigmas, renoise, euler_step, seam_spread,  # noqa: F401
                      upscale_loop)
from .sp import padded_tokens, send_heads, gather_heads, sp_layer, head_share  # noqa: F401
