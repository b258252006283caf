"""Planted mistakes in the oracle must make a pin fail (CPU only).

Each test patches one plausible error into the oracle (a wrong ramp, a
non-strict overlap test, offsets taken over the wrong rows, a RoPE sign, a
wrong softmax scale, a dropped 1/k weight, a swapped projection) and runs the
pin that should catch it, expecting that pin to fail.  The oracle's own code is
untouched outside each test.
"""
import numpy as np
import pytest

import oracle
import oracle.blend as oblend
import oracle.denoise as oden
import oracle.tile_plan as oplan
import tests.test_oracle_attention as tatt
import tests.test_oracle_blend as tblend
import tests.test_oracle_plan as tplan


def _wrong_ramp(L, n, o, i):
    w = _ORIG_DIM_WEIGHTS(L, n, o, i)
    if n > 1 and o > 0:
        w = w.copy()
        a, _ = oplan.dim_boxes(L, n, o)[i]
        if i > 0:      # ramp up with (k+1)/(2o) instead of (2k+1)/(2o)
            s = oplan._cores(L, n)[i] - o // 2
            for k in range(o):
                w[s + k - a] = np.float32(k + 1) / np.float32(2 * o)
    return w


_ORIG_DIM_WEIGHTS = oplan.dim_weights


def test_wrong_ramp_is_caught(monkeypatch):
    monkeypatch.setattr(oplan, "dim_weights", _wrong_ramp)
    with pytest.raises(AssertionError):
        tplan.test_masks_sum_to_one_exactly("tiny_2x16x16")


def test_non_strict_overlap_is_caught(monkeypatch):
    def keeps(cond_pos, j, ext_s, ext_e):
        s, e = cond_pos[j, :, 0], cond_pos[j, :, 1]
        return bool(s[0] < 0 or all(s[d] <= ext_e[d] and e[d] >= ext_s[d] for d in range(3)))
    monkeypatch.setattr(oplan, "_keeps", keeps)
    with pytest.raises(AssertionError):
        for name in ["tiny_2x16x16", "d64_8x32x32", "audio_32x48x80"]:
            tplan.test_keep_rule_brute_force(name)


def test_missing_negative_time_rule_is_caught(monkeypatch):
    def keeps(cond_pos, j, ext_s, ext_e):
        s, e = cond_pos[j, :, 0], cond_pos[j, :, 1]
        return bool(all(s[d] < ext_e[d] and e[d] > ext_s[d] for d in range(3)))
    monkeypatch.setattr(oplan, "_keeps", keeps)
    with pytest.raises(AssertionError):
        tplan.test_keep_rule_brute_force("tiny_2x16x16")


def test_offset_over_all_rows_is_caught(monkeypatch):
    orig = oplan.plan

    def plan(grid, tiling, cond_pos=None, normalize_positions=True, world_size=1, rank=0):
        p = orig(grid, tiling, cond_pos, normalize_positions, world_size, rank)
        if normalize_positions:   # re-base every tile on the min start over ALL its rows
            for t in range(p.tile_id.size):
                r0, r1 = p.tile_row_begin[t], p.tile_row_begin[t + 1]
                raw = p.row_pos[r0:r1] + p.tile_offset[t][None, :, None]
                off = raw[:, :, 0].min(axis=0)
                p.row_pos[r0:r1] = raw - off[None, :, None]
                p.tile_offset[t] = off
        return p
    monkeypatch.setattr(oplan, "plan", plan)
    monkeypatch.setattr(oracle, "plan", plan)
    with pytest.raises(AssertionError):
        tplan.test_normalization_invariants("audio_32x48x80")


def test_rope_sign_error_is_caught(monkeypatch):
    def bad_rope(x, angles):
        x = np.asarray(x, dtype=np.float64)
        c, s = np.cos(angles), np.sin(angles)
        out = np.empty_like(x)
        out[:, 0::2] = x[:, 0::2] * c + x[:, 1::2] * s      # sign flipped here only
        out[:, 1::2] = x[:, 0::2] * s + x[:, 1::2] * c
        return out
    monkeypatch.setattr(oden, "apply_rope", bad_rope)
    monkeypatch.setattr(oracle, "apply_rope", bad_rope)
    with pytest.raises(AssertionError):
        tatt.test_rope_matches_complex_rotation_and_keeps_norms(64)
    with pytest.raises(AssertionError):
        tatt.test_attention_brute_force(False, 12)


def test_rope_axis_mixup_is_caught(monkeypatch):
    orig = oden.rope_angles

    def bad_angles(pos, head_dim, base=10000.0):
        pos = np.asarray(pos)[:, [1, 0, 2], :]              # time and height swapped
        return orig(pos, head_dim, base)
    monkeypatch.setattr(oden, "rope_angles", bad_angles)
    with pytest.raises(AssertionError):
        tatt.test_attention_brute_force(False, 12)


def test_softmax_scale_error_is_caught(monkeypatch):
    orig = oden._softmax_rows
    monkeypatch.setattr(oden, "_softmax_rows", lambda z: orig(z * np.sqrt(2.0)))
    with pytest.raises(AssertionError):
        tatt.test_equal_positions_reduce_to_textbook_attention()


def test_swapped_projection_is_caught(monkeypatch):
    orig = oden.tile_forward

    def bad(x, pos, xa, wq, wk, wv, wo, *a, **k):
        return orig(x, pos, xa, wq, wv, wk, wo, *a, **k)     # K and V weights swapped
    monkeypatch.setattr(oracle, "tile_forward", bad)
    with pytest.raises(AssertionError):
        tatt.test_attention_brute_force(True, 6)


def test_dropped_inverse_k_weight_is_caught(monkeypatch):
    orig = oplan.plan

    def plan(*a, **k):
        p = orig(*a, **k)
        n_gen = p.grid[0] * p.grid[1] * p.grid[2]
        p.row_weight[p.row_src >= n_gen] = 1.0
        return p
    monkeypatch.setattr(oracle, "plan", plan)
    with pytest.raises(AssertionError):
        tblend.test_identity_reconstructs_latent("d64_8x32x32")


def test_blend_row_mixup_is_caught(monkeypatch):
    orig = oblend.blend_tiles

    def bad(y_tiles, p, n_dst=None, y_global=None):
        y = np.array(y_tiles, copy=True)
        y[:, :-1] = y[:, 1:]                                  # off-by-one row
        return orig(y, p, n_dst, y_global)
    monkeypatch.setattr(oracle, "blend_tiles", bad)
    with pytest.raises(AssertionError):
        tblend.test_identity_reconstructs_latent("tiny_2x16x16")


def test_unbalanced_split_is_caught(monkeypatch):
    # taking the smallest divisor above 1 instead of the one nearest sqrt(n)
    def split(n):
        h = next((d for d in range(2, n + 1) if n % d == 0), 1)
        return (min(h, n // h), max(h, n // h))
    monkeypatch.setattr(oracle, "balanced_tile_split", split)
    with pytest.raises(AssertionError):
        tplan.test_balanced_split_brute_force()


def test_transposed_split_is_caught(monkeypatch):
    orig = oplan.balanced_tile_split
    monkeypatch.setattr(oracle, "balanced_tile_split", lambda n: orig(n)[::-1])
    with pytest.raises(AssertionError):
        tplan.test_balanced_split_special_cases()


# ---- the per-tile transformer block ----

import dataclasses as _dc  # noqa: E402

import oracle.block as oblock  # noqa: E402
import tests.test_oracle_block as tblock  # noqa: E402


def _mutated_block(monkeypatch, **changes):
    """Replace block_forward by a copy with one planted change."""
    def block(x, pos, text, mod, lay, heads, head_dim):
        x = np.asarray(x, dtype=np.float64)
        shift_a, scale_a, gate_a, shift_f, scale_f, gate_f = mod
        one = 0.0 if changes.get("no_one_plus") else 1.0
        h = oblock.rms_norm(x) * (one + scale_a) + shift_a
        a, _ = oracle.tile_forward(h, pos, None, lay.wq, lay.wk, lay.wv, lay.wo, heads, head_dim)
        x = x + gate_a * a
        c = oblock.cross_attn(oblock.rms_norm(x), text, lay.cq, lay.ck, lay.cv, lay.co, heads,
                              head_dim)
        x = c if changes.get("no_cross_residual") else x + c
        h = oblock.rms_norm(x) * (one + scale_f) + shift_f
        f = oblock.ffn(h, lay.w1, lay.w2)
        return x + (f if changes.get("ungated_ffn") else gate_f * f)
    monkeypatch.setattr(oblock, "block_forward", block)


def test_scale_without_one_is_caught(monkeypatch):
    _mutated_block(monkeypatch, no_one_plus=True)
    with pytest.raises(AssertionError):
        tblock.test_block_self_attention_branch_is_the_hot_path_layer()


def test_missing_cross_residual_is_caught(monkeypatch):
    _mutated_block(monkeypatch, no_cross_residual=True)
    with pytest.raises(AssertionError):
        tblock.test_block_with_closed_gates_is_identity()


def test_ungated_ffn_is_caught(monkeypatch):
    _mutated_block(monkeypatch, ungated_ffn=True)
    with pytest.raises(AssertionError):
        tblock.test_block_with_closed_gates_is_identity()


def test_gelu_without_cubic_term_is_caught(monkeypatch):
    monkeypatch.setattr(oblock, "gelu_tanh",
                        lambda u: 0.5 * np.asarray(u) * (1 + np.tanh(np.sqrt(2 / np.pi) * np.asarray(u))))
    with pytest.raises(AssertionError):
        tblock.test_gelu_tanh_against_erf_gelu_and_odd_part()


def test_cross_attn_scale_by_d_is_caught(monkeypatch):
    orig = oblock.cross_attn
    monkeypatch.setattr(oblock, "cross_attn",
                        lambda h, t, wq, wk, wv, wo, heads, d: orig(h, t, wq / np.sqrt(d), wk, wv, wo,
                                                                    heads, d))
    with pytest.raises(AssertionError):
        tblock.test_cross_attn_brute_force()


def test_rms_eps_outside_root_is_caught(monkeypatch):
    monkeypatch.setattr(oblock, "rms_norm",
                        lambda x, eps=oblock.RMS_EPS: np.asarray(x) / (
                            np.sqrt(np.mean(np.asarray(x) ** 2, axis=-1, keepdims=True)) + eps))
    with pytest.raises(AssertionError):
        tblock.test_rms_norm_closed_forms()


# --------------------------------------------------------------------------
# the upscale loop
# --------------------------------------------------------------------------

import oracle.upscale as oup  # noqa: E402
import tests.test_oracle_upscale as tup  # noqa: E402

_SIGMAS = oup.linear_sigmas(0.8, 3)


def test_euler_sign_error_is_caught(monkeypatch):
    def step(x, v, sigma, sigma_next, n_gen):
        out = np.array(x, dtype=np.float64, copy=True)
        out[:, :n_gen] += (np.float64(sigma) - np.float64(sigma_next)) * v[:, :n_gen]
        return out
    monkeypatch.setattr(oup, "euler_step", step)
    with pytest.raises(AssertionError):
        tup.test_straight_path_is_followed_exactly(_SIGMAS)


def test_renoise_without_signal_decay_is_caught(monkeypatch):
    def renoise(x1, noise, sigma0, n_gen):
        x = np.array(x1, dtype=np.float64, copy=True)
        x[:, :n_gen] += np.float64(sigma0) * noise
        return x
    monkeypatch.setattr(oup, "renoise", renoise)
    with pytest.raises(AssertionError):
        tup.test_straight_path_is_followed_exactly(_SIGMAS)


def test_euler_on_conditioning_rows_is_caught(monkeypatch):
    def step(x, v, sigma, sigma_next, n_gen):
        return np.asarray(x, dtype=np.float64) + (np.float64(sigma_next) - np.float64(sigma)) * v
    monkeypatch.setattr(oup, "euler_step", step)
    with pytest.raises(AssertionError):
        tup.test_straight_path_is_followed_exactly(_SIGMAS)


def test_unweighted_seam_spread_is_caught(monkeypatch):
    def seam(y_tiles, p, n_gen):
        q = _dc.replace(p, row_weight=np.ones_like(p.row_weight))
        return _ORIG_SEAM(y_tiles, q, n_gen)
    monkeypatch.setattr(oup, "seam_spread", seam)
    with pytest.raises(AssertionError):
        tup.test_seam_spread_two_tile_closed_form()


def test_timestep_without_scale_is_caught(monkeypatch):
    monkeypatch.setattr(oup, "TAU_PER_SIGMA", 1.0)
    with pytest.raises(AssertionError):
        tup.test_one_step_is_the_block_step()


_ORIG_SEAM = oup.seam_spread


# --------------------------------------------------------------------------
# sequence parallelism
# --------------------------------------------------------------------------

import oracle.sp as osp  # noqa: E402
import tests.test_oracle_sp as tsp  # noqa: E402


def test_unmasked_padding_is_caught(monkeypatch):
    def softmax_all(logits, n_valid):
        m = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - m)
        return e / e.sum(axis=1, keepdims=True)
    monkeypatch.setattr(osp, "_softmax_masked", softmax_all)
    with pytest.raises(AssertionError):
        tsp.test_sp_layer_equals_untiled_layer(30, 4)


def test_exchange_to_the_wrong_rank_is_caught(monkeypatch):
    def send(x_local, rank, world, t_pad, dst):
        t_loc, heads, _ = x_local.shape
        hw = heads // world
        for s in range(world):
            src = (s + 1) % world
            dst[s][rank * t_loc:(rank + 1) * t_loc] = x_local[:, src * hw:(src + 1) * hw]
    monkeypatch.setattr(osp, "send_heads", send)
    with pytest.raises(AssertionError):
        tsp.test_exchange_definition_and_round_trip(24, 4, 8, 4)
