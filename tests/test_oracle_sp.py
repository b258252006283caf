"""Pins of the sequence-parallel oracle (CPU only).

  * padding: closed forms;
  * the exchange: every element checked against its definition by explicit
    loops, and the round trip gather(send(x)) == x byte for byte (the guide's
    exactness claim);
  * the SP layer equals the untiled attention layer (oracle.tile_forward on
    the whole sequence, itself pinned by brute force) for several world
    sizes, including a token count that needs padding (padded keys masked);
  * the per-rank head shares (each rank's heads over all tokens, output
    projected with those heads' rows of Wo) sum to the full layer.
"""
import numpy as np
import pytest

import oracle
import oracle.sp as osp

RNG = np.random.default_rng(5)


def test_padded_tokens_closed_forms():
    assert osp.padded_tokens(6144, 8) == 6144
    assert osp.padded_tokens(6145, 8) == 6152
    assert osp.padded_tokens(10, 3) == 12
    assert osp.padded_tokens(1, 7) == 7
    for bad in [(0, 2), (5, 0)]:
        with pytest.raises(ValueError):
            osp.padded_tokens(*bad)


@pytest.mark.parametrize("T,W,H,d", [(24, 4, 8, 4), (12, 3, 6, 2), (8, 1, 4, 4), (16, 8, 8, 2)])
def test_exchange_definition_and_round_trip(T, W, H, d):
    t_loc, hw = T // W, H // W
    xs = [RNG.standard_normal((t_loc, H, d)).astype(np.float32) for _ in range(W)]
    bufs = [np.full((T, hw, d), np.nan, np.float32) for _ in range(W)]
    for r in range(W):
        osp.send_heads(xs[r], r, W, T, bufs)
    for s in range(W):
        for t in range(T):
            for j in range(hw):
                assert np.array_equal(bufs[s][t, j], xs[t // t_loc][t % t_loc, s * hw + j])
    for r in range(W):
        back = osp.gather_heads(bufs, r, W, t_loc)
        assert back.dtype == np.float32
        assert np.array_equal(back.view(np.uint32), xs[r].view(np.uint32))


def test_exchange_rejects_bad_shapes():
    with pytest.raises(ValueError):
        osp.send_heads(np.zeros((4, 6, 2)), 0, 4, 16, [np.zeros((16, 1, 2))] * 4)   # 6 % 4
    with pytest.raises(ValueError):
        osp.send_heads(np.zeros((4, 8, 2)), 0, 4, 12, [np.zeros((12, 2, 2))] * 4)   # 4 * 4 != 12


def _layer_inputs(T, C, H, d):
    x = RNG.standard_normal((T, C))
    pos = np.zeros((T, 3, 2))
    f, h, w = np.unravel_index(np.arange(T), (2, 3, -(-T // 6)))
    pos[:, 0] = np.stack([f, f + 1], -1)
    pos[:, 1] = np.stack([h, h + 1], -1)
    pos[:, 2] = np.stack([w, w + 1], -1)
    ws = [RNG.standard_normal((C, H * d)) / np.sqrt(C) for _ in range(3)]
    wo = RNG.standard_normal((H * d, C)) / np.sqrt(H * d)
    return x, pos, ws, wo


@pytest.mark.parametrize("T,W", [(24, 1), (24, 2), (24, 4), (30, 4), (29, 2)])
def test_sp_layer_equals_untiled_layer(T, W):
    C, H, d = 16, 4, 64
    x, pos, (wq, wk, wv), wo = _layer_inputs(T, C, H, d)
    want, _ = oracle.tile_forward(x, pos, None, wq, wk, wv, wo, H, d)
    got = osp.sp_layer(x, pos, wq, wk, wv, wo, H, d, W)
    assert got.shape == want.shape
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_head_shares_sum_to_the_layer():
    T, C, H, d, W = 20, 16, 8, 64, 4
    x, pos, (wq, wk, wv), wo = _layer_inputs(T, C, H, d)
    want, _ = oracle.tile_forward(x, pos, None, wq, wk, wv, wo, H, d)
    total = np.zeros_like(want)
    seen = []
    for r in range(W):
        hs = osp.head_share(H, W, r)
        seen += list(range(H))[hs]
        cols = slice(hs.start * d, hs.stop * d)
        part, _ = oracle.tile_forward(x, pos, None, wq[:, cols], wk[:, cols], wv[:, cols],
                                      wo[cols], H // W, d)
        total += part
    assert sorted(seen) == list(range(H))
    assert np.allclose(total, want, rtol=1e-12, atol=1e-12)
