"""CPU checks of the host-side pool layout conversions (include/tv.h): the element order
inside a tile -- K element (entry e, channel c) at ((c/32)*64 + e)*32 + c%32, V element
(c, e) at ((e/16)*d + c)*16 + e%16 -- as the binding's converters produce it, their
inverses, and the contiguous-pool tile placement.  Layout only; no arithmetic of the path."""
import numpy as np
import pytest
import torch

from tree_speculative_decoding_amd import tv


@pytest.mark.parametrize("d", [64, 128])
def test_k_tile_order(d):
    x = np.arange(2 * 64 * d).reshape(2, 64, d)
    y = tv.k_to_tiles(x).reshape(2, -1)
    for e in range(64):
        for c in range(d):
            assert y[1, ((c // 32) * 64 + e) * 32 + c % 32] == x[1, e, c]
    assert (tv.k_from_tiles(tv.k_to_tiles(x)) == x).all()
    t = torch.from_numpy(x)
    assert torch.equal(tv.k_from_tiles(tv.k_to_tiles(t)), t)


@pytest.mark.parametrize("d", [64, 128])
def test_v_tile_order(d):
    v = np.arange(3 * d * 64).reshape(3, d, 64)
    z = tv.vt_to_tiles(v).reshape(3, -1)
    for c in range(d):
        for e in range(64):
            assert z[2, ((e // 16) * d + c) * 16 + e % 16] == v[2, c, e]
    assert (tv.vt_from_tiles(tv.vt_to_tiles(v)) == v).all()


def test_tile_vt_round_trip_zero_fills():
    rng = np.random.default_rng(0)
    v = rng.standard_normal((2, 3, 150, 64)).astype(np.float32)
    t = tv.tile_vt(v, 192)
    assert t.shape == (2, 3, 3, 64, 64)
    back = tv.untile_vt(t)
    assert (back[..., :150, :] == v).all() and (back[..., 150:, :] == 0).all()


def test_contiguous_tile_index_is_a_permutation():
    for B, H, cap in [(3, 2, 64 * 37), (1, 8, 64 * 16), (5, 1, 64 * 5)]:
        idx = tv.contiguous_tile_index(B, H, cap)
        assert sorted(idx.reshape(-1).tolist()) == list(range(B * H * cap // 64))
