"""Pins for oracle.layout: round trips, bit-disjointness of the tiled V
layout, the hi/lo nibble identity, and single codes placed at byte/bit
positions worked out by hand from the layout definition."""
import numpy as np
import pytest

from oracle import layout


def test_nibble_identity():
    q = np.arange(256, dtype=np.uint8)
    hi, lo = layout.split_planes(q, 8)
    assert np.array_equal(hi, q >> 4) and np.array_equal(lo, q & 15)
    assert np.array_equal(((hi.astype(np.int32) << 4) | lo), q)
    assert np.array_equal(layout.join_planes(hi, lo, 8), q)
    assert (hi[0x4D], lo[0x4D]) == (4, 13)


@pytest.mark.parametrize("w,d", [(4, 64), (4, 128), (2, 64), (2, 128),
                                 (1, 128)])
def test_k_plane_round_trip(w, d):
    rng = np.random.default_rng(w * d)
    vals = rng.integers(0, 1 << w, (40, d)).astype(np.uint8)
    raw = layout.pack_k_plane(vals, w)
    assert raw.shape == (40, d * w // 8)
    assert np.array_equal(layout.unpack_k_plane(raw, w, d), vals)


def test_k_plane_hand_placed():
    # w=2, channel 13 of token 1 -> byte 13//4 = 3 of row 1, bit 2*(13%4) = 2
    vals = np.zeros((2, 64), np.uint8)
    vals[1, 13] = 3
    raw = layout.pack_k_plane(vals, 2)
    assert np.argwhere(raw).tolist() == [[1, 3]] and raw[1, 3] == 3 << 2
    # w=4: odd channel 9 -> byte 4, high nibble
    vals = np.zeros((1, 64), np.uint8)
    vals[0, 9] = 0xA
    raw = layout.pack_k_plane(vals, 4)
    assert raw[0, 4] == 0xA0 and raw.sum() == 0xA0


@pytest.mark.parametrize("w,d", [(4, 64), (4, 128), (2, 64), (2, 128),
                                 (1, 64), (1, 128)])
def test_v_tile_bits_disjoint_and_round_trip(w, d):
    dw, bit = layout.v_tile_index(d, w)
    cells = set()
    for j in range(32):
        for c in range(d):
            for k in range(w):
                cells.add((int(dw[j, c]), int(bit[j, c]) + k))
    assert len(cells) == 32 * d * w                       # no overlap
    assert max(b for _, b in cells) < 32                  # inside a dword
    assert max(x for x, _ in cells) == d * w - 1          # dense tile
    rng = np.random.default_rng(w + d)
    vals = rng.integers(0, 1 << w, (96, d)).astype(np.uint8)
    raw = layout.pack_v_plane(vals, w)
    assert raw.shape == (3, 4 * d * w)
    assert np.array_equal(layout.unpack_v_plane(raw, w, d), vals)


def test_v_tile_hand_placed():
    # w=4, d=128: token j=5 (g=1, i=1, h=0), channel 35 (r=3, m=2):
    # lane 16+3 = 19, dword 19*8 + 2 = 154, bit 4 -> byte 616, high nibble.
    vals = np.zeros((32, 128), np.uint8)
    vals[5, 35] = 0xB
    raw = layout.pack_v_plane(vals, 4)[0]
    assert np.argwhere(raw).ravel().tolist() == [616] and raw[616] == 0xB0
    # token 21 (h=1, same g, i) lands 16 bits higher: byte 618, high nibble
    vals[:] = 0
    vals[21, 35] = 0x7
    raw = layout.pack_v_plane(vals, 4)[0]
    assert np.argwhere(raw).ravel().tolist() == [618] and raw[618] == 0x70
    # w=1, d=128: token 2 (g=0, i=2, h=0), channel 100 (r=4, m=6):
    # per=4, lane 4, dword 4*2 + 6//4 = 9, bit 1*(4*(6%4)+2) = 10 -> byte 37
    # bit 2.
    vals = np.zeros((32, 128), np.uint8)
    vals[2, 100] = 1
    raw = layout.pack_v_plane(vals, 1)[0]
    assert np.argwhere(raw).ravel().tolist() == [37] and raw[37] == 1 << 2


def test_v_sz_round_trip_and_position():
    rng = np.random.default_rng(0)
    s = rng.standard_normal((64, 2)).astype(np.float16)
    z = rng.standard_normal((64, 2)).astype(np.float16)
    raw = layout.pack_v_sz(s, z)
    assert raw.shape == (2, 2, 4, 4, 2, 2)
    s2, z2 = layout.unpack_v_sz(raw)
    assert np.array_equal(s2, s) and np.array_equal(z2, z)
    # token 21 of tile 1: g = (21 % 16) // 4 = 1, i = 1, h = 1
    assert raw[1, 0, 1, 1, 0, 1] == s[32 + 21, 0]
    assert raw[1, 1, 1, 1, 1, 1] == z[32 + 21, 1]
    # token 5 shares that u32 as its low half (g = 1, i = 1, h = 0)
    assert raw[1, 0, 1, 1, 0, 0] == s[32 + 5, 0]


def test_v_res_tile_round_trip_and_position():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((32, 128)).astype(np.float16)
    tile = layout.pack_v_res_tile(v)
    assert np.array_equal(layout.unpack_v_res_tile(tile, 128), v)
    assert len(set(layout.v_res_index(128).ravel().tolist())) == 32 * 128
    # slot 18 (g=0, i=2, h=1), channel 17 (r=1, m=1): (0+1)*64 + 8 + 4 + 1
    assert tile[77] == v[18, 17]


def test_k_sz_pairs():
    s = np.array([[1.5, 2.0]], np.float16)
    z = np.array([[-1.0, 0.25]], np.float16)
    raw = layout.pack_k_sz(s, z)
    assert raw.tolist() == [[[1.5, -1.0], [2.0, 0.25]]]
