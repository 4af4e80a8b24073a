"""Device byte layouts of the quantized cache, written from their definition.

The library's C header defines where every code, scale and residual value
lives.  This module packs logical arrays into those bytes and unpacks them,
independently of the HIP code, so GPU buffers can be compared bit for bit.

Definitions (per (b, kvh) block; LSB-first bit packing; w = bits per code
in a plane: 4 for 8-bit codes split into hi/lo nibble planes, else 2 or 1):

  K plane       u8 [L_max][d*w/8]: channel c in byte c // (8/w) at bit
                w * (c % (8/w)).
  K scale/zero  fp16 [L_max/G][d][2] = (s, z).
  V plane tile  u8 [4*d*w] per 32 tokens; token j, channel c:
                g=(j%16)//4, i=j%4, h=j//16, r=c%16, m=c//16, per=4//w,
                u32 index (16g+r)*(d*w//64) + m//per, bit 16h + w*(4*(m%per)+i).
  V scale/zero  fp16 [L_max/32][2][4][4][d/Gv][2] per tile, indexed
                [part][g][i][group][h]: part 0 = scales, 1 = zero-points,
                token j = 16h + 4g + i.
  k_res         fp16 [ring][d], slot = position % ring.
  v_res tile    fp16 [32*d] per 32 slots; slot j, channel c at half index
                (16g+r)*(d//2) + 8m + 2i + h.

Pinned by (tests/test_oracle_layout.py): pack/unpack round trips, every
(token, channel) mapping to a distinct bit, the hi/lo nibble identity
q == (hi << 4) | lo, and hand-placed single codes at positions worked out
from the definition by hand.
"""
from __future__ import annotations

import numpy as np

__all__ = ["plane_width", "split_planes", "join_planes", "pack_k_plane",
           "unpack_k_plane", "v_tile_index", "pack_v_plane", "unpack_v_plane",
           "pack_k_sz", "unpack_k_sz", "pack_v_sz", "unpack_v_sz",
           "v_res_index", "pack_v_res_tile", "unpack_v_res_tile"]


def plane_width(bits: int) -> int:
    return {8: 4, 2: 2, 1: 1}[bits]


def split_planes(q: np.ndarray, bits: int):
    """Logical codes -> per-plane values: (hi, lo) for 8-bit, (q, None)."""
    q = q.astype(np.uint8)
    if bits == 8:
        return q >> 4, q & 15
    return q, None


def join_planes(hi: np.ndarray, lo: np.ndarray | None, bits: int):
    if bits == 8:
        return ((hi.astype(np.uint16) << 4) | lo).astype(np.uint8)
    return hi.astype(np.uint8)


# ---- K planes: token-major rows ------------------------------------------

def pack_k_plane(vals: np.ndarray, w: int) -> np.ndarray:
    """vals: (N, d) codes of one plane (each < 2**w) -> u8 (N, d*w/8)."""
    N, d = vals.shape
    per = 8 // w
    v = vals.astype(np.uint8).reshape(N, d // per, per)
    out = np.zeros((N, d // per), np.uint8)
    for k in range(per):
        out |= (v[:, :, k] << (w * k)).astype(np.uint8)
    return out


def unpack_k_plane(raw: np.ndarray, w: int, d: int) -> np.ndarray:
    N = raw.shape[0]
    per = 8 // w
    mask = (1 << w) - 1
    out = np.empty((N, d // per, per), np.uint8)
    for k in range(per):
        out[:, :, k] = (raw >> (w * k)) & mask
    return out.reshape(N, d)


# ---- V planes: 32-token tiles --------------------------------------------

def v_tile_index(d: int, w: int):
    """(u32 index, bit) arrays of shape (32, d) for a V plane tile."""
    j = np.arange(32)[:, None]
    c = np.arange(d)[None, :]
    g = (j % 16) // 4
    i = j % 4
    h = j // 16
    r = c % 16
    m = c // 16
    per = 4 // w
    lane = 16 * g + r
    dword = lane * (d * w // 64) + m // per
    bit = 16 * h + w * (4 * (m % per) + i)
    return np.broadcast_to(dword, (32, d)), np.broadcast_to(bit, (32, d))


def pack_v_plane(vals: np.ndarray, w: int) -> np.ndarray:
    """vals: (N, d) codes of one plane, N a multiple of 32 -> u8 (N/32,
    4*d*w)."""
    N, d = vals.shape
    nt = N // 32
    dw, bit = v_tile_index(d, w)
    words = np.zeros((nt, d * w), np.uint64)
    v = vals.reshape(nt, 32, d).astype(np.uint64)
    shifted = v << bit.astype(np.uint64)[None]
    flat_idx = dw.reshape(-1)
    for t in range(nt):
        np.add.at(words[t], flat_idx, shifted[t].reshape(-1))
    return words.astype(np.uint32).view(np.uint8).reshape(nt, 4 * d * w)


def unpack_v_plane(raw: np.ndarray, w: int, d: int) -> np.ndarray:
    nt = raw.shape[0]
    words = np.ascontiguousarray(raw).view(np.uint32).reshape(nt, d * w)
    dw, bit = v_tile_index(d, w)
    mask = (1 << w) - 1
    vals = (words[:, dw] >> bit[None].astype(np.uint32)) & mask
    return vals.reshape(nt * 32, d).astype(np.uint8)


# ---- scale/zero ------------------------------------------------------------

def pack_k_sz(s: np.ndarray, z: np.ndarray) -> np.ndarray:
    """(N/G, d) s, z -> fp16 (N/G, d, 2)."""
    return np.stack([s.astype(np.float16), z.astype(np.float16)], axis=-1)


def unpack_k_sz(raw: np.ndarray):
    return raw[..., 0].copy(), raw[..., 1].copy()


def _v_sz_index():
    """(g, i, h) of tile token j for the scale/zero planes."""
    j = np.arange(32)
    return (j % 16) // 4, j % 4, j // 16


def pack_v_sz(s: np.ndarray, z: np.ndarray) -> np.ndarray:
    """(N, d/Gv) s, z -> fp16 (N/32, 2, 4, 4, d/Gv, 2)."""
    N, ng = s.shape
    nt = N // 32
    st = s.reshape(nt, 32, ng).astype(np.float16)
    zt = z.reshape(nt, 32, ng).astype(np.float16)
    out = np.empty((nt, 2, 4, 4, ng, 2), np.float16)
    for j, (g, i, h) in enumerate(zip(*_v_sz_index())):
        out[:, 0, g, i, :, h] = st[:, j]
        out[:, 1, g, i, :, h] = zt[:, j]
    return out


def unpack_v_sz(raw: np.ndarray):
    nt, _, _, _, ng, _ = raw.shape
    s = np.empty((nt, 32, ng), np.float16)
    z = np.empty_like(s)
    for j, (g, i, h) in enumerate(zip(*_v_sz_index())):
        s[:, j] = raw[:, 0, g, i, :, h]
        z[:, j] = raw[:, 1, g, i, :, h]
    return s.reshape(nt * 32, ng), z.reshape(nt * 32, ng)


# ---- residual V ring tiles ----------------------------------------------------

def v_res_index(d: int):
    """Half index (32, d) of slot j, channel c inside a v_res tile."""
    j = np.arange(32)[:, None]
    c = np.arange(d)[None, :]
    g = (j % 16) // 4
    i = j % 4
    h = j // 16
    r = c % 16
    m = c // 16
    return (16 * g + r) * (d // 2) + 8 * m + 2 * i + h


def pack_v_res_tile(vals: np.ndarray) -> np.ndarray:
    """(32, d) fp16 -> (32*d,) fp16 tile."""
    d = vals.shape[1]
    out = np.empty(32 * d, np.float16)
    out[v_res_index(d)] = vals
    return out


def unpack_v_res_tile(tile: np.ndarray, d: int) -> np.ndarray:
    return tile[v_res_index(d)].astype(np.float16)
