"""Append / flush / rollback replay of the hierarchical quantized cache.

Source: QuantSpec page, Approach — recent tokens stay in a full-precision
double buffer of size 2G; the oldest tokens are quantized when it overflows;
rejected draft tokens are rolled back without requantizing.  Reading used
(the pages give no exact rule): after appending, while the residual holds
more than R tokens, its oldest G tokens are quantized as one key group (per
channel) and G value groups (per token).  Rollback pops the newest tokens
of the residual only.

State per (b, kvh) block is kept as logical numpy arrays (codes, scales,
zeros, fp16 residual).  ``device_image`` packs it into the bytes the library
stores (via ``oracle.layout``) for bit-exact comparison.

Pinned by (tests/test_oracle_cache.py): a group's codes do not depend on
when it was flushed (one bulk append == many small appends), rollback never
changes quantized data, the counters follow the flush rule's closed form, and
the quantized store equals quantizing the first n_q tokens directly.
"""
from __future__ import annotations

import numpy as np

from . import layout, quant

__all__ = ["Replay", "device_image"]


class Replay:
    def __init__(self, B, Hkv, d, G, Gv, bits, R):
        self.B, self.Hkv, self.d = B, Hkv, d
        self.G, self.Gv, self.bits, self.R = G, Gv, bits, R
        ng = d // Gv
        self.kq = np.zeros((B, Hkv, 0, d), np.uint8)
        self.ks = np.zeros((B, Hkv, 0, d), np.float16)
        self.kz = np.zeros((B, Hkv, 0, d), np.float16)
        self.vq = np.zeros((B, Hkv, 0, d), np.uint8)
        self.vs = np.zeros((B, Hkv, 0, ng), np.float16)
        self.vz = np.zeros((B, Hkv, 0, ng), np.float16)
        self.rk = np.zeros((B, Hkv, 0, d), np.float16)
        self.rv = np.zeros((B, Hkv, 0, d), np.float16)

    @property
    def n_q(self) -> int:
        return self.kq.shape[2]

    @property
    def n_r(self) -> int:
        return self.rk.shape[2]

    def append(self, k_new: np.ndarray, v_new: np.ndarray) -> int:
        """k_new, v_new: fp16 (B, n, Hkv, d), the token-major order the
        library takes.  Returns the number of groups flushed."""
        kn = np.transpose(np.asarray(k_new, np.float16), (0, 2, 1, 3))
        vn = np.transpose(np.asarray(v_new, np.float16), (0, 2, 1, 3))
        self.rk = np.concatenate([self.rk, kn], axis=2)
        self.rv = np.concatenate([self.rv, vn], axis=2)
        flushed = 0
        while self.n_r - flushed * self.G > self.R:
            flushed += 1
        if flushed:
            self._flush(flushed * self.G)
        return flushed

    def _flush(self, n: int):
        B, H, d = self.B, self.Hkv, self.d
        kq = np.empty((B, H, n, d), np.uint8)
        ks = np.empty((B, H, n // self.G, d), np.float16)
        kz = np.empty_like(ks)
        vq = np.empty((B, H, n, d), np.uint8)
        vs = np.empty((B, H, n, d // self.Gv), np.float16)
        vz = np.empty_like(vs)
        for b in range(B):
            for h in range(H):
                kq[b, h], ks[b, h], kz[b, h] = quant.quantize_keys(
                    self.rk[b, h, :n], self.G, self.bits)
                vq[b, h], vs[b, h], vz[b, h] = quant.quantize_values(
                    self.rv[b, h, :n], self.Gv, self.bits)
        self.kq = np.concatenate([self.kq, kq], axis=2)
        self.ks = np.concatenate([self.ks, ks], axis=2)
        self.kz = np.concatenate([self.kz, kz], axis=2)
        self.vq = np.concatenate([self.vq, vq], axis=2)
        self.vs = np.concatenate([self.vs, vs], axis=2)
        self.vz = np.concatenate([self.vz, vz], axis=2)
        self.rk = self.rk[:, :, n:]
        self.rv = self.rv[:, :, n:]

    def rollback(self, m: int):
        if m > self.n_r:
            raise ValueError("rollback longer than the residual")
        keep = self.n_r - m
        self.rk = self.rk[:, :, :keep]
        self.rv = self.rv[:, :, :keep]


def device_image(rep: Replay, ring: int):
    """Expected device bytes of the defined region of every buffer.

    Returns a dict of per-block arrays (leading dims B, Hkv):
      k_hi, k_lo: u8 (n_q, d*w/8) rows      v_hi, v_lo: u8 (n_q/32, 4*d*w)
      k_sz: fp16 (n_q/G, d, 2)              v_sz: fp16 (n_q/32, 2, 4, 4, ng, 2)
      k_res: fp16 (n_r, d) with slots ``res_slots``
      v_res: fp16 (n_r, d) values of the same slots (read back with
             oracle.layout.unpack_v_res_tile)
    """
    w = layout.plane_width(rep.bits)
    B, H = rep.B, rep.Hkv
    out = {k: [] for k in ("k_hi", "k_lo", "v_hi", "v_lo", "k_sz", "v_sz")}
    for b in range(B):
        row = {k: [] for k in out}
        for h in range(H):
            khi, klo = layout.split_planes(rep.kq[b, h], rep.bits)
            vhi, vlo = layout.split_planes(rep.vq[b, h], rep.bits)
            row["k_hi"].append(layout.pack_k_plane(khi, w))
            row["v_hi"].append(layout.pack_v_plane(vhi, w))
            if rep.bits == 8:
                row["k_lo"].append(layout.pack_k_plane(klo, w))
                row["v_lo"].append(layout.pack_v_plane(vlo, w))
            row["k_sz"].append(layout.pack_k_sz(rep.ks[b, h], rep.kz[b, h]))
            row["v_sz"].append(layout.pack_v_sz(rep.vs[b, h], rep.vz[b, h]))
        for k in out:
            out[k].append(row[k])
    img = {k: (np.array(v) if v[0] else None) for k, v in out.items()}
    img["res_slots"] = (rep.n_q + np.arange(rep.n_r)) % ring
    img["k_res"] = rep.rk.copy()
    img["v_res"] = rep.rv.copy()
    return img
