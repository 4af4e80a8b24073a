"""On-demand reconstruction of a token subset, binary32-exact.

Source: MSpecKV page, Abstract — offloaded KV stays in quantized form and
only the subsets that are needed are reconstructed on demand.  Reading used
(the page gives no formula): the rebuilt row is the cache's own dequantized
value, rounded once more to fp16, with the same binary32 sequence the top-k
keys use:

  p < n_q (quantized):   x^ = fp16_rne( f32(z + f32(code * s)) )
      code = q (target: every stored bit) or 16*(q >> 4) + 7.5 (draft4:
      the INT4 view the QuantSpec draft reads); (s, z) of the token's key
      group (keys) or value group (values)
  n_q <= p < n_q + n_r:  the fp16 residual value itself
  any other p:           NaN

Every * and + is one numpy float32 operation (IEEE binary32, round to
nearest even, no fused multiply-add); the cast to float16 rounds to nearest
even.

Pinned by (tests/test_oracle_gather.py): residual rows equal the appended
fp16 tokens bit for bit; quantized rows are within s/2 (target) or 8 s
(draft4) of the original tokens plus the fp16 rounding of the result; rows
agree with the exact rational value z + code*s to within one fp16 rounding;
a hand-worked group gives the values computed on paper; positions outside
the cache give NaN.
"""
from __future__ import annotations

import numpy as np

__all__ = ["gather_block", "gather"]


def _codes(q: np.ndarray, path: str) -> np.ndarray:
    if path == "target":
        return q.astype(np.float32)
    if path == "draft4":
        return (np.float32(16.0) * (q.astype(np.int32) >> 4).astype(np.float32)
                + np.float32(7.5))
    raise ValueError(path)


def _rebuild(code: np.ndarray, s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    prod = code.astype(np.float32) * s16.astype(np.float32)     # one f32 multiply
    return (z16.astype(np.float32) + prod).astype(np.float16)  # one f32 add, RNE


def gather_block(rep, b: int, h: int, pos: np.ndarray, path: str):
    """fp16 (K, V) rows, each (len(pos), d), of block (b, h) of a
    ``oracle.cache.Replay`` at token positions ``pos``."""
    d, G, Gv = rep.d, rep.G, rep.Gv
    n_q, n_r = rep.n_q, rep.n_r
    K = np.full((len(pos), d), np.nan, np.float16)
    V = np.full((len(pos), d), np.nan, np.float16)
    for i, p in enumerate(np.asarray(pos, np.int64)):
        if 0 <= p < n_q:
            kc = _codes(rep.kq[b, h, p], path)
            vc = _codes(rep.vq[b, h, p], path)
            K[i] = _rebuild(kc, rep.ks[b, h, p // G], rep.kz[b, h, p // G])
            grp = np.arange(d) // Gv
            V[i] = _rebuild(vc, rep.vs[b, h, p][grp], rep.vz[b, h, p][grp])
        elif n_q <= p < n_q + n_r:
            K[i] = rep.rk[b, h, p - n_q]
            V[i] = rep.rv[b, h, p - n_q]
    return K, V


def gather(rep, idx: np.ndarray, path: str):
    """idx: int (B, Hkv, n) positions.  Returns fp16 (K, V), each
    (B, Hkv, n, d)."""
    B, H, n = idx.shape
    K = np.empty((B, H, n, rep.d), np.float16)
    V = np.empty_like(K)
    for b in range(B):
        for h in range(H):
            K[b, h], V[b, h] = gather_block(rep, b, h, idx[b, h], path)
    return K, V
