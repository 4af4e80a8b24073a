"""Speculative verify / draft attention over the quantized cache, float64.

Sources: QuantSpec page, Approach (the draft attends over the upper-4-bit
cache, the target verifies gamma+1 tokens over the INT8 cache, recent tokens
in an fp16 buffer); SpeCache page, Approach (output token plus speculative
token decoded together over the low-bit copy).  FlashDecoding's split-K is
an evaluation order of the same softmax, so the oracle is the plain
definition, with no splitting:

  kvh(h)   = h // (Hq // Hkv)                         (GQA, contiguous groups)
  pos(t)   = L - T + t    (the T query tokens are the last T cache tokens)
  logit    = sm_scale * q[t, h] . k^[j]     for j <= pos(t), else excluded
  out[t,h] = sum_j softmax_j(logit) v^[j]
  lse[h,t] = log sum_j exp(logit)

k^, v^: dequantized codes (target: z + q*s; draft4: z + (16*(q>>4)+7.5)*s)
for j < n_q, and the fp16 values themselves for residual tokens j >= n_q.

Pinned by (tests/test_oracle_attention.py): equality with torch's
scaled_dot_product_attention (float64, CPU) when the whole context is in the
residual buffer, equality with the same routine applied to the dequantized
cache, row t of a verify equal to a T=1 decode over the first pos(t)+1
tokens, GQA equal to MHA with repeated kv heads, and the draft ignoring the
low nibble plane.  Exact substitution (``attend_exact``): no positions gives
``attend``; substituting every quantized token by its original fp16 value
gives SDPA over the original tokens for that row and leaves the other rows
as they were; substituting a token by its own dequantized value (when that
value is an fp16 number) changes nothing.
"""
from __future__ import annotations

import numpy as np

from . import quant

__all__ = ["block_kv", "attend_block", "attend", "attend_exact",
           "max_value_scale", "VALUE_SCALE_LIMIT"]

# Domain of the inputs (a reading, with finiteness): every value group's
# scale is at most 63.  The library's attention multiplies fp16
# probabilities scaled to at most 2^10 by the value scale in fp16, which
# stays finite up to 63; the oracle itself has no such limit.
VALUE_SCALE_LIMIT = 63.0


def max_value_scale(rep) -> float:
    """Largest value-group scale in an ``oracle.cache.Replay`` (0 when
    nothing is quantized), to check inputs against VALUE_SCALE_LIMIT."""
    return float(rep.vs.max()) if rep.vs.size else 0.0


def block_kv(kq, ks, kz, vq, vs, vz, rk, rv, G, Gv, path):
    """Float64 (K, V) of one block: dequantized prefix then fp16 residual.
    kq/vq: (n_q, d) codes; ks/kz (n_q/G, d); vs/vz (n_q, d/Gv); rk/rv
    (n_r, d) fp16.  path: "target" or "draft4"."""
    if path == "target":
        Kq = quant.dequant(kq, ks, kz, "key", G)
        Vq = quant.dequant(vq, vs, vz, "value", Gv)
    elif path == "draft4":
        Kq = quant.dequant_draft4(kq, ks, kz, "key", G)
        Vq = quant.dequant_draft4(vq, vs, vz, "value", Gv)
    else:
        raise ValueError(path)
    K = np.concatenate([Kq, rk.astype(np.float64)], axis=0)
    V = np.concatenate([Vq, rv.astype(np.float64)], axis=0)
    return K, V


def attend_block(q16: np.ndarray, K: np.ndarray, V: np.ndarray,
                 sm_scale: float):
    """q16: (T, gs, d) queries of the gs heads sharing this kv block.
    K, V: (L, d) float64.  Returns out (T, gs, d) and lse (gs, T), float64."""
    T, gs, d = q16.shape
    L = K.shape[0]
    q = q16.astype(np.float64)
    logits = np.einsum("thc,jc->thj", q, K) * float(sm_scale)
    pos = L - T + np.arange(T)
    visible = np.arange(L)[None, :] <= pos[:, None]          # (T, L)
    logits = np.where(visible[:, None, :], logits, -np.inf)
    m = logits.max(axis=2, keepdims=True)
    p = np.exp(logits - m)
    l = p.sum(axis=2, keepdims=True)
    out = np.einsum("thj,jc->thc", p, V) / l
    lse = (m + np.log(l))[:, :, 0].T
    return out, lse


def attend(rep, q16: np.ndarray, path: str, sm_scale: float):
    """Whole-cache attention for an ``oracle.cache.Replay``.
    q16: (B, T, Hq, d).  Returns out (B, T, Hq, d), lse (B, Hq, T)."""
    B, T, Hq, d = q16.shape
    gs = Hq // rep.Hkv
    out = np.empty((B, T, Hq, d), np.float64)
    lse = np.empty((B, Hq, T), np.float64)
    for b in range(B):
        for h in range(rep.Hkv):
            K, V = block_kv(rep.kq[b, h], rep.ks[b, h], rep.kz[b, h],
                            rep.vq[b, h], rep.vs[b, h], rep.vz[b, h],
                            rep.rk[b, h], rep.rv[b, h], rep.G, rep.Gv, path)
            o, s = attend_block(q16[b, :, h * gs:(h + 1) * gs], K, V, sm_scale)
            out[b, :, h * gs:(h + 1) * gs] = o
            lse[b, h * gs:(h + 1) * gs] = s
    return out, lse


def attend_exact(rep, q16: np.ndarray, path: str, sm_scale: float,
                 idx: np.ndarray, k_exact: np.ndarray, v_exact: np.ndarray,
                 t_exact: int = 0):
    """``attend`` with exact substitution for one query row (SpeCache page,
    Approach: the KV pairs the speculative token ranks highest are fetched
    in full precision and used for the output token).  Query row t_exact
    reads the fp16 values k_exact/v_exact at the quantized positions
    idx[b, kvh] (entries < 0 are skipped) instead of their dequantized
    values; every other row reads the cache as ``attend`` does.
    idx: (B, Hkv, n) int, distinct positions < n_q per block;
    k_exact, v_exact: (B, Hkv, n, d) fp16.  Returns out, lse as ``attend``."""
    out, lse = attend(rep, q16, path, sm_scale)
    B, T, Hq, d = q16.shape
    gs = Hq // rep.Hkv
    for b in range(B):
        for h in range(rep.Hkv):
            K, V = block_kv(rep.kq[b, h], rep.ks[b, h], rep.kz[b, h],
                            rep.vq[b, h], rep.vs[b, h], rep.vz[b, h],
                            rep.rk[b, h], rep.rv[b, h], rep.G, rep.Gv, path)
            sel = np.asarray(idx[b, h])
            keep = sel >= 0
            assert (sel[keep] < rep.n_q).all()
            assert len(np.unique(sel[keep])) == keep.sum()
            K[sel[keep]] = k_exact[b, h][keep].astype(np.float64)
            V[sel[keep]] = v_exact[b, h][keep].astype(np.float64)
            o, s = attend_block(q16[b, :, h * gs:(h + 1) * gs], K, V, sm_scale)
            out[b, t_exact, h * gs:(h + 1) * gs] = o[t_exact]
            lse[b, h * gs:(h + 1) * gs, t_exact] = s[:, t_exact]
    return out, lse
