"""Speculative-token top-k over low-bit scores, per kv head.

Source: SpeCache page, Approach — a speculative token decoded alongside the
output token is scored against the low-bit KV copy, and the top-k KV pairs
of that score are the ones prefetched for the next step.  Readings (the
pages leave these open):
  * candidates are the quantized tokens 0..n_q-1 (residual tokens are fp16 on
    the GPU already, so nothing needs fetching);
  * the GQA heads sharing a kv head are pooled by the max of their logits;
  * the key is a canonical binary32 computation so GPU and CPU agree to the
    bit:  k^_jc = f32(z + f32(code*s))  (code*s is exact for codes < 2^9),
        logit_hj = (((0 + q_h0 k^_j0) + q_h1 k^_j1) + ...)   channel order,
        each product and each sum one IEEE binary32 op;
        key_j = max_h logit_hj + 0.0   (-0 folded to +0);
  * order: key descending, then index ascending (ties go to the lower
    index); slots past n_q hold index -1 and key -inf.

numpy float32 ufuncs do one IEEE op each (numpy has no FMA), so the loop
below is the definition.

Pinned by (tests/test_oracle_topk.py): brute force on tiny shapes (Python
sorted over exact rational scores when they are far apart), agreement with
torch.topk over float64 softmax probabilities for one head, the binary32
error bound against the float64 dot product, tie and padding rules.
Pinned to the bit by (tests/test_oracle_bitlevel.py): two hand-derived
blocks (tests/golden/topk_key_rounding.json) whose keys and order change if
the channel sum is taken pairwise or with fused multiply-adds.
"""
from __future__ import annotations

import numpy as np

from . import quant

__all__ = ["canonical_keys", "select", "topk_block"]


def canonical_keys(qg16: np.ndarray, codes: np.ndarray, ks: np.ndarray,
                   kz: np.ndarray, G: int, path: str) -> np.ndarray:
    """qg16: (gs, d) fp16 speculative-token queries of one kv group.
    codes: (N, d) u8 key codes, ks/kz: (N/G, d) fp16.  Returns f32 (N,)."""
    N, d = codes.shape
    if path == "target":
        code32 = codes.astype(np.float32)
    elif path == "draft4":
        code32 = quant.draft4_code(codes).astype(np.float32)
    else:
        raise ValueError(path)
    s32 = np.repeat(ks.astype(np.float32), G, axis=0)[:N]
    z32 = np.repeat(kz.astype(np.float32), G, axis=0)[:N]
    khat = z32 + code32 * s32                       # (N, d) float32
    q32 = qg16.astype(np.float32)                   # (gs, d)
    acc = np.zeros((q32.shape[0], N), np.float32)
    for c in range(d):
        acc = acc + q32[:, c:c + 1] * khat[None, :, c]
    return acc.max(axis=0) + np.float32(0.0)


def select(key: np.ndarray, k: int):
    """Indices and keys of the k largest keys, ties to the lower index,
    padded with (-1, -inf)."""
    N = key.shape[0]
    order = np.argsort(-key, kind="stable")[:k]
    idx = np.full(k, -1, np.int32)
    val = np.full(k, -np.inf, np.float32)
    idx[: order.shape[0]] = order
    val[: order.shape[0]] = key[order]
    return idx, val


def topk_block(qg16, codes, ks, kz, G, path, k):
    return select(canonical_keys(qg16, codes, ks, kz, G, path), k)
