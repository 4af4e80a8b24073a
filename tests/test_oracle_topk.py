"""Pins for oracle.topk: exact rational brute force on tiny shapes, the
binary32 error bound, agreement with torch.topk over float64 softmax
probabilities, and the tie / -0 / padding rules."""
from fractions import Fraction

import numpy as np
import torch

from oracle import quant, topk


def _cache(rng, N, d, G, bits, scale=1.0):
    K = (rng.standard_normal((N, d)) * scale).astype(np.float16)
    return quant.quantize_keys(K, G, bits)


def _exact_logits(q16, codes, ks, kz, G, path):
    """Exact rational q . k^ with k^ = z + code*s evaluated exactly."""
    N, d = codes.shape
    out = np.empty((q16.shape[0], N), object)
    for h in range(q16.shape[0]):
        for j in range(N):
            g = j // G
            acc = Fraction(0)
            for c in range(d):
                code = Fraction(int(codes[j, c]))
                if path == "draft4":
                    code = 16 * (int(codes[j, c]) >> 4) + Fraction(15, 2)
                kh = Fraction(float(kz[g, c])) + code * Fraction(float(ks[g, c]))
                acc += Fraction(float(q16[h, c])) * kh
            out[h, j] = acc
    return out


def test_brute_force_tiny():
    rng = np.random.default_rng(0)
    N, d, G, gs, k = 64, 8, 32, 2, 10
    checked = 0
    for bits, path in ((8, "target"), (8, "draft4"), (2, "target"),
                       (1, "target")):
        codes, ks, kz = _cache(rng, N, d, G, bits)
        q = rng.standard_normal((gs, d)).astype(np.float16)
        key = topk.canonical_keys(q, codes, ks, kz, G, path)
        exact = _exact_logits(q, codes, ks, kz, G, path)
        pooled = [max(exact[:, j]) for j in range(N)]
        # binary32 bound: one rounding in k^, d products, d sums
        for j in range(N):
            mag = max(sum(abs(Fraction(float(q[h, c]))) * abs(
                Fraction(float(kz[j // G, c])) + abs(Fraction(float(ks[j // G, c])))
                * 256) for c in range(d)) for h in range(gs))
            assert abs(Fraction(float(key[j])) - pooled[j]) <= (d + 3) * mag / 2**24
        # brute-force order by exact score, ties to lower index
        order = sorted(range(N), key=lambda j: (-pooled[j], j))
        idx, val = topk.select(key, k)
        # the orders agree wherever exact scores are well separated
        gap_ok = all(pooled[order[i]] - pooled[order[i + 1]] > Fraction(1, 10**4)
                     for i in range(k))
        if gap_ok:
            assert idx.tolist() == order[:k]
            checked += 1
        assert np.array_equal(val, key[idx])
    assert checked == 4


def test_matches_torch_topk_on_softmax_probabilities():
    """One head (no pooling): the k tokens with the largest float64 softmax
    probabilities are the top-k keys (checked where ranks are separated)."""
    rng = np.random.default_rng(1)
    N, d, G, k = 2048, 128, 128, 64
    codes, ks, kz = _cache(rng, N, d, G, 8, scale=2.0)
    q = rng.standard_normal((1, d)).astype(np.float16)
    key = topk.canonical_keys(q, codes, ks, kz, G, "target")
    idx, _ = topk.select(key, k)
    Kh = quant.dequant(codes, ks, kz, "key", G)
    logits = torch.from_numpy(Kh @ q[0].astype(np.float64) / np.sqrt(d))
    p = torch.softmax(logits, 0)
    vals, ref = torch.topk(p, k + 1)
    assert (vals[k - 1] - vals[k]) / vals[k] > 1e-5
    assert sorted(idx.tolist()) == sorted(ref[:k].tolist())


def test_ties_negative_zero_and_padding():
    d, G = 8, 32
    codes = np.zeros((32, d), np.uint8)
    ks = np.ones((1, d), np.float16)
    kz = np.zeros((1, d), np.float16)
    codes[[3, 9, 20]] = 2          # three identical best tokens
    codes[[5, 11]] = 1             # two identical runners-up
    q = np.ones((1, d), np.float16)
    key = topk.canonical_keys(q, codes, ks, kz, G, "target")
    idx, val = topk.select(key, 6)
    assert idx.tolist() == [3, 9, 20, 5, 11, 0]
    assert val.tolist() == [16.0, 16.0, 16.0, 8.0, 8.0, 0.0]
    # a zero logit made of negative products is folded to +0
    q2 = -np.ones((1, d), np.float16)
    key2 = topk.canonical_keys(q2, np.zeros((32, d), np.uint8), ks, kz, G,
                               "target")
    assert not np.signbit(key2).any()
    # fewer candidates than k: padded with -1 / -inf
    idx, val = topk.select(key[:4], 6)
    assert idx.tolist()[4:] == [-1, -1] and np.isneginf(val[4:]).all()


def test_max_pooling_over_group_heads():
    rng = np.random.default_rng(2)
    N, d, G = 96, 16, 32
    codes, ks, kz = _cache(rng, N, d, G, 2)
    q = rng.standard_normal((3, d)).astype(np.float16)
    pooled = topk.canonical_keys(q, codes, ks, kz, G, "target")
    single = [topk.canonical_keys(q[h:h + 1], codes, ks, kz, G, "target")
              for h in range(3)]
    assert np.array_equal(pooled, np.maximum.reduce(single))
