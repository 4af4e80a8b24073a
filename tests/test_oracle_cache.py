"""Pins for oracle.cache: the flush rule's closed form, flush-time
independence of group codes, rollback leaving quantized data untouched."""
import math

import numpy as np
import pytest

from oracle import cache, quant


def _tokens(rng, B, n, H, d):
    return (rng.standard_normal((B, n, H, d)) * 2).astype(np.float16)


@pytest.mark.parametrize("L,G,R,expect", [
    (256, 32, 32, (224, 32)),          # tiny workload
    (8192, 128, 256, (7936, 256)),     # Llama-2-7B-shaped, 8K
    (32768, 128, 256, (32512, 256)),   # Llama-3-8B GQA, 32K
    (131072, 128, 256, (130816, 256)), # LWM-7B, 128K
    (32768, 32, 32, (32736, 32)),      # SpeCache-style batch
    (100, 32, 256, (0, 100)),          # everything still residual
])
def test_flush_closed_form(L, G, R, expect):
    # closed form: n_q = G * max(0, ceil((L - R) / G)), n_r = L - n_q
    n_q = G * max(0, math.ceil((L - R) / G))
    assert (n_q, L - n_q) == expect
    rep = cache.Replay(1, 1, 64, G, 32, 8, R)
    z = np.zeros((1, L, 1, 64), np.float16)
    rep.append(z, z)
    assert (rep.n_q, rep.n_r) == expect


def test_bulk_equals_incremental_with_rollback():
    rng = np.random.default_rng(5)
    B, H, d, G, Gv, R, bits = 2, 2, 64, 32, 32, 64, 8
    L = 700
    K = _tokens(rng, B, L, H, d)
    V = _tokens(rng, B, L, H, d)
    bulk = cache.Replay(B, H, d, G, Gv, bits, R)
    bulk.append(K, V)
    inc = cache.Replay(B, H, d, G, Gv, bits, R)
    pos = 0
    while pos < L:
        n = int(min(L - pos, rng.integers(1, 40)))
        inc.append(K[:, pos:pos + n], V[:, pos:pos + n])
        pos += n
        if rng.random() < 0.4:
            m = int(rng.integers(0, min(n, inc.n_r) + 1))
            inc.rollback(m)             # reject m draft tokens ...
            pos -= m                    # ... and decode them again
    for name in ("kq", "ks", "kz", "vq", "vs", "vz", "rk", "rv"):
        assert np.array_equal(getattr(bulk, name), getattr(inc, name)), name


def test_store_equals_direct_quantization():
    rng = np.random.default_rng(6)
    B, H, d, G, Gv, R = 1, 3, 128, 128, 64, 256
    L = 1000
    K = _tokens(rng, B, L, H, d)
    V = _tokens(rng, B, L, H, d)
    rep = cache.Replay(B, H, d, G, Gv, 8, R)
    rep.append(K, V)
    for h in range(H):
        q, s, z = quant.quantize_keys(K[0, :rep.n_q, h], G, 8)
        assert np.array_equal(rep.kq[0, h], q) and np.array_equal(rep.ks[0, h], s)
        q, s, z = quant.quantize_values(V[0, :rep.n_q, h], Gv, 8)
        assert np.array_equal(rep.vq[0, h], q) and np.array_equal(rep.vz[0, h], z)
        assert np.array_equal(rep.rk[0, h], K[0, rep.n_q:, h])


def test_rollback_only_touches_residual():
    rng = np.random.default_rng(7)
    rep = cache.Replay(1, 1, 64, 32, 32, 2, 64)
    K = _tokens(rng, 1, 150, 1, 64)
    rep.append(K, K)
    snap = [getattr(rep, n).copy() for n in ("kq", "ks", "kz", "vq", "vs", "vz")]
    n_r = rep.n_r
    rep.rollback(5)
    assert rep.n_r == n_r - 5
    for a, n in zip(snap, ("kq", "ks", "kz", "vq", "vs", "vz")):
        assert np.array_equal(a, getattr(rep, n))
    with pytest.raises(ValueError):
        rep.rollback(rep.n_r + 1)


def test_device_image_shapes():
    rng = np.random.default_rng(8)
    rep = cache.Replay(1, 2, 128, 128, 64, 8, 256)
    K = _tokens(rng, 1, 600, 2, 128)
    rep.append(K, K)
    img = cache.device_image(rep, ring=288)
    assert img["k_hi"].shape == (1, 2, 384, 64)
    assert img["v_lo"].shape == (1, 2, 12, 4 * 128 * 4)
    assert img["v_sz"].shape == (1, 2, 12, 2, 4, 4, 2, 2)
    # 600 tokens, R=256, G=128: ceil(344/128) = 3 groups flushed
    assert (rep.n_q, rep.n_r) == (384, 216)
    assert img["res_slots"].tolist() == [(384 + i) % 288 for i in range(216)]
