"""Pins for oracle.quant: closed-form invariants of the asymmetric min/max
quantizer, the grouping axes, and a hand-derived worked example."""
import json
import os

import numpy as np
import pytest

from oracle import quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden",
                      "quant_worked_example.json")


def _groups(rng, n_groups, size, kind):
    if kind == "normal":
        x = rng.standard_normal((n_groups, size))
    elif kind == "outlier":
        x = rng.standard_normal((n_groups, size)) * 10.0 ** rng.integers(
            -2, 3, (n_groups, 1))
    elif kind == "skew":
        x = rng.lognormal(0, 1.5, (n_groups, size)) - 1.0
    else:
        raise ValueError(kind)
    return x.astype(np.float16)


@pytest.mark.parametrize("bits", [1, 2, 8])
@pytest.mark.parametrize("kind", ["normal", "outlier", "skew"])
def test_value_groups_invariants(bits, kind):
    rng = np.random.default_rng(10 * bits + len(kind))
    Lv = (1 << bits) - 1
    N, Gv, d = 96, 32, 128
    V = _groups(rng, N * d // Gv, Gv, kind).reshape(N, d)
    q, s, z = quant.quantize_values(V, Gv, bits)
    assert q.dtype == np.uint8 and q.max() <= Lv
    assert s.shape == (N, d // Gv) and z.shape == s.shape
    g = V.reshape(N, d // Gv, Gv)
    qg = q.reshape(N, d // Gv, Gv)
    # zero is the group minimum, stored exactly
    assert np.array_equal(z, g.min(axis=2))
    nondeg = s > 0
    assert nondeg.all()
    # end codes: the minimum gets 0, the maximum gets Lv
    amin = g.argmin(axis=2)[..., None]
    amax = g.argmax(axis=2)[..., None]
    assert (np.take_along_axis(qg, amin, 2) == 0).all()
    assert (np.take_along_axis(qg, amax, 2) == Lv).all()
    # reconstruction error within half a step (normal-range scales)
    xh = quant.dequant(q, s, z, "value", Gv)
    err = np.abs(V.astype(np.float64) - xh)
    bound = np.repeat(s.astype(np.float64), Gv, axis=1) * 0.5 * (1 + 2.0 ** -9)
    assert (err <= bound).all()


@pytest.mark.parametrize("bits", [1, 2, 8])
def test_key_groups_invariants(bits):
    rng = np.random.default_rng(bits)
    Lv = (1 << bits) - 1
    N, G, d = 256, 32, 64
    K = (rng.standard_normal((N, d)) * np.where(np.arange(d) % 17 == 0, 10, 1)
         ).astype(np.float16)
    q, s, z = quant.quantize_keys(K, G, bits)
    assert s.shape == (N // G, d)
    g = K.reshape(N // G, G, d)
    qg = q.reshape(N // G, G, d)
    assert np.array_equal(z, g.min(axis=1))
    amin = g.argmin(axis=1)[:, None, :]
    amax = g.argmax(axis=1)[:, None, :]
    assert (np.take_along_axis(qg, amin, 1) == 0).all()
    assert (np.take_along_axis(qg, amax, 1) == Lv).all()
    xh = quant.dequant(q, s, z, "key", G)
    err = np.abs(K.astype(np.float64) - xh)
    bound = np.repeat(s.astype(np.float64), G, axis=0) * 0.5 * (1 + 2.0 ** -9)
    assert (err <= bound).all()


def test_draft4_error_bound():
    """x^4 = z + (16*hi+7.5)*s lies within 8 s of x (half of the 16-code
    step the upper nibble keeps)."""
    rng = np.random.default_rng(7)
    N, G, d = 512, 128, 128
    K = (rng.standard_normal((N, d)) * 3).astype(np.float16)
    q, s, z = quant.quantize_keys(K, G, 8)
    x4 = quant.dequant_draft4(q, s, z, "key", G)
    err = np.abs(K.astype(np.float64) - x4)
    bound = np.repeat(s.astype(np.float64), G, axis=0) * 8 * (1 + 2.0 ** -9)
    assert (err <= bound).all()
    # the draft needs only the upper nibble: changing the low nibble of a
    # code leaves x^4 unchanged
    q2 = (q & 0xF0) | ((q + 5) & 0x0F)
    assert np.array_equal(quant.dequant_draft4(q2, s, z, "key", G), x4)


def test_degenerate_and_tiny_groups():
    # constant group: s == 0, all codes 0, exact reconstruction
    V = np.full((2, 32), 0.3, np.float16)
    for bits in (1, 2, 8):
        q, s, z = quant.quantize_values(V, 32, bits)
        assert (s == 0).all() and (q == 0).all()
        assert np.array_equal(quant.dequant(q, s, z, "value", 32),
                              V.astype(np.float64))
    # range so small that s underflows fp16: treated as degenerate
    x = np.zeros((1, 32), np.float16)
    x[0, 5] = np.float16(2.0 ** -24)          # smallest fp16 subnormal
    q, s, z = quant.quantize_values(x, 32, 8)
    assert s[0, 0] == 0 and (q == 0).all()
    # subnormal scale: general bound 0.5 s + Lv |s - range/Lv| + 2^-23 range
    x[0, 5] = np.float16(3e-4)
    x[0, 9] = np.float16(-1e-4)
    q, s, z = quant.quantize_values(x, 32, 8)
    sv = float(s[0, 0])
    rng_ = float(x.max()) - float(x.min())
    bound = 0.5 * sv + 255 * abs(sv - rng_ / 255) + 2.0 ** -23 * rng_
    err = np.abs(quant.dequant(q, s, z, "value", 32) - x.astype(np.float64))
    assert err.max() <= bound


def test_grouping_axes():
    """Keys are grouped per (channel, G tokens); values per (token, Gv
    channels): perturbing one element moves only its own group's params."""
    rng = np.random.default_rng(3)
    N, G, Gv, d = 128, 32, 32, 128
    X = rng.standard_normal((N, d)).astype(np.float16)
    _, ks, kz = quant.quantize_keys(X, G, 8)
    _, vs, vz = quant.quantize_values(X, Gv, 8)
    Y = X.copy()
    Y[37, 70] = np.float16(50.0)
    _, ks2, kz2 = quant.quantize_keys(Y, G, 8)
    _, vs2, vz2 = quant.quantize_values(Y, Gv, 8)
    dk = np.argwhere(ks2 != ks)
    dv = np.argwhere(vs2 != vs)
    assert dk.tolist() == [[37 // G, 70]]
    assert dv.tolist() == [[37, 70 // Gv]]
    assert np.array_equal(kz, kz2) and np.array_equal(vz, vz2)


def test_worked_example():
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        x = np.array([c["x"]], np.float16)
        q, s, z = quant.quantize_values(x, x.shape[1], c["bits"])
        assert float(s[0, 0]) == c["scale"], c["name"]
        assert float(z[0, 0]) == c["zero"], c["name"]
        assert q[0].tolist() == c["codes"], c["name"]
        xh = quant.dequant(q, s, z, "value", x.shape[1])
        assert xh[0].tolist() == c["dequant"], c["name"]
        if "draft_code" in c:
            assert quant.draft4_code(q)[0].tolist() == c["draft_code"]
            assert (q[0] >> 4).tolist() == c["hi"]
            assert (q[0] & 15).tolist() == c["lo"]
        # the same group laid out along tokens quantizes identically as keys
        qk, sk, zk = quant.quantize_keys(x.T.copy(), x.shape[1], c["bits"])
        assert qk[:, 0].tolist() == c["codes"]
        assert float(sk[0, 0]) == c["scale"]
