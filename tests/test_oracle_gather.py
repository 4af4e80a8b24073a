"""Pins for oracle.gather (on-demand reconstruction of a token subset):
closed-form error bounds against the original tokens, exact rational
arithmetic, a hand-worked group, residual rows and out-of-range positions."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import cache as ocache, gather


def _replay(bits, d=64, G=32, Gv=32, R=64, L=300, seed=0, scale_ch=None):
    rng = np.random.default_rng(seed)
    B, H = 1, 2
    K = rng.standard_normal((B, L, H, d))
    if scale_ch is not None:
        K[..., scale_ch] *= 10.0
    K = K.astype(np.float16)
    V = rng.standard_normal((B, L, H, d)).astype(np.float16)
    rep = ocache.Replay(B, H, d, G, Gv, bits, R)
    for p0 in range(0, L, 37):                      # ragged appends
        rep.append(K[:, p0:p0 + 37], V[:, p0:p0 + 37])
    return rep, K, V


def _ulp16(x):
    """Spacing of fp16 values at |x| (normal range)."""
    a = np.abs(x.astype(np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


@pytest.mark.parametrize("bits", [8, 2, 1])
def test_residual_rows_are_the_appended_tokens(bits):
    rep, K, V = _replay(bits, d=128 if bits == 1 else 64)
    pos = np.arange(rep.n_q, rep.n_q + rep.n_r)
    for h in range(2):
        Kg, Vg = gather.gather_block(rep, 0, h, pos, "target")
        assert np.array_equal(Kg.view(np.uint16), K[0, pos, h].view(np.uint16))
        assert np.array_equal(Vg.view(np.uint16), V[0, pos, h].view(np.uint16))


@pytest.mark.parametrize("bits,path", [(8, "target"), (8, "draft4"),
                                       (2, "target"), (1, "target")])
def test_quantized_rows_within_quantizer_bounds(bits, path):
    """|x^ - x| <= (half a step, or 8 steps for the INT4 view) + the fp16
    rounding of x^, with the step bounded from the original group's range:
    s <= (max - min)/Lv rounded up to fp16."""
    d = 128 if bits == 1 else 64
    G, Gv = 64, 32
    rep, K, V = _replay(bits, d=d, G=G, Gv=Gv, R=128, scale_ch=[3, 17])
    Lv = (1 << bits) - 1
    n_q = rep.n_q
    assert n_q >= 2 * G
    pos = np.arange(n_q)
    steps = 8.0 if path == "draft4" else 0.5
    for h in range(2):
        Kg, Vg = gather.gather_block(rep, 0, h, pos, path)
        x = K[0, :n_q, h].astype(np.float64)
        grp = x.reshape(n_q // G, G, d)
        s_k = np.repeat((grp.max(1) - grp.min(1)) / Lv, G, axis=0) * (1 + 2.0 ** -10)
        err = np.abs(Kg.astype(np.float64) - x)
        assert (err <= steps * s_k + 0.5 * _ulp16(Kg) + 1e-12).all()
        y = V[0, :n_q, h].astype(np.float64)
        vg = y.reshape(n_q, d // Gv, Gv)
        s_v = np.repeat((vg.max(2) - vg.min(2)) / Lv, Gv, axis=1) * (1 + 2.0 ** -10)
        err = np.abs(Vg.astype(np.float64) - y)
        assert (err <= steps * s_v + 0.5 * _ulp16(Vg) + 1e-12).all()


@pytest.mark.parametrize("path", ["target", "draft4"])
def test_rows_round_the_exact_rational_value(path):
    """Each rebuilt value is within one fp16 step of z + code*s computed
    exactly (one binary32 rounding, then one fp16 rounding)."""
    rep, _, _ = _replay(8, d=64)
    rng = np.random.default_rng(3)
    pos = rng.integers(0, rep.n_q, 40)
    G, Gv = rep.G, rep.Gv
    for h in range(2):
        Kg, Vg = gather.gather_block(rep, 0, h, pos, path)
        for i, p in enumerate(pos):
            for c in range(0, 64, 7):
                for got, q, s, z in (
                        (Kg[i, c], rep.kq[0, h, p, c], rep.ks[0, h, p // G, c],
                         rep.kz[0, h, p // G, c]),
                        (Vg[i, c], rep.vq[0, h, p, c], rep.vs[0, h, p, c // Gv],
                         rep.vz[0, h, p, c // Gv])):
                    code = (Fraction(16 * (int(q) >> 4)) + Fraction(15, 2)
                            if path == "draft4" else Fraction(int(q)))
                    exact = Fraction(float(z)) + code * Fraction(float(s))
                    tol = _ulp16(np.array([float(exact)]))[0]
                    assert abs(Fraction(float(got)) - exact) <= Fraction(tol)


def test_hand_worked_key_group():
    """One key group of 32 tokens; channel 0 holds 0.25 t at token t < 31,
    10 at token 5 and 63.75 at token 31, so min = 0 and max = 63.75:
    s = 63.75/255 = 0.25 exactly and z = 0, every code is 4x and the target
    row gives x back.  The INT4 view of x = 10 (code 40, hi = 2) is
    (32 + 7.5) * 0.25 = 9.875, of x = 63.75 (code 255, hi = 15) is
    (240 + 7.5) * 0.25 = 61.875, of x = 0 (hi = 0) is 7.5 * 0.25 = 1.875."""
    G, d = 32, 64
    x = np.zeros((1, G, 1, d), np.float16)
    vals = np.array([0.25 * t for t in range(31)] + [63.75])
    x[0, :, 0, 0] = vals
    x[0, 5, 0, 0] = 10.0
    rep = ocache.Replay(1, 1, d, G, 32, 8, 0)
    rep.append(x, x)
    assert rep.n_q == G
    assert float(rep.ks[0, 0, 0, 0]) == 0.25 and float(rep.kz[0, 0, 0, 0]) == 0.0
    Kt, _ = gather.gather_block(rep, 0, 0, np.arange(G), "target")
    assert np.array_equal(Kt[:, 0].astype(np.float64), x[0, :, 0, 0].astype(np.float64))
    Kd, _ = gather.gather_block(rep, 0, 0, np.array([5, 31, 0]), "draft4")
    assert [float(v) for v in Kd[:, 0]] == [9.875, 61.875, 1.875]


def test_positions_outside_the_cache_are_nan():
    rep, _, _ = _replay(8)
    L = rep.n_q + rep.n_r
    Kg, Vg = gather.gather_block(rep, 0, 1, np.array([-1, L, L + 50, 0]), "target")
    assert np.isnan(Kg[:3]).all() and np.isnan(Vg[:3]).all()
    assert not np.isnan(Kg[3]).any() and not np.isnan(Vg[3]).any()
