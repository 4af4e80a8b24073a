"""Bit-level pins of the oracle: the two binary32 definitions the GPU must
meet to the bit.

* The quantizer's code is rint_even of the correctly rounded quotient
  (x - z) / s (SpeCache page, Approach; QuantSpec page, Approach and
  "Builds on: KIVI").  tests/golden/quant_divide_ties.json holds two groups
  whose quotient is an exact half-integer: a reciprocal-multiply moves it
  off the tie and changes the code.
* The top-k key sums the channel products in channel order with one
  binary32 rounding per product and per sum (SpeCache page, Approach: the
  speculative token's scores choose the pairs to fetch).
  tests/golden/topk_key_rounding.json holds two blocks whose order flips
  under a pairwise sum or under fused multiply-adds.

The golden values were derived by hand; the helpers below re-derive them
with exact rationals and one explicit rounding per operation, so the files
cannot drift, and show that each case tells the definition apart from the
named alternative.  A scalar pure-Python quantizer brute-forces the tiny
workload against the vectorized oracle.
"""
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import kvq_synth as synth
from oracle import quant, topk

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)["cases"]


# ---- exact rational rounding ----------------------------------------------

def rne(x: Fraction, mant_bits: int, emin: int) -> Fraction:
    """Round x to the nearest binary floating-point number with mant_bits
    significand bits (implicit bit included) and minimum normal exponent
    emin, ties to even; subnormals keep the spacing 2^(emin - mant_bits + 1).
    No overflow handling (the values here are small)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    # fix the floating estimate of floor(log2(a))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - mant_bits + 1)
    m = a / ulp
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def f32(x: Fraction) -> Fraction:
    return rne(Fraction(x), 24, -126)


def f16(x: Fraction) -> Fraction:
    return rne(Fraction(x), 11, -14)


def rint_even(x: Fraction) -> int:
    fl = x.numerator // x.denominator
    rem = x - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


# ---- quantizer divide ------------------------------------------------------

@pytest.mark.parametrize("case", _load("quant_divide_ties.json"),
                         ids=lambda c: c["name"])
def test_quantizer_rounds_the_true_quotient(case):
    x = np.array([case["x"]], np.float16)
    bits = case["bits"]
    Lv = (1 << bits) - 1
    # the oracle, against the hand-derived golden
    q, s, z = quant.quantize_values(x, x.shape[1], bits)
    assert float(s[0, 0]) == case["scale"] and float(z[0, 0]) == case["zero"]
    assert q[0].tolist() == case["codes"]
    qk, sk, _ = quant.quantize_keys(x.T.copy(), x.shape[1], bits)
    assert qk[:, 0].tolist() == case["codes"] and float(sk[0, 0]) == case["scale"]
    if "hi" in case:
        assert (q[0] >> 4).tolist() == case["hi"]
        assert (q[0] & 15).tolist() == case["lo"]
    # re-derivation in exact rationals, one rounding per step
    xs = [Fraction(float(v)) for v in x[0]]
    zr = min(xs)
    sr = f16(f32(f32(f32(max(xs)) - f32(zr)) / Lv))
    assert sr == Fraction(case["scale"])
    codes = [min(max(rint_even(f32((xv - zr) / sr)), 0), Lv) for xv in xs]
    assert codes == case["codes"]
    # the case separates the definition from a reciprocal-multiply
    recip = f32(1 / sr)
    alt = [min(max(rint_even(f32((xv - zr) * recip)), 0), Lv) for xv in xs]
    assert alt == case["reciprocal_codes"] != case["codes"]
    assert any(((xv - zr) / sr).denominator == 2 for xv in xs)   # an exact tie


# ---- top-k key -------------------------------------------------------------

def _case_arrays(case):
    q = np.array(case["q"], np.float16)
    codes = np.array(case["codes"], np.uint8)
    ks = np.array([case["s"]], np.float16)
    kz = np.array([case["z"]], np.float16)
    return q, codes, ks, kz


def _khat(case, j):
    return [f32(Fraction(float(np.float16(z))) +
                f32(c * Fraction(float(np.float16(s)))))
            for z, s, c in zip(case["z"], case["s"], case["codes"][j])]


def _prods(case, h, j):
    return [f32(Fraction(float(np.float16(qv))) * k)
            for qv, k in zip(case["q"][h], _khat(case, j))]


def key_sequential(case, j):
    best = None
    for h in range(len(case["q"])):
        acc = Fraction(0)
        for p in _prods(case, h, j):
            acc = f32(acc + p)
        best = acc if best is None else max(best, acc)
    return best


def key_pairwise(case, j):
    best = None
    for h in range(len(case["q"])):
        v = _prods(case, h, j)
        while len(v) > 1:
            v = [f32(v[i] + v[i + 1]) for i in range(0, len(v), 2)]
        best = v[0] if best is None else max(best, v[0])
    return best


def key_fused(case, j):
    best = None
    for h in range(len(case["q"])):
        acc = Fraction(0)
        for qv, k in zip(case["q"][h], _khat(case, j)):
            acc = f32(acc + Fraction(float(np.float16(qv))) * k)
        best = acc if best is None else max(best, acc)
    return best


@pytest.mark.parametrize("case", _load("topk_key_rounding.json"),
                         ids=lambda c: c["name"])
def test_topk_key_is_the_sequential_unfused_sum(case):
    q, codes, ks, kz = _case_arrays(case)
    key = topk.canonical_keys(q, codes, ks, kz, case["G"], "target")
    assert key.dtype == np.float32
    assert key.tolist() == case["keys"]
    assert not np.signbit(key).any()
    idx, val = topk.select(key, len(case["idx"]))
    assert idx.tolist() == case["idx"]
    assert val.tolist() == [case["keys"][i] for i in case["idx"]]
    # re-derivation, one rounding per product and per sum
    N = codes.shape[0]
    assert [float(key_sequential(case, j)) for j in range(N)] == case["keys"]
    # the case separates the definition from the named alternative
    if "pairwise_keys" in case:
        alt = [float(key_pairwise(case, j)) for j in range(N)]
        assert alt == case["pairwise_keys"] != case["keys"]
    if "fused_keys" in case:
        alt = [float(key_fused(case, j)) for j in range(N)]
        assert alt == case["fused_keys"] != case["keys"]


# ---- scalar brute force of the quantizer ------------------------------------

def _r32(v: float) -> float:
    """Round a Python float to binary32 (C cast: nearest, ties to even).
    For +, -, *, / of two binary32 operands the binary64 result rounded to
    binary32 is the correctly rounded binary32 result."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


def _r16(v: float) -> float:
    return struct.unpack("<e", struct.pack("<e", v))[0]


def _scalar_group(xs, Lv):
    mn, mx = min(xs), max(xs)
    s = _r16(_r32(_r32(_r32(mx) - _r32(mn)) / Lv))
    codes = []
    for x in xs:
        if s == 0.0:
            codes.append(0)
            continue
        t = _r32(_r32(x - mn) / s)
        r = round(t)                     # Python rounds half to even
        codes.append(min(max(r, 0), Lv))
    return codes, s, mn


@pytest.mark.parametrize("bits", [8, 2, 1])
def test_quantizer_scalar_loop_tiny_workload(bits):
    """Element-by-element Python loop over the tiny workload's K (per
    channel over G tokens) and V (per token over Gv channels)."""
    w = synth.WORKLOADS["tiny"]
    K, V = synth.kv_all(w, 0)
    K = K[0, 0].astype(np.float16)
    V = V[0, 0].astype(np.float16)
    Lv = (1 << bits) - 1
    N, d = K.shape
    N -= N % w.G
    qk, sk, zk = quant.quantize_keys(K[:N], w.G, bits)
    qv, sv, zv = quant.quantize_values(V[:N], w.Gv, bits)
    for g in range(N // w.G):
        for c in range(d):
            xs = [float(v) for v in K[g * w.G:(g + 1) * w.G, c]]
            codes, s, z = _scalar_group(xs, Lv)
            assert s == float(sk[g, c]) and z == float(zk[g, c])
            assert codes == qk[g * w.G:(g + 1) * w.G, c].tolist()
    for t in range(N):
        for g in range(d // w.Gv):
            xs = [float(v) for v in V[t, g * w.Gv:(g + 1) * w.Gv]]
            codes, s, z = _scalar_group(xs, Lv)
            assert s == float(sv[t, g]) and z == float(zv[t, g])
            assert codes == qv[t, g * w.Gv:(g + 1) * w.Gv].tolist()
