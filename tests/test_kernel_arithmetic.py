"""Host checks of floating-point identities the HIP kernels rely on.

The quantize-on-append kernel computes each code clip(rint(RN((x - z)/s)))
without a per-element divide: a reciprocal RN(1/s) per group, one fma
correction step (Markstein's division theorem), and rounding by an add of
2^23.  tests/quotient_identity.c checks both identities over every positive
fp16 scale and the numerators where a code could flip; the GPU parity tests
then check the kernel's codes against the oracle's correctly rounded divide.

The attention kernel's 1/2-bit paths rely on two fp16 facts, checked here
with exact float64 arithmetic:
* 2-bit key groups rebuild Q' = q c0 s as hi' = RN16(qh s) and
  lo' = RN16(RN16(qh s - hi') + ql s), which carries ~22 bits only if the
  residual qh s - hi' of two fp16 values is itself an fp16 value (outside
  the subnormal range);
* 1-bit codes carry their key scale as fma(1 + code/2, s, -s), exact when
  s/2 is an fp16 value, i.e. for every normal s (and subnormal s with an
  even significand).
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_quotient_and_rounding_identities(tmp_path):
    exe = tmp_path / "quotient_identity"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", str(exe),
                    os.path.join(HERE, "quotient_identity.c"), "-lm"],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " 0 mismatches" in r.stdout, r.stdout


def _all_fp16(lo_exp, hi_exp):
    """Every positive finite fp16 value with exponent in [lo_exp, hi_exp]."""
    bits = np.arange(0x0001, 0x7C00, dtype=np.uint16)
    v = bits.view(np.float16).astype(np.float64)
    return v[(v >= 2.0 ** lo_exp) & (v < 2.0 ** (hi_exp + 1))]


def test_fp16_product_residual_is_fp16():
    """For fp16 a, b with a product in fp16's normal range, the residual
    a b - RN16(a b) is exactly representable in fp16 (when it is not below
    the smallest normal): every significand of one binade of b against
    sampled a from every binade, plus random pairs."""
    rng = np.random.default_rng(0)
    b = _all_fp16(0, 0)                          # all 1024 significands in [1, 2)
    a_all = _all_fp16(-14, 15)
    a = np.concatenate([a_all[::97], -a_all[::101]])
    p = np.multiply.outer(a, b).ravel()
    x = rng.standard_normal(2_000_000) * np.exp(rng.uniform(-7, 7, 2_000_000))
    y = np.abs(rng.standard_normal(2_000_000)) * np.exp(rng.uniform(-8, 4, 2_000_000))
    p = np.concatenate([p, x.astype(np.float16).astype(np.float64) *
                        y.astype(np.float16).astype(np.float64)])
    p = p[np.isfinite(p) & (np.abs(p) < 65504) & (np.abs(p) >= 2.0 ** -14)]
    hi = p.astype(np.float16).astype(np.float64)
    r = p - hi                                    # exact in float64
    normal = np.abs(r) >= 2.0 ** -14
    assert normal.sum() > 100_000
    r16 = r.astype(np.float16).astype(np.float64)
    assert np.array_equal(r16[normal], r[normal])


def test_onebit_scaled_code_is_exact():
    """fma(1 + code/2, s, -s) = code s / 2 for codes 0, 1 and every normal
    fp16 scale: the product and the sum are exact, so the one rounding to
    fp16 returns s/2 itself."""
    s = _all_fp16(-13, 15)                        # s/2 stays a normal fp16
    for code in (0, 1):
        x = 1.0 + code / 2.0                      # an fp16 value
        exact = x * s - s                         # float64: exact
        got = exact.astype(np.float16).astype(np.float64)
        assert np.array_equal(got, code * s / 2.0)
