"""Host checks of binary32 identities the HIP quantizer relies on.

The quantize-on-append kernel computes each code clip(rint(RN((x - z)/s)))
without a per-element divide: a reciprocal RN(1/s) per group, one fma
correction step (Markstein's division theorem), and rounding by an add of
2^23.  tests/quotient_identity.c checks both identities over every positive
fp16 scale and the numerators where a code could flip; the GPU parity tests
then check the kernel's codes against the oracle's correctly rounded divide.
"""
import os
import shutil
import subprocess

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
