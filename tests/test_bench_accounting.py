"""The benchmark's algorithmic byte counts (the numerator of the reported
HBM roofline fraction) against per-step figures worked out by hand from the
cache layout: codes at the bits a path reads, fp16 scale/zero amortized per
group, fp16 residual tokens, fp16 q and out.  Fill levels are those the
flush rule gives after appending the whole context (n_q a multiple of G,
the residual holding the rest)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (imports torch only inside its GPU functions)

# (Hkv, Hq, d, G, Gv, n_q, n_r, T, bits read, batch, bytes per step)
CASES = [
    ("llama2_8k int8 T=9", 32, 32, 128, 128, 64, 7936, 256, 9, 8, 1, 72_400_896),
    ("llama2_8k int4 T=1", 32, 32, 128, 128, 64, 7936, 256, 1, 4, 1, 39_763_968),
    ("llama3_32k int4 T=1", 8, 32, 128, 128, 64, 32512, 256, 1, 4, 1, 37_478_400),
    ("llama3_32k int8 T=7", 8, 32, 128, 128, 64, 32512, 256, 7, 8, 1, 70_868_992),
    ("lwm_128k int8 T=6", 32, 32, 128, 128, 64, 130816, 256, 6, 8, 1, 1_126_170_624),
    ("lwm_128k int4 T=1", 32, 32, 128, 128, 64, 130816, 256, 1, 4, 1, 590_266_368),
    ("specache 1-bit T=2", 8, 32, 128, 32, 32, 32736, 32, 2, 1, 36, 609_288_192),
    ("specache 2-bit T=2", 8, 32, 128, 32, 32, 32736, 32, 2, 2, 36, 910_983_168),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_algorithmic_bytes(case):
    _, Hkv, Hq, d, G, Gv, n_q, n_r, T, bits, B, want = case
    assert B * bench.algorithmic_bytes(Hkv, Hq, d, G, Gv, n_q, n_r, T, bits) == want


def test_per_token_bytes():
    """Per quantized token per kv head at d = 128: INT8 268 B (G = 128,
    Gv = 64), INT4 draft 140 B, 1-bit 64 B and 2-bit 96 B (G = Gv = 32); an
    fp16 residual token 512 B."""
    one = lambda G, Gv, bits: bench.algorithmic_bytes(1, 1, 128, G, Gv, 1, 0, 0, bits)
    assert one(128, 64, 8) == 268
    assert one(128, 64, 4) == 140
    assert one(32, 32, 1) == 64
    assert one(32, 32, 2) == 96
    assert bench.algorithmic_bytes(1, 1, 128, 128, 64, 0, 1, 0, 8) == 512
