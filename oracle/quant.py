"""KIVI-style asymmetric group quantizer, emulated exactly in IEEE float32.

Sources: SpeCache page, Approach ("1-bit KIVI", zero-point and scale);
QuantSpec page, Experimental setup ("Builds on: KIVI") and Approach (the
upper 4 bits of an 8-bit code are the INT4 draft code).  The pages give no
formula; the reading used here is the plain asymmetric min/max one:

    z = min(x)                       (an fp16 value, stored exactly)
    s = fp16_rne(f32(f32(max) - f32(min)) / f32(Lv)),   Lv = 2**bits - 1
    q = 0 if s == 0 else clip(rint_even(f32(f32(x) - f32(z)) / f32(s)), 0, Lv)

numpy float32 ufuncs perform exactly one IEEE operation each (numpy has no
fused multiply-add), division is correctly rounded, ``np.rint`` rounds half to
even and ``astype(float16)`` rounds to nearest even, so this matches the
definition bit for bit.

Groups: keys per (channel, G consecutive tokens); values per (token, Gv
consecutive channels).

Pinned by (tests/test_oracle_quant.py): code range, end codes hitting 0 and
Lv in every non-degenerate group, |x - x^| <= s/2 (1 + 2^-9),
|x - x^4| <= 8 s (1 + 2^-9), degenerate groups, the grouping axes, and a
hand-derived worked example (tests/golden/quant_worked_example.json).
Pinned to the bit by (tests/test_oracle_bitlevel.py): two hand-derived
groups whose quotient (x - z)/s is an exact half-integer, where a
reciprocal-multiply would give another code
(tests/golden/quant_divide_ties.json), and a scalar pure-Python loop over
the tiny workload at 1, 2 and 8 bits.
"""
from __future__ import annotations

import numpy as np

__all__ = ["levels", "group_params", "codes_for", "quantize_keys",
           "quantize_values", "dequant", "dequant_draft4", "draft4_code"]


def levels(bits: int) -> int:
    if bits not in (1, 2, 8):
        raise ValueError("bits must be 1, 2 or 8")
    return (1 << bits) - 1


def group_params(mn16: np.ndarray, mx16: np.ndarray, Lv: int):
    """(scale, zero) as fp16 from the fp16 group minimum and maximum."""
    mn16 = np.asarray(mn16, np.float16)
    mx16 = np.asarray(mx16, np.float16)
    span = mx16.astype(np.float32) - mn16.astype(np.float32)
    s = (span / np.float32(Lv)).astype(np.float16)
    return s, mn16.copy()


def codes_for(x16: np.ndarray, s16: np.ndarray, z16: np.ndarray, Lv: int):
    """Codes of fp16 values x against broadcastable fp16 scale/zero."""
    num = x16.astype(np.float32) - z16.astype(np.float32)
    s32 = np.broadcast_to(s16.astype(np.float32), num.shape)
    safe = np.where(s32 == 0, np.float32(1.0), s32)
    r = np.rint(num / safe)
    q = np.clip(r, np.float32(0), np.float32(Lv))
    q = np.where(s32 == 0, np.float32(0), q)
    return q.astype(np.uint8)


def quantize_keys(K16: np.ndarray, G: int, bits: int):
    """Per-channel key groups.  K16: fp16 (N, d), N a multiple of G.
    Returns codes u8 (N, d), scale fp16 (N/G, d), zero fp16 (N/G, d)."""
    N, d = K16.shape
    if N % G:
        raise ValueError("N must be a multiple of G")
    Lv = levels(bits)
    Kg = K16.reshape(N // G, G, d)
    s, z = group_params(Kg.min(axis=1), Kg.max(axis=1), Lv)
    q = codes_for(Kg, s[:, None, :], z[:, None, :], Lv)
    return q.reshape(N, d), s, z


def quantize_values(V16: np.ndarray, Gv: int, bits: int):
    """Per-token value groups.  V16: fp16 (N, d), d a multiple of Gv.
    Returns codes u8 (N, d), scale fp16 (N, d/Gv), zero fp16 (N, d/Gv)."""
    N, d = V16.shape
    if d % Gv:
        raise ValueError("d must be a multiple of Gv")
    Lv = levels(bits)
    Vg = V16.reshape(N, d // Gv, Gv)
    s, z = group_params(Vg.min(axis=2), Vg.max(axis=2), Lv)
    q = codes_for(Vg, s[:, :, None], z[:, :, None], Lv)
    return q.reshape(N, d), s, z


def _expand(param: np.ndarray, N: int, d: int, axis_group: str, group: int):
    """Broadcast per-group params to (N, d)."""
    p = param.astype(np.float64)
    if axis_group == "token":       # keys: (N/G, d) -> (N, d)
        return np.repeat(p, group, axis=0)
    return np.repeat(p, group, axis=1)  # values: (N, d/Gv) -> (N, d)


def dequant(q: np.ndarray, s: np.ndarray, z: np.ndarray, kind: str,
            group: int) -> np.ndarray:
    """x^ = z + q*s in float64 (exact).  kind: "key" (group = G tokens) or
    "value" (group = Gv channels)."""
    N, d = q.shape
    ax = "token" if kind == "key" else "channel"
    S = _expand(s, N, d, ax, group)
    Z = _expand(z, N, d, ax, group)
    return Z + q.astype(np.float64) * S


def draft4_code(q: np.ndarray) -> np.ndarray:
    """INT4 draft reconstruction point of 8-bit codes: 16*(q>>4) + 7.5."""
    return 16.0 * (q.astype(np.int32) >> 4).astype(np.float64) + 7.5


def dequant_draft4(q: np.ndarray, s: np.ndarray, z: np.ndarray, kind: str,
                   group: int) -> np.ndarray:
    """x^4 = z + (16*hi + 7.5)*s in float64, hi = q >> 4 (the upper nibble
    the draft reads, QuantSpec page, Approach)."""
    N, d = q.shape
    ax = "token" if kind == "key" else "channel"
    S = _expand(s, N, d, ax, group)
    Z = _expand(z, N, d, ax, group)
    return Z + draft4_code(q) * S
