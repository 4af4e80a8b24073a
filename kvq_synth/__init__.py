"""Seeded synthetic workloads for quantized-KV decode/verify attention.

This module only draws random numbers and names shapes.  It holds none of
the method's arithmetic (no quantization, attention or selection), so both
the CPU oracle and the GPU tests/benchmark can take their inputs from it.

Workloads (shapes from the model families the pages evaluate: Llama-2-7B,
Llama-3-8B, LWM-7B-128K, Mistral-7B at 32K; QuantSpec page, Experimental
setup and Measured-effects table; SpeCache page, Key results):

  tiny            B=1  Hq=4  Hkv=1 d=64  L=256    G=32  Gv=32 R=32  INT8
  llama2_7b_8k    B=1  Hq=32 Hkv=32 d=128 L=8192  G=128 Gv=64 R=256 INT8
  llama3_8b_32k   B=1  Hq=32 Hkv=8 d=128 L=32768  G=128 Gv=64 R=256 INT8
  lwm_7b_128k     B=1  Hq=32 Hkv=32 d=128 L=131072 G=128 Gv=64 R=256 INT8
  specache_1bit / specache_2bit
                  B=36 Hq=32 Hkv=8 d=128 L=32768  G=32  Gv=32 R=32  1/2-bit

Random streams (numpy PCG64 via SeedSequence), one per (b, kvh) block so
that a large workload can be generated block by block:
  [seed, b, kvh, 0]: K then V, each standard_normal((L, d), float32)
  [seed, b, kvh, 1]: 4 outlier channels (choice(d, 4, replace=False)), then
                     per-token K drift lognormal(0, 0.5, L)
  [seed, 999]:       queries standard_normal((B, T, Hq, d), float32)
Distribution "outlier" scales K's outlier channels by 10; "outlier_drift"
also multiplies each K row by its drift factor.  Values are cast to fp16
last.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

__all__ = ["Workload", "WORKLOADS", "kv_block", "kv_all", "queries"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    L: int          # context length in tokens (includes the T query tokens)
    G: int          # key group (tokens per channel scale)
    Gv: int         # value group (channels per token scale)
    R: int          # residual capacity
    bits: int       # 8, 2 or 1
    dist: str       # "normal" | "outlier" | "outlier_drift"
    # (path, T) pairs run on this workload: path is "target" or "draft4"
    runs: tuple = field(default_factory=tuple)
    topk: int = 0   # k of the per-kv-head top-k (0: none)

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 1, 4, 1, 64, 256, 32, 32, 32, 8, "normal",
                 runs=(("target", 1), ("draft4", 1))),
        Workload("llama2_7b_8k", 1, 32, 32, 128, 8192, 128, 64, 256, 8,
                 "outlier", runs=(("target", 9), ("draft4", 1))),
        Workload("llama3_8b_32k", 1, 32, 8, 128, 32768, 128, 64, 256, 8,
                 "outlier_drift", runs=(("draft4", 1), ("target", 7))),
        Workload("lwm_7b_128k", 1, 32, 32, 128, 131072, 128, 64, 256, 8,
                 "outlier", runs=tuple([("target", t) for t in range(1, 7)]
                                       + [("draft4", 1)])),
        Workload("specache_1bit", 36, 32, 8, 128, 32768, 32, 32, 32, 1,
                 "normal", runs=(("target", 2),), topk=64),
        Workload("specache_2bit", 36, 32, 8, 128, 32768, 32, 32, 32, 2,
                 "normal", runs=(("target", 2),), topk=64),
    ]
}


def kv_block(w: Workload, seed: int, b: int, kvh: int, L: int | None = None):
    """fp16 (K, V) of shape (L, d) for block (b, kvh).  A different L gives
    different values (V is drawn after all of K); slice a full draw when a
    prefix is needed."""
    L = w.L if L is None else L
    rng = np.random.default_rng(np.random.SeedSequence([seed, b, kvh, 0]))
    K = rng.standard_normal((L, w.d), dtype=np.float32)
    V = rng.standard_normal((L, w.d), dtype=np.float32)
    if w.dist in ("outlier", "outlier_drift"):
        rng1 = np.random.default_rng(np.random.SeedSequence([seed, b, kvh, 1]))
        ch = rng1.choice(w.d, 4, replace=False)
        K[:, ch] *= np.float32(10.0)
        if w.dist == "outlier_drift":
            drift = rng1.lognormal(0.0, 0.5, L).astype(np.float32)
            K *= drift[:, None]
    elif w.dist != "normal":
        raise ValueError(f"unknown distribution {w.dist!r}")
    return K.astype(np.float16), V.astype(np.float16)


def kv_all(w: Workload, seed: int, L: int | None = None):
    """fp16 (K, V) of shape (B, Hkv, L, d) for small workloads."""
    L = w.L if L is None else L
    K = np.empty((w.B, w.Hkv, L, w.d), np.float16)
    V = np.empty_like(K)
    for b in range(w.B):
        for h in range(w.Hkv):
            K[b, h], V[b, h] = kv_block(w, seed, b, h, L)
    return K, V


def queries(w: Workload, seed: int, T: int):
    """fp16 queries (B, T, Hq, d)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 999]))
    return rng.standard_normal((w.B, T, w.Hq, w.d), dtype=np.float32).astype(
        np.float16)
