"""Helpers for the GPU tests: build caches from the seeded workloads and read
device buffers back into the oracle's logical arrays (through oracle.layout,
which implements the documented byte layout independently of the HIP code).
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import kvq_synth as synth
import quantized_kv_attention_quant_amd as kq
from oracle import layout


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def shape_for(w: synth.Workload, L_max: int | None = None, max_append=32):
    L_max = L_max or int(math.ceil(w.L / w.G) * w.G)
    return kq.Shape(B=w.B, Hkv=w.Hkv, d=w.d, G=w.G, Gv=w.Gv, bits=w.bits,
                    R=w.R, L_max=L_max, max_append=max_append)


def host_tokens(w: synth.Workload, seed: int, L: int | None = None):
    """fp16 K, V as (B, L, Hkv, d) host arrays (the append layout)."""
    L = w.L if L is None else L
    K = np.empty((w.B, L, w.Hkv, w.d), np.float16)
    V = np.empty_like(K)
    for b in range(w.B):
        for h in range(w.Hkv):
            kb, vb = synth.kv_block(w, seed, b, h, L)
            K[b, :, h] = kb
            V[b, :, h] = vb
    return K, V


def to_dev(x: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def read_block(cache: kq.QuantKVCache, b: int, h: int):
    """Logical contents of block (b, h): codes, scales, zeros, residual."""
    s, c = cache.shape, cache.c
    d, w = s.d, layout.plane_width(s.bits)
    n_q, n_r, ring = c.n_q, c.n_r, c.ring
    blk = b * s.Hkv + h

    def sl(t, per_block, lo, hi):
        return t[blk * per_block + lo: blk * per_block + hi].cpu().numpy()

    row = d * w // 8
    kh = sl(cache.k_hi, s.L_max * row, 0, n_q * row).reshape(n_q, row)
    kq_ = layout.unpack_k_plane(kh, w, d)
    tile = 4 * d * w
    nt = n_q // 32
    vh = sl(cache.v_hi, (s.L_max // 32) * tile, 0, nt * tile).reshape(nt, tile)
    vq = layout.unpack_v_plane(vh, w, d)
    if s.bits == 8:
        kl = sl(cache.k_lo, s.L_max * row, 0, n_q * row).reshape(n_q, row)
        kq_ = layout.join_planes(kq_, layout.unpack_k_plane(kl, w, d), 8)
        vl = sl(cache.v_lo, (s.L_max // 32) * tile, 0, nt * tile).reshape(nt, tile)
        vq = layout.join_planes(vq, layout.unpack_v_plane(vl, w, d), 8)
    ksz_b = (s.L_max // s.G) * d * 4
    ksz = sl(cache.k_sz, ksz_b, 0, (n_q // s.G) * d * 4).view(np.float16)
    ks, kz = layout.unpack_k_sz(ksz.reshape(n_q // s.G, d, 2))
    ng = d // s.Gv
    vsz_tile = 32 * ng * 4
    vsz = sl(cache.v_sz, (s.L_max // 32) * vsz_tile, 0, nt * vsz_tile)
    vs, vz = layout.unpack_v_sz(vsz.view(np.float16).reshape(nt, 2, 4, 4, ng, 2))
    res_b = ring * d * 2
    kr_all = sl(cache.k_res, res_b, 0, res_b).view(np.float16).reshape(ring, d)
    vr_all = sl(cache.v_res, res_b, 0, res_b).view(np.float16).reshape(
        ring // 32, 32 * d)
    slots = (n_q + np.arange(n_r)) % ring
    rk = kr_all[slots]
    vtiles = np.stack([layout.unpack_v_res_tile(t, d) for t in vr_all])
    rv = vtiles[slots // 32, slots % 32]
    return dict(kq=kq_, ks=ks, kz=kz, vq=vq, vs=vs, vz=vz, rk=rk, rv=rv)


def assert_attn_close(got, ref, what="attention"):
    """max|got - ref| <= 2e-3 * max|ref| (fp32 accumulate, fp16 output)."""
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref).max()
    bound = 2e-3 * np.abs(ref).max()
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert err <= bound, f"{what}: max|err| {err:.3e} > {bound:.3e}"
    return err / np.abs(ref).max()


def lse_tolerance(rep, q16, path, sm_scale):
    """Bound on |lse_gpu - lse_oracle| (B, Hq, T), derived from the kernel's
    arithmetic.  Scores use Q' = q*s*c0 (quantized keys) or q*c0 (fp16 keys)
    split into two fp16 parts, so each channel term carries a relative error
    of at most 2^-21; the MFMA accumulates terms Q' * a in fp32 (a = 1024 +
    code <= 1279 for 8-bit codes, a = code for 1-bit, and for 2-bit codes
    a = 4 (1 + code/4) <= 7 against 4 Q', with 4 sum_c q c0 s taken out of
    the start), whose partial sums stay below max(a) * sum_c |Q'_c| and take
    ~16 roundings of 2^-24.  Every logit, and so the log-sum-exp, moves by
    at most 2^-21 sm sum_c|q_c k^_jc| + e sm sum_c |q_c| s_gc, with
    e = 16 2^-24 max(a), plus 4 2^-21 for 2-bit codes (their start takes
    the exact q c0 s, not its two rounded fp16 parts); the bound doubles
    that and adds 2e-6 for exp2/log2 and the merge."""
    from oracle import attention as oatt
    B, T, Hq, d = q16.shape
    gs = Hq // rep.Hkv
    tol = np.empty((B, Hq, T))
    for b in range(B):
        for h in range(rep.Hkv):
            K, _ = oatt.block_kv(rep.kq[b, h], rep.ks[b, h], rep.kz[b, h],
                                 rep.vq[b, h], rep.vs[b, h], rep.vz[b, h],
                                 rep.rk[b, h], rep.rv[b, h], rep.G, rep.Gv,
                                 path)
            qa = np.abs(q16[b, :, h * gs:(h + 1) * gs].astype(np.float64))
            mag = np.einsum("thc,jc->thj", qa, np.abs(K)).max(axis=2)
            s = rep.ks[b, h].astype(np.float64)
            # largest MFMA operand against Q': 1024 + code for 8-bit codes,
            # the code for 1-bit, 4 (1 + 3/4) for 2-bit
            top = {8: 1279.0, 2: 7.0, 1: 1.0}[rep.bits]
            e = 16 * 2.0 ** -24 * top + (4 * 2.0 ** -21 if rep.bits == 2 else 0.0)
            acc = (np.einsum("thc,gc->thg", qa, s).max(axis=2) if s.size
                   else np.zeros_like(mag))
            bound = sm_scale * (2.0 ** -21 * mag + e * acc)
            tol[b, h * gs:(h + 1) * gs] = (2 * bound).T
    return tol + 2e-6


def assert_block_bytes(cache: kq.QuantKVCache, b: int, h: int, rep,
                       rb: int = 0, rh: int = 0, what: str = ""):
    """Block (b, h) of the device cache equals block (rb, rh) of an oracle
    replay: codes bit for bit, scales and zeros as fp16 values, residual
    tokens bit for bit."""
    got = read_block(cache, b, h)
    for name in ("kq", "vq"):
        assert np.array_equal(got[name], getattr(rep, name)[rb, rh]), (what, name)
    for name in ("rk", "rv"):
        assert np.array_equal(got[name].view(np.uint16),
                              getattr(rep, name)[rb, rh].view(np.uint16)), (what, name)
    for name in ("ks", "kz", "vs", "vz"):
        assert np.array_equal(got[name], getattr(rep, name)[rb, rh]), (what, name)
