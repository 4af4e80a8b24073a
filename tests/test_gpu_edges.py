"""GPU parity at the edges the method defines, against the oracle:

* degenerate groups: constant key channels and value groups (s = 0, all
  codes 0) and spans so small that s underflows fp16, through the HIP
  quantizer (bytes), attention and top-k;
* split-count invariance: one block attended alone (many splits) and inside
  a batch of blocks (few splits);
* GQA equal to MHA with the kv heads repeated;
* value scales at the attention kernels' limit (s = 63, where the fp16
  product of a probability scaled to 2^10 and s is largest);
* key scales times queries near the range the key operands hold in fp16.
"""
import numpy as np
import pytest
import torch

import kvq_synth as synth
import quantized_kv_attention_quant_amd as kq
from oracle import attention, cache as ocache, topk as otopk
from kvq_testlib import (assert_attn_close, assert_block_bytes, host_tokens,
                         lse_tolerance, say, shape_for, to_dev)

pytestmark = pytest.mark.gpu

W = synth.Workload
TINY = np.float16(2.0 ** -24)                  # smallest fp16 subnormal


def _degenerate_tokens(w, seed):
    """Seeded tokens with degenerate key channels and value groups."""
    K, V = host_tokens(w, seed)
    G = w.G
    for h in range(w.Hkv):
        # key group 1: channels 0..7 constant over the group (s = 0)
        for c in range(8):
            K[:, G:2 * G, h, c] = np.float16(0.25 * c - 1.0)
        # key group 2: channel 9 in {0, 2^-24}: (max - min)/Lv underflows fp16
        # for 8 and 2 bits (1 bit: s = 2^-24, a subnormal scale)
        K[:, 2 * G:3 * G, h, 9] = np.where(np.arange(G) % 3 == 0, TINY,
                                           np.float16(0))
        # key group 3: channel 20 all -0.0 and +0.0
        K[:, 3 * G:4 * G, h, 20] = np.where(np.arange(G) % 2 == 0,
                                            np.float16(-0.0), np.float16(0.0))
        # values: token 300 has its first value group constant, token 301
        # its second group in {0, 2^-24}, token 302 every group constant
        V[:, 300, h, :w.Gv] = np.float16(0.75)
        V[:, 301, h, w.Gv:2 * w.Gv] = np.where(np.arange(w.Gv) % 5 == 0, TINY,
                                               np.float16(0))
        V[:, 302, h, :] = np.float16(-1.5)
    return K, V


DEGEN = [
    W("degen_int8", 1, 8, 2, 128, 1000, 128, 64, 256, 8, "outlier"),
    W("degen_2bit", 1, 8, 2, 128, 1000, 32, 32, 32, 2, "normal"),
    W("degen_1bit", 1, 8, 2, 128, 1000, 32, 32, 32, 1, "normal"),
]


@pytest.mark.parametrize("w", DEGEN, ids=[w.name for w in DEGEN])
def test_degenerate_groups(w):
    say(f"[gpu] degenerate groups {w.name}")
    K, V = _degenerate_tokens(w, 2)
    cache = kq.QuantKVCache(shape_for(w, max_append=64))
    rep = ocache.Replay(w.B, w.Hkv, w.d, w.G, w.Gv, w.bits, w.R)
    # a bulk append, then small appends that flush one group at a time
    for lo, hi in ((0, 600), (600, 700), (700, 1000)):
        cache.append(to_dev(K[:, lo:hi]), to_dev(V[:, lo:hi]))
        rep.append(K[:, lo:hi], V[:, lo:hi])
    torch.cuda.synchronize()
    # the cases are what they claim in the oracle's store
    G = w.G
    assert (rep.ks[0, 0, 1, :8] == 0).all() and (rep.kq[0, 0, G:2 * G, :8] == 0).all()
    if w.bits != 1:
        assert rep.ks[0, 0, 2, 9] == 0
    assert rep.ks[0, 0, 3, 20] == 0
    assert (rep.vs[0, 0, 302] == 0).all() and rep.vs[0, 0, 300, 0] == 0
    for h in range(w.Hkv):
        assert_block_bytes(cache, 0, h, rep, 0, h, f"{w.name} block {h}")
    sm = w.d ** -0.5
    for path, T in (("target", 2), ("draft4", 1)):
        if path == "draft4" and w.bits != 8:
            continue
        q16 = synth.queries(w, 7, T)
        out, lse = cache.verify(to_dev(q16), path=path, want_lse=True)
        torch.cuda.synchronize()
        ref, ref_lse = attention.attend(rep, q16, path, sm)
        assert_attn_close(out.cpu().numpy(), ref, f"{w.name} {path}")
        assert (np.abs(lse.cpu().numpy() - ref_lse)
                <= lse_tolerance(rep, q16, path, sm)).all()
    q16 = synth.queries(w, 8, 1)[:, 0]
    idx, key = cache.topk(to_dev(q16), 32)
    torch.cuda.synchronize()
    gs = w.Hq // w.Hkv
    for h in range(w.Hkv):
        ri, rk = otopk.topk_block(q16[0, h * gs:(h + 1) * gs], rep.kq[0, h],
                                  rep.ks[0, h], rep.kz[0, h], w.G, "target", 32)
        assert np.array_equal(idx.cpu().numpy()[0, h], ri)
        assert np.array_equal(key.cpu().numpy()[0, h].view(np.uint32),
                              rk.view(np.uint32))


def test_split_count_invariance():
    """Block (2, 5) of a 4 x 8-block INT8 cache at 8K, T=7 GQA-4: inside the
    batch the launcher gives each block a few splits, alone it gives the
    block many; both agree with the oracle and with each other."""
    w = W("split_batch", 4, 32, 8, 128, 8192, 128, 64, 256, 8, "outlier_drift")
    b0, h0, T = 2, 5, 7
    gs = w.Hq // w.Hkv
    say("[gpu] split-count invariance: 8K INT8 block alone vs in a batch of 32")
    K, V = host_tokens(w, 4)
    q16 = synth.queries(w, 9, T)
    big = kq.QuantKVCache(shape_for(w))
    big.append(to_dev(K), to_dev(V))
    wa = W("split_alone", 1, gs, 1, 128, 8192, 128, 64, 256, 8, "outlier_drift")
    alone = kq.QuantKVCache(shape_for(wa))
    Ka = np.ascontiguousarray(K[b0:b0 + 1, :, h0:h0 + 1])
    Va = np.ascontiguousarray(V[b0:b0 + 1, :, h0:h0 + 1])
    alone.append(to_dev(Ka), to_dev(Va))
    qa = np.ascontiguousarray(q16[b0:b0 + 1, :, h0 * gs:(h0 + 1) * gs])
    ob, lb = big.verify(to_dev(q16), want_lse=True)
    oa, la = alone.verify(to_dev(qa), want_lse=True)
    torch.cuda.synchronize()
    got_b = ob.cpu().numpy()[b0:b0 + 1, :, h0 * gs:(h0 + 1) * gs]
    got_a = oa.cpu().numpy()
    rep = ocache.Replay(1, 1, w.d, w.G, w.Gv, w.bits, w.R)
    rep.append(Ka, Va)
    sm = w.d ** -0.5
    ref, ref_lse = attention.attend(rep, qa, "target", sm)
    assert_attn_close(got_b, ref, "in batch")
    assert_attn_close(got_a, ref, "alone")
    assert_attn_close(got_a, got_b.astype(np.float64), "alone vs in batch")
    tol = lse_tolerance(rep, qa, "target", sm)
    lbb = lb.cpu().numpy()[b0:b0 + 1, h0 * gs:(h0 + 1) * gs]
    assert (np.abs(lbb - ref_lse) <= tol).all()
    assert (np.abs(la.cpu().numpy() - ref_lse) <= tol).all()
    assert (np.abs(la.cpu().numpy() - lbb) <= 2 * tol).all()
    assert big.n_q == alone.n_q


@pytest.mark.parametrize("path,T", [("target", 7), ("draft4", 1)])
def test_gqa_equals_mha_with_repeated_kv_heads(path, T):
    w = W("gqa4", 1, 8, 2, 128, 2000, 128, 64, 256, 8, "outlier")
    say(f"[gpu] GQA == MHA with repeated kv heads, {path} T={T}")
    K, V = host_tokens(w, 6)
    gs = w.Hq // w.Hkv
    Km = np.ascontiguousarray(np.repeat(K, gs, axis=2))
    Vm = np.ascontiguousarray(np.repeat(V, gs, axis=2))
    wm = W("mha8", 1, 8, 8, 128, 2000, 128, 64, 256, 8, "outlier")
    gqa = kq.QuantKVCache(shape_for(w))
    mha = kq.QuantKVCache(shape_for(wm))
    gqa.append(to_dev(K), to_dev(V))
    mha.append(to_dev(Km), to_dev(Vm))
    q16 = synth.queries(w, 3, T)
    og, _ = gqa.verify(to_dev(q16), path=path)
    om, _ = mha.verify(to_dev(q16), path=path)
    torch.cuda.synchronize()
    rep = ocache.Replay(1, w.Hkv, w.d, w.G, w.Gv, w.bits, w.R)
    rep.append(K, V)
    ref, _ = attention.attend(rep, q16, path, w.d ** -0.5)
    assert_attn_close(og.cpu().numpy(), ref, "GQA")
    assert_attn_close(om.cpu().numpy(), ref, "MHA")
    assert_attn_close(og.cpu().numpy(), om.cpu().numpy().astype(np.float64),
                      "GQA vs MHA")


@pytest.mark.parametrize("bits", [8, 2, 1])
def test_value_scale_at_the_limit(bits):
    """Value groups whose scale is exactly 63, the largest the attention
    kernels take (their PV step multiplies fp16 probabilities scaled to at
    most 2^10 by s in fp16): finite outputs within the bar."""
    G = 128 if bits == 8 else 32
    Gv = 64 if bits == 8 else 32
    w = W(f"vlimit_{bits}", 1, 8, 2, 128, 900, G, Gv, 256 if bits == 8 else 32,
          bits, "normal")
    say(f"[gpu] value scale 63, {bits}-bit")
    K, V = host_tokens(w, 5)
    Lv = (1 << bits) - 1
    half = np.float16(63 * Lv / 2)               # range 63 * Lv: s = 63
    rng = np.random.default_rng(1)
    rows = rng.choice(800, 200, replace=False)
    for r in rows:
        V[0, r, :, 0] = -half
        V[0, r, :, 1] = half
    cache = kq.QuantKVCache(shape_for(w))
    cache.append(to_dev(K), to_dev(V))
    rep = ocache.Replay(1, w.Hkv, w.d, w.G, w.Gv, w.bits, w.R)
    rep.append(K, V)
    assert attention.max_value_scale(rep) == 63.0
    q16 = synth.queries(w, 2, 2)
    out, _ = cache.verify(to_dev(q16))
    torch.cuda.synchronize()
    ref, _ = attention.attend(rep, q16, "target", w.d ** -0.5)
    assert_attn_close(out.cpu().numpy(), ref, f"value scale 63, {bits}-bit")


@pytest.mark.parametrize("bits", [8, 2, 1])
def test_lowbit_key_range(bits):
    """One key group with a large scale and a large query component on its
    channel: q c0 s at 90% of what a 2-bit cache's key operands hold in
    fp16 (4 q c0 s < 65504, c0 = sm_scale log2 e), one token's logit ahead
    of every other by thousands.  Outputs finite and within the bar (the
    row's attention is that token's value), for every code width."""
    G = 128 if bits == 8 else 32
    Gv = 64 if bits == 8 else 32
    w = W(f"krange_{bits}", 1, 8, 2, 128, 900, G, Gv, 256 if bits == 8 else 32,
          bits, "normal")
    say(f"[gpu] key scale x query near the fp16 range, {bits}-bit")
    K, V = host_tokens(w, 6)
    A = np.float16(1500.0)
    g0 = 2 * G                                   # a quantized group
    K[0, g0:g0 + G, :, 0] = 0
    K[0, g0 + 5, :, 0] = A                       # the dominant token
    K[0, g0 + 9, :, 0] = -A
    cache = kq.QuantKVCache(shape_for(w))
    cache.append(to_dev(K), to_dev(V))
    rep = ocache.Replay(1, w.Hkv, w.d, w.G, w.Gv, w.bits, w.R)
    rep.append(K, V)
    assert g0 + G <= rep.n_q
    s = float(rep.ks[0, 0, g0 // G, 0])
    sm = w.d ** -0.5
    c0 = sm * np.log2(np.e)
    qv = 0.9 * 65504 / (4 * c0 * s)
    assert 10 < qv < 60000
    q16 = synth.queries(w, 3, 2)
    q16[..., 0] = np.float16(qv)
    out, lse = cache.verify(to_dev(q16), want_lse=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isfinite(got).all() and np.isfinite(lse.cpu().numpy()).all()
    ref, ref_lse = attention.attend(rep, q16, "target", sm)
    assert_attn_close(got, ref, f"key range, {bits}-bit")
    tol = lse_tolerance(rep, q16, "target", sm)
    assert (np.abs(lse.cpu().numpy() - ref_lse) <= tol).all()


@pytest.mark.parametrize("bits", [8, 2])
def test_quantizer_divide_ties(bits):
    """The hand-derived groups whose quotient (x - z)/s is an exact
    half-integer (tests/golden/quant_divide_ties.json), laid along key
    tokens and value channels: the HIP quantizer must give the correctly
    rounded divide's codes (a reciprocal-multiply alone would not)."""
    import json
    import os
    cases = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                        "quant_divide_ties.json")))["cases"]
    case = [c for c in cases if c["bits"] == bits][0]
    x = np.array(case["x"], np.float16)
    w = W(f"ties{bits}", 1, 4, 1, 64, 96, 32, 16, 32, bits, "normal")
    say(f"[gpu] divide ties, {bits}-bit")
    K, V = host_tokens(w, 1)
    K[0, :32, 0, :] = np.tile(x, 8)[:, None]             # every key channel
    V[0, :64, 0, :16] = np.tile(x, 4)[None, :]            # value group 0
    cache = kq.QuantKVCache(shape_for(w, max_append=96))
    cache.append(to_dev(K), to_dev(V))
    rep = ocache.Replay(w.B, w.Hkv, w.d, w.G, w.Gv, w.bits, w.R)
    rep.append(K, V)
    torch.cuda.synchronize()
    assert rep.kq[0, 0, :4, 0].tolist() == case["codes"]
    assert rep.vq[0, 0, 0, :4].tolist() == case["codes"]
    assert_block_bytes(cache, 0, 0, rep, 0, 0, f"ties {bits}-bit")
