"""GPU parity at small sizes: quantize-on-append bytes, verify/draft attention
and top-k indices against the CPU oracle on the same seeded inputs.

Sizes span several tiles, key groups and splits plus a ragged residual tail;
shapes cover d = 64/128, 8/2/1-bit codes, MHA and GQA, T up to the 32-row
limit.  Every case prints its name before touching the GPU.
"""
import numpy as np
import pytest
import torch

import kvq_synth as synth
import quantized_kv_attention_quant_amd as kq
from oracle import attention, cache as ocache, quant, topk as otopk
from kvq_testlib import (assert_attn_close, host_tokens, lse_tolerance,
                         read_block, say, shape_for, to_dev)

pytestmark = pytest.mark.gpu

W = synth.Workload

SMALL = {
    "tiny": synth.WORKLOADS["tiny"],
    "gqa_d128_int8": W("gqa_d128_int8", 2, 8, 2, 128, 1200, 128, 64, 256, 8,
                       "outlier_drift"),
    "mha_d64_int8": W("mha_d64_int8", 1, 3, 3, 64, 777, 64, 32, 128, 8,
                      "outlier"),
    "gqa_2bit": W("gqa_2bit", 2, 8, 2, 128, 1000, 32, 32, 32, 2, "normal"),
    "gqa_1bit": W("gqa_1bit", 2, 8, 2, 128, 1000, 32, 32, 32, 1, "normal"),
    "d64_2bit": W("d64_2bit", 1, 4, 2, 64, 500, 32, 16, 64, 2, "normal"),
    "gv128": W("gv128", 1, 4, 1, 128, 700, 64, 128, 64, 8, "outlier"),
    # key groups of 96 tokens: not a power of two, and groups straddle the
    # top-k's 1024-token chunks
    "g96": W("g96", 1, 8, 2, 128, 2400, 96, 64, 192, 8, "outlier"),
    "g96_2bit": W("g96_2bit", 1, 8, 2, 128, 2000, 96, 32, 96, 2, "normal"),
    # two query heads per kv head: T = 16 fills the 32-row limit
    "gqa2": W("gqa2", 1, 4, 2, 128, 900, 64, 64, 128, 8, "outlier"),
    # bulk appends of many small key groups with a flush count that is not
    # a multiple of 4 or 2: 81 groups of 32 and 71 groups of 64
    "g32_bulk": W("g32_bulk", 1, 4, 2, 128, 2600, 32, 32, 32, 2, "normal"),
    "g64_bulk": W("g64_bulk", 1, 4, 2, 128, 4560, 64, 64, 64, 8, "outlier"),
    # 10 top-k chunks: top-256 candidates overflow one merge pass
    "long_2bit": W("long_2bit", 1, 8, 2, 128, 9500, 32, 32, 32, 2, "normal"),
    # key groups longer than 128 tokens: 16 rows per quantizer thread at
    # head dim 128 (read again in batches of 8), 8 rows at head dim 64
    "g256": W("g256", 1, 4, 2, 128, 1800, 256, 64, 256, 8, "outlier"),
    "d64_g256_2bit": W("d64_g256_2bit", 1, 4, 2, 64, 1500, 256, 32, 256, 2,
                       "normal"),
    # 8 query heads per kv head: T * 8 rows above 32 run as head subsets
    "gqa8": W("gqa8", 1, 16, 2, 128, 1500, 64, 64, 128, 8, "outlier"),
    # group sizes that are not powers of two (top-k pads them to 4 and 8)
    "gqa3_2bit": W("gqa3_2bit", 1, 6, 2, 128, 2000, 32, 32, 32, 2, "normal"),
    "gqa7": W("gqa7", 1, 14, 2, 128, 1500, 64, 64, 128, 8, "outlier"),
    # 1/2-bit caches with 8 query heads per kv head: head subsets
    "gqa8_2bit": W("gqa8_2bit", 1, 16, 2, 128, 1500, 32, 32, 32, 2, "normal"),
    "gqa8_1bit": W("gqa8_1bit", 1, 16, 2, 128, 1500, 32, 32, 32, 1, "normal"),
}


def build(w, seed=0, chunks=None):
    """GPU cache + oracle replay after appending w.L tokens (in one call or
    in the given chunk sizes)."""
    K, V = host_tokens(w, seed)
    cache = kq.QuantKVCache(shape_for(w, max_append=64))
    rep = ocache.Replay(w.B, w.Hkv, w.d, w.G, w.Gv, w.bits, w.R)
    pos = 0
    for n in (chunks or [w.L]):
        kd, vd = to_dev(K[:, pos:pos + n]), to_dev(V[:, pos:pos + n])
        cache.append(kd, vd)
        rep.append(K[:, pos:pos + n], V[:, pos:pos + n])
        pos += n
    assert pos == w.L
    torch.cuda.synchronize()
    assert (cache.n_q, cache.n_r) == (rep.n_q, rep.n_r)
    return cache, rep


def check_bytes(cache, rep):
    """Codes bit-exact, scales/zeros equal as fp16 values, residual exact."""
    for b in range(rep.B):
        for h in range(rep.Hkv):
            got = read_block(cache, b, h)
            for name, ref in (("kq", rep.kq[b, h]), ("vq", rep.vq[b, h]),
                              ("rk", rep.rk[b, h]), ("rv", rep.rv[b, h])):
                assert np.array_equal(got[name].view(np.uint8) if name[0] != "r"
                                      else got[name], ref), (name, b, h)
            for name, ref in (("ks", rep.ks), ("kz", rep.kz), ("vs", rep.vs),
                              ("vz", rep.vz)):
                assert np.array_equal(got[name], ref[b, h]), (name, b, h)


@pytest.mark.parametrize("name", list(SMALL))
def test_append_bulk_bit_exact(name):
    say(f"[gpu] append bulk {name}")
    cache, rep = build(SMALL[name])
    check_bytes(cache, rep)


@pytest.mark.parametrize("name", ["tiny", "gqa_d128_int8", "gqa_2bit",
                                  "gqa_1bit", "mha_d64_int8", "g96", "g256"])
def test_append_incremental_and_rollback(name):
    w = SMALL[name]
    say(f"[gpu] append incremental {name}")
    rng = np.random.default_rng(11)
    K, V = host_tokens(w, 1)
    cache = kq.QuantKVCache(shape_for(w, max_append=64))
    rep = ocache.Replay(w.B, w.Hkv, w.d, w.G, w.Gv, w.bits, w.R)
    pos = 0
    steps = 0
    while pos < w.L:
        n = int(min(w.L - pos, rng.integers(1, 80)))
        cache.append(to_dev(K[:, pos:pos + n]), to_dev(V[:, pos:pos + n]))
        rep.append(K[:, pos:pos + n], V[:, pos:pos + n])
        pos += n
        if rng.random() < 0.5 and rep.n_r > 0:
            m = int(rng.integers(0, min(n, rep.n_r) + 1))
            cache.rollback(m)
            rep.rollback(m)
            pos -= m
        steps += 1
    torch.cuda.synchronize()
    assert (cache.n_q, cache.n_r) == (rep.n_q, rep.n_r)
    check_bytes(cache, rep)
    assert steps > 10


RUNS = [("tiny", "target", 1), ("tiny", "draft4", 1), ("tiny", "target", 8),
        ("gqa_d128_int8", "target", 7), ("gqa_d128_int8", "draft4", 1),
        ("gqa_d128_int8", "target", 2), ("gqa_d128_int8", "draft4", 8),
        ("mha_d64_int8", "target", 9), ("mha_d64_int8", "draft4", 3),
        ("gqa_2bit", "target", 2), ("gqa_2bit", "target", 8),
        ("gqa_1bit", "target", 2), ("d64_2bit", "target", 5),
        ("gv128", "target", 4), ("gv128", "draft4", 8),
        ("g96", "target", 7), ("g96", "draft4", 1), ("g96_2bit", "target", 2),
        # T = 16, the largest speculative block: 16 rows (MHA) and 32 (GQA 2)
        ("mha_d64_int8", "target", 16), ("gqa2", "target", 16),
        ("gqa2", "draft4", 16),
        ("g256", "target", 5), ("g256", "draft4", 1),
        ("d64_g256_2bit", "target", 3),
        # 40 rows (heads 0-5, then 6-7), 64 rows (2 x 4 heads), 128 rows
        ("gqa8", "target", 5), ("gqa8", "target", 8), ("gqa8", "draft4", 16),
        ("gqa3_2bit", "target", 2), ("gqa7", "target", 4),
        # 1-bit codes in two-wave streams (32 rows); 1/2-bit codes over head
        # subsets: 40 rows (6 + 2 heads), 48 rows (5 + 3 heads)
        ("gqa_1bit", "target", 8), ("gqa8_2bit", "target", 5),
        ("gqa8_1bit", "target", 6)]


@pytest.mark.parametrize("name,path,T", RUNS)
def test_attention_matches_oracle(name, path, T):
    w = SMALL[name]
    say(f"[gpu] attention {name} {path} T={T}")
    cache, rep = build(w)
    q16 = synth.queries(w, 0, T)
    out, lse = cache.verify(to_dev(q16), path=path, want_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = attention.attend(rep, q16, path, w.d ** -0.5)
    rel = assert_attn_close(out.cpu().numpy(), ref, f"{name} {path} T={T}")
    tol = lse_tolerance(rep, q16, path, w.d ** -0.5)
    lerr = np.abs(lse.cpu().numpy() - ref_lse)
    say(f"    rel err {rel:.2e}; lse err {lerr.max():.2e} (tol {tol.min():.2e}"
        f"..{tol.max():.2e})")
    assert (lerr <= tol).all()


def test_attention_all_residual_and_short_prefix():
    w = W("short", 1, 4, 2, 128, 300, 128, 64, 256, 8, "outlier")
    for L in (5, 40, 256, 257, 300):
        ww = w.scaled(L=L)
        say(f"[gpu] attention short L={L}")
        cache, rep = build(ww)
        T = min(4, L)
        q16 = synth.queries(ww, 3, T)
        out, _ = cache.verify(to_dev(q16), path="target")
        ref, _ = attention.attend(rep, q16, "target", 0.1)
        # default scale is d**-0.5; recompute reference with it
        ref, _ = attention.attend(rep, q16, "target", ww.d ** -0.5)
        assert_attn_close(out.cpu().numpy(), ref, f"L={L}")


def test_draft_ignores_low_planes_and_is_deterministic():
    w = SMALL["gqa_d128_int8"]
    say("[gpu] draft invariance to lo planes")
    cache, _ = build(w)
    q = to_dev(synth.queries(w, 5, 1))
    a, _ = cache.verify(q, path="draft4")
    a2, _ = cache.verify(q, path="draft4")
    t, _ = cache.verify(q, path="target")
    cache.k_lo.copy_(torch.randint_like(cache.k_lo, 0, 256))
    cache.v_lo.copy_(torch.randint_like(cache.v_lo, 0, 256))
    b_, _ = cache.verify(q, path="draft4")
    t2, _ = cache.verify(q, path="target")
    torch.cuda.synchronize()
    assert torch.equal(a, a2)
    assert torch.equal(a, b_)
    assert not torch.equal(t, t2)


def test_verify_row_equals_prefix_decode():
    w = SMALL["gqa_d128_int8"]
    say("[gpu] verify row vs prefix decode")
    T = 6
    cache, _ = build(w)
    q16 = synth.queries(w, 7, T)
    full, _ = cache.verify(to_dev(q16), path="target")
    full = full.cpu().numpy().astype(np.float64)
    for t in range(T):
        c2, _ = build(w)
        c2.rollback(T - 1 - t)
        one, _ = c2.verify(to_dev(q16[:, t:t + 1]), path="target")
        assert_attn_close(one.cpu().numpy()[:, 0], full[:, t], f"row {t}")


@pytest.mark.parametrize("name,path,k", [
    ("gqa_d128_int8", "target", 64), ("gqa_d128_int8", "draft4", 64),
    ("gqa_2bit", "target", 64), ("gqa_1bit", "target", 100),
    ("mha_d64_int8", "target", 256), ("tiny", "target", 300 // 2),
    ("g96", "target", 64), ("g96", "draft4", 64), ("g96_2bit", "target", 200),
    ("g32_bulk", "target", 128), ("long_2bit", "target", 256),
    ("g256", "target", 64), ("d64_g256_2bit", "target", 32),
    ("gqa3_2bit", "target", 64), ("gqa7", "target", 100),
    ("gqa7", "draft4", 64), ("gqa8_2bit", "target", 64),
    ("gqa8_1bit", "target", 32)])
def test_topk_bit_exact(name, path, k):
    w = SMALL[name]
    say(f"[gpu] topk {name} {path} k={k}")
    cache, _ = build(w)
    qs16 = synth.queries(w, 9, 1)[:, 0]
    idx, key = cache.topk(to_dev(qs16), k, path=path)
    torch.cuda.synchronize()
    idx, key = idx.cpu().numpy(), key.cpu().numpy()
    gs = w.Hq // w.Hkv
    for b in range(w.B):
        for h in range(w.Hkv):
            blk = read_block(cache, b, h)
            ref_i, ref_k = otopk.topk_block(qs16[b, h * gs:(h + 1) * gs],
                                            blk["kq"], blk["ks"], blk["kz"],
                                            w.G, path, k)
            assert np.array_equal(idx[b, h], ref_i), (b, h)
            assert np.array_equal(key[b, h].view(np.uint32),
                                  ref_k.view(np.uint32)), (b, h)


def test_topk_ties_and_padding():
    w = W("ties", 1, 2, 1, 128, 200, 32, 32, 32, 1, "normal")
    say("[gpu] topk ties / padding")
    K = np.zeros((1, 200, 1, 128), np.float16)
    K[0, ::3, 0, :] = 1.0              # every third token identical
    K[0, 1::3, 0, 5] = -1.0
    cache = kq.QuantKVCache(shape_for(w))
    cache.append(to_dev(K), to_dev(K))
    q = to_dev(np.ones((1, 2, 128), np.float16))
    idx, key = cache.topk(q, 256)
    torch.cuda.synchronize()
    blk = read_block(cache, 0, 0)
    ref_i, ref_k = otopk.topk_block(np.ones((2, 128), np.float16), blk["kq"],
                                    blk["ks"], blk["kz"], 32, "target", 256)
    # 200 tokens, G = R = 32: ceil(168/32) = 6 groups quantized
    assert cache.n_q == 192
    assert np.array_equal(idx.cpu().numpy()[0, 0], ref_i)
    assert (idx.cpu().numpy()[0, 0, 192:] == -1).all()
    assert np.isneginf(key.cpu().numpy()[0, 0, 192:]).all()
