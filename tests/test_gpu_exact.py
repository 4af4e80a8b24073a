"""GPU parity of the SpeCache-style prefetch path: kv_fetch_rows (rows of a
host-resident fp16 copy, bit for bit) and kv_attn_verify_exact (one query
row reads the fetched exact values) against oracle.attention.attend_exact,
small over every code width and at the full batched 32K 2-bit size as one
pipeline: top-k of the speculative token -> fetch -> exact verify."""
import numpy as np
import pytest
import torch

import kvq_synth as synth
import quantized_kv_attention_quant_amd as kq
from oracle import attention, cache as ocache, topk as otopk
from kvq_testlib import (assert_attn_close, host_tokens, lse_tolerance, say,
                         shape_for, to_dev)

pytestmark = pytest.mark.gpu

W = synth.Workload

CASES = [
    ("tiny", synth.WORKLOADS["tiny"], "target", 2, 0),
    ("tiny_draft", synth.WORKLOADS["tiny"], "draft4", 2, 0),
    ("gqa_d128_int8", W("gqa_d128_int8", 2, 8, 2, 128, 1200, 128, 64, 256, 8,
                        "outlier_drift"), "target", 7, 0),
    ("gqa_2bit", W("gqa_2bit", 2, 8, 2, 128, 1000, 32, 32, 32, 2, "normal"),
     "target", 2, 0),
    ("gqa_1bit_row1", W("gqa_1bit", 2, 8, 2, 128, 1000, 32, 32, 32, 1, "normal"),
     "target", 3, 1),
    ("mha_d64", W("mha_d64_int8", 1, 3, 3, 64, 777, 64, 32, 128, 8, "outlier"),
     "target", 2, 0),
    # T = 16: the substituted row is the last of 32 rows, or a middle one
    ("gqa2_t16_last", W("gqa2", 1, 4, 2, 128, 900, 64, 64, 128, 8, "outlier"),
     "target", 16, 15),
    # 8 query heads per kv head at T = 6: 48 rows, run as two head subsets
    ("gqa8_t6", W("gqa8", 1, 16, 2, 128, 1500, 64, 64, 128, 8, "outlier"),
     "target", 6, 4),
    ("mha_d64_t16_draft", W("mha_d64_int8", 1, 3, 3, 64, 777, 64, 32, 128, 8,
                            "outlier"), "draft4", 16, 7),
    # 1-bit codes in two-wave streams (32 rows), and a 2-bit cache with 8
    # query heads per kv head at T = 5 (40 rows: head subsets of 6 and 2)
    ("gqa_1bit_t8", W("gqa_1bit", 2, 8, 2, 128, 1000, 32, 32, 32, 1, "normal"),
     "target", 8, 5),
    ("gqa8_2bit_t5", W("gqa8_2bit", 1, 16, 2, 128, 1500, 32, 32, 32, 2,
                       "normal"), "target", 5, 2),
]


def _picks(rng, B, H, n_q, n):
    """Distinct quantized positions per block, then a -1 and an out-of-range
    entry (both skipped by the substitution)."""
    idx = np.empty((B, H, n + 2), np.int32)
    for b in range(B):
        for h in range(H):
            idx[b, h, :n] = rng.choice(n_q, n, replace=False)
            idx[b, h, n:] = (-1, n_q + 5)
    return idx


def test_fetch_rows_bit_exact():
    say("[gpu] fetch rows from pinned host memory")
    w = CASES[2][1]
    shape = shape_for(w)
    mirror = kq.HostMirror(shape, w.L)
    K, V = host_tokens(w, 0)
    mirror.write(0, K, V)
    cache = kq.QuantKVCache(shape)
    rng = np.random.default_rng(4)
    idx = rng.integers(0, w.L, (w.B, w.Hkv, 50)).astype(np.int32)
    idx[:, :, :3] = (-1, w.L, 0)
    kf, vf = mirror.fetch(cache, torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    kf, vf = kf.cpu().numpy(), vf.cpu().numpy()
    for b in range(w.B):
        for h in range(w.Hkv):
            for i, p in enumerate(idx[b, h]):
                if 0 <= p < w.L:
                    assert np.array_equal(kf[b, h, i].view(np.uint16),
                                          K[b, p, h].view(np.uint16))
                    assert np.array_equal(vf[b, h, i].view(np.uint16),
                                          V[b, p, h].view(np.uint16))
                else:
                    assert np.isnan(kf[b, h, i]).all() and np.isnan(vf[b, h, i]).all()
    # pageable memory is refused before any launch
    pageable = torch.zeros(8, dtype=torch.float16)
    with pytest.raises(kq.KvqError):
        kq.kv_fetch_rows(cache.c, pageable, pageable, 1, torch.from_numpy(idx).cuda(),
                         idx.shape[2], torch.from_numpy(kf).cuda(),
                         torch.from_numpy(vf).cuda())


@pytest.mark.parametrize("name,w,path,T,t_exact", CASES, ids=[c[0] for c in CASES])
def test_verify_exact_matches_oracle(name, w, path, T, t_exact):
    say(f"[gpu] exact substitution {name} {path} T={T} row {t_exact}")
    K, V = host_tokens(w, 0)
    shape = shape_for(w, max_append=64)
    cache = kq.QuantKVCache(shape)
    rep = ocache.Replay(w.B, w.Hkv, w.d, w.G, w.Gv, w.bits, w.R)
    cache.append(to_dev(K), to_dev(V))
    rep.append(K, V)
    mirror = kq.HostMirror(shape, w.L)
    mirror.write(0, K, V)
    idx = _picks(np.random.default_rng(9), w.B, w.Hkv, rep.n_q, 20)
    idx_d = torch.from_numpy(idx).cuda()
    kx, vx = mirror.fetch(cache, idx_d)
    q16 = synth.queries(w, 5, T)
    out, lse = cache.verify_exact(to_dev(q16), idx_d, kx, vx, t_exact=t_exact,
                                  path=path, want_lse=True)
    torch.cuda.synchronize()
    keep = (idx >= 0) & (idx < rep.n_q)
    idx_o = np.where(keep, idx, -1)
    kxo = np.zeros((w.B, w.Hkv, idx.shape[2], w.d), np.float16)
    vxo = np.zeros_like(kxo)
    for b in range(w.B):
        for h in range(w.Hkv):
            for i in np.nonzero(keep[b, h])[0]:
                kxo[b, h, i] = K[b, idx[b, h, i], h]
                vxo[b, h, i] = V[b, idx[b, h, i], h]
    ref, ref_lse = attention.attend_exact(rep, q16, path, w.d ** -0.5, idx_o,
                                          kxo, vxo, t_exact)
    rel = assert_attn_close(out.cpu().numpy(), ref, f"{name} exact")
    tol = lse_tolerance(rep, q16, path, w.d ** -0.5)
    lerr = np.abs(lse.cpu().numpy() - ref_lse)
    say(f"    rel err {rel:.2e}; lse err {lerr.max():.2e}")
    assert (lerr <= tol).all()
    # the substitution moves the substituted row (for low-bit codes) and
    # only that row
    base, _ = attention.attend(rep, q16, path, w.d ** -0.5)
    others = [t for t in range(T) if t != t_exact]
    assert np.abs(ref[:, others] - base[:, others]).max() == 0.0


def test_specache_pipeline_full_size():
    """B=36, 8 kv heads, 32K tokens of 2-bit codes: top-64 of the speculative
    token per kv head, fetch those rows from the pinned host copy, verify
    T=2 with the output token reading them exactly; sampled blocks against
    the oracle."""
    w = synth.WORKLOADS["specache_2bit"]
    say("[gpu] full size specache_2bit: top-64 -> fetch -> exact verify")
    sampled = [(0, 0), (20, 5)]
    g = torch.Generator(device="cuda")
    g.manual_seed(123)
    Kd = torch.randn((w.B, w.L, w.Hkv, w.d), generator=g, device="cuda").half()
    Vd = torch.randn((w.B, w.L, w.Hkv, w.d), generator=g, device="cuda").half()
    host = {}
    for (b, h) in sampled:
        kb, vb = synth.kv_block(w, 0, b, h, w.L)
        Kd[b, :, h] = torch.from_numpy(kb).cuda()
        Vd[b, :, h] = torch.from_numpy(vb).cuda()
        host[(b, h)] = (kb, vb)
    shape = shape_for(w, max_append=32)
    cache = kq.QuantKVCache(shape)
    cache.append(Kd[:, :w.L - 2].contiguous(), Vd[:, :w.L - 2].contiguous())
    cache.append(Kd[:, w.L - 2:].contiguous(), Vd[:, w.L - 2:].contiguous())
    mirror = kq.HostMirror(shape, w.L)
    for b in range(w.B):                       # device tokens -> pinned copy
        mirror.k[b].copy_(Kd[b].permute(1, 0, 2).contiguous())
        mirror.v[b].copy_(Vd[b].permute(1, 0, 2).contiguous())
    del Kd, Vd
    torch.cuda.synchronize()
    q16 = synth.queries(w, 3, 2)
    qs = torch.from_numpy(np.ascontiguousarray(q16[:, 1])).cuda()
    idx, _ = cache.topk(qs, w.topk)
    kx, vx = mirror.fetch(cache, idx)
    out, lse = cache.verify_exact(to_dev(q16), idx, kx, vx, t_exact=0,
                                  want_lse=True)
    torch.cuda.synchronize()
    idx, out, lse = idx.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()
    gs = w.Hq // w.Hkv
    for (b, h), (kb, vb) in host.items():
        rep = ocache.Replay(1, 1, w.d, w.G, w.Gv, w.bits, w.R)
        rep.append(kb[None, :w.L - 2, None], vb[None, :w.L - 2, None])
        rep.append(kb[None, w.L - 2:, None], vb[None, w.L - 2:, None])
        qb = q16[b:b + 1, :, h * gs:(h + 1) * gs]
        ref_i, _ = otopk.topk_block(qb[0, 1], rep.kq[0, 0], rep.ks[0, 0],
                                    rep.kz[0, 0], w.G, "target", w.topk)
        assert np.array_equal(idx[b, h], ref_i), (b, h)
        sel = idx[b, h][None, None]
        ref, ref_lse = attention.attend_exact(
            rep, qb, "target", w.d ** -0.5, sel, kb[sel[0, 0]][None, None],
            vb[sel[0, 0]][None, None], 0)
        rel = assert_attn_close(out[b:b + 1, :, h * gs:(h + 1) * gs], ref,
                                f"pipeline ({b},{h})")
        tol = lse_tolerance(rep, qb, "target", w.d ** -0.5)
        lerr = np.abs(lse[b:b + 1, h * gs:(h + 1) * gs] - ref_lse)
        say(f"    ({b},{h}): rel err {rel:.2e}, lse err {lerr.max():.2e}")
        assert (lerr <= tol).all(), (b, h)


def test_verify_exact_without_substitutions_equals_verify():
    """No fetched rows (n = 0), or only skipped entries (-1): the
    substitution partial is empty (m = -inf, l = 0, o = 0), so the merge adds
    exact zeros and out and lse equal plain verify bit for bit."""
    w = CASES[2][1]
    say("[gpu] exact verify with nothing substituted")
    shape = shape_for(w)
    cache = kq.QuantKVCache(shape)
    K, V = host_tokens(w, 3)
    cache.append(to_dev(K), to_dev(V))
    q = to_dev(synth.queries(w, 4, 7))
    ref, ref_lse = cache.verify(q, want_lse=True)
    for n, fill in ((0, 0), (5, -1)):
        idx = torch.full((w.B, w.Hkv, n), fill, dtype=torch.int32, device="cuda")
        kx = torch.zeros((w.B, w.Hkv, n, w.d), dtype=torch.float16, device="cuda")
        out, lse = cache.verify_exact(q, idx, kx, kx.clone(), t_exact=0,
                                      want_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), n
        assert torch.equal(lse, ref_lse), n


@pytest.mark.parametrize("bits", [1, 2])
def test_verify_exact_dominant_fetched_token(bits):
    """A fetched token that carries almost all of the low-bit attention mass
    of the substituted row while its exact logit is small: the query is
    aligned with that token's dequantized key, whose exact key sits near the
    middle of every group's range.  The substituted row must then follow
    the exact softmax, where that token is negligible (within 2e-3 of the
    oracle: no cancellation between its quantized and exact terms)."""
    w = W(f"dominant_{bits}bit", 1, 8, 2, 128, 1000, 32, 32, 32, bits, "normal")
    T, t_exact, jstar = 2, 0, 333
    top = 25.0 if bits == 1 else 45.0        # jstar's low-bit logit
    say(f"[gpu] exact substitution, dominant fetched token, {bits}-bit")
    K, V = host_tokens(w, 0)
    K[:, jstar] = np.float16(0.1)            # mid-range: its low-bit codes round up
    shape = shape_for(w, max_append=64)
    cache = kq.QuantKVCache(shape)
    rep = ocache.Replay(w.B, w.Hkv, w.d, w.G, w.Gv, w.bits, w.R)
    cache.append(to_dev(K), to_dev(V))
    rep.append(K, V)
    assert jstar < rep.n_q
    sm = w.d ** -0.5
    gs = w.Hq // w.Hkv
    q16 = synth.queries(w, 5, T)
    for h in range(w.Hkv):                   # row t_exact: along k^(jstar)
        kh = attention.block_kv(rep.kq[0, h], rep.ks[0, h], rep.kz[0, h],
                                rep.vq[0, h], rep.vs[0, h], rep.vz[0, h],
                                rep.rk[0, h], rep.rv[0, h], w.G, w.Gv,
                                "target")[0][jstar]
        q16[0, t_exact, h * gs:(h + 1) * gs] = (
            top / (sm * np.linalg.norm(kh)) * kh / np.linalg.norm(kh)).astype(np.float16)
    rng = np.random.default_rng(3)
    n = 12
    idx = np.empty((w.B, w.Hkv, n), np.int32)
    for h in range(w.Hkv):
        others = rng.choice([p for p in range(rep.n_q) if p != jstar], n - 1,
                            replace=False)
        idx[0, h] = np.concatenate([[jstar], others])
    kxo = np.stack([[K[0, idx[0, h], h] for h in range(w.Hkv)]])
    vxo = np.stack([[V[0, idx[0, h], h] for h in range(w.Hkv)]])
    out, lse = cache.verify_exact(to_dev(q16), to_dev(idx), to_dev(kxo),
                                  to_dev(vxo), t_exact=t_exact, want_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = attention.attend_exact(rep, q16, "target", sm, idx, kxo, vxo,
                                          t_exact)
    base, _ = attention.attend(rep, q16, "target", sm)
    # the case is what it claims: the quantized softmax of the row puts
    # almost all of its mass on jstar, the exact one almost none
    Kq, _ = attention.block_kv(rep.kq[0, 0], rep.ks[0, 0], rep.kz[0, 0],
                               rep.vq[0, 0], rep.vs[0, 0], rep.vz[0, 0],
                               rep.rk[0, 0], rep.rv[0, 0], w.G, w.Gv, "target")
    lq = sm * Kq[:rep.n_q] @ q16[0, t_exact, 0].astype(np.float64)
    assert lq[jstar] - np.log(np.exp(lq - lq.max()).sum()) - lq.max() > -0.01
    le = sm * K[0, :rep.n_q, 0].astype(np.float64) @ q16[0, t_exact, 0].astype(np.float64)
    assert le[jstar] < le.max() - 3
    assert np.abs(ref[0, t_exact] - base[0, t_exact]).max() > 0.1
    rel = assert_attn_close(out.cpu().numpy(), ref, f"dominant {bits}-bit")
    lerr = np.abs(lse.cpu().numpy() - ref_lse)
    say(f"    rel err {rel:.2e}; lse err {lerr.max():.2e}")
    assert lerr.max() <= 1e-3
