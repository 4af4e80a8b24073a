"""kv_attn_verify_noalloc: the attention entry point for callers that cannot
allocate (its partials live in a static device scratch) against the
workspace entry point kv_attn_verify on the same caches and queries, three
calls in a row, each on a smaller input than the one before, plus its size
limit (checked before any HIP call)."""
import numpy as np
import pytest
import torch

import kvq_synth as synth
import quantized_kv_attention_quant_amd as kq
from oracle import attention, cache as ocache
from kvq_testlib import (assert_attn_close, host_tokens, say, shape_for,
                         to_dev)

W = synth.Workload

# a GQA INT8 verify over several splits, then a smaller one with 8 query
# heads per kv head (48 rows: two launch pairs over head subsets), then a
# smaller MHA-group draft
CASES = [
    ("gqa_int8_t7", W("gqa_int8_t7", 2, 8, 2, 128, 3000, 128, 64, 256, 8,
                      "outlier_drift"), 7, "target"),
    ("gqa8_int8_t6", W("gqa8_int8_t6", 1, 16, 2, 128, 1500, 64, 64, 128, 8,
                       "outlier"), 6, "target"),
    ("tiny_draft_t1", synth.WORKLOADS["tiny"], 1, "draft4"),
]


def _cache(w, seed):
    K, V = host_tokens(w, seed)
    cache = kq.QuantKVCache(shape_for(w, max_append=64))
    cache.append(to_dev(K), to_dev(V))
    rep = ocache.Replay(w.B, w.Hkv, w.d, w.G, w.Gv, w.bits, w.R)
    rep.append(K, V)
    return cache, rep


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point():
    sh = torch.cuda.current_stream().cuda_stream
    for name, w, T, path in CASES:
        say(f"[no-alloc] {name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} d={w.d} "
            f"L={w.L} T={T} {path}")
        cache, rep = _cache(w, 3)
        q16 = synth.queries(w, 5, T)
        q = to_dev(q16)
        sm = w.d ** -0.5
        p = kq.KVQ_TARGET if path == "target" else kq.KVQ_DRAFT4
        ref_out, ref_lse = torch.empty_like(q), torch.empty(
            (w.B, w.Hq, T), dtype=torch.float32, device=q.device)
        ws = cache.attn_workspace(T, w.Hq)
        kq.kv_attn_verify(cache.c, q, T, w.Hq, p, sm, ref_out, ref_lse, ws, sh)
        # garbage in the outputs first: the call must write every element
        out = torch.full_like(q, float("nan"))
        lse = torch.full((w.B, w.Hq, T), float("nan"), dtype=torch.float32,
                         device=q.device)
        kq.kv_attn_verify_noalloc(cache.c, q, T, w.Hq, p, sm, out, lse, sh)
        torch.cuda.synchronize()
        got, ref = out.cpu().numpy(), ref_out.cpu().numpy()
        assert_attn_close(got, ref.astype(np.float64), f"{name} vs kv_attn_verify")
        assert np.isfinite(lse.cpu().numpy()).all()
        assert np.abs(lse.cpu().numpy() - ref_lse.cpu().numpy()).max() <= 1e-4
        # and both against the oracle
        oref, _ = attention.attend(rep, q16, path, sm)
        assert_attn_close(got, oref, f"{name} vs oracle")
        say(f"[no-alloc] {name}: identical to kv_attn_verify: "
            f"{bool(np.array_equal(got, ref))}")
        del cache, ws


def test_noalloc_rejects_calls_beyond_the_scratch():
    """B*Hkv*rows_pad*(d+2)*4 bytes per split slot with fewer than two slots
    in the 32 MiB scratch: KVQ_EWORKSPACE before any HIP call (placeholder
    pointers, never dereferenced)."""
    c = kq.KvqCacheStruct()
    for k, v in dict(B=64, Hkv=64, d=128, G=128, Gv=64, bits=8, R=256,
                     L_max=4096, max_append=32).items():
        setattr(c, k, v)
    kq.kv_cache_layout(c)
    for name in ("k_hi", "k_lo", "v_hi", "v_lo", "k_sz", "v_sz", "k_res",
                 "v_res"):
        setattr(c, name, 0x1000)
    c.n_q, c.n_r = 1024, 40

    class FakeT:
        def data_ptr(self):
            return 0x2000

    # 4096 blocks x 32 rows x 130 floats: 68 MB per slot
    with pytest.raises(kq.KvqError) as e:
        kq.kv_attn_verify_noalloc(c, FakeT(), 16, 128, kq.KVQ_TARGET, 0.088,
                                  FakeT(), None, 0)
    assert e.value.code == kq.KVQ_EWORKSPACE
    assert "scratch" in kq.kv_last_error()
    # the ordinary argument checks come first, as in kv_attn_verify
    with pytest.raises(kq.KvqError) as e:
        kq.kv_attn_verify_noalloc(c, FakeT(), 0, 128, kq.KVQ_TARGET, 0.088,
                                  FakeT(), None, 0)
    assert e.value.code == kq.KVQ_EINVAL
