"""Pins for oracle.attention against torch's scaled_dot_product_attention
(float64, CPU) and against structural invariants of verify attention."""
import numpy as np
import pytest
import torch

from oracle import attention, cache, quant


def _build(B, H, d, G, Gv, bits, R, L, seed=0, scale=1.0):
    rng = np.random.default_rng(seed)
    K = (rng.standard_normal((B, L, H, d)) * scale).astype(np.float16)
    V = rng.standard_normal((B, L, H, d)).astype(np.float16)
    rep = cache.Replay(B, H, d, G, Gv, bits, R)
    rep.append(K, V)
    return rep, K, V


def _sdpa(q16, K64, V64, Hkv, sm_scale):
    """torch SDPA in float64 on CPU with the verify mask (row t of T sees
    positions <= L - T + t).  q16: (B, T, Hq, d); K64/V64: (B, Hkv, L, d)."""
    B, T, Hq, d = q16.shape
    L = K64.shape[2]
    gs = Hq // Hkv
    q = torch.from_numpy(q16.astype(np.float64)).permute(0, 2, 1, 3)
    k = torch.from_numpy(K64).repeat_interleave(gs, dim=1)
    v = torch.from_numpy(V64).repeat_interleave(gs, dim=1)
    pos = L - T + torch.arange(T)
    mask = torch.arange(L)[None, :] <= pos[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=mask, scale=sm_scale)
    logits = (q @ k.transpose(-1, -2)) * sm_scale
    lse = torch.logsumexp(logits.masked_fill(~mask, -torch.inf), dim=-1)
    return o.permute(0, 2, 1, 3).numpy(), lse.numpy()


def test_all_residual_equals_sdpa():
    """L <= R: nothing is quantized, so the result is plain softmax
    attention over the fp16 K/V."""
    B, H, Hq, d, L, T = 2, 2, 8, 64, 40, 5
    rep, K, V = _build(B, H, d, 32, 32, 8, 64, L)
    assert rep.n_q == 0
    q = np.random.default_rng(1).standard_normal((B, T, Hq, d)).astype(np.float16)
    out, lse = attention.attend(rep, q, "target", 0.125)
    Kt = np.transpose(K, (0, 2, 1, 3)).astype(np.float64)
    Vt = np.transpose(V, (0, 2, 1, 3)).astype(np.float64)
    ref, ref_lse = _sdpa(q, Kt, Vt, H, 0.125)
    assert np.abs(out - ref).max() < 1e-12
    assert np.abs(lse - ref_lse).max() < 1e-12


@pytest.mark.parametrize("path,bits", [("target", 8), ("draft4", 8),
                                       ("target", 2), ("target", 1)])
def test_quantized_equals_sdpa_on_dequantized(path, bits):
    B, H, Hq, d, G, Gv, R, L, T = 1, 2, 4, 128, 32, 32, 32, 300, 3
    rep, K, V = _build(B, H, d, G, Gv, bits, R, L, seed=2)
    deq = quant.dequant if path == "target" else quant.dequant_draft4
    K64 = np.empty((B, H, L, d))
    V64 = np.empty((B, H, L, d))
    for h in range(H):
        K64[0, h, :rep.n_q] = deq(rep.kq[0, h], rep.ks[0, h], rep.kz[0, h], "key", G)
        V64[0, h, :rep.n_q] = deq(rep.vq[0, h], rep.vs[0, h], rep.vz[0, h], "value", Gv)
        K64[0, h, rep.n_q:] = rep.rk[0, h]
        V64[0, h, rep.n_q:] = rep.rv[0, h]
    q = np.random.default_rng(3).standard_normal((B, T, Hq, d)).astype(np.float16)
    out, lse = attention.attend(rep, q, path, d ** -0.5)
    ref, ref_lse = _sdpa(q, K64, V64, H, d ** -0.5)
    assert np.abs(out - ref).max() < 1e-12
    assert np.abs(lse - ref_lse).max() < 1e-11


def test_verify_row_equals_prefix_decode():
    """Row t of a T-token verify equals a T=1 decode over the first
    L-T+t+1 tokens (causal among the speculative tokens)."""
    B, H, Hq, d, G, R, T = 1, 1, 2, 64, 32, 64, 4
    rng = np.random.default_rng(4)
    L = 200
    K = rng.standard_normal((B, L, H, d)).astype(np.float16)
    V = rng.standard_normal((B, L, H, d)).astype(np.float16)
    q = rng.standard_normal((B, T, Hq, d)).astype(np.float16)
    rep = cache.Replay(B, H, d, G, 32, 8, R)
    rep.append(K, V)
    full, _ = attention.attend(rep, q, "target", 0.1)
    for t in range(T):
        r = cache.Replay(B, H, d, G, 32, 8, R)
        r.append(K, V)
        r.rollback(T - 1 - t)        # drop the later speculative tokens
        one, _ = attention.attend(r, q[:, t:t + 1], "target", 0.1)
        assert np.abs(one[:, 0] - full[:, t]).max() < 1e-13


def test_gqa_equals_mha_with_repeated_heads():
    B, H, gs, d, G, R, L, T = 1, 2, 3, 64, 32, 32, 160, 2
    rng = np.random.default_rng(5)
    K = rng.standard_normal((B, L, H, d)).astype(np.float16)
    V = rng.standard_normal((B, L, H, d)).astype(np.float16)
    q = rng.standard_normal((B, T, H * gs, d)).astype(np.float16)
    gqa = cache.Replay(B, H, d, G, 32, 8, R)
    gqa.append(K, V)
    mha = cache.Replay(B, H * gs, d, G, 32, 8, R)
    mha.append(np.repeat(K, gs, axis=2), np.repeat(V, gs, axis=2))
    a, la = attention.attend(gqa, q, "target", 0.1)
    b, lb = attention.attend(mha, q, "target", 0.1)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_draft_ignores_low_nibbles():
    rep, _, _ = _build(1, 1, 64, 32, 32, 8, 32, 192, seed=6)
    q = np.random.default_rng(7).standard_normal((1, 1, 2, 64)).astype(np.float16)
    a, _ = attention.attend(rep, q, "draft4", 0.125)
    t, _ = attention.attend(rep, q, "target", 0.125)
    rep.kq = (rep.kq & 0xF0) | (~rep.kq & 0x0F)
    rep.vq = (rep.vq & 0xF0) | ((rep.vq * 7) & 0x0F)
    b, _ = attention.attend(rep, q, "draft4", 0.125)
    t2, _ = attention.attend(rep, q, "target", 0.125)
    assert np.array_equal(a, b)
    assert np.abs(t - t2).max() > 1e-4
