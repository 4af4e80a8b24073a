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


def test_exact_substitution_pins():
    """attend_exact: nothing selected == attend; every quantized token
    replaced by its original value == SDPA over the original tokens for the
    substituted row, other rows unchanged; a token replaced by its own
    dequantized value (an fp16 number here) changes nothing."""
    B, H, Hq, d, G, Gv, R, L, T = 1, 2, 8, 64, 32, 32, 32, 200, 2
    rep, K, V = _build(B, H, d, G, Gv, 2, R, L, seed=5)
    n_q = rep.n_q
    q = np.random.default_rng(6).standard_normal((B, T, Hq, d)).astype(np.float16)
    base, base_lse = attention.attend(rep, q, "target", 0.125)
    none = -np.ones((B, H, 3), np.int64)
    z = np.zeros((B, H, 3, d), np.float16)
    o, s = attention.attend_exact(rep, q, "target", 0.125, none, z, z)
    assert np.array_equal(o, base) and np.array_equal(s, base_lse)
    # every quantized token replaced by the original fp16 token
    idx = np.tile(np.arange(n_q), (B, H, 1))
    kx = np.transpose(K[:, :n_q], (0, 2, 1, 3))
    vx = np.transpose(V[:, :n_q], (0, 2, 1, 3))
    o, s = attention.attend_exact(rep, q, "target", 0.125, idx, kx, vx, t_exact=0)
    Kt = np.transpose(K, (0, 2, 1, 3)).astype(np.float64)
    Vt = np.transpose(V, (0, 2, 1, 3)).astype(np.float64)
    ref, ref_lse = _sdpa(q, Kt, Vt, H, 0.125)
    assert np.abs(o[:, 0] - ref[:, 0]).max() < 1e-12
    assert np.abs(s[:, :, 0] - ref_lse[:, :, 0]).max() < 1e-12
    assert np.array_equal(o[:, 1], base[:, 1]) and np.array_equal(s[:, :, 1], base_lse[:, :, 1])
    assert np.abs(o[:, 0] - base[:, 0]).max() > 1e-3     # 2-bit codes do differ
    # substituting a token by its own dequantized value: pick tokens whose
    # dequantized K and V rows are exactly fp16 numbers
    Kq = quant.dequant(rep.kq[0, 0], rep.ks[0, 0], rep.kz[0, 0], "key", G)
    Vq = quant.dequant(rep.vq[0, 0], rep.vs[0, 0], rep.vz[0, 0], "value", Gv)
    fits = [j for j in range(n_q)
            if (Kq[j].astype(np.float16).astype(np.float64) == Kq[j]).all()
            and (Vq[j].astype(np.float16).astype(np.float64) == Vq[j]).all()]
    assert len(fits) >= 1
    sel = np.array(fits[:4])
    idx1 = -np.ones((B, H, len(sel)), np.int64)
    idx1[0, 0] = sel
    k1 = np.zeros((B, H, len(sel), d), np.float16)
    v1 = np.zeros_like(k1)
    k1[0, 0] = Kq[sel].astype(np.float16)
    v1[0, 0] = Vq[sel].astype(np.float16)
    o, s = attention.attend_exact(rep, q, "target", 0.125, idx1, k1, v1)
    assert np.abs(o - base).max() < 1e-13 and np.abs(s - base_lse).max() < 1e-13
