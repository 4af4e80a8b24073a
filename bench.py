#!/usr/bin/env python3
"""Benchmark: speculative verify step over a 32K-context quantized KV cache.

Workload (one GPU): a Llama-3-8B-shaped GQA attention layer, B=1, Hq=32,
Hkv=8, d=128, context 32768, key groups G=128, value groups of 64 channels,
fp16 residual of R=256 tokens, INT8 codes in two nibble planes.  Synthetic
seeded K/V (N(0,1), 4 outlier key channels x10, per-token lognormal(0,0.5)
key drift), random queries.

One step = one pass of the hot path for a gamma = 6 speculative step:
  kv_quant_append  of the 7 new tokens (fp16 ring write; no flush is due)
  kv_attn_verify   INT4 draft attention, T=1 (upper nibble plane only)
  kv_attn_verify   INT8 target verify attention, T=7 (causal among the 7)
  kv_rollback      of the 7 tokens (host counters; the next step reuses them)
The layer's cache has 8 copies (0.57 GB), standing for 8 layers of a model.
Step i appends to and drafts on copy i mod 8, and verifies and rolls back
copy (i - 4) mod 8, whose draft ran 4 steps earlier: as in a model, where
the draft pass over every layer runs between a layer's draft and its
verify, neither attention call finds its cache in the 256 MB Infinity Cache
(about 430 MB of other copies are read in between).  A verify timed right
after the draft on the same copy (warm) is reported beside it.

The JSON line reports us/step (wall clock over the timed steps), the
dominant kernel's duration (HIP events on its stream) against the HBM
roofline, and the CPU oracle timed on the host on one full step.  Beside the
step ("comparators", not part of the step's value): the same attention with
the whole context in the fp16 residual buffer (the FP16 comparator), and
kv_dequant_gather of 64 positions per kv head.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np

METRIC = ("verify-attention µs/step and achieved HBM GB/s (% peak), "
          "32K ctx INT4/INT8")
PEAK_GBPS = 8000.0
WORKLOAD = "llama3_8b_32k"
T_VERIFY, T_DRAFT = 7, 1
N_COPIES = 8
LAG = N_COPIES // 2          # a copy's verify runs LAG steps after its draft


def algorithmic_bytes(Hkv, Hq, d, G, Gv, n_q, n_r, T, bits_read):
    """Bytes one attention launch must move: codes at the bits the path
    reads per element of K and V, fp16 scale/zero amortized per group,
    fp16 residual K and V, fp16 q and out."""
    per_tok = 2 * d * bits_read // 8 + 4 * d // G + 4 * (d // Gv)
    return Hkv * (n_q * per_tok + n_r * 4 * d) + 2 * T * Hq * d * 2


def build_caches(w, seed, device):
    """N_COPIES device caches holding the first L-7 tokens, the host fp16
    token streams (B, L, Hkv, d) they were built from, and the HIP-event
    time (us) of the bulk quantize-on-append that filled the first cache."""
    import torch
    import kvq_synth as synth
    import quantized_kv_attention_quant_amd as kq
    K = np.empty((w.B, w.L, w.Hkv, w.d), np.float16)
    V = np.empty_like(K)
    for b in range(w.B):
        for h in range(w.Hkv):
            K[b, :, h], V[b, :, h] = synth.kv_block(w, seed, b, h, w.L)
    L0 = w.L - T_VERIFY
    shape = kq.Shape(B=w.B, Hkv=w.Hkv, d=w.d, G=w.G, Gv=w.Gv, bits=w.bits,
                     R=w.R, L_max=w.L, max_append=32)
    base = kq.QuantKVCache(shape, device=device)
    kd = torch.from_numpy(np.ascontiguousarray(K[:, :L0])).to(device)
    vd = torch.from_numpy(np.ascontiguousarray(V[:, :L0])).to(device)
    stream = torch.cuda.current_stream()
    # an untimed append first: the first launch also loads the code object
    scratch = kq.QuantKVCache(shape, device=device)
    scratch.append(kd[:, :2 * w.G].contiguous(), vd[:, :2 * w.G].contiguous())
    # bulk quantize-on-append of the prefix, timed as 6 back-to-back fills of
    # a scratch cache (kv_cache_layout empties it): after the first, the host
    # launch latency hides behind the previous fill; median of the last 5
    torch.cuda.synchronize()
    evs = []
    for _ in range(6):
        kq.kv_cache_layout(scratch.c)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        kq.kv_quant_append(scratch.c, kd, vd, L0, stream.cuda_stream)
        e[1].record(stream)
        evs.append(e)
    torch.cuda.synchronize()
    prefill_us = float(np.median([e[0].elapsed_time(e[1]) * 1e3
                                  for e in evs[1:]]))
    del scratch
    base.append(kd, vd)                  # the prefix of the timed caches
    torch.cuda.synchronize()
    del kd, vd
    caches = [base] + [base.clone() for _ in range(N_COPIES - 1)]
    torch.cuda.synchronize()
    return caches, K, V, prefill_us


def _oracle_steps(args):
    """One worker of the CPU baseline: replay the prefix of kv heads
    [h0, h1) (untimed), then run full steps on them until `budget_s` of
    wall time has passed.  Returns (steps, seconds)."""
    w, K, V, q_draft, q_verify, k_new, v_new, h0, h1, budget_s = args
    from threadpoolctl import threadpool_limits
    from oracle import attention as oatt
    from oracle import cache as ocache
    gs = w.Hq // w.Hkv
    qd = np.ascontiguousarray(q_draft[:, :, h0 * gs:h1 * gs])
    qv = np.ascontiguousarray(q_verify[:, :, h0 * gs:h1 * gs])
    with threadpool_limits(limits=1):
        rep = ocache.Replay(w.B, h1 - h0, w.d, w.G, w.Gv, w.bits, w.R)
        rep.append(np.ascontiguousarray(K[:, :, h0:h1]),
                   np.ascontiguousarray(V[:, :, h0:h1]))
        kn = np.ascontiguousarray(k_new[:, :, h0:h1])
        vn = np.ascontiguousarray(v_new[:, :, h0:h1])
        steps, t0 = 0, time.perf_counter()
        while True:
            rep.append(kn, vn)
            oatt.attend(rep, qd, "draft4", w.d ** -0.5)
            oatt.attend(rep, qv, "target", w.d ** -0.5)
            rep.rollback(T_VERIFY)
            steps += 1
            dt = time.perf_counter() - t0
            if dt >= budget_s:
                return steps, dt


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, seed, K, V, q_draft, q_verify, k_new, v_new,
                 budget_s=10.0):
    """Time the CPU oracle on full steps (append the 7 tokens to the
    replayed cache, draft + verify attention in float64, rollback) on the
    host's cores: the 8 kv-head blocks are independent, so P worker
    processes (P = the cores this process may run on, at most one per kv
    head and at most 16) each take Hkv/P heads and run steps for
    ~budget_s; a step takes the slowest worker's time per step.  The
    oracle's numpy code is unchanged (one BLAS thread per worker).  The
    replay of the 32K-token prefix is set-up, not timed."""
    import multiprocessing as mp
    visible = len(os.sched_getaffinity(0))
    P = max(1, min(visible, 16, w.Hkv))
    while w.Hkv % P:
        P -= 1
    per = w.Hkv // P
    jobs = [(w, K, V, q_draft, q_verify, k_new, v_new, i * per, (i + 1) * per,
             budget_s) for i in range(P)]
    with mp.get_context("spawn").Pool(P) as pool:
        res = pool.map(_oracle_steps, jobs)
    per_step = max(dt / n for n, dt in res)
    steps = min(n for n, _ in res)
    return {"value": round(per_step * 1e6, 1), "unit": "us/step",
            "cores": P, "kind": "oracle",
            "cpu_model": _cpu_model(), "host_cpus_visible": visible,
            "sample": f"{steps}+ full steps per worker (append 7, INT4 draft "
                      "T=1, INT8 verify T=7, rollback 7) over the 32K cache, "
                      f"{P} worker processes of {per} kv head(s) each, "
                      "float64 numpy, one BLAS thread per worker; prefix "
                      "replay untimed"}


def traffic_from_profile():
    """HBM bytes per verify launch from the committed rocprofv3 counter
    summary, or None when the attention source changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic_verify_int8_t7_llama3_32k.json")
    src = os.path.join(ROOT, "quantized_kv_attention_quant_amd", "csrc",
                       "kvq_attn.hip")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        prof = json.load(f)
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if prof.get("kvq_attn_sha256") != sha:
        return None
    return prof["hbm_bytes_per_launch"]


def calibrate_copy(nbytes=256 << 20, reps=3):
    """A plain device copy of known size, for scaling FETCH_SIZE/WRITE_SIZE
    in a profiled run (it shows up as its own kernel)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").random_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()


def comparators(w, seed, K, V, caches, q_draft, q_verify, k_new, v_new,
                steps=50):
    """Two side measurements on the same workload (not part of the step):
      fp16 comparator: the same attention with the whole 32K context in the
        fp16 residual buffer (no quantized prefix), T=7 and T=1, against the
        INT8 / INT4 paths over the quantized cache;
      on-demand reconstruction: kv_dequant_gather of 64 positions per kv
        head (a top-k fetch), target path, on the quantized cache copies.
    Both use HIP events on the launch stream; each call reads a different
    cache copy, as in the step."""
    import torch
    import quantized_kv_attention_quant_amd as kq
    dev = q_draft.device
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    L0 = w.L - T_VERIFY
    shape = kq.Shape(B=w.B, Hkv=w.Hkv, d=w.d, G=w.G, Gv=w.Gv, bits=w.bits,
                     R=w.L, L_max=w.G, max_append=32)
    base = kq.QuantKVCache(shape, device=dev)
    base.append(torch.from_numpy(np.ascontiguousarray(K[:, :L0])).to(dev),
                torch.from_numpy(np.ascontiguousarray(V[:, :L0])).to(dev))
    n_fp16 = 4                                   # 4 x 134 MB > Infinity Cache
    fcs = [base] + [base.clone() for _ in range(n_fp16 - 1)]
    assert base.n_q == 0 and base.n_r == L0
    sm = w.d ** -0.5
    ws = fcs[0].attn_workspace(T_VERIFY, w.Hq)
    out_v, out_d = torch.empty_like(q_verify), torch.empty_like(q_draft)

    def timed(fn, n):
        ts = []
        for i in range(n + 5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn(i)
            e1.record(stream)
            ts.append((e0, e1))
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in ts[5:]]) * 1e3

    # time only the attention: record around the verify call
    def fp16_attn(T, q, out):
        ts = []
        for i in range(steps + 5):
            c = fcs[i % n_fp16]
            kq.kv_quant_append(c.c, k_new, v_new, T_VERIFY, sh)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            kq.kv_attn_verify(c.c, q, T, w.Hq, kq.KVQ_TARGET, sm, out, None, ws, sh)
            e1.record(stream)
            kq.kv_rollback(c.c, T_VERIFY)
            ts.append((e0, e1))
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in ts[5:]]) * 1e3

    f7 = fp16_attn(T_VERIFY, q_verify, out_v)
    f1 = fp16_attn(T_DRAFT, q_draft, out_d)
    bytes_f7 = algorithmic_bytes(w.Hkv, w.Hq, w.d, w.G, w.Gv, 0, w.L, T_VERIFY, 8)
    bytes_f1 = algorithmic_bytes(w.Hkv, w.Hq, w.d, w.G, w.Gv, 0, w.L, T_DRAFT, 8)
    del fcs, base
    torch.cuda.empty_cache()

    rng = np.random.default_rng(seed + 7)
    n_g = 64
    idx = torch.from_numpy(rng.integers(0, w.L, (w.B, w.Hkv, n_g)).astype(np.int32)).to(dev)
    k_out = torch.empty((w.B, w.Hkv, n_g, w.d), dtype=torch.float16, device=dev)
    v_out = torch.empty_like(k_out)
    for c in caches:
        kq.kv_quant_append(c.c, k_new, v_new, T_VERIFY, sh)
    g = timed(lambda i: kq.kv_dequant_gather(caches[i % N_COPIES].c, idx, n_g,
                                             kq.KVQ_TARGET, k_out, v_out, sh),
              steps)
    for c in caches:
        kq.kv_rollback(c.c, T_VERIFY)
    torch.cuda.synchronize()
    return {
        "fp16_verify_t7_us": round(float(np.median(f7)), 3),
        "fp16_decode_t1_us": round(float(np.median(f1)), 3),
        "fp16_verify_t7_gbps": round(bytes_f7 / (f7.mean() * 1e-6) / 1e9, 1),
        "fp16_decode_t1_gbps": round(bytes_f1 / (f1.mean() * 1e-6) / 1e9, 1),
        "gather_64_per_head_us": round(float(np.median(g)), 3),
    }


def specache_pipeline(seed, name="specache_2bit", steps=30):
    """The SpeCache-style prefetch path at the batched 32K 1-bit or 2-bit
    size (B=36, Hq=32, Hkv=8, d=128, G=Gv=R=32, T=2: output token +
    speculative token):
      kv_topk           top-64 positions per kv head from the speculative
                        token's 2-bit scores
      kv_fetch_rows     those rows' fp16 K and V from a pinned host copy
      kv_attn_verify_exact  T=2 with the output token reading them exactly
    beside plain kv_attn_verify on the same cache.  K/V are a seeded device
    draw (only shapes matter for the timing); HIP events on the launch
    stream, each call timed alone."""
    import torch
    import kvq_synth as synth
    import quantized_kv_attention_quant_amd as kq
    w = synth.WORKLOADS[name]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    g = torch.Generator(device=dev)
    g.manual_seed(seed + 11)
    shape = kq.Shape(B=w.B, Hkv=w.Hkv, d=w.d, G=w.G, Gv=w.Gv, bits=w.bits,
                     R=w.R, L_max=w.L, max_append=32)
    cache = kq.QuantKVCache(shape, device=dev)
    mirror = kq.HostMirror(shape, w.L)
    T = 2
    for lo, hi in ((0, w.L - T), (w.L - T, w.L)):
        K = torch.randn((w.B, hi - lo, w.Hkv, w.d), generator=g, device=dev).half()
        V = torch.randn((w.B, hi - lo, w.Hkv, w.d), generator=g, device=dev).half()
        cache.append(K, V)
        mirror.k[:, :, lo:hi].copy_(K.permute(0, 2, 1, 3).cpu())
        mirror.v[:, :, lo:hi].copy_(V.permute(0, 2, 1, 3).cpu())
        del K, V
    q = torch.from_numpy(synth.queries(w, seed + 3, T)).to(dev)
    q_spec = q[:, T - 1].contiguous()
    k = w.topk
    idx = torch.empty((w.B, w.Hkv, k), dtype=torch.int32, device=dev)
    kx = torch.empty((w.B, w.Hkv, k, w.d), dtype=torch.float16, device=dev)
    vx = torch.empty_like(kx)
    out = torch.empty_like(q)
    tws = cache.topk_workspace(w.Hq, k)
    aws = cache.attn_workspace(T, w.Hq)
    torch.cuda.synchronize()
    calls = {
        "topk": lambda: cache.topk(q_spec, k, idx=idx, ws=tws),
        "fetch": lambda: mirror.fetch(cache, idx, kx, vx),
        "verify_exact": lambda: cache.verify_exact(q, idx, kx, vx, t_exact=0,
                                                   out=out, ws=aws),
        "verify": lambda: cache.verify(q, out=out, ws=aws),
    }
    ts = {name: [] for name in calls}
    for i in range(steps + 3):
        for name, fn in calls.items():
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            if i >= 3:
                ts[name].append((e0, e1))
    torch.cuda.synchronize()
    us = {n: float(np.median([a.elapsed_time(b) for a, b in v])) * 1e3
          for n, v in ts.items()}
    fetch_bytes = 2 * w.B * w.Hkv * k * w.d * 2

    # A contiguous host -> device copy of as many bytes as the fetch moves
    # (the page's sparse-vs-full transfer comparison).
    flat = mirror.k.view(-1)[:fetch_bytes // 2]
    dst = torch.empty(fetch_bytes // 2, dtype=torch.float16, device=dev)
    cts = []
    for i in range(steps + 3):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dst.copy_(flat, non_blocking=True)
        e1.record(stream)
        if i >= 3:
            cts.append((e0, e1))
    torch.cuda.synchronize()
    contig_us = float(np.median([a.elapsed_time(b) for a, b in cts])) * 1e3

    # Pipelined steps: step i's output token attends with the rows fetched
    # for step i-1's top-k; step i's top-k then starts the next fetch on a
    # second stream (default priority), which runs while step i+1's mask and
    # split pass do: only the exact-term kernel waits for it (rows_ready).
    copy = torch.cuda.Stream(device=dev)
    idxs = [torch.empty_like(idx) for _ in range(2)]
    kxs = [torch.empty_like(kx) for _ in range(2)]
    vxs = [torch.empty_like(vx) for _ in range(2)]
    e_topk = [torch.cuda.Event() for _ in range(2)]
    e_fetch = [torch.cuda.Event() for _ in range(2)]

    def start_fetch(cur):
        cache.topk(q_spec, k, idx=idxs[cur], ws=tws)
        e_topk[cur].record(stream)
        copy.wait_event(e_topk[cur])
        mirror.fetch(cache, idxs[cur], kxs[cur], vxs[cur], stream=copy)
        e_fetch[cur].record(copy)

    def pipe_step(i):
        prev = (i - 1) % 2
        cache.verify_exact(q, idxs[prev], kxs[prev], vxs[prev], t_exact=0,
                           out=out, ws=aws, rows_ready=e_fetch[prev])
        start_fetch(i % 2)

    start_fetch(1)                       # the step before the first
    for i in range(3):
        pipe_step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(3, 3 + steps):
        pipe_step(i)
    stream.wait_event(e_fetch[(2 + steps) % 2])
    e1.record(stream)
    torch.cuda.synchronize()
    overlapped_us = e0.elapsed_time(e1) * 1e3 / steps
    verify_bytes = w.B * algorithmic_bytes(w.Hkv, w.Hq, w.d, w.G, w.Gv,
                                           cache.n_q, cache.n_r, T, w.bits)
    res = {
        "workload": f"SpeCache-style batched {w.bits}-bit cache: B=36 Hq=32 "
                    "Hkv=8 d=128 L=32768 G=Gv=R=32, T=2, top-64 per kv head",
        "topk_us": round(us["topk"], 3),
        "fetch_us": round(us["fetch"], 3),
        "fetch_host_gbps": round(fetch_bytes / (us["fetch"] * 1e-6) / 1e9, 2),
        "verify_exact_us": round(us["verify_exact"], 3),
        "verify_us": round(us["verify"], 3),
        "verify_gbps": round(verify_bytes / (us["verify"] * 1e-6) / 1e9, 1),
        "pipeline_us": round(us["topk"] + us["fetch"] + us["verify_exact"], 3),
        "pipeline_overlapped_us": round(overlapped_us, 3),
        "contiguous_copy_us": round(contig_us, 3),
        "sparse_vs_contiguous_time": round(us["fetch"] / contig_us, 2),
    }
    del cache, mirror
    torch.cuda.empty_cache()
    return res


def lwm_128k_steps(seed, steps=64):
    """The LWM-7B-shaped 128K layer (B=1, Hq=Hkv=32, d=128, G=128, Gv=64,
    R=256, INT8) as a speculative state machine: from a prefill of
    L - 4*steps tokens, `steps` steps of {append 6, INT8 verify T=6,
    rollback 2}, which end at L = 131072 and cross flushes of G=128 tokens
    (an append that pushes the residual past R quantizes its oldest group);
    then an INT4 draft at T=1 on the full cache.  K/V are a seeded
    device draw (only shapes matter for the timing); HIP events around each
    call."""
    import torch
    import kvq_synth as synth
    import quantized_kv_attention_quant_amd as kq
    w = synth.WORKLOADS["lwm_7b_128k"]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    g = torch.Generator(device=dev)
    g.manual_seed(seed + 13)
    shape = kq.Shape(B=w.B, Hkv=w.Hkv, d=w.d, G=w.G, Gv=w.Gv, bits=w.bits,
                     R=w.R, L_max=w.L, max_append=32)
    cache = kq.QuantKVCache(shape, device=dev)
    p0 = w.L - 4 * steps
    K = torch.randn((w.B, p0, w.Hkv, w.d), generator=g, device=dev).half()
    V = torch.randn((w.B, p0, w.Hkv, w.d), generator=g, device=dev).half()
    cache.append(K, V)
    del K, V
    kn = torch.randn((steps, w.B, 6, w.Hkv, w.d), generator=g, device=dev).half()
    vn = torch.randn((steps, w.B, 6, w.Hkv, w.d), generator=g, device=dev).half()
    q6 = torch.from_numpy(synth.queries(w, seed + 5, 6)).to(dev)
    q1 = torch.from_numpy(synth.queries(w, seed + 6, 1)).to(dev)
    out6, out1 = torch.empty_like(q6), torch.empty_like(q1)
    ws = cache.attn_workspace(6, w.Hq)
    sm = w.d ** -0.5
    torch.cuda.synchronize()
    rec = []
    for i in range(steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        nq0 = cache.n_q
        e[0].record(stream)
        kq.kv_quant_append(cache.c, kn[i], vn[i], 6, sh)
        e[1].record(stream)
        kq.kv_attn_verify(cache.c, q6, 6, w.Hq, kq.KVQ_TARGET, sm, out6, None,
                          ws, sh)
        e[2].record(stream)
        rec.append((e, cache.n_q > nq0, cache.n_q, cache.n_r))
        cache.rollback(2)
    assert cache.n_q + cache.n_r == w.L
    d1 = []
    for i in range(20):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        kq.kv_attn_verify(cache.c, q1, 1, w.Hq, kq.KVQ_DRAFT4, sm, out1, None,
                          ws, sh)
        e[1].record(stream)
        d1.append(e)
    # the INT8 verify at T = 1..6 on the full cache (the T query tokens are
    # the last T of the residual; 1.1 GB per call, more than the Infinity
    # Cache, so every call is cold)
    sweep = {}
    for T in range(1, 7):
        qT = torch.from_numpy(synth.queries(w, seed + 20 + T, T)).to(dev)
        oT = torch.empty_like(qT)
        ev = []
        for i in range(12):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(stream)
            kq.kv_attn_verify(cache.c, qT, T, w.Hq, kq.KVQ_TARGET, sm, oT,
                              None, ws, sh)
            e[1].record(stream)
            if i >= 2:
                ev.append(e)
        sweep[T] = ev
    torch.cuda.synchronize()
    app = [(e[0].elapsed_time(e[1]) * 1e3, fl) for e, fl, _, _ in rec]
    ver = [e[1].elapsed_time(e[2]) * 1e3 for e, _, _, _ in rec]
    # the verify's algorithmic bytes at each step's fill level
    vb = [algorithmic_bytes(w.Hkv, w.Hq, w.d, w.G, w.Gv, nq, nr, 6, 8)
          for _, _, nq, nr in rec]
    draft_us = float(np.median([e[0].elapsed_time(e[1]) * 1e3 for e in d1]))
    draft_bytes = algorithmic_bytes(w.Hkv, w.Hq, w.d, w.G, w.Gv, cache.n_q,
                                    cache.n_r, 1, 4)
    flush = [a for a, fl in app if fl]
    sweep_us = {T: float(np.median([e[0].elapsed_time(e[1]) * 1e3 for e in ev]))
                for T, ev in sweep.items()}
    res = {
        "workload": "LWM-7B-shaped 128K layer: B=1 Hq=Hkv=32 d=128 "
                    "L=131072 G=128 Gv=64 R=256 INT8; steps of append 6 / "
                    "verify T=6 / rollback 2",
        "steps": steps,
        "flushes": len(flush),
        "append6_us": round(float(np.median([a for a, fl in app if not fl])), 3),
        "append6_flush_us": round(float(np.median(flush)), 3) if flush else None,
        "verify_int8_t6_us": round(float(np.median(ver)), 3),
        "verify_int8_t6_gbps": round(float(np.mean(vb)) / (float(np.mean(ver)) * 1e-6) / 1e9, 1),
        "draft_int4_t1_us": round(draft_us, 3),
        "draft_int4_t1_gbps": round(draft_bytes / (draft_us * 1e-6) / 1e9, 1),
        "verify_int8_by_T_us": {str(T): round(u, 3) for T, u in sweep_us.items()},
        "verify_int8_by_T_gbps": {
            str(T): round(algorithmic_bytes(w.Hkv, w.Hq, w.d, w.G, w.Gv,
                                            cache.n_q, cache.n_r, T, 8)
                          / (u * 1e-6) / 1e9, 1) for T, u in sweep_us.items()},
    }
    del cache, kn, vn
    torch.cuda.empty_cache()
    return res


def llama2_8k(seed, steps=50):
    """The Llama-2-7B-shaped 8K layer (B=1, Hq=Hkv=32, d=128, G=128, Gv=64,
    R=256, INT8): INT8 verify at T=9 and INT4 draft at T=1, each call on one
    of 4 cache copies (4 x 72 MB, more than the Infinity Cache) appended
    with the T query tokens and rolled back after.  K/V are a seeded device
    draw; HIP events around each attention call."""
    import torch
    import kvq_synth as synth
    import quantized_kv_attention_quant_amd as kq
    w = synth.WORKLOADS["llama2_7b_8k"]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    g = torch.Generator(device=dev)
    g.manual_seed(seed + 17)
    T = 9
    shape = kq.Shape(B=w.B, Hkv=w.Hkv, d=w.d, G=w.G, Gv=w.Gv, bits=w.bits,
                     R=w.R, L_max=w.L, max_append=32)
    base = kq.QuantKVCache(shape, device=dev)
    K = torch.randn((w.B, w.L - T, w.Hkv, w.d), generator=g, device=dev).half()
    V = torch.randn((w.B, w.L - T, w.Hkv, w.d), generator=g, device=dev).half()
    base.append(K, V)
    del K, V
    caches = [base] + [base.clone() for _ in range(3)]
    kn = torch.randn((w.B, T, w.Hkv, w.d), generator=g, device=dev).half()
    vn = torch.randn((w.B, T, w.Hkv, w.d), generator=g, device=dev).half()
    q9 = torch.from_numpy(synth.queries(w, seed + 7, T)).to(dev)
    q1 = torch.from_numpy(synth.queries(w, seed + 8, 1)).to(dev)
    out9, out1 = torch.empty_like(q9), torch.empty_like(q1)
    ws = base.attn_workspace(T, w.Hq)
    sm = w.d ** -0.5

    def run(path, TT, q, out):
        ts = []
        for i in range(steps + 5):
            c = caches[i % 4]
            kq.kv_quant_append(c.c, kn, vn, T, sh)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            kq.kv_attn_verify(c.c, q, TT, w.Hq, path, sm, out, None, ws, sh)
            e1.record(stream)
            kq.kv_rollback(c.c, T)
            if i >= 5:
                ts.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ts])) * 1e3

    v_us = run(kq.KVQ_TARGET, T, q9, out9)
    d_us = run(kq.KVQ_DRAFT4, 1, q1, out1)
    n_q, n_r = base.n_q, base.n_r + T
    vb = algorithmic_bytes(w.Hkv, w.Hq, w.d, w.G, w.Gv, n_q, n_r, T, 8)
    db = algorithmic_bytes(w.Hkv, w.Hq, w.d, w.G, w.Gv, n_q, n_r, 1, 4)
    del caches, base
    torch.cuda.empty_cache()
    return {
        "workload": "Llama-2-7B-shaped 8K layer: B=1 Hq=Hkv=32 d=128 L=8192 "
                    "G=128 Gv=64 R=256 INT8",
        "verify_int8_t9_us": round(v_us, 3),
        "verify_int8_t9_gbps": round(vb / (v_us * 1e-6) / 1e9, 1),
        "draft_int4_t1_us": round(d_us, 3),
        "draft_int4_t1_gbps": round(db / (d_us * 1e-6) / 1e9, 1),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-comparators", action="store_true",
                    help="skip the side measurements (fp16 comparator, "
                         "gather, prefetch pipeline, 128K and 8K layers)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 256 MiB device copy (profiling scale)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the verify path shards by kv head "
              "with no communication, so --gpus above 1 is not run here",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import kvq_synth as synth
    import quantized_kv_attention_quant_amd as kq

    kq.lib()   # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[WORKLOAD]
    caches, K, V, prefill_us = build_caches(w, args.seed, dev)
    L0 = w.L - T_VERIFY
    Kn = np.ascontiguousarray(K[:, L0:])       # the 7 speculative tokens
    Vn = np.ascontiguousarray(V[:, L0:])
    qd16 = synth.queries(w, args.seed, T_DRAFT)
    qv16 = synth.queries(w, args.seed + 1, T_VERIFY)
    k_new, v_new = torch.from_numpy(Kn).to(dev), torch.from_numpy(Vn).to(dev)
    q_draft, q_verify = torch.from_numpy(qd16).to(dev), torch.from_numpy(qv16).to(dev)
    out_d = torch.empty_like(q_draft)
    out_v = torch.empty_like(q_verify)
    ws = caches[0].attn_workspace(T_VERIFY, w.Hq)   # large enough for both
    assert ws.numel() >= kq.kv_attn_workspace_bytes(caches[0].c, T_DRAFT, w.Hq)
    sm = w.d ** -0.5
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    n_q, n_r = caches[0].n_q, caches[0].n_r + T_VERIFY
    bytes_draft = algorithmic_bytes(w.Hkv, w.Hq, w.d, w.G, w.Gv, n_q, n_r,
                                    T_DRAFT, 4)
    bytes_verify = algorithmic_bytes(w.Hkv, w.Hq, w.d, w.G, w.Gv, n_q, n_r,
                                     T_VERIFY, 8)
    bytes_append = 2 * 2 * T_VERIFY * w.B * w.Hkv * w.d * 2
    # bulk prefill: read the fp16 K and V of the prefix, write the codes and
    # scale/zero of the quantized part and the fp16 ring of the rest
    per_tok_q = 2 * w.d * (8 if w.bits == 8 else w.bits) // 8 + 4 * w.d // w.G \
        + 4 * (w.d // w.Gv)
    bytes_prefill = w.B * w.Hkv * (L0 * 4 * w.d + n_q * per_tok_q
                                   + (L0 - n_q) * 4 * w.d)

    events = []

    def prime(i):
        kq.kv_quant_append(caches[i % N_COPIES].c, k_new, v_new, T_VERIFY, sh)

    def step(i, timed):
        a = caches[i % N_COPIES]            # append + draft
        b = caches[(i - LAG) % N_COPIES]    # verify + rollback (drafted LAG steps ago)
        if timed:
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            e[0].record(stream)
        kq.kv_quant_append(a.c, k_new, v_new, T_VERIFY, sh)
        if timed:
            e[1].record(stream)
        kq.kv_attn_verify(a.c, q_draft, T_DRAFT, w.Hq, kq.KVQ_DRAFT4, sm,
                          out_d, None, ws, sh)
        if timed:
            e[2].record(stream)
        kq.kv_attn_verify(b.c, q_verify, T_VERIFY, w.Hq, kq.KVQ_TARGET, sm,
                          out_v, None, ws, sh)
        if timed:
            e[3].record(stream)
            events.append(e)
        kq.kv_rollback(b.c, T_VERIFY)

    # prime the pipeline: the LAG copies before step 0 hold their appended
    # tokens (their drafts belong to the untimed prefix)
    for i in range(-LAG, 0):
        prime(i)
    i = 0
    for _ in range(args.warmup):
        step(i, False)
        i += 1
    torch.cuda.synchronize()
    # 1) wall clock over K plain steps (no events in the stream)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(i, False)
        i += 1
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    # 2) the same steps with per-kernel HIP events on the launch stream
    for _ in range(args.steps):
        step(i, True)
        i += 1
    torch.cuda.synchronize()
    # drain: verify and roll back the copies still holding appended tokens
    for j in range(i - LAG, i):
        kq.kv_rollback(caches[j % N_COPIES].c, T_VERIFY)
    app = np.array([e[0].elapsed_time(e[1]) for e in events]) * 1e3
    drf = np.array([e[1].elapsed_time(e[2]) for e in events]) * 1e3
    ver = np.array([e[2].elapsed_time(e[3]) for e in events]) * 1e3
    gpu_step = app + drf + ver
    # 3) warm verify, for comparison only: right after the draft on the same
    # copy, which has just read 37.5 MB of the verify's 70.9 MB
    warm = []
    for j in range(60):
        c = caches[j % N_COPIES]
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        kq.kv_quant_append(c.c, k_new, v_new, T_VERIFY, sh)
        kq.kv_attn_verify(c.c, q_draft, T_DRAFT, w.Hq, kq.KVQ_DRAFT4, sm,
                          out_d, None, ws, sh)
        e[0].record(stream)
        kq.kv_attn_verify(c.c, q_verify, T_VERIFY, w.Hq, kq.KVQ_TARGET, sm,
                          out_v, None, ws, sh)
        e[1].record(stream)
        kq.kv_rollback(c.c, T_VERIFY)
        if j >= 10:
            warm.append(e)
    torch.cuda.synchronize()
    ver_warm = np.array([e[0].elapsed_time(e[1]) for e in warm]) * 1e3

    achieved = bytes_verify / (ver.mean() * 1e-6) / 1e9
    res = {
        "metric": METRIC,
        "value": round(wall * 1e6, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "Llama-3-8B GQA layer at 32K: B=1 Hq=32 Hkv=8 d=128 "
                        "L=32768 G=128 Gv=64 R=256; INT4 draft T=1 + INT8 "
                        "verify T=7 + append/rollback of 7 tokens",
            "cache_copies": N_COPIES,
            "bytes_per_step": bytes_append + bytes_draft + bytes_verify,
        },
        "kernels_us": {
            "append_t7": round(float(np.median(app)), 3),
            "draft_int4_t1": round(float(np.median(drf)), 3),
            "verify_int8_t7": round(float(np.median(ver)), 3),
            "verify_int8_t7_p10_p90": [round(float(np.percentile(ver, 10)), 3),
                                       round(float(np.percentile(ver, 90)), 3)],
            "verify_int8_t7_warm": round(float(np.median(ver_warm)), 3),
            "gpu_step_events": round(float(gpu_step.mean()), 3),
            "prefill_32k": round(prefill_us, 3),
        },
        "hbm_gbps": {
            "draft_int4_t1": round(bytes_draft / (drf.mean() * 1e-6) / 1e9, 1),
            "verify_int8_t7": round(achieved, 1),
            "step_events": round((bytes_append + bytes_draft + bytes_verify)
                                 / (gpu_step.mean() * 1e-6) / 1e9, 1),
            "prefill_32k": round(bytes_prefill / (prefill_us * 1e-6) / 1e9, 1),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "kv_attn_verify INT8 T=7",
            "achieved": round(achieved, 1),
            "peak": PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_GBPS, 4),
            "traffic": traffic_from_profile(),
            "bytes_per_launch": bytes_verify,
        },
    }
    if not args.no_comparators:
        comp = comparators(w, args.seed, K, V, caches, q_draft, q_verify,
                           k_new, v_new)
        ku = res["kernels_us"]
        comp["int8_vs_fp16_speedup"] = round(comp["fp16_verify_t7_us"]
                                             / ku["verify_int8_t7"], 3)
        comp["int4_vs_fp16_speedup"] = round(comp["fp16_decode_t1_us"]
                                             / ku["draft_int4_t1"], 3)
        comp["specache_prefetch"] = specache_pipeline(args.seed, "specache_2bit")
        comp["specache_prefetch_1bit"] = specache_pipeline(args.seed, "specache_1bit")
        comp["lwm_128k"] = lwm_128k_steps(args.seed)
        comp["llama2_8k"] = llama2_8k(args.seed)
        res["comparators"] = comp
    if args.calibrate_copy:
        calibrate_copy()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(
            w, args.seed, np.ascontiguousarray(K[:, :L0]),
            np.ascontiguousarray(V[:, :L0]), qd16, qv16, Kn, Vn)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
