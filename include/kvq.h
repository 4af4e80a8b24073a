/*
 * kvq.h — C ABI of libkvq: decode/verify attention read directly from a
 * group-quantized KV cache, for one AMD MI355X (gfx950).
 *
 * The library implements the kernel-level hot path shared by three
 * KV-quantized speculative decoders described on public pages:
 *
 *   [QS]  "QuantSpec: Self-Speculative Decoding with Hierarchical Quantized
 *         KV Cache" (summary page).  Approach: the upper 4 bits of each code
 *         are the INT4 draft cache and upper+lower 4 bits rebuild the INT8
 *         target cache, so no second copy is stored; a double full-precision
 *         buffer of size 2G keeps recent tokens unquantized and avoids
 *         requantizing on rollback.  Measured-effects table, "INT4 attention
 *         kernel that loads the upper 4-bit KV cache" rows.  Experimental
 *         setup, "Builds on: FlashDecoding, KIVI".
 *   [SC]  "SpeCache: Speculative Key-Value Caching for Efficient Generation
 *         of LLMs" (summary page).  Approach: a low-bit (1/2-bit KIVI) copy
 *         of the KV cache stays on the GPU; a speculative token decoded
 *         alongside the output token scores that copy and its top-k KV pairs
 *         are the ones to prefetch.
 *   [MS]  "MSpecKV" (project page).  Abstract: KV-cache traffic dominates
 *         long-context decoding; offloaded KV is stored quantized and only
 *         the subsets that are needed are reconstructed on demand.
 *
 * Three entry points do the work: kv_quant_append (quantize-on-append),
 * kv_attn_verify (split-K attention over the quantized prefix plus the
 * fp16 residual buffer, merged by log-sum-exp) and kv_topk (per-kv-head
 * top-k over low-bit scores).  kv_dequant_gather rebuilds fp16 rows of a
 * requested token subset; kv_fetch_rows copies rows of a host-resident fp16
 * copy and kv_attn_verify_exact substitutes them for one query row.  The
 * rest is host-side bookkeeping.
 *
 * Conventions for every call
 *   - Ownership: the caller owns every buffer (host struct and device
 *     memory).  The library never allocates or frees memory.  Its only
 *     global state is the thread-local message of kv_last_error and, for
 *     kv_attn_verify_noalloc, a static device array on each GPU (32 MiB,
 *     held until the process ends) with its address looked up once per
 *     device.
 *   - Pointers named "device" are HIP device addresses; `stream` is a
 *     hipStream_t handle (NULL = the null stream).  All device work is
 *     enqueued on `stream` and is asynchronous to the host.
 *   - Return value: KVQ_OK (0) or a negative KVQ_E* code.  Arguments are
 *     validated before any HIP call; on error nothing is enqueued and the
 *     struct is unchanged.  No C++ exception crosses the ABI.
 *   - A kvq_cache must not be used by two host threads at once.
 *
 * Quantizer (KIVI-style asymmetric min/max, [SC] Approach "1-bit KIVI",
 * [QS] "Builds on: KIVI").  For one group x of fp16 values and b stored bits
 * (Lv = 2^b - 1):
 *     z = min(x)                                   (stored fp16, exact)
 *     s = fp16_rne( f32(f32(max x) - f32(min x)) / f32(Lv) )
 *     q = 0                                  if s == 0
 *       = clamp(rint_even( f32(f32(x) - f32(z)) / f32(s) ), 0, Lv)  otherwise
 *   every op is one IEEE binary32 operation (no fused multiply-add), the
 *   division is correctly rounded, rint_even rounds half to even, and the
 *   codes are computed against the stored (fp16-rounded) scale.
 *   Keys: one group per (channel, G consecutive tokens).  Values: one group
 *   per (token, Gv consecutive channels).
 *   Dequantized value: x^ = z + q*s.  INT4 draft view of an 8-bit code
 *   ([QS] Approach: the draft reads only the upper 4 bits): hi = q >> 4,
 *   x^4 = z + (16*hi + 7.5)*s, the centre of the 16 codes sharing hi.
 *   Inputs must be finite with (max-min)/Lv representable in fp16.
 *
 * Device layouts.  A "block" is one (b, kvh) pair; blocks are stored
 * b-major then kvh, each block at a fixed stride.  Bit packing is LSB-first.
 *   w = bits per code in a plane: 4 for bits==8 (two nibble planes: *_hi
 *       holds q>>4, *_lo holds q&15), 2 for bits==2, 1 for bits==1 (only a
 *       *_hi plane; *_lo must be NULL).
 *   K planes k_hi/k_lo: u8 [B][Hkv][L_max][d*w/8], token-major; channel c of
 *       a token sits in byte c/(8/w) at bit w*(c%(8/w)).
 *   K scale/zero k_sz: fp16 pairs [B][Hkv][L_max/G][d][2] = {s, z}.
 *   V planes v_hi/v_lo: u8 [B][Hkv][L_max/32][4*d*w], one 4*d*w-byte tile per
 *       32 consecutive tokens.  Token j (0..31) of a tile and channel c:
 *           g = (j%16)/4, i = j%4, h = j/16, r = c%16, m = c/16,
 *           per = 4/w, lane = 16*g + r,
 *           dword = lane*(d*w/64) + m/per,  bit = 16*h + w*(4*(m%per) + i)
 *       (dword = little-endian u32 index inside the tile).
 *   V scale/zero v_sz: fp16 [B][Hkv][L_max/32][2][4][4][d/Gv][2], per tile
 *       [part][g][i][group][h] with part 0 = scales, 1 = zero-points: the
 *       value of token j = 16*h + 4*g + i (h, g, i as above), so each u32
 *       holds one part of the token pair (4g+i, 16+4g+i) of one group.
 *   Residual ring: slot of absolute token position p is p % ring.
 *     k_res: fp16 [B][Hkv][ring][d], token-major.
 *     v_res: fp16 [B][Hkv][ring/32][32*d], one tile per 32 slots; slot j of
 *       a tile and channel c (g, i, h, r, m as above) sit at half index
 *           (16*g + r)*(d/2) + 8*m + 2*i + h.
 *   Supported shapes: see kv_cache_layout.
 *
 * Cache state.  Tokens 0..n_q-1 are quantized (n_q a multiple of G); tokens
 * n_q..n_q+n_r-1 are fp16 in the ring.  Appending then flushing follows the
 * [QS] double buffer: after an append, while n_r > R the oldest G residual
 * tokens are quantized as one key group (and G value groups).  Rollback only
 * shortens the residual ([QS] Approach: no requantization on rollback).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  KVQ_OK = 0,
  KVQ_EINVAL = -1,       /* bad argument or shape */
  KVQ_ECAPACITY = -2,    /* append would pass L_max quantized tokens */
  KVQ_EROLLBACK = -3,    /* rollback longer than the residual */
  KVQ_EWORKSPACE = -4,   /* workspace missing or too small */
  KVQ_EUNSUPPORTED = -5, /* valid request outside what the kernels cover */
  KVQ_EHIP = -6          /* a HIP launch failed */
};

enum {
  KVQ_TARGET = 0, /* attend over every stored bit of the codes */
  KVQ_DRAFT4 = 1  /* bits==8 only: attend over the upper nibble (x^4) */
};

typedef struct kvq_cache {
  /* Shape, filled by the caller before kv_cache_layout. */
  int32_t B, Hkv, d;
  int32_t G;          /* key group: tokens per (channel) scale/zero */
  int32_t Gv;         /* value group: channels per (token) scale/zero */
  int32_t bits;       /* 8, 2 or 1 */
  int32_t R;          /* residual capacity (flush threshold), tokens */
  int32_t L_max;      /* quantized-store capacity, tokens, multiple of G */
  int32_t max_append; /* largest append staged through the ring in one go */
  /* Derived by kv_cache_layout. */
  int32_t ring;          /* ring slots: multiple of 32, >= R + max_append */
  int64_t bytes_k_plane; /* bytes of k_hi (and of k_lo when bits == 8) */
  int64_t bytes_v_plane; /* bytes of v_hi (and of v_lo when bits == 8) */
  int64_t bytes_k_sz, bytes_v_sz, bytes_k_res, bytes_v_res;
  /* Host counters, maintained by the library. */
  int64_t n_q, n_r;
  /* Device buffers, allocated by the caller with the sizes above. */
  void *k_hi, *k_lo, *v_hi, *v_lo;
  void *k_sz, *v_sz;
  void *k_res, *v_res;
} kvq_cache;

/* Validate the shape, derive `ring` and the byte size of every buffer, and
 * set n_q = n_r = 0.  Host only.  Shape rules: B, Hkv >= 1; d in {64, 128};
 * bits in {8, 2, 1} (bits == 1 needs d == 128); G a positive multiple of
 * 32; L_max a positive multiple of G, at most 2^24; Gv a multiple of 16
 * dividing d with d/Gv <= 4; G <= R; 1 <= max_append.  The ring needs no
 * initial contents.  KVQ_EINVAL (message in kv_last_error) when a rule
 * fails. */
int kv_cache_layout(kvq_cache* c);

/* Quantize-on-append ([QS] Approach; quantizer and grouping as above).
 * k_new, v_new: device fp16 [B][n][Hkv][d] (token-major, as a model's
 * projection writes them).  Appends n >= 1 tokens to every block, then
 * quantizes f = max(0, ceil((n_r + n - R)/G)) groups of the oldest residual
 * tokens into the store, reading them from the ring or straight from
 * k_new/v_new (bulk prefill).  Counters are updated at enqueue time.
 * KVQ_ECAPACITY if n_q + f*G > L_max.  One launch when n_r + n <= ring,
 * otherwise two (flush, then ring write). */
int kv_quant_append(kvq_cache* c, const void* k_new, const void* v_new, int n,
                    void* stream);

/* Drop the m most recent tokens (rejected draft tokens): n_r -= m.  Never
 * touches quantized groups ([QS] Approach).  KVQ_EROLLBACK if m > n_r.
 * Host only. */
int kv_rollback(kvq_cache* c, int m);

/* Workspace bytes kv_attn_verify (and kv_attn_verify_exact) needs for this
 * cache at any fill level: one fp32 partial (m, l, o for up to 32 rows) per
 * split of every block, for as many splits as the launcher may choose on a
 * device with up to 512 resident workgroup slots (it uses fewer on larger
 * devices), plus one spare slot per block for the substitution partial,
 * then one bit per token slot (L_max/32 words per block) for the
 * substitution's mask of fetched positions.
 * 0 if the shape is invalid.  Host only. */
size_t kv_attn_workspace_bytes(const kvq_cache* c, int T, int Hq);

/* Speculative verify / draft attention ([QS] Approach; [SC] Approach for
 * T = 2 over a 1/2-bit cache; split-K with a log-sum-exp merge per
 * [QS] "Builds on: FlashDecoding").
 *   q:   device fp16 [B][T][Hq][d].  Query row t sits at absolute position
 *        L - T + t (L = n_q + n_r: the T tokens are already appended) and
 *        sees positions 0..L-T+t (causal among the T).
 *   GQA: query head h reads kv head h / (Hq/Hkv).
 *   path: KVQ_TARGET (all stored bits) or KVQ_DRAFT4 (bits == 8 only).
 *   logits = sm_scale * q . k^ (k^ dequantized per path, fp16 values for
 *   residual tokens); out = softmax(logits) . v^, fp32 accumulation.
 *   out: device fp16 [B][T][Hq][d].  lse: device fp32 [B][Hq][T] natural-log
 *   log-sum-exp of the logits, or NULL.
 *   ws: device workspace of >= kv_attn_workspace_bytes(c, T, Hq) bytes;
 *   it needs no initial contents and holds scratch between the call's two
 *   launches (split pass, then log-sum-exp merge).  Calls sharing one ws
 *   must be ordered (same stream).
 *   Range: value groups need scale s <= 63 (the PV step multiplies fp16
 *   probabilities scaled to at most 2^10 by s in fp16); per channel, the
 *   query times sm_scale * log2(e) times the key scale s of the channel's
 *   group must stay below 65504 in magnitude (below 16376 for 2-bit
 *   caches: the product is kept as fp16 parts, for 2-bit codes times 4);
 *   every input finite.
 *   Rows: one launch pair handles the T * Hq/Hkv query rows of a kv head
 *   up to 32; above that, the query heads of each kv group run in
 *   consecutive launch pairs of 32 / T heads (each reading the cache).
 * Requires 1 <= T <= 16, T <= n_r, Hq % Hkv == 0. */
int kv_attn_verify(const kvq_cache* c, const void* q, int T, int Hq, int path,
                   float sm_scale, void* out, float* lse, void* ws,
                   size_t ws_bytes, void* stream);

/* kv_attn_verify for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, semantics and results as kv_attn_verify
 * without ws/ws_bytes: the split partials go to a static device scratch of
 * 32 MiB that the library holds on every GPU it runs on until the process
 * ends.  Nothing is allocated or freed, by the library or otherwise.
 *   Limit: a call needs B*Hkv*rows_pad*(d+2)*4 bytes per split slot, rows_pad
 *   = 16 when T*Hq/Hkv <= 16 else 32, and at least 2 slots in the scratch;
 *   otherwise KVQ_EWORKSPACE (before any HIP call).  Within that, the split
 *   count is the one kv_attn_verify plans whenever the scratch holds it.
 *   Concurrency: every call on one GPU shares that GPU's scratch, so calls
 *   that may overlap on one GPU (different streams, other threads) race;
 *   order them.  The scratch keeps the last call's partials; a call needs
 *   no initial contents. */
int kv_attn_verify_noalloc(const kvq_cache* c, const void* q, int T, int Hq,
                           int path, float sm_scale, void* out, float* lse,
                           void* stream);

/* Verify / draft attention with exact substitution for one query row
 * ([SC] Approach: the KV pairs the speculative token ranks highest are
 * fetched in full precision and used for the output token).  Same as
 * kv_attn_verify (same arguments, workspace and result layout), except that
 * query row t_exact (0 <= t_exact < T) reads the fp16 values
 * k_exact/v_exact[b][kvh][i] instead of the quantized ones at the
 * positions idx[b][kvh][i], i < n; the other rows are unchanged.
 *   idx: device int32 [B][Hkv][n]; each block's entries must be distinct
 *        (as kv_topk returns them); entries outside [0, n_q) are skipped
 *        (kv_topk's -1 padding).
 *   k_exact, v_exact: device fp16 [B][Hkv][n][d] (e.g. from kv_fetch_rows).
 *   rows_ready: NULL, or a hipEvent_t recorded (on any stream) after
 *        k_exact/v_exact are written: the call reads idx at once but waits
 *        for the event only before the launch that reads the rows, so a
 *        transfer of the rows (kv_fetch_rows on another stream) overlaps
 *        the split pass ([SC] Approach: the fetch runs in parallel with
 *        computation).  With NULL the rows must be ready in stream order.
 * Two more launches than kv_attn_verify: a mask of the fetched positions
 * before the split pass, which leaves them out of row t_exact, and the
 * partial of their exact terms after it (into a spare workspace slot),
 * which the log-sum-exp merge adds.  (No quantized term is subtracted, so
 * the row stays accurate when a fetched token held most of its low-bit
 * attention mass.)
 * Requires 0 <= n <= 256. */
int kv_attn_verify_exact(const kvq_cache* c, const void* q, int T, int Hq,
                         int path, float sm_scale, int t_exact,
                         const int32_t* idx, int n, const void* k_exact,
                         const void* v_exact, void* out, float* lse, void* ws,
                         size_t ws_bytes, void* rows_ready, void* stream);

/* Workspace bytes kv_topk needs for this cache at any fill level. */
size_t kv_topk_workspace_bytes(const kvq_cache* c, int Hq, int k);

/* Top-k of the speculative token's low-bit scores per kv head ([SC]
 * Approach: the speculative token predicts the KV pairs the next step
 * attends to most).  For block (b, kvh) and quantized token j < n_q, with
 * q_h = f32 of q_spec[b][h] for the Hq/Hkv heads h of the group and
 * k^_jc = f32(z + f32(code*s)) (code per path; DRAFT4 uses 16*hi + 7.5):
 *     logit_hj = (((0 + q_h0*k^_j0) + q_h1*k^_j1) + ...) + q_h,d-1*k^_j,d-1
 *   (each * and + one IEEE binary32 op, channel order 0..d-1, no fusing),
 *     key_j = max_h logit_hj + 0.0   (folds -0 to +0).
 * idx: device int32 [B][Hkv][k], the k tokens with the largest key, ordered
 * by key descending then index ascending (ties go to the lower index);
 * slots past n_q hold -1.  key: device fp32 [B][Hkv][k] or NULL (the keys
 * of idx; -inf in padded slots).  Tokens still in the residual ring are
 * fp16 already and are not candidates.
 * ws: >= kv_topk_workspace_bytes(c, Hq, k) bytes; it needs no initial
 * contents and holds the per-chunk candidates between the call's two
 * launches (scoring, then merge).  Calls sharing one ws must be ordered
 * (same stream).  Requires 1 <= k <= 256, Hq % Hkv == 0, Hq/Hkv <= 8. */
int kv_topk(const kvq_cache* c, const void* q_spec, int Hq, int path, int k,
            int32_t* idx, float* key, void* ws, size_t ws_bytes, void* stream);

/* On-demand reconstruction of a token subset ([MS] Abstract: KV kept in
 * quantized form, only the subsets that are needed rebuilt on demand).  For
 * every block (b, kvh) and request i < n, with p = idx[b][kvh][i]:
 *   0 <= p < n_q (quantized):  k_out/v_out[b][kvh][i][c] =
 *       fp16_rne( f32(z + f32(code*s)) )   (one IEEE binary32 multiply, one
 *       add, no fusing), with the token's key-group / value-group (s, z) and
 *       code = q (KVQ_TARGET, every stored bit) or 16*hi + 7.5 (KVQ_DRAFT4,
 *       bits == 8 only: the INT4 draft view);
 *   n_q <= p < n_q + n_r (residual):  the fp16 values in the ring;
 *   any other p:  fp16 NaN in every channel (nothing outside the cache is
 *       read).
 * idx: device int32 [B][Hkv][n]; k_out, v_out: device fp16 [B][Hkv][n][d]
 * (token-major rows, written in full).  n = 0 enqueues nothing.  No
 * workspace.  Requires 0 <= n <= 2^24. */
int kv_dequant_gather(const kvq_cache* c, const int32_t* idx, int n, int path,
                      void* k_out, void* v_out, void* stream);

/* Fetch rows of a full-precision copy of the cache held in host memory
 * ([SC] Approach: the full KV stays off the GPU; the pairs the speculative
 * token selects are fetched).  host_k, host_v: fp16 [B][Hkv][host_len][d],
 * in pinned host memory the device can read (hipHostMalloc, or torch
 * tensors with pin_memory), each B*Hkv*host_len*d halves; the call looks
 * up their device addresses (hipPointerGetAttributes) and returns
 * KVQ_EINVAL for memory the device cannot read.  For every block and i < n,
 * with
 * p = idx[b][kvh][i] (device int32 [B][Hkv][n]): k_out/v_out[b][kvh][i] =
 * host row p, or fp16 NaN rows when p is outside [0, host_len).  k_out,
 * v_out: device fp16 [B][Hkv][n][d].  Only the cache's shape fields are
 * used.  Enqueue it on a second stream to overlap the transfer with other
 * work.  Requires 0 <= n <= 2^24. */
int kv_fetch_rows(const kvq_cache* c, const void* host_k, const void* host_v,
                  int64_t host_len, const int32_t* idx, int n, void* k_out,
                  void* v_out, void* stream);

/* Message for the last non-zero return on this thread ("" if none). */
const char* kv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
