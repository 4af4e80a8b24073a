// C ABI of libkvq (declared in include/kvq.h): argument validation, cache
// bookkeeping, launch planning.  Every check runs before the first HIP call,
// so a rejected call enqueues nothing and leaves the struct untouched.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "kvq_internal.h"

#define KVQ_API extern "C" __attribute__((visibility("default")))

namespace {

using kvq::cdiv;

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

// Fewest unit streams an attention workgroup runs (8 waves sharing streams in
// pairs); the split planner gives every stream at least one unit, so no call
// has more splits than units / kMinStreams.
constexpr int kMinStreams = 4;
constexpr int kTopkChunk = 1024;       // tokens per top-k workgroup
constexpr int kMaxTopk = 256;

int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// Shape rules of kv_cache_layout; returns KVQ_OK or an error with message.
int check_shape(const kvq_cache* c) {
  if (!c) return fail(KVQ_EINVAL, "cache is NULL");
  if (c->B < 1 || c->Hkv < 1) return fail(KVQ_EINVAL, "B and Hkv must be >= 1");
  if (c->d != 64 && c->d != 128) return fail(KVQ_EINVAL, "d must be 64 or 128");
  if (c->bits != 8 && c->bits != 2 && c->bits != 1)
    return fail(KVQ_EINVAL, "bits must be 8, 2 or 1");
  if (c->bits == 1 && c->d != 128)
    return fail(KVQ_EINVAL, "1-bit codes need d == 128");
  if (c->G < 32 || c->G % 32) return fail(KVQ_EINVAL, "G must be a multiple of 32");
  if (c->L_max < c->G || c->L_max % c->G)
    return fail(KVQ_EINVAL, "L_max must be a positive multiple of G");
  if (c->L_max > (1LL << 24))
    return fail(KVQ_EINVAL, "L_max must be <= 2^24 tokens");
  if (c->Gv < 16 || c->Gv % 16 || c->d % c->Gv || c->d / c->Gv > 4)
    return fail(KVQ_EINVAL,
                "Gv must be a multiple of 16 dividing d with d/Gv <= 4");
  if (c->R < c->G) return fail(KVQ_EINVAL, "R must be >= G");
  if (c->max_append < 1) return fail(KVQ_EINVAL, "max_append must be >= 1");
  return KVQ_OK;
}

// A cache handed to a work call must have gone through kv_cache_layout and
// have every buffer set.
int check_cache(const kvq_cache* c) {
  int rc = check_shape(c);
  if (rc) return rc;
  if (c->ring != round_up((int64_t)c->R + c->max_append, 32))
    return fail(KVQ_EINVAL, "cache not laid out (call kv_cache_layout)");
  if (c->n_q < 0 || c->n_r < 0 || c->n_q % c->G || c->n_q > c->L_max ||
      c->n_r > c->ring)
    return fail(KVQ_EINVAL, "cache counters are inconsistent");
  if (!c->k_hi || !c->v_hi || !c->k_sz || !c->v_sz || !c->k_res || !c->v_res)
    return fail(KVQ_EINVAL, "a cache buffer pointer is NULL");
  if ((c->bits == 8) != (c->k_lo != nullptr) ||
      (c->bits == 8) != (c->v_lo != nullptr))
    return fail(KVQ_EINVAL, "k_lo/v_lo must be set exactly when bits == 8");
  return KVQ_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(KVQ_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// ---- attention split plan --------------------------------------------------
// The launcher picks the split count per block from the device's resident
// workgroup slots (plan_splits); the workspace holds one partial per split,
// sized for up to kSlotsBound slots (256 CUs x 2 workgroups) and never more
// splits than the cache has units of work for.
constexpr int kSlotsBound = 512;

int rows_pad_of(int T, int Hq, int Hkv) {
  return T * (Hq / Hkv) <= 16 ? 16 : 32;
}

int s_alloc_of(const kvq_cache* c) {
  const int64_t nb = (int64_t)c->B * c->Hkv;
  const int64_t ring = round_up((int64_t)c->R + c->max_append, 32);
  const int64_t units_max = 2 * cdiv(ring, 32) + cdiv(c->L_max, 32);
  int64_t s = 4 * cdiv(kSlotsBound, nb);
  const int64_t by_units = cdiv(units_max, kMinStreams);
  if (s > by_units) s = by_units;
  if (s > kvq::kMaxSplits - 1) s = kvq::kMaxSplits - 1;
  if (s < 1) s = 1;
  return (int)s + 1;   // one spare slot: the exact-substitution partial
}

}  // namespace

KVQ_API int kv_cache_layout(kvq_cache* c) {
  int rc = check_shape(c);
  if (rc) return rc;
  const int64_t blocks = (int64_t)c->B * c->Hkv;
  const int w = kvq::plane_width(c->bits);
  const int64_t ring = round_up((int64_t)c->R + c->max_append, 32);
  if (ring > (1 << 30)) return fail(KVQ_EINVAL, "R + max_append too large");
  c->ring = (int32_t)ring;
  c->bytes_k_plane = blocks * c->L_max * c->d * w / 8;
  c->bytes_v_plane = c->bytes_k_plane;
  c->bytes_k_sz = blocks * (c->L_max / c->G) * c->d * 4;
  c->bytes_v_sz = blocks * c->L_max * (c->d / c->Gv) * 4;
  c->bytes_k_res = blocks * ring * c->d * 2;
  c->bytes_v_res = c->bytes_k_res;
  c->n_q = 0;
  c->n_r = 0;
  return KVQ_OK;
}

KVQ_API int kv_quant_append(kvq_cache* c, const void* k_new, const void* v_new,
                            int n, void* stream) {
  int rc = check_cache(c);
  if (rc) return rc;
  if (!k_new || !v_new) return fail(KVQ_EINVAL, "k_new/v_new is NULL");
  if (n < 1) return fail(KVQ_EINVAL, "n must be >= 1");
  const int64_t total = c->n_r + (int64_t)n;
  const int64_t f = total > c->R ? cdiv(total - c->R, c->G) : 0;
  if (c->n_q + f * c->G > c->L_max)
    return fail(KVQ_ECAPACITY, "append of %d tokens needs %lld quantized slots, "
                "L_max is %d", n, (long long)(c->n_q + f * c->G), c->L_max);
  if (f * c->G / 32 > INT32_MAX)
    return fail(KVQ_EUNSUPPORTED, "append too large for one call");

  kvq::AppendArgs a;
  a.g = kvq::geom_of(c);
  a.p = kvq::ptrs_of(c);
  a.k_new = (const __half*)k_new;
  a.v_new = (const __half*)v_new;
  a.n = n;
  a.q0 = c->n_q;
  a.new0 = c->n_q + c->n_r;
  a.groups = (int)f;
  const int64_t keep0 = c->n_q + f * c->G;          // first surviving position
  a.wr_first = (int)(keep0 > a.new0 ? keep0 - a.new0 : 0);
  a.wr_count = n - a.wr_first;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (total <= c->ring) {
    e = kvq::launch_append(a, true, true, s);
  } else {
    e = kvq::launch_append(a, true, false, s);
    if (e == hipSuccess) e = kvq::launch_append(a, false, true, s);
  }
  if (e != hipSuccess) return hip_fail(e, "kv_quant_append launch");
  c->n_q += f * c->G;
  c->n_r = total - f * c->G;
  return KVQ_OK;
}

KVQ_API int kv_rollback(kvq_cache* c, int m) {
  if (!c) return fail(KVQ_EINVAL, "cache is NULL");
  if (m < 0) return fail(KVQ_EINVAL, "m must be >= 0");
  if (m > c->n_r)
    return fail(KVQ_EROLLBACK, "rollback of %d tokens, residual holds %lld", m,
                (long long)c->n_r);
  c->n_r -= m;
  return KVQ_OK;
}

namespace {

// Workspace: the split partials [B*Hkv][s_alloc][rows_pad][d + 2] floats,
// then (exact substitution) one bit per quantized token of every block.
size_t partial_bytes(const kvq_cache* c, int T, int Hq) {
  return (size_t)c->B * c->Hkv * s_alloc_of(c) * rows_pad_of(T, Hq, c->Hkv) *
         (c->d + 2) * sizeof(float);
}

}  // namespace

KVQ_API size_t kv_attn_workspace_bytes(const kvq_cache* c, int T, int Hq) {
  if (check_shape(c) || T < 1 || Hq < 1 || Hq % c->Hkv) return 0;
  return partial_bytes(c, T, Hq) +
         (size_t)c->B * c->Hkv * (c->L_max / 32) * sizeof(uint32_t);
}


namespace {

// Validation and argument set-up shared by the attention entry points
// (check_ws = false: the caller supplies the partial slots itself).
int attn_setup(const kvq_cache* c, const void* q, int T, int Hq, int path,
               float sm_scale, void* out, float* lse, void* ws, size_t ws_bytes,
               kvq::AttnArgs& a, bool check_ws = true) {
  int rc = check_cache(c);
  if (rc) return rc;
  if (!q || !out) return fail(KVQ_EINVAL, "q/out is NULL");
  if (T < 1 || T > 16) return fail(KVQ_EINVAL, "T must be in [1, 16]");
  if (T > c->n_r)
    return fail(KVQ_EINVAL, "T = %d exceeds the %lld residual tokens", T,
                (long long)c->n_r);
  if (Hq < 1 || Hq % c->Hkv) return fail(KVQ_EINVAL, "Hq must be a multiple of Hkv");
  if (path != KVQ_TARGET && path != KVQ_DRAFT4)
    return fail(KVQ_EINVAL, "unknown path %d", path);
  if (path == KVQ_DRAFT4 && c->bits != 8)
    return fail(KVQ_EINVAL, "the draft path reads 8-bit caches only");
  if (!std::isfinite(sm_scale)) return fail(KVQ_EINVAL, "sm_scale not finite");
  const size_t need = kv_attn_workspace_bytes(c, T, Hq);
  if (check_ws && (!ws || ws_bytes < need))
    return fail(KVQ_EWORKSPACE, "workspace needs %zu bytes", need);

  a.g = kvq::geom_of(c);
  a.p = kvq::ptrs_of(c);
  a.q = (const __half*)q;
  a.out = (__half*)out;
  a.lse = lse;
  a.ws = (float*)ws;
  a.n_q = c->n_q;
  a.n_r = c->n_r;
  a.T = T;
  a.Hq = Hq;
  a.gs = Hq / c->Hkv;
  a.h0 = 0;
  a.hs = a.gs;
  a.rows = T * a.gs;   // above 32, launch_attn splits the heads
  a.path = path;
  a.c0 = sm_scale * 1.4426950408889634f;
  a.S = 0;
  a.s_alloc = s_alloc_of(c);
  a.rows_pad = rows_pad_of(T, Hq, c->Hkv);
  a.n_exact = -1;
  a.t_exact = 0;
  a.idx_exact = nullptr;
  a.k_exact = a.v_exact = nullptr;
  a.xmask = nullptr;
  a.rows_ready = nullptr;
  return KVQ_OK;
}

}  // namespace

KVQ_API int kv_attn_verify(const kvq_cache* c, const void* q, int T, int Hq,
                           int path, float sm_scale, void* out, float* lse,
                           void* ws, size_t ws_bytes, void* stream) {
  kvq::AttnArgs a;
  const int rc = attn_setup(c, q, T, Hq, path, sm_scale, out, lse, ws, ws_bytes, a);
  if (rc) return rc;
  hipError_t e = kvq::launch_attn(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kv_attn_verify launch");
  return KVQ_OK;
}

KVQ_API int kv_attn_verify_noalloc(const kvq_cache* c, const void* q, int T,
                                   int Hq, int path, float sm_scale, void* out,
                                   float* lse, void* stream) {
  kvq::AttnArgs a;
  const int rc = attn_setup(c, q, T, Hq, path, sm_scale, out, lse, nullptr, 0, a,
                            false);
  if (rc) return rc;
  // Partial slots per block that fit the static scratch (at most as many as
  // the workspace entry point plans with, so the split count is the same
  // whenever the scratch holds it).
  const size_t slot = (size_t)c->B * c->Hkv * rows_pad_of(T, Hq, c->Hkv) *
                      (c->d + 2) * sizeof(float);
  const size_t fit = kvq::kScratchBytes / slot;
  if (fit < 2)
    return fail(KVQ_EWORKSPACE, "call needs %zu bytes per split slot and at "
                "least 2 slots; the static scratch holds %zu bytes", slot,
                kvq::kScratchBytes);
  if ((size_t)a.s_alloc > fit) a.s_alloc = (int)fit;
  void* scr = nullptr;
  hipError_t e = kvq::attn_scratch(&scr);
  if (e != hipSuccess) return hip_fail(e, "kv_attn_verify_noalloc scratch");
  a.ws = (float*)scr;
  e = kvq::launch_attn(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kv_attn_verify_noalloc launch");
  return KVQ_OK;
}

KVQ_API int kv_attn_verify_exact(const kvq_cache* c, const void* q, int T, int Hq,
                                 int path, float sm_scale, int t_exact,
                                 const int32_t* idx, int n, const void* k_exact,
                                 const void* v_exact, void* out, float* lse,
                                 void* ws, size_t ws_bytes, void* rows_ready,
                                 void* stream) {
  kvq::AttnArgs a;
  const int rc = attn_setup(c, q, T, Hq, path, sm_scale, out, lse, ws, ws_bytes, a);
  if (rc) return rc;
  if (t_exact < 0 || t_exact >= T) return fail(KVQ_EINVAL, "t_exact must be in [0, T)");
  if (n < 0 || n > kvq::kMaxExact)
    return fail(KVQ_EINVAL, "n must be in [0, %d]", kvq::kMaxExact);
  if (n > 0 && (!idx || !k_exact || !v_exact))
    return fail(KVQ_EINVAL, "idx/k_exact/v_exact is NULL");
  a.n_exact = n;
  a.t_exact = t_exact;
  a.idx_exact = idx;
  a.k_exact = (const __half*)k_exact;
  a.v_exact = (const __half*)v_exact;
  a.xmask = (unsigned*)((char*)ws + partial_bytes(c, T, Hq));
  a.rows_ready = rows_ready;
  hipError_t e = kvq::launch_attn(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kv_attn_verify_exact launch");
  return KVQ_OK;
}

KVQ_API size_t kv_topk_workspace_bytes(const kvq_cache* c, int Hq, int k) {
  if (check_shape(c) || Hq < 1 || k < 1) return 0;
  const int64_t chunks = cdiv(c->L_max, kTopkChunk);
  return (size_t)c->B * c->Hkv * chunks * k * sizeof(unsigned long long);
}

KVQ_API int kv_topk(const kvq_cache* c, const void* q_spec, int Hq, int path,
                    int k, int32_t* idx, float* key, void* ws, size_t ws_bytes,
                    void* stream) {
  int rc = check_cache(c);
  if (rc) return rc;
  if (!q_spec || !idx) return fail(KVQ_EINVAL, "q_spec/idx is NULL");
  if (k < 1 || k > kMaxTopk) return fail(KVQ_EINVAL, "k must be in [1, 256]");
  if (Hq < 1 || Hq % c->Hkv) return fail(KVQ_EINVAL, "Hq must be a multiple of Hkv");
  const int gs = Hq / c->Hkv;
  if (gs > 8) return fail(KVQ_EUNSUPPORTED, "Hq/Hkv must be at most 8");
  if (path != KVQ_TARGET && path != KVQ_DRAFT4)
    return fail(KVQ_EINVAL, "unknown path %d", path);
  if (path == KVQ_DRAFT4 && c->bits != 8)
    return fail(KVQ_EINVAL, "the draft path reads 8-bit caches only");
  const size_t need = kv_topk_workspace_bytes(c, Hq, k);
  if (!ws || ws_bytes < need)
    return fail(KVQ_EWORKSPACE, "workspace needs %zu bytes", need);

  kvq::TopkArgs a;
  a.g = kvq::geom_of(c);
  a.p = kvq::ptrs_of(c);
  a.q = (const __half*)q_spec;
  a.idx = idx;
  a.key = key;
  a.cand = (unsigned long long*)ws;
  a.n_q = c->n_q;
  a.Hq = Hq;
  a.gs = gs;
  a.k = k;
  a.path = path;
  a.chunk = kTopkChunk;
  a.chunks = (int)(c->n_q > 0 ? cdiv(c->n_q, kTopkChunk) : 1);
  hipError_t e = kvq::launch_topk(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kv_topk launch");
  return KVQ_OK;
}

KVQ_API int kv_dequant_gather(const kvq_cache* c, const int32_t* idx, int n,
                              int path, void* k_out, void* v_out, void* stream) {
  int rc = check_cache(c);
  if (rc) return rc;
  if (n < 0) return fail(KVQ_EINVAL, "n must be >= 0");
  if (n > 0 && (!idx || !k_out || !v_out))
    return fail(KVQ_EINVAL, "idx/k_out/v_out is NULL");
  if (path != KVQ_TARGET && path != KVQ_DRAFT4)
    return fail(KVQ_EINVAL, "unknown path %d", path);
  if (path == KVQ_DRAFT4 && c->bits != 8)
    return fail(KVQ_EINVAL, "the draft path reads 8-bit caches only");
  if (n > (1 << 24)) return fail(KVQ_EINVAL, "n must be at most 2^24");

  kvq::GatherArgs a;
  a.g = kvq::geom_of(c);
  a.p = kvq::ptrs_of(c);
  a.idx = idx;
  a.k_out = (__half*)k_out;
  a.v_out = (__half*)v_out;
  a.n_q = c->n_q;
  a.n_r = c->n_r;
  a.n = n;
  a.path = path;
  hipError_t e = kvq::launch_gather(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kv_dequant_gather launch");
  return KVQ_OK;
}

KVQ_API int kv_fetch_rows(const kvq_cache* c, const void* host_k,
                          const void* host_v, int64_t host_len, const int32_t* idx,
                          int n, void* k_out, void* v_out, void* stream) {
  int rc = check_shape(c);
  if (rc) return rc;
  if (n < 0 || n > (1 << 24)) return fail(KVQ_EINVAL, "n must be in [0, 2^24]");
  if (host_len < 0) return fail(KVQ_EINVAL, "host_len must be >= 0");
  if (n > 0 && (!host_k || !host_v || !idx || !k_out || !v_out))
    return fail(KVQ_EINVAL, "host_k/host_v/idx/k_out/v_out is NULL");
  // The host buffers must be pinned allocations the device can read: look
  // up their device addresses instead of trusting the pointers, so pageable
  // memory is refused here rather than faulting in the kernel.
  const void* dev[2] = {nullptr, nullptr};
  if (n > 0) {
    const void* hp[2] = {host_k, host_v};
    for (int i = 0; i < 2; ++i) {
      hipPointerAttribute_t at;
      hipError_t e = hipPointerGetAttributes(&at, hp[i]);
      if (e != hipSuccess || at.type != hipMemoryTypeHost || !at.devicePointer) {
        (void)hipGetLastError();
        return fail(KVQ_EINVAL, "host_k/host_v must be pinned host memory the "
                                "device can read");
      }
      dev[i] = at.devicePointer;
    }
  }
  kvq::FetchArgs a;
  a.host_k = (const __half*)dev[0];
  a.host_v = (const __half*)dev[1];
  a.host_len = host_len;
  a.idx = idx;
  a.k_out = (__half*)k_out;
  a.v_out = (__half*)v_out;
  a.B = c->B;
  a.Hkv = c->Hkv;
  a.d = c->d;
  a.n = n;
  hipError_t e = kvq::launch_fetch(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kv_fetch_rows launch");
  return KVQ_OK;
}

KVQ_API const char* kv_last_error(void) { return g_err.c_str(); }
