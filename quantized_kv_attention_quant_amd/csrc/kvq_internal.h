// Internal definitions shared by the libkvq HIP sources (not part of the
// public ABI).  Layouts and arithmetic are those documented in kvq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

constexpr int kTile = 32;       // tokens per V tile / ring tile
constexpr int kWave = 64;       // CDNA wavefront width
constexpr int kMaxSplits = 1024;   // split partials per block; their weights fit the merge LDS
constexpr int kMaxExact = 256;     // positions per block in an exact substitution

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) {
  return (a + b - 1) / b;
}

// Bits per code in one stored plane: 8-bit codes live in two nibble planes.
__host__ __device__ inline int plane_width(int bits) {
  return bits == 8 ? 4 : bits;
}

// Geometry of one cache, flattened for kernels (all strides in elements of
// the buffer's own type).
struct CacheGeom {
  int B, Hkv, d, G, Gv, bits, R, ring;
  int64_t L_max;
  int w;                      // plane width in bits
  int64_t k_row_bytes;        // d*w/8
  int64_t k_block_bytes;      // L_max * k_row_bytes
  int64_t v_tile_bytes;       // 4*d*w
  int64_t v_block_bytes;      // (L_max/32) * v_tile_bytes
  int64_t ksz_block;          // half2 per block in k_sz: (L_max/G)*d
  int64_t vsz_tile;           // half2 per tile in v_sz: 32*(d/Gv)
  int64_t vsz_block;          // (L_max/32)*vsz_tile
  int64_t res_block;          // halfs per block in k_res / v_res: ring*d
};

inline CacheGeom geom_of(const kvq_cache* c) {
  CacheGeom g;
  g.B = c->B; g.Hkv = c->Hkv; g.d = c->d; g.G = c->G; g.Gv = c->Gv;
  g.bits = c->bits; g.R = c->R; g.ring = c->ring; g.L_max = c->L_max;
  g.w = plane_width(c->bits);
  g.k_row_bytes = (int64_t)c->d * g.w / 8;
  g.k_block_bytes = g.L_max * g.k_row_bytes;
  g.v_tile_bytes = 4LL * c->d * g.w;
  g.v_block_bytes = (g.L_max / kTile) * g.v_tile_bytes;
  g.ksz_block = (g.L_max / c->G) * c->d;
  g.vsz_tile = (int64_t)kTile * (c->d / c->Gv);
  g.vsz_block = (g.L_max / kTile) * g.vsz_tile;
  g.res_block = (int64_t)c->ring * c->d;
  return g;
}

// Raw device pointers of a cache.
struct CachePtrs {
  uint8_t *k_hi, *k_lo, *v_hi, *v_lo;
  __half2 *k_sz, *v_sz;
  __half *k_res, *v_res;
};

inline CachePtrs ptrs_of(const kvq_cache* c) {
  CachePtrs p;
  p.k_hi = (uint8_t*)c->k_hi; p.k_lo = (uint8_t*)c->k_lo;
  p.v_hi = (uint8_t*)c->v_hi; p.v_lo = (uint8_t*)c->v_lo;
  p.k_sz = (__half2*)c->k_sz; p.v_sz = (__half2*)c->v_sz;
  p.k_res = (__half*)c->k_res; p.v_res = (__half*)c->v_res;
  return p;
}

// Half index of (slot j in a 32-slot ring tile, channel c) in v_res.
__host__ __device__ inline int vres_index(int j, int c, int d) {
  int g = (j & 15) >> 2, i = j & 3, h = j >> 4, r = c & 15, m = c >> 4;
  return (16 * g + r) * (d / 2) + 8 * m + 2 * i + h;
}

// ---- one quantized element, read straight from the device layouts --------
// Code of channel c of quantized token pos (< n_q) of block blk, as the path
// reads it: every stored bit (q) or the INT4 draft view 16*(q >> 4) + 7.5.
__device__ inline float code_value(unsigned hi, unsigned lo, bool two, bool draft) {
  if (draft) return 16.f * (float)hi + 7.5f;
  return (float)(two ? (hi << 4) | lo : hi);
}

// Key: byte c / (8/w) of the token's plane row, bits w * (c % (8/w)); its
// key group's (s, z) pair.
__device__ inline float key_code(const CacheGeom& g, const CachePtrs& p,
                                 int64_t blk, int64_t pos, int c, bool draft) {
  const int per_byte = 8 / g.w, sh = g.w * (c % per_byte);
  const unsigned mask = (1u << g.w) - 1u;
  const int64_t row = blk * g.k_block_bytes + pos * g.k_row_bytes + c / per_byte;
  const unsigned hi = ((unsigned)p.k_hi[row] >> sh) & mask;
  const unsigned lo = g.bits == 8 ? ((unsigned)p.k_lo[row] >> sh) & mask : 0u;
  return code_value(hi, lo, g.bits == 8, draft);
}
__device__ inline __half2 key_sz(const CacheGeom& g, const CachePtrs& p,
                                 int64_t blk, int64_t pos, int c) {
  return p.k_sz[blk * g.ksz_block + (pos / g.G) * g.d + c];
}

// Value: token j = pos % 32 of its 32-token tile (g = (j%16)/4, i = j%4,
// h = j/16), channel c (r = c%16, m = c/16): dword (16g + r)*(d w/64) + m/per
// of the tile, bits 16h + w (4 (m%per) + i), per = 4/w.
__device__ inline float value_code(const CacheGeom& g, const CachePtrs& p,
                                   int64_t blk, int64_t pos, int c, bool draft) {
  const int j = (int)(pos % kTile);
  const int jg = (j % 16) / 4, ji = j % 4, jh = j / 16, r = c % 16, m = c / 16;
  const int per = 4 / g.w;
  const int dw = (16 * jg + r) * (g.d * g.w / 64) + m / per;
  const int sh = 16 * jh + g.w * (4 * (m % per) + ji);
  const unsigned mask = (1u << g.w) - 1u;
  const int64_t tile = blk * g.v_block_bytes + (pos / kTile) * g.v_tile_bytes;
  const unsigned hi = (((const uint32_t*)(p.v_hi + tile))[dw] >> sh) & mask;
  const unsigned lo =
      g.bits == 8 ? (((const uint32_t*)(p.v_lo + tile))[dw] >> sh) & mask : 0u;
  return code_value(hi, lo, g.bits == 8, draft);
}
// The value group's (s, z): halves [part][g][i][group][h] of the tile.
__device__ inline float2 value_sz(const CacheGeom& g, const CachePtrs& p,
                                  int64_t blk, int64_t pos, int c) {
  const int j = (int)(pos % kTile);
  const int jg = (j % 16) / 4, ji = j % 4, jh = j / 16;
  const int ngv = g.d / g.Gv, gg = c / g.Gv;
  const __half* t = (const __half*)(p.v_sz + blk * g.vsz_block + (pos / kTile) * g.vsz_tile);
  const int so = (jg * 4 + ji) * ngv * 2 + gg * 2 + jh;
  const int zo = ((4 + jg) * 4 + ji) * ngv * 2 + gg * 2 + jh;
  return make_float2(__half2float(t[so]), __half2float(t[zo]));
}

// ---- launchers (defined in the .hip files; return hipError_t) ----------

// Append/flush: see kv_quant_append.  Items [flush_begin, flush_end) are
// groups of G tokens to quantize starting at absolute position q0; ring
// items write tokens [wr_begin, wr_end) of k_new/v_new to the ring.
struct AppendArgs {
  CacheGeom g;
  CachePtrs p;
  const __half* k_new;
  const __half* v_new;
  int n;            // tokens in k_new/v_new
  int64_t q0;       // first position to quantize (= n_q before the call)
  int64_t new0;     // absolute position of k_new[0] (= n_q + n_r before)
  int groups;       // K groups to flush (each G tokens)
  int wr_first;     // first k_new index that goes to the ring
  int wr_count;     // how many k_new tokens go to the ring
};
hipError_t launch_append(const AppendArgs& a, bool flush, bool ring_write,
                         hipStream_t s);

struct AttnArgs {
  CacheGeom g;
  CachePtrs p;
  const __half* q;
  __half* out;
  float* lse;
  float* ws;        // partials: [B*Hkv][s_alloc][rows_pad][d + 2] float
  int64_t n_q, n_r;
  int T, Hq, gs, rows;
  int h0, hs;       // this launch's query heads of each kv group: h0 .. h0+hs-1
                    // (rows = T * hs; all gs heads unless rows would pass 32)
  int path;         // KVQ_TARGET / KVQ_DRAFT4
  float c0;         // sm_scale * log2(e)
  int S;            // split workgroups per block (set by the launcher)
  int s_alloc;      // partial slots per block in the workspace
  int rows_pad;     // 16 * row tiles
  int nq_mod;       // n_q mod ring: ring slot of the first residual token
  int grp_shift;    // log2(G / 32) when G / 32 is a power of two, else -1
  // exact substitution (kv_attn_verify_exact); n_exact < 0: none
  int n_exact;              // positions per block in idx_exact
  int t_exact;              // the query row that reads the exact values
  const int32_t* idx_exact; // [B][Hkv][n_exact] quantized positions (-1: skip)
  const __half* k_exact;    // [B][Hkv][n_exact][d]
  const __half* v_exact;    // [B][Hkv][n_exact][d]
  unsigned* xmask;          // [B*Hkv][L_max/32] fetched-position bits, or NULL
  void* rows_ready;         // hipEvent_t after k_exact/v_exact are written, or NULL
};
// Splits per block for nb blocks on `slots` resident workgroup slots, with
// `units` units of work per block, nw waves per workgroup, at most cap.
int plan_splits(int64_t nb, int64_t slots, int64_t units, int nw, int cap);
hipError_t launch_attn(const AttnArgs& a, hipStream_t s);
// Static device scratch of kv_attn_verify_noalloc: kScratchBytes per GPU;
// attn_scratch returns its address on the current device (looked up once
// per device).
constexpr size_t kScratchBytes = size_t(32) << 20;
hipError_t attn_scratch(void** ptr);

// On-demand reconstruction: see kv_dequant_gather.
struct GatherArgs {
  CacheGeom g;
  CachePtrs p;
  const int32_t* idx;   // [B][Hkv][n] token positions
  __half* k_out;        // [B][Hkv][n][d]
  __half* v_out;        // [B][Hkv][n][d]
  int64_t n_q, n_r;
  int n;
  int path;             // KVQ_TARGET / KVQ_DRAFT4
};
hipError_t launch_gather(const GatherArgs& a, hipStream_t s);

// Rows of host-resident fp16 K/V: see kv_fetch_rows.
struct FetchArgs {
  const __half* host_k;   // [B][Hkv][host_len][d], device-accessible host memory
  const __half* host_v;
  int64_t host_len;
  const int32_t* idx;     // [B][Hkv][n]
  __half* k_out;          // [B][Hkv][n][d]
  __half* v_out;
  int B, Hkv, d, n;
};
hipError_t launch_fetch(const FetchArgs& a, hipStream_t s);

struct TopkArgs {
  CacheGeom g;
  CachePtrs p;
  const __half* q;   // [B][Hq][d]
  int32_t* idx;
  float* key;
  unsigned long long* cand;  // [B*Hkv][chunks][k]
  int64_t n_q;
  int Hq, gs, k, path;
  int chunk;         // tokens per workgroup
  int chunks;        // workgroups per block
};
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);

}  // namespace kvq
