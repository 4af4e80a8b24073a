// Quantize-on-append for the hierarchical quantized KV cache.
//
// QuantSpec page, Approach: recent tokens stay in a double fp16 buffer; when
// it overflows its oldest tokens are quantized once (no requantization on
// rollback); the upper nibble of each 8-bit code is the INT4 draft code.
// SpeCache page, Approach / KIVI: keys are quantized per channel over token
// groups, values per token over channel groups, with a zero-point and scale.
//
// One launch covers three kinds of work item (blockIdx.x), each for one
// (b = blockIdx.z, kvh = blockIdx.y) block:
//   K-group items: one group of G tokens; thread t owns the channels of
//     output byte t of a plane row, finds their min/max over the group and
//     writes codes row by row.
//   V-tile items:  32 tokens; thread (j, grp) owns the Gv channels of one
//     token's value group; codes are assembled in LDS into the tiled plane
//     layout and stored with coalesced dword writes.
//   Ring items:    one appended token copied into the fp16 residual ring.
// The arithmetic is the exact binary32 sequence of the quantizer definition
// (correctly rounded subtract and divide, round-half-even, RNE to fp16).
#include "kvq_internal.h"

// Bit-exact binary32 arithmetic: built with -ffp-contract=off as well.
#pragma clang fp contract(off)

namespace kvq {
namespace {

constexpr int kThreads = 256;

__device__ inline float stored_scale(float mn, float mx, int Lv) {
  float span = __fsub_rn(mx, mn);
  float s = __fdiv_rn(span, (float)Lv);
  return __half2float(__float2half_rn(s));
}

__device__ inline unsigned code_of(float x, float z, float s, int Lv) {
  if (s == 0.f) return 0u;
  float r = rintf(__fdiv_rn(__fsub_rn(x, z), s));
  r = fminf(fmaxf(r, 0.f), (float)Lv);
  return (unsigned)r;
}

struct Item {
  int k_items, v_items, ring_items;
};

__device__ inline const __half* key_row(const AppendArgs& a, int b, int kvh,
                                        int64_t p) {
  const CacheGeom& g = a.g;
  if (p >= a.new0)
    return a.k_new + (((int64_t)b * a.n + (p - a.new0)) * g.Hkv + kvh) * g.d;
  int64_t slot = p % g.ring;
  return a.p.k_res + ((int64_t)b * g.Hkv + kvh) * g.res_block + slot * g.d;
}

__device__ inline float value_at(const AppendArgs& a, int b, int kvh,
                                 int64_t p, int c) {
  const CacheGeom& g = a.g;
  if (p >= a.new0)
    return __half2float(
        a.v_new[(((int64_t)b * a.n + (p - a.new0)) * g.Hkv + kvh) * g.d + c]);
  int64_t slot = p % g.ring;
  const __half* base = a.p.v_res + ((int64_t)b * g.Hkv + kvh) * g.res_block +
                       (slot / kTile) * (int64_t)kTile * g.d;
  return __half2float(base[vres_index((int)(slot % kTile), c, g.d)]);
}

// Load `cpt` consecutive halfs (cpt in {2, 4, 8}) as floats.
__device__ inline void load_chans(const __half* src, int cpt, float* out) {
  if (cpt == 2) {
    __half2 v = *(const __half2*)src;
    out[0] = __low2float(v); out[1] = __high2float(v);
  } else if (cpt == 4) {
    uint2 raw = *(const uint2*)src;
    const __half* h = (const __half*)&raw;
#pragma unroll
    for (int k = 0; k < 4; ++k) out[k] = __half2float(h[k]);
  } else {
    uint4 raw = *(const uint4*)src;
    const __half* h = (const __half*)&raw;
#pragma unroll
    for (int k = 0; k < 8; ++k) out[k] = __half2float(h[k]);
  }
}

__device__ void key_group(const AppendArgs& a, int item, int b, int kvh) {
  const CacheGeom& g = a.g;
  const int cpt = 8 / g.w;          // channels per output byte
  const int t = threadIdx.x;
  if (t >= g.d / cpt) return;       // no barriers in this item
  const int Lv = (1 << g.bits) - 1;
  const int64_t p0 = a.q0 + (int64_t)item * g.G;
  const int64_t blk = (int64_t)b * g.Hkv + kvh;
  float mn[8], mx[8], x[8], s[8], z[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) { mn[k] = INFINITY; mx[k] = -INFINITY; }
  for (int tok = 0; tok < g.G; ++tok) {
    load_chans(key_row(a, b, kvh, p0 + tok) + t * cpt, cpt, x);
    for (int k = 0; k < cpt; ++k) {
      mn[k] = fminf(mn[k], x[k]);
      mx[k] = fmaxf(mx[k], x[k]);
    }
  }
  __half2* ksz = a.p.k_sz + blk * g.ksz_block + (p0 / g.G) * g.d + t * cpt;
  for (int k = 0; k < cpt; ++k) {
    z[k] = mn[k];
    s[k] = stored_scale(mn[k], mx[k], Lv);
    ksz[k] = __halves2half2(__float2half_rn(s[k]), __float2half_rn(z[k]));
  }
  uint8_t* hi = a.p.k_hi + blk * g.k_block_bytes + t;
  uint8_t* lo = g.bits == 8 ? a.p.k_lo + blk * g.k_block_bytes + t : nullptr;
  for (int tok = 0; tok < g.G; ++tok) {
    const int64_t p = p0 + tok;
    load_chans(key_row(a, b, kvh, p) + t * cpt, cpt, x);
    unsigned bh = 0, bl = 0;
    for (int k = 0; k < cpt; ++k) {
      unsigned q = code_of(x[k], z[k], s[k], Lv);
      if (g.bits == 8) {
        bh |= (q >> 4) << (4 * k);
        bl |= (q & 15u) << (4 * k);
      } else {
        bh |= q << (g.w * k);
      }
    }
    hi[p * g.k_row_bytes] = (uint8_t)bh;
    if (lo) lo[p * g.k_row_bytes] = (uint8_t)bl;
  }
}

__device__ void value_tile(const AppendArgs& a, int item, int b, int kvh,
                           unsigned* lds_hi, unsigned* lds_lo) {
  const CacheGeom& g = a.g;
  const int Lv = (1 << g.bits) - 1;
  const int ng = g.d / g.Gv;
  const int words = g.d * g.w;             // dwords per plane tile
  const int64_t p0 = a.q0 + (int64_t)item * kTile;
  const int64_t tile = p0 / kTile;
  const int64_t blk = (int64_t)b * g.Hkv + kvh;
  for (int i = threadIdx.x; i < words; i += kThreads) {
    lds_hi[i] = 0u;
    lds_lo[i] = 0u;
  }
  __syncthreads();
  const int j = threadIdx.x % kTile, grp = threadIdx.x / kTile;
  if (grp < ng) {
    const int64_t p = p0 + j;
    float mn = INFINITY, mx = -INFINITY;
    for (int c = grp * g.Gv; c < (grp + 1) * g.Gv; ++c) {
      float x = value_at(a, b, kvh, p, c);
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    const float z = mn, s = stored_scale(mn, mx, Lv);
    const int gg = (j & 15) >> 2, i = j & 3, h = j >> 4;
    // [part][g][i][group][h]: scale plane then zero-point plane
    __half* sz = (__half*)(a.p.v_sz + blk * g.vsz_block + tile * g.vsz_tile);
    const int at = ((gg * 4 + i) * ng + grp) * 2 + h;
    sz[at] = __float2half_rn(s);
    sz[32 * ng + at] = __float2half_rn(z);
    const int per = 4 / g.w;
    for (int c = grp * g.Gv; c < (grp + 1) * g.Gv; ++c) {
      unsigned q = code_of(value_at(a, b, kvh, p, c), z, s, Lv);
      const int r = c & 15, m = c >> 4;
      const int dw = (16 * gg + r) * (g.d * g.w / 64) + m / per;
      const int bit = 16 * h + g.w * (4 * (m % per) + i);
      if (g.bits == 8) {
        atomicOr(&lds_hi[dw], (q >> 4) << bit);
        atomicOr(&lds_lo[dw], (q & 15u) << bit);
      } else {
        atomicOr(&lds_hi[dw], q << bit);
      }
    }
  }
  __syncthreads();
  unsigned* ghi = (unsigned*)(a.p.v_hi + blk * g.v_block_bytes +
                              tile * g.v_tile_bytes);
  unsigned* glo = g.bits == 8 ? (unsigned*)(a.p.v_lo + blk * g.v_block_bytes +
                                            tile * g.v_tile_bytes)
                              : nullptr;
  for (int i = threadIdx.x; i < words; i += kThreads) {
    ghi[i] = lds_hi[i];
    if (glo) glo[i] = lds_lo[i];
  }
}

__device__ void ring_token(const AppendArgs& a, int item, int b, int kvh) {
  const CacheGeom& g = a.g;
  const int ni = a.wr_first + item;
  const int64_t p = a.new0 + ni;
  const int64_t slot = p % g.ring;
  const int64_t blk = (int64_t)b * g.Hkv + kvh;
  const int64_t src = (((int64_t)b * a.n + ni) * g.Hkv + kvh) * g.d;
  __half* kd = a.p.k_res + blk * g.res_block + slot * g.d;
  __half* vd = a.p.v_res + blk * g.res_block +
               (slot / kTile) * (int64_t)kTile * g.d;
  const int j = (int)(slot % kTile);
  for (int c = threadIdx.x; c < g.d; c += kThreads) {
    kd[c] = a.k_new[src + c];
    vd[vres_index(j, c, g.d)] = a.v_new[src + c];
  }
}

__global__ void __launch_bounds__(kThreads)
append_kernel(AppendArgs a, Item it) {
  __shared__ unsigned lds_hi[128 * 4];
  __shared__ unsigned lds_lo[128 * 4];
  const int b = blockIdx.z, kvh = blockIdx.y;
  int x = blockIdx.x;
  if (x < it.k_items) { key_group(a, x, b, kvh); return; }
  x -= it.k_items;
  if (x < it.v_items) { value_tile(a, x, b, kvh, lds_hi, lds_lo); return; }
  x -= it.v_items;
  if (x < it.ring_items) ring_token(a, x, b, kvh);
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, bool flush, bool ring_write,
                         hipStream_t s) {
  Item it;
  it.k_items = flush ? a.groups : 0;
  it.v_items = flush ? (int)((int64_t)a.groups * a.g.G / kTile) : 0;
  it.ring_items = ring_write ? a.wr_count : 0;
  const int64_t nx = (int64_t)it.k_items + it.v_items + it.ring_items;
  if (nx == 0) return hipSuccess;
  dim3 grid((unsigned)nx, a.g.Hkv, a.g.B);
  hipLaunchKernelGGL(append_kernel, grid, dim3(kThreads), 0, s, a, it);
  return hipGetLastError();
}

}  // namespace kvq
