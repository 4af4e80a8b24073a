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
//   K-group items: one group of G tokens; thread (t, qt) owns 8 channels
//     over token slice qt, the slices' min/max meet in LDS, and each thread
//     writes its slice's codes as whole words of the plane rows.
//   V-tile items:  32 tokens, 8 threads per token over the channels; a
//     value group's min/max meet by lane shuffles; codes are assembled in
//     LDS into the tiled plane layout and stored with coalesced dword
//     writes.
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

// Work items of one launch.  Bulk appends give each V-tile workgroup vt
// tiles and each ring workgroup rt tokens (fewer, larger workgroups: a
// 32K-token prefill would otherwise dispatch ~100K tiny ones); a per-step
// append keeps one tile and one token per workgroup for latency.
struct Item {
  int k_items, v_items, ring_items;
  int v_tiles, r_tokens;   // totals
  int vt, rt;              // tiles / tokens per workgroup
};

// Key row of position p: the appended tokens for p >= new0, else the ring
// slot `slot` (= p mod ring, tracked by the caller: there is no 64-bit
// divide instruction, and its software sequence per token dominated).
__device__ inline const __half* key_row(const AppendArgs& a, int b, int kvh,
                                        int64_t p, int slot) {
  const CacheGeom& g = a.g;
  if (p >= a.new0)
    return a.k_new + (((int64_t)b * a.n + (p - a.new0)) * g.Hkv + kvh) * g.d;
  return a.p.k_res + ((int64_t)b * g.Hkv + kvh) * g.res_block + (int64_t)slot * g.d;
}

// Value channel c of position p, given p's ring slot (p mod ring).
__device__ inline float value_at(const AppendArgs& a, int b, int kvh,
                                 int64_t p, int slot, int c) {
  const CacheGeom& g = a.g;
  if (p >= a.new0)
    return __half2float(
        a.v_new[(((int64_t)b * a.n + (p - a.new0)) * g.Hkv + kvh) * g.d + c]);
  const __half* base = a.p.v_res + ((int64_t)b * g.Hkv + kvh) * g.res_block +
                       (int64_t)(slot / kTile) * kTile * g.d;
  return __half2float(base[vres_index(slot % kTile, c, g.d)]);
}

// Load CPT consecutive halfs (CPT in {2, 4, 8}) as floats.
template <int CPT>
__device__ inline void load_chans(const __half* src, float* out) {
  constexpr int cpt = CPT;
  if constexpr (cpt == 2) {
    __half2 v = *(const __half2*)src;
    out[0] = __low2float(v); out[1] = __high2float(v);
  } else if constexpr (cpt == 4) {
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

// K-group item: threads = channel column t (8 consecutive channels, one
// 16-byte load per token row) x token slice qt (G / NQ consecutive tokens).
// Each thread takes the min/max of its slice, the slices meet in LDS, and
// each thread then writes its slice's codes: the 8 channels' codes are one
// whole word of a plane row (a dword for 8-bit codes in nibble planes, 16
// bits for 2-bit, a byte for 1-bit).  The token loops are unrolled so
// several rows are in flight.
template <int W>   // bits per code in a plane: 4 (8-bit codes), 2, 1
__device__ void key_group(const AppendArgs& a, int item, int b, int kvh,
                          float* s_mn, float* s_mx) {
  const CacheGeom& g = a.g;
  constexpr int CH = 8;                       // channels per thread
  constexpr int BITS = W == 4 ? 8 : W;
  const int cols = g.d / CH;                  // channel columns (8 or 16)
  const int nq = kThreads / cols;             // token slices (16 or 32)
  const int tpq = g.G / nq;                   // tokens per slice (>= 1)
  const int t = threadIdx.x % cols, qt = threadIdx.x / cols;
  const int c0 = t * CH;
  constexpr int Lv = (1 << BITS) - 1;
  const int64_t p0 = a.q0 + (int64_t)item * g.G;
  const int64_t ps = p0 + (int64_t)qt * tpq;
  const int64_t blk = (int64_t)b * g.Hkv + kvh;
  float mn[CH], mx[CH], x[CH], s[CH], z[CH];
#pragma unroll
  for (int k = 0; k < CH; ++k) { mn[k] = INFINITY; mx[k] = -INFINITY; }
  // ring slot of ps (one divide, only when the slice starts in the ring;
  // appended rows never use it)
  const int slot0 = ps < a.new0 ? (int)(ps % g.ring) : 0;
  auto slot_of = [&](int tok) {                 // (slot0 + tok) mod ring
    int sl = slot0 + tok;
    while (sl >= g.ring) sl -= g.ring;
    return sl;
  };
#pragma unroll 8
  for (int tok = 0; tok < tpq; ++tok) {
    load_chans<CH>(key_row(a, b, kvh, ps + tok, slot_of(tok)) + c0, x);
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      mn[k] = fminf(mn[k], x[k]);
      mx[k] = fmaxf(mx[k], x[k]);
    }
  }
  // min/max over the token slices: across the slices of this wave first
  // (lanes cols, 2 cols, ... apart hold the same channels), then across
  // the kThreads / 64 waves through LDS
#pragma unroll
  for (int k = 0; k < CH; ++k)
    for (int o = cols; o < kWave; o <<= 1) {
      mn[k] = fminf(mn[k], __shfl_xor(mn[k], o));
      mx[k] = fmaxf(mx[k], __shfl_xor(mx[k], o));
    }
  const int wv = threadIdx.x / kWave;
  if ((threadIdx.x % kWave) < cols) {
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      s_mn[wv * g.d + c0 + k] = mn[k];
      s_mx[wv * g.d + c0 + k] = mx[k];
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    float lo = INFINITY, hi = -INFINITY;
#pragma unroll
    for (int r = 0; r < kThreads / kWave; ++r) {
      lo = fminf(lo, s_mn[r * g.d + c0 + k]);
      hi = fmaxf(hi, s_mx[r * g.d + c0 + k]);
    }
    z[k] = lo;
    s[k] = stored_scale(lo, hi, Lv);
  }
  if (qt == 0) {
    __half2* ksz = a.p.k_sz + blk * g.ksz_block + (p0 / g.G) * g.d + c0;
#pragma unroll
    for (int k = 0; k < CH; ++k)
      ksz[k] = __halves2half2(__float2half_rn(s[k]), __float2half_rn(z[k]));
  }
  // byte offset of the column's word in a plane row
  uint8_t* hi = a.p.k_hi + blk * g.k_block_bytes + c0 * W / 8;
  uint8_t* lo = BITS == 8 ? a.p.k_lo + blk * g.k_block_bytes + c0 * W / 8 : nullptr;
  // codes in batches of KB tokens: the batch's rows are loaded before its
  // codes are stored (the compiler cannot reorder a load above a store that
  // may alias it, so token-by-token the loads would wait in turn)
  constexpr int KB = 8;
  for (int t0 = 0; t0 < tpq; t0 += KB) {
    float xb[KB][CH];
#pragma unroll
    for (int u = 0; u < KB; ++u)
      if (t0 + u < tpq)
        load_chans<CH>(key_row(a, b, kvh, ps + t0 + u, slot_of(t0 + u)) + c0, xb[u]);
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if (t0 + u >= tpq) break;
      const int64_t p = ps + t0 + u;
      unsigned bh = 0, bl = 0;
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        unsigned q = code_of(xb[u][k], z[k], s[k], Lv);
        if constexpr (BITS == 8) {
          bh |= (q >> 4) << (4 * k);
          bl |= (q & 15u) << (4 * k);
        } else {
          bh |= q << (W * k);
        }
      }
      if constexpr (W == 4) {
        *(unsigned*)(hi + p * g.k_row_bytes) = bh;
        *(unsigned*)(lo + p * g.k_row_bytes) = bl;
      } else if constexpr (W == 2) {
        *(unsigned short*)(hi + p * g.k_row_bytes) = (unsigned short)bh;
      } else {
        hi[p * g.k_row_bytes] = (uint8_t)bh;
      }
    }
  }
}

// V-tile item: 32 tokens, 8 threads per token; thread (j, u) holds the d/8
// channels u*d/8 .. of token j, a value group spans Gv/(d/8) threads whose
// min/max meet by lane shuffles.  Codes are assembled in LDS into the tiled
// plane layout and stored with coalesced dword writes.
__device__ void value_tile(const AppendArgs& a, int item, int b, int kvh,
                           unsigned* lds_hi, unsigned* lds_lo) {
  const CacheGeom& g = a.g;
  const int Lv = (1 << g.bits) - 1;
  const int ng = g.d / g.Gv;
  const int words = g.d * g.w;             // dwords per plane tile
  const int cpv = g.d / 8;                 // channels per thread (8 or 16)
  const int tpg = g.Gv / cpv;              // threads per value group (1..8)
  const int64_t p0 = a.q0 + (int64_t)item * kTile;
  const int64_t tile = p0 / kTile;
  const int64_t blk = (int64_t)b * g.Hkv + kvh;
  for (int i = threadIdx.x; i < words; i += kThreads) {
    lds_hi[i] = 0u;
    lds_lo[i] = 0u;
  }
  __syncthreads();
  const int j = threadIdx.x / 8, u = threadIdx.x % 8;
  const int c0 = u * cpv, grp = c0 / g.Gv;
  const int64_t p = p0 + j;
  float x[16];
  if (p >= a.new0) {   // appended token: token-major, 16-byte loads
    const __half* src =
        a.v_new + (((int64_t)b * a.n + (p - a.new0)) * g.Hkv + kvh) * g.d + c0;
    load_chans<8>(src, x);
    if (cpv == 16) load_chans<8>(src + 8, x + 8);
  } else {             // ring token: one divide per thread for its slot
    const int slot = (int)(p % g.ring);
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (k < cpv) x[k] = value_at(a, b, kvh, p, slot, c0 + k);
  }
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    if (k < cpv) {
      mn = fminf(mn, x[k]);
      mx = fmaxf(mx, x[k]);
    }
  }
  for (int o = 1; o < tpg; o <<= 1) {      // lanes of one group: aligned runs
    mn = fminf(mn, __shfl_xor(mn, o));
    mx = fmaxf(mx, __shfl_xor(mx, o));
  }
  const float z = mn, s = stored_scale(mn, mx, Lv);
  const int gg = (j & 15) >> 2, i = j & 3, h = j >> 4;
  if (u % tpg == 0) {
    // [part][g][i][group][h]: scale plane then zero-point plane
    __half* sz = (__half*)(a.p.v_sz + blk * g.vsz_block + tile * g.vsz_tile);
    const int at = ((gg * 4 + i) * ng + grp) * 2 + h;
    sz[at] = __float2half_rn(s);
    sz[32 * ng + at] = __float2half_rn(z);
  }
  const int per = 4 / g.w;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    if (k < cpv) {
      const int c = c0 + k;
      const unsigned q = code_of(x[k], z, s, Lv);
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
  __shared__ float s_mn[16 * 128], s_mx[16 * 128];   // K slices' min/max
  const int b = blockIdx.z, kvh = blockIdx.y;
  int x = blockIdx.x;
  if (x < it.k_items) {
    if (a.g.w == 4) key_group<4>(a, x, b, kvh, s_mn, s_mx);
    else if (a.g.w == 2) key_group<2>(a, x, b, kvh, s_mn, s_mx);
    else key_group<1>(a, x, b, kvh, s_mn, s_mx);
    return;
  }
  x -= it.k_items;
  if (x < it.v_items) {
    for (int k = 0; k < it.vt; ++k) {
      const int tl = x * it.vt + k;
      if (tl >= it.v_tiles) break;              // uniform in the workgroup
      if (k > 0) __syncthreads();               // LDS of the last tile read out
      value_tile(a, tl, b, kvh, lds_hi, lds_lo);
    }
    return;
  }
  x -= it.v_items;
  if (x < it.ring_items) {
    for (int k = 0; k < it.rt; ++k) {
      const int r = x * it.rt + k;
      if (r >= it.r_tokens) break;
      ring_token(a, r, b, kvh);
    }
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, bool flush, bool ring_write,
                         hipStream_t s) {
  Item it;
  it.k_items = flush ? a.groups : 0;
  it.v_tiles = flush ? (int)((int64_t)a.groups * a.g.G / kTile) : 0;
  it.r_tokens = ring_write ? a.wr_count : 0;
  it.vt = it.v_tiles >= 64 ? 4 : 1;
  it.rt = it.r_tokens >= 64 ? 8 : 1;
  it.v_items = (int)cdiv(it.v_tiles, it.vt);
  it.ring_items = (int)cdiv(it.r_tokens, it.rt);
  const int64_t nx = (int64_t)it.k_items + it.v_items + it.ring_items;
  if (nx == 0) return hipSuccess;
  dim3 grid((unsigned)nx, a.g.Hkv, a.g.B);
  hipLaunchKernelGGL(append_kernel, grid, dim3(kThreads), 0, s, a, it);
  return hipGetLastError();
}

}  // namespace kvq
