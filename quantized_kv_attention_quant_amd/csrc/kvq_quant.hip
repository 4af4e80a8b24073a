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
//     over token slice qt, the slices' fp16 min/max meet by lane shuffles
//     and one LDS step, one thread per channel derives (s, z, 1/s), and
//     each thread writes its slice's codes as whole words of the plane rows.
//   V-tile items:  32-token tiles, 8 threads per token over the channels; a
//     value group's min/max meet by lane shuffles; codes are assembled in
//     LDS into the tiled plane layout and stored with coalesced dword
//     writes, the next tile's rows already in flight.
//   Ring items:    one appended token copied into the fp16 residual ring.
// The arithmetic is the exact binary32 sequence of the quantizer definition
// (correctly rounded subtract and quotient, round-half-even, RNE to fp16).
#include "kvq_internal.h"

// Bit-exact binary32 arithmetic: built with -ffp-contract=off as well.
#pragma clang fp contract(off)

namespace kvq {
namespace {

constexpr int kThreads = 256;
typedef _Float16 hv2 __attribute__((ext_vector_type(2)));   // two fp16 lanes

__device__ inline float stored_scale(float mn, float mx, int Lv) {
  float span = __fsub_rn(mx, mn);
  float s = __fdiv_rn(span, (float)Lv);
  return __half2float(__float2half_rn(s));
}

// Key groups per K item: when G divides 128 (head dim 128), 128/G groups
// side by side, so every group's threads hold 8 rows each; else one.
__host__ __device__ inline int kgroups_per_item(int d, int G) {
  return (d == 128 && G < 128 && 128 % G == 0) ? 128 / G : 1;
}

// RN(1/s) of a group's stored scale, once per group; 0 for s = 0, which
// makes every code of the group 0 in code_word below.
__device__ inline float recip_of(float s) {
  return s == 0.f ? 0.f : __fdiv_rn(1.f, s);
}

// Code of x in a group (z, s), r = RN(1/s): clip(rint(RN((x - z) / s)))
// in the low bits of the returned word (the bits above are those of 2^23:
// mask them off).  The correctly rounded quotient comes without a divide
// per element: q1 = RN(num r) is within one ulp of num / s, its remainder
// e = num - q1 s is exact in binary32 (one fma), and RN(q1 + e r) is then
// the correctly rounded quotient (Markstein's division theorem, which
// needs r to be the correctly rounded reciprocal and no underflow).  No
// operand underflows here: num = RN(x - z) of fp16 values is 0 or at
// least 2^-24, s is an fp16 value, and the quotient is at most 1.5 Lv.
// tests/quotient_identity.c checks this against the divide for every
// positive fp16 scale, at the numerators around every k s and (k + 1/2) s,
// k <= 400, and at random ones in [0, 400 s] (2.1e9 cases).  A degenerate group
// (s = 0, r = 0) gives q1 = 0, e = num and a quotient of 0: no branch.
// The clip comes before the rounding (0 and Lv are integers, so the two
// commute), and the rounding is the add of 2^23, which rounds a value in
// [0, 2^22] to an integer, ties to even, exactly as rint does.
__device__ inline unsigned code_word(float x, float z, float s, float r,
                                     float Lv) {
  const float num = __builtin_fmaf(x, 1.f, -z);      // RN(x - z)
  const float q1 = __fmul_rn(num, r);
  const float e = __builtin_fmaf(-q1, s, num);
  const float q = __builtin_fmaf(e, r, q1);
  return __float_as_uint(__fadd_rn(fminf(fmaxf(q, 0.f), Lv), 8388608.f));
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

// K-group item: kgroups_per_item(d, G) key groups of G tokens side by side,
// each in its own run of threads, thread = channel column t (8 consecutive
// channels, one 16-byte load per token row) x token slice qt.  Each thread
// takes the fp16 min/max of its slice (packed, two channels per
// instruction: exact), the slices meet by lane shuffles within a wave and
// through LDS across the group's waves, one thread per channel then derives
// the group's (s, z) and RN(1/s) once, and each thread writes its slice's
// codes: the 8 channels' codes are one whole word of a plane row (a dword
// for 8-bit codes in nibble planes, 16 bits for 2-bit, a byte for 1-bit).
// Slices of at most KB tokens stay in registers between the two passes;
// longer ones are read again in batches of KB rows.
template <int D, int W, int NGI>   // head dim; bits per code in a plane:
                                   // 4 (8-bit codes), 2, 1; groups per item
__device__ __forceinline__ void key_group(const AppendArgs& a, int item, int b, int kvh,
                          float* s_mn, float* s_mx) {
  const CacheGeom& g = a.g;
  constexpr int CH = 8;                       // channels per thread
  constexpr int KB = 8;                       // rows per batch
  constexpr int BITS = W == 4 ? 8 : W;
  constexpr int cols = D / CH;                // channel columns (8 or 16)
  constexpr int RB = D * W / 8;               // bytes per plane row
  constexpr int tps = kThreads / NGI;         // threads per group (>= 64)
  const int sg = threadIdx.x / tps, ti = threadIdx.x % tps;
  constexpr int wps = tps / kWave;            // waves per group
  const int tpq = g.G / (tps / cols);         // tokens per slice (>= 1)
  const int t = ti % cols, qt = ti / cols;
  const int c0 = t * CH;
  constexpr int Lv = (1 << BITS) - 1;
  const int gi = item * NGI + sg;             // this run's key group
  const bool valid = gi < a.groups;           // the last item may be short
  const int64_t p0 = a.q0 + (int64_t)gi * g.G;
  const int64_t ps = p0 + (int64_t)qt * tpq;
  const int64_t blk = (int64_t)b * g.Hkv + kvh;
  // ring slot of ps (one divide, only when the slice starts in the ring;
  // appended rows never use it)
  const int slot0 = valid && ps < a.new0 ? (int)(ps % g.ring) : 0;
  auto slot_of = [&](int tok) {                 // (slot0 + tok) mod ring
    int sl = slot0 + tok;
    while (sl >= g.ring) sl -= g.ring;
    return sl;
  };
  auto row = [&](int tok) {
    return *(const uint4*)(key_row(a, b, kvh, ps + tok, slot_of(tok)) + c0);
  };
  hv2 mn[CH / 2], mx[CH / 2];
#pragma unroll
  for (int k = 0; k < CH / 2; ++k) {
    mn[k] = hv2{(_Float16)INFINITY, (_Float16)INFINITY};
    mx[k] = -mn[k];
  }
  auto fold = [&](uint4 r) {
    const hv2* h = (const hv2*)&r;
#pragma unroll
    for (int k = 0; k < CH / 2; ++k) {
      mn[k] = __builtin_elementwise_min(mn[k], h[k]);
      mx[k] = __builtin_elementwise_max(mx[k], h[k]);
    }
  };
  const bool keep = tpq <= KB;                  // uniform
  uint4 xr[KB];
  if (keep) {
#pragma unroll
    for (int u = 0; u < KB; ++u)
      if (valid && u < tpq) xr[u] = row(u);
#pragma unroll
    for (int u = 0; u < KB; ++u)
      if (valid && u < tpq) fold(xr[u]);
  } else if (valid) {
#pragma unroll 8
    for (int tok = 0; tok < tpq; ++tok) fold(row(tok));
  }
  // min/max over the token slices: across the slices of this wave first
  // (lanes cols, 2 cols, ... apart hold the same channels; a wave lies in
  // one group), then across the group's waves through LDS
#pragma unroll
  for (int k = 0; k < CH / 2; ++k)
    for (int o = cols; o < kWave; o <<= 1) {
      const unsigned lo = __shfl_xor(__builtin_bit_cast(unsigned, mn[k]), o);
      const unsigned hi = __shfl_xor(__builtin_bit_cast(unsigned, mx[k]), o);
      mn[k] = __builtin_elementwise_min(mn[k], __builtin_bit_cast(hv2, lo));
      mx[k] = __builtin_elementwise_max(mx[k], __builtin_bit_cast(hv2, hi));
    }
  const int wv = threadIdx.x / kWave;
  unsigned* w_mn = (unsigned*)s_mn;             // [wave][d/2] half2 words
  unsigned* w_mx = (unsigned*)s_mx;
  float* par = s_mn + 256 + sg * 3 * D;         // [3][d]: s, z, RN(1/s)
  if ((threadIdx.x % kWave) < cols) {
#pragma unroll
    for (int k = 0; k < CH / 2; ++k) {
      w_mn[wv * (D / 2) + c0 / 2 + k] = __builtin_bit_cast(unsigned, mn[k]);
      w_mx[wv * (D / 2) + c0 / 2 + k] = __builtin_bit_cast(unsigned, mx[k]);
    }
  }
  __syncthreads();
  for (int c = ti; c < D; c += tps) {           // one thread per channel
    const __half* hmn = (const __half*)w_mn;
    const __half* hmx = (const __half*)w_mx;
    float lo = INFINITY, hi = -INFINITY;
    for (int r = sg * wps; r < (sg + 1) * wps; ++r) {
      lo = fminf(lo, __half2float(hmn[r * D + c]));
      hi = fmaxf(hi, __half2float(hmx[r * D + c]));
    }
    const float sc = stored_scale(lo, hi, Lv);
    par[c] = sc;
    par[D + c] = lo;
    par[2 * D + c] = recip_of(sc);
    if (valid)
      a.p.k_sz[blk * g.ksz_block + (p0 / g.G) * D + c] =
          __halves2half2(__float2half_rn(sc), __float2half_rn(lo));
  }
  __syncthreads();
  float s[CH], z[CH], rs[CH];
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    s[k] = par[c0 + k];
    z[k] = par[D + c0 + k];
    rs[k] = par[2 * D + c0 + k];
  }
  // byte offset of the column's word in a plane row
  uint8_t* hi = a.p.k_hi + blk * g.k_block_bytes + c0 * W / 8;
  uint8_t* lo = BITS == 8 ? a.p.k_lo + blk * g.k_block_bytes + c0 * W / 8 : nullptr;
  auto emit = [&](int tok, uint4 r) {
    const int64_t p = ps + tok;
    const __half* h = (const __half*)&r;
    unsigned bh = 0, bl = 0;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const unsigned q = code_word(__half2float(h[k]), z[k], s[k], rs[k], (float)Lv);
      if constexpr (BITS == 8) {
        bh |= ((q >> 4) & 15u) << (4 * k);
        bl |= (q & 15u) << (4 * k);
      } else {
        bh |= (q & (unsigned)Lv) << (W * k);
      }
    }
    if constexpr (W == 4) {
      *(unsigned*)(hi + p * RB) = bh;
      *(unsigned*)(lo + p * RB) = bl;
    } else if constexpr (W == 2) {
      *(unsigned short*)(hi + p * RB) = (unsigned short)bh;
    } else {
      hi[p * RB] = (uint8_t)bh;
    }
  };
  if (!valid) return;
  if (keep) {
#pragma unroll
    for (int u = 0; u < KB; ++u)
      if (u < tpq) emit(u, xr[u]);
    return;
  }
  // long slices: codes in batches of KB tokens, the batch's rows loaded
  // before its codes are stored (the compiler cannot reorder a load above a
  // store that may alias it, so token-by-token the loads would wait in turn)
  for (int t0 = 0; t0 < tpq; t0 += KB) {
    uint4 xb[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u)
      if (t0 + u < tpq) xb[u] = row(t0 + u);
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if (t0 + u >= tpq) break;
      emit(t0 + u, xb[u]);
    }
  }
}

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS
// operations, not for its outstanding global loads (a full __syncthreads
// would also drain the next tile's prefetched rows).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The value of lane l ^ M (M = 1, 2 or 8) of this wave: one DPP move
// (quad permutations for 1 and 2, a rotation by 8 within each 16-lane row).
template <int M>
__device__ __forceinline__ unsigned lane_xor(unsigned v) {
  static_assert(M == 1 || M == 2 || M == 8, "DPP lane xor");
  constexpr int ctrl = M == 1 ? 0xB1 : M == 2 ? 0x4E : 0x128;
  return (unsigned)__builtin_amdgcn_mov_dpp((int)v, ctrl, 0xF, 0xF, false);
}
// v OR-ed with the value of lane l ^ 16 (the 16-lane rows swapped).
__device__ __forceinline__ unsigned lane_xor16(unsigned v) {
  const auto s = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return s[0] | s[1];
}

// V-tile items: `count` consecutive 32-token tiles from tile `first`, 8
// threads per token; thread (j, u) holds the CPV = D/8 channels u*CPV.. of
// token j, a value group spans Gv/CPV threads whose min/max meet by lane
// shuffles.  Codes are assembled in LDS into the tiled plane layout and
// stored with coalesced dword writes.  The next tile's rows are loaded
// before the current tile is processed, so their latency overlaps it.
template <int D, int W>   // head dim; bits per code in a plane
__device__ __forceinline__ void value_tiles(const AppendArgs& a, int first,
                                            int count, int b, int kvh,
                                            unsigned* lds_hi, unsigned* lds_lo) {
  const CacheGeom& g = a.g;
  constexpr int BITS = W == 4 ? 8 : W;
  constexpr int Lv = (1 << BITS) - 1;
  constexpr int CPV = D / 8;               // channels per thread (8 or 16)
  constexpr int NL = CPV / 8;              // 16-byte row pieces per thread
  constexpr int WORDS = D * W;             // dwords per plane tile
  constexpr int PER = 4 / W;               // 16-channel groups per dword
  // lane xor that steps m % PER (m = c / 16): u for head dim 128, u / 2 for 64
  constexpr int MX1 = D == 128 ? 1 : 2;
  static_assert(PER < 4 || D == 128, "1-bit codes need head dim 128");
  constexpr bool FULL = W == 1;            // whole halves by one lane, no atomics
  const int ng = D / g.Gv;
  const int tpg = g.Gv / CPV;              // threads per value group (1..8)
  const int64_t blk = (int64_t)b * g.Hkv + kvh;
  // thread (j, u): token j, channels u*CPV..  For 8-bit codes wave w takes
  // the tokens j = 4n + w (one i = j % 4 per wave), so the lanes of one LDS
  // atomic meet in a word at most two at a time (h = 0, 1); otherwise a
  // wave takes 8 consecutive tokens, which puts the 4 i of a word in one
  // wave (for 1/2-bit codes the lane combining below relies on that, and
  // it measured faster for 2-bit codes)
  const int u = threadIdx.x % 8;
  const int j = BITS != 8 ? threadIdx.x / 8
                          : 4 * ((threadIdx.x % kWave) / 8) + threadIdx.x / kWave;
  const int c0 = u * CPV, grp = c0 / g.Gv;
  const int gg = (j & 15) >> 2, i = j & 3, h = j >> 4;
  // fp16 channels c0.. of token j of tile tl (appended rows: 16-byte
  // loads; ring rows: the permuted ring layout, one divide for the slot)
  auto load = [&](int tl, uint4 (&xr)[NL]) {
    const int64_t p = a.q0 + (int64_t)tl * kTile + j;
    if (p >= a.new0) {
      const uint4* src = (const uint4*)(
          a.v_new + (((int64_t)b * a.n + (p - a.new0)) * g.Hkv + kvh) * D + c0);
#pragma unroll
      for (int n = 0; n < NL; ++n) xr[n] = src[n];
    } else {
      const int slot = (int)(p % g.ring);
      const __half* base = a.p.v_res + blk * g.res_block +
                           (int64_t)(slot / kTile) * kTile * D;
      unsigned short e[CPV];
#pragma unroll
      for (int k = 0; k < CPV; ++k)
        e[k] = __half_as_ushort(base[vres_index(slot % kTile, c0 + k, D)]);
#pragma unroll
      for (int n = 0; n < NL; ++n)
        xr[n] = uint4{e[8 * n] | (unsigned)e[8 * n + 1] << 16,
                      e[8 * n + 2] | (unsigned)e[8 * n + 3] << 16,
                      e[8 * n + 4] | (unsigned)e[8 * n + 5] << 16,
                      e[8 * n + 6] | (unsigned)e[8 * n + 7] << 16};
    }
  };
  uint4 cur[NL], nxt[NL];
  load(first, cur);
  for (int k = 0; k < count; ++k) {
    const int tl = first + k;
    const int64_t tile = a.q0 / kTile + tl;  // q0 is a multiple of G
    if (k + 1 < count) load(tl + 1, nxt);
    if (k > 0) lds_barrier();              // the last tile's words read out
    if constexpr (!FULL) {                 // atomics OR into cleared words
      for (int w = threadIdx.x; w < WORDS; w += kThreads) {
        lds_hi[w] = 0u;
        if constexpr (BITS == 8) lds_lo[w] = 0u;
      }
    }
    // group min/max: packed fp16 (exact), then across the group's lanes
    hv2 m2 = __builtin_bit_cast(hv2, cur[0].x), x2 = m2;
#pragma unroll
    for (int n = 0; n < NL; ++n) {
      const hv2* hp = (const hv2*)&cur[n];
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        m2 = __builtin_elementwise_min(m2, hp[k2]);
        x2 = __builtin_elementwise_max(x2, hp[k2]);
      }
    }
    float mn = fminf((float)m2[0], (float)m2[1]);
    float mx = fmaxf((float)x2[0], (float)x2[1]);
    for (int o = 1; o < tpg; o <<= 1) {    // lanes of one group: aligned runs
      mn = fminf(mn, __shfl_xor(mn, o));
      mx = fmaxf(mx, __shfl_xor(mx, o));
    }
    const float z = mn, sc = stored_scale(mn, mx, Lv), rs = recip_of(sc);
    if (u % tpg == 0) {
      // [part][g][i][group][h]: scale plane then zero-point plane
      __half* sz = (__half*)(a.p.v_sz + blk * g.vsz_block + tile * g.vsz_tile);
      const int at = ((gg * 4 + i) * ng + grp) * 2 + h;
      sz[at] = __float2half_rn(sc);
      sz[32 * ng + at] = __float2half_rn(z);
    }
    // Each half (h) of a tile dword holds the codes of the 4 tokens i of one
    // (g, h) and the PER channel groups m % PER of one channel r: lanes of
    // this wave that differ in i (lane bits 3-4) and in m % PER (lane bits
    // from MX1).  With 1-bit codes (16 lanes per half) the contributions are
    // OR-ed across those lanes and one lane writes the whole half, so no
    // word needs clearing or an atomic update; with 2-bit codes they are
    // OR-ed across m % PER and the 4 lanes left OR theirs into the cleared
    // word; 8-bit codes go to LDS by atomic OR directly (4 lanes per word:
    // there the lane moves cost more than the atomics' conflicts).
    if constexpr (!FULL) lds_barrier();    // cleared words for the atomics
    const __half* hx = (const __half*)cur;
    const bool lead_m = PER == 1 || (threadIdx.x & (MX1 * (PER - 1))) == 0;
#pragma unroll
    for (int k2 = 0; k2 < CPV; ++k2) {
      const int c = c0 + k2;
      const unsigned q = code_word(__half2float(hx[k2]), z, sc, rs, (float)Lv) & 255u;
      const int r = c & 15, m = c >> 4;
      const int dw = (16 * gg + r) * (D * W / 64) + m / PER;
      const int pos = W * (4 * (m % PER) + i);
      if constexpr (BITS == 8) {
        atomicOr(&lds_hi[dw], (q >> 4) << (16 * h + pos));
        atomicOr(&lds_lo[dw], (q & 15u) << (16 * h + pos));
      } else {
        unsigned v = q << pos;
        if constexpr (PER >= 2) v |= lane_xor<MX1>(v);
        if constexpr (PER == 4) v |= lane_xor<2 * MX1>(v);
        if constexpr (FULL) {
          v |= lane_xor<8>(v);
          v |= lane_xor16(v);
          if (i == 0 && lead_m) ((unsigned short*)lds_hi)[2 * dw + h] = (unsigned short)v;
        } else if (lead_m) {
          atomicOr(&lds_hi[dw], v << (16 * h));
        }
      }
    }
    lds_barrier();                           // the tile's words complete
    unsigned* ghi = (unsigned*)(a.p.v_hi + blk * g.v_block_bytes +
                                tile * g.v_tile_bytes);
    unsigned* glo = (unsigned*)(a.p.v_lo + blk * g.v_block_bytes +
                                tile * g.v_tile_bytes);
    for (int w = threadIdx.x; w < WORDS; w += kThreads) {
      ghi[w] = lds_hi[w];
      if constexpr (BITS == 8) glo[w] = lds_lo[w];
    }
    if (k + 1 < count) {
#pragma unroll
      for (int n = 0; n < NL; ++n) cur[n] = nxt[n];
    }
  }
}

__device__ __forceinline__ void ring_token(const AppendArgs& a, int item, int b, int kvh) {
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

// One kernel per (head dim, code width, key groups per item): a launch runs
// only its own item code (a single kernel holding every instantiation
// measured slower on the low-bit fills).  The 8-bit and 1-bit kernels are
// held to 96 VGPRs for five waves per SIMD (117 and 107 unconstrained, four
// waves): the registers spilled cost less than the fifth wave gains (32K
// prefill 54.0 against 56.1 us, batched 1-bit fill 1.33 against 1.40 ms);
// the 2-bit kernels (108) keep four, where five measured 1-2% slower.
template <int D, int W, int NGI>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(W == 2 ? 4 : 5)))
append_kernel(AppendArgs a, Item it) {
  __shared__ unsigned lds_hi[128 * 4];
  __shared__ unsigned lds_lo[128 * 4];
  // K groups: the waves' fp16 min/max words, then the channels' (s, z, 1/s)
  __shared__ float s_mn[256 + 4 * 3 * 128], s_mx[256];
  const int b = blockIdx.z, kvh = blockIdx.y;
  int x = blockIdx.x;
  if (x < it.k_items) {
    key_group<D, W, NGI>(a, x, b, kvh, s_mn, s_mx);
    return;
  }
  x -= it.k_items;
  if (x < it.v_items) {
    const int first = x * it.vt;
    const int count = min(it.vt, it.v_tiles - first);
    value_tiles<D, W>(a, first, count, b, kvh, lds_hi, lds_lo);
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

template <int D, int W, int NGI>
hipError_t go(const AppendArgs& a, const Item& it, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((append_kernel<D, W, NGI>), grid, dim3(kThreads), 0, s, a, it);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, bool flush, bool ring_write,
                         hipStream_t s) {
  Item it;
  const int ngi = kgroups_per_item(a.g.d, a.g.G);
  it.k_items = flush ? (int)cdiv(a.groups, ngi) : 0;
  it.v_tiles = flush ? (int)((int64_t)a.groups * a.g.G / kTile) : 0;
  it.r_tokens = ring_write ? a.wr_count : 0;
  it.vt = it.v_tiles >= 64 ? 4 : 1;
  it.rt = it.r_tokens >= 64 ? 8 : 1;
  it.v_items = (int)cdiv(it.v_tiles, it.vt);
  it.ring_items = (int)cdiv(it.r_tokens, it.rt);
  const int64_t nx = (int64_t)it.k_items + it.v_items + it.ring_items;
  if (nx == 0) return hipSuccess;
  const dim3 grid((unsigned)nx, a.g.Hkv, a.g.B);
  const int w = a.g.w;
  if (a.g.d == 64) {                  // 8-bit or 2-bit codes, one group per item
    if (w == 4) return go<64, 4, 1>(a, it, grid, s);
    if (w == 2) return go<64, 2, 1>(a, it, grid, s);
    return hipErrorInvalidValue;
  }
  if (a.g.d != 128) return hipErrorInvalidValue;
  if (ngi == 4) {
    if (w == 4) return go<128, 4, 4>(a, it, grid, s);
    if (w == 2) return go<128, 2, 4>(a, it, grid, s);
    return go<128, 1, 4>(a, it, grid, s);
  }
  if (ngi == 2) {
    if (w == 4) return go<128, 4, 2>(a, it, grid, s);
    if (w == 2) return go<128, 2, 2>(a, it, grid, s);
    return go<128, 1, 2>(a, it, grid, s);
  }
  if (w == 4) return go<128, 4, 1>(a, it, grid, s);
  if (w == 2) return go<128, 2, 1>(a, it, grid, s);
  return go<128, 1, 1>(a, it, grid, s);
}

}  // namespace kvq
