// Split-K decode/verify attention read directly from the quantized cache.
//
// QuantSpec page, Approach: the draft attends over the upper-4-bit codes, the
// target verifies gamma+1 tokens over the 8-bit codes plus the fp16 buffer of
// recent tokens; Experimental setup, "Builds on: FlashDecoding" (split the
// context across workgroups, merge partial softmax statistics by
// log-sum-exp).  SpeCache page, Approach: output + speculative token (T = 2)
// over a 1/2-bit KIVI copy.
//
// Work decomposition (grid = splits x Hkv x B, 4 waves per workgroup):
//   * quantized splits: each wave walks a run of 32-token tiles of the
//     quantized prefix; residual splits: each wave takes one 32-slot tile of
//     the fp16 ring (where the causal mask among the T query tokens lives).
//   * per tile the wave computes S^T = K * Q'^T on MFMA (16x16x32 f16, two
//     16-token subtiles x up to two 16-row tiles), runs the online softmax on
//     the S^T accumulators in place, and feeds P'^T straight back as the B
//     operand of O^T += V^T * P'^T: the accumulator layout of the score MFMA
//     (lane = row, 4 consecutive tokens) is exactly the operand layout the PV
//     MFMA needs once the V tile is stored token-permuted, so no data crosses
//     lanes.  Rows are query tokens x GQA heads (T * Hq/Hkv <= 32).
//   * codes are turned into fp16 MFMA operands in registers with the
//     "0x6400 | code" trick (fp16 1024 + code); per-channel key scales are
//     folded into Q' = q * s * sm_scale * log2(e) once per key group, kept as
//     two fp16 parts (hi + lo, two MFMAs) so the scores carry ~22 bits of Q'
//     (one fp16 part alone moves outlier-channel logits by ~1e-2); the 1024
//     offset and the zero-points go into the accumulator's initial value; per-
//     token value scales are folded into P' = p * s * 2^10 and value zero-
//     points into a per-row fp32 side sum.
//   * the 4 waves merge in registers through LDS, write one partial
//     (m, l, o) per workgroup, and the last workgroup of each (b, kvh) block
//     (atomic ticket, self-resetting) merges all partials and writes fp16
//     output and the natural-log LSE.
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef unsigned u4v __attribute__((ext_vector_type(4)));

constexpr int NW = 4;
constexpr int NT = NW * kWave;
constexpr unsigned kMagic = 0x64006400u;       // fp16 pair (1024, 1024)
constexpr unsigned kMinus1024 = 0xE400E400u;   // fp16 pair (-1024, -1024)
constexpr unsigned kMinusDraft = 0xE3F1E3F1u;  // fp16 pair (-1016.5, -1016.5)
constexpr float kPScale = 1024.f;              // P' = p * s * 2^10
constexpr float kLn2 = 0.693147180559945309f;

enum Path { P_T8 = 0, P_D4 = 1, P_L2 = 2, P_L1 = 3 };

__device__ __forceinline__ f4v mfma16(u4v a, u4v b, f4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(
      __builtin_bit_cast(h8v, a), __builtin_bit_cast(h8v, b), c, 0, 0, 0);
}

__device__ __forceinline__ unsigned hadd2(unsigned x, unsigned y) {
  h2v r = __builtin_bit_cast(h2v, x) + __builtin_bit_cast(h2v, y);
  return __builtin_bit_cast(unsigned, r);
}

__device__ __forceinline__ unsigned pack2(float lo, float hi) {
  h2v r;
  r[0] = (_Float16)lo;
  r[1] = (_Float16)hi;
  return __builtin_bit_cast(unsigned, r);
}

__device__ __forceinline__ float h_lo(unsigned x) {
  return (float)__builtin_bit_cast(h2v, x)[0];
}
__device__ __forceinline__ float h_hi(unsigned x) {
  return (float)__builtin_bit_cast(h2v, x)[1];
}

// The fp32 value as materialised in a register.  Splitting x into fp16
// hi = fp16(x) and lo = fp16(x - hi) needs both parts to see the same x,
// but the compiler may fold a product feeding an fp16 conversion into one
// mixed-precision FMA (v_fma_mixlo_f16, a single rounding of the exact
// product) for one use and round the fp32 product for the other; on an
// fp16 rounding midpoint the two differ and lo gets the wrong sign.
__device__ __forceinline__ float opaque(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

__device__ __forceinline__ float xor_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}
__device__ __forceinline__ float xor_sum(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

// 8-bit codes split over a hi and a lo nibble dword (nibble n = channel or
// token n of the dword).  Pair j = nibbles (j, j+4) as fp16 (1024 + code).
__device__ __forceinline__ void dec8(unsigned H, unsigned L, unsigned* r) {
  const unsigned ce = ((H << 4) & 0xF0F0F0F0u) | (L & 0x0F0F0F0Fu);
  const unsigned co = (H & 0xF0F0F0F0u) | ((L >> 4) & 0x0F0F0F0Fu);
  r[0] = (ce & 0x00FF00FFu) | kMagic;
  r[1] = (co & 0x00FF00FFu) | kMagic;
  r[2] = ((ce >> 8) & 0x00FF00FFu) | kMagic;
  r[3] = ((co >> 8) & 0x00FF00FFu) | kMagic;
}

// Upper nibbles only: pair j = nibbles (j, j+4) as fp16 (1024 + 16*hi).
__device__ __forceinline__ void dec4(unsigned H, unsigned* r) {
  r[0] = ((H << 4) & 0x00F000F0u) | kMagic;
  r[1] = (H & 0x00F000F0u) | kMagic;
  r[2] = ((H >> 4) & 0x00F000F0u) | kMagic;
  r[3] = ((H >> 8) & 0x00F000F0u) | kMagic;
}

// W-bit codes: the pair at bits (W*i, 16 + W*i) as exact fp16 codes.
template <int W>
__device__ __forceinline__ unsigned declow(unsigned H, int i) {
  constexpr unsigned mask = ((1u << W) - 1u) * 0x00010001u;
  return hadd2(((H >> (W * i)) & mask) | kMagic, kMinus1024);
}

template <int N>
__device__ __forceinline__ void ldg(const void* p, unsigned* o) {
  if constexpr (N == 1) {
    o[0] = *(const unsigned*)p;
  } else if constexpr (N == 2) {
    uint2 v = *(const uint2*)p;
    o[0] = v.x; o[1] = v.y;
  } else {
    static_assert(N % 4 == 0, "dword count");
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
      uint4 v = ((const uint4*)p)[k];
      o[4 * k] = v.x; o[4 * k + 1] = v.y; o[4 * k + 2] = v.z; o[4 * k + 3] = v.w;
    }
  }
}

template <int PATH, int D, int NRT, int NG>
struct Cfg {
  static constexpr int W = PATH == P_L2 ? 2 : PATH == P_L1 ? 1 : 4;
  static constexpr bool TWO = PATH == P_T8;   // hi + lo planes
  static constexpr int KS = D / 32;           // MFMA k-steps per subtile
  static constexpr int NDK = D * W / 128;     // K dwords / lane / plane / subtile
  static constexpr int NDV = D * W / 64;      // V dwords / lane / plane / tile
  static constexpr int MT = D / 16;           // 16-channel output tiles
  static constexpr int PERK = 16 / W;         // code pairs per K dword
  static constexpr int RP = 16 * NRT;         // padded rows
  static constexpr int NSZ = 8 * NG;          // V scale dwords / lane / tile
  static constexpr float KBIAS =
      PATH == P_T8 ? 1024.f : PATH == P_D4 ? 1016.5f : 0.f;
};

template <class C>
struct QTile {
  unsigned kh[2][C::NDK];
  unsigned kl[2][C::TWO ? C::NDK : 1];
  unsigned vh[C::NDV];
  unsigned vl[C::TWO ? C::NDV : 1];
  unsigned sz[C::NSZ];
};

template <int PATH, int D, int NRT, int NG>
__global__ void __launch_bounds__(NT) attn_kernel(const AttnArgs a) {
  using C = Cfg<PATH, D, NRT, NG>;
  constexpr int RP = C::RP;
  __shared__ __align__(16) __half s_q[RP * D];
  __shared__ __align__(16) float s_slab[2 * RP * D];
  __shared__ float s_ml[2 * 2 * RP];
  __shared__ int s_flag;

  const CacheGeom& g = a.g;
  const int b = blockIdx.z, kvh = blockIdx.y, split = blockIdx.x;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int l16 = lane & 15, gq = lane >> 4;
  const int64_t blk = (int64_t)b * g.Hkv + kvh;
  const int S = a.s_q + a.s_r;
  const int64_t L = a.n_q + a.n_r;

  // ---- stage this block's query rows in LDS (row = t * gs + head-in-group)
  for (int e = tid; e < RP * D; e += NT) {
    const int row = e / D, c = e % D;
    __half v = __float2half(0.f);
    if (row < a.rows) {
      const int t = row / a.gs, hl = row % a.gs;
      v = a.q[(((int64_t)b * a.T + t) * a.Hq + kvh * a.gs + hl) * D + c];
    }
    s_q[e] = v;
  }
  __syncthreads();

  float m_run[NRT], l_run[NRT];
  f4v acc[NRT][C::MT];
  float zacc[NRT][NG];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) acc[rt][mt] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) zacc[rt][gg] = 0.f;
  }
  const bool residual = split >= a.s_q;
  float oscale = 1.f;

  // Online-softmax update of row tile rt from the S^T accumulators of the
  // two subtiles; returns the probabilities in place.
  auto softmax_update = [&](int rt, f4v& s0, f4v& s1) {
    float mx = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                     fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
    mx = xor_max(mx);
    const float mnew = fmaxf(m_run[rt], mx);
    const float mref = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = fast_exp2(m_run[rt] - mref);
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s0[i] = fast_exp2(s0[i] - mref);
      s1[i] = fast_exp2(s1[i] - mref);
      ps += s0[i] + s1[i];
    }
    l_run[rt] = l_run[rt] * alpha + ps;
    m_run[rt] = mnew;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) acc[rt][mt] *= alpha;
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) zacc[rt][gg] *= alpha;
    }
  };

  if (!residual) {
    // ================= quantized prefix ===================================
    oscale = 1.f / kPScale;
    const int64_t nqt = a.n_q / kTile;
    const int64_t t0 = (int64_t)split * NW * a.tpw + (int64_t)wave * a.tpw;
    const int64_t t1 = t0 + a.tpw < nqt ? t0 + a.tpw : nqt;
    const uint8_t* kh_base = a.p.k_hi + blk * g.k_block_bytes;
    const uint8_t* kl_base = C::TWO ? a.p.k_lo + blk * g.k_block_bytes : nullptr;
    const uint8_t* vh_base = a.p.v_hi + blk * g.v_block_bytes;
    const uint8_t* vl_base = C::TWO ? a.p.v_lo + blk * g.v_block_bytes : nullptr;
    const __half2* vsz_base = a.p.v_sz + blk * g.vsz_block;
    const __half2* ksz_base = a.p.k_sz + blk * g.ksz_block;
    const int64_t krow = D * C::W / 8;
    const int kofs = gq * (D * C::W / 32);
    const int vofs = lane * (D * C::W / 16);

    auto load_tile = [&](QTile<C>& tl, int64_t t) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int64_t tok = t * kTile + 16 * st + l16;
        ldg<C::NDK>(kh_base + tok * krow + kofs, tl.kh[st]);
        if constexpr (C::TWO) ldg<C::NDK>(kl_base + tok * krow + kofs, tl.kl[st]);
      }
      ldg<C::NDV>(vh_base + t * g.v_tile_bytes + vofs, tl.vh);
      if constexpr (C::TWO) ldg<C::NDV>(vl_base + t * g.v_tile_bytes + vofs, tl.vl);
      ldg<C::NSZ>(vsz_base + t * g.vsz_tile + gq * C::NSZ, tl.sz);
    };

    u4v bq[NRT][C::KS], bql[NRT][C::KS];   // Q' = hi + lo (two fp16 parts)
    float bias[NRT];
    int64_t cur_group = -1;

    // Q' and the accumulator's initial value for key group kg.
    auto prepare_group = [&](int64_t kg) {
      unsigned sz[D / 4];
      ldg<D / 4>(ksz_base + kg * D + gq * (D / 4), sz);
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const __half* qr = s_q + (l16 + 16 * rt) * D + gq * (D / 4);
        float sum_q = 0.f, sum_z = 0.f;
#pragma unroll
        for (int p = 0; p < D / 8; ++p) {
          const int ca = (p / C::PERK) * 2 * C::PERK + p % C::PERK;
          const int cb = ca + C::PERK;
          const float qa = __half2float(qr[ca]) * a.c0;
          const float qb = __half2float(qr[cb]) * a.c0;
          const float xa = opaque(qa * h_lo(sz[ca]));
          const float xb = opaque(qb * h_lo(sz[cb]));
          const unsigned hi = pack2(xa, xb);
          const unsigned lo = pack2(xa - h_lo(hi), xb - h_hi(hi));
          bq[rt][p / 4][p % 4] = hi;
          bql[rt][p / 4][p % 4] = lo;
          sum_q += (h_lo(hi) + h_hi(hi)) + (h_lo(lo) + h_hi(lo));
          sum_z += qa * h_hi(sz[ca]) + qb * h_hi(sz[cb]);
        }
        bias[rt] = xor_sum(sum_z) - C::KBIAS * xor_sum(sum_q);
      }
    };

    auto compute_tile = [&](const QTile<C>& tl, int64_t t) {
      const int64_t kg = t * kTile / g.G;
      if (kg != cur_group) {
        prepare_group(kg);
        cur_group = kg;
      }
      // ---- scores S^T = K Q'^T
      f4v sc[2][NRT];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        u4v ak[C::KS];
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          unsigned r[4];
          if constexpr (PATH == P_T8) {
            dec8(tl.kh[st][ks], tl.kl[st][ks], r);
          } else if constexpr (PATH == P_D4) {
            dec4(tl.kh[st][ks], r);
          } else {
            constexpr int KPD = C::PERK / 4;   // k-steps per dword
#pragma unroll
            for (int j = 0; j < 4; ++j)
              r[j] = declow<C::W>(tl.kh[st][ks / KPD], 4 * (ks % KPD) + j);
          }
          ak[ks] = u4v{r[0], r[1], r[2], r[3]};
        }
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          f4v s = f4v{bias[rt], bias[rt], bias[rt], bias[rt]};
#pragma unroll
          for (int ks = 0; ks < C::KS; ++ks) {
            s = mfma16(ak[ks], bq[rt][ks], s);
            s = mfma16(ak[ks], bql[rt][ks], s);
          }
          sc[st][rt] = s;
        }
      }
      // ---- softmax and P' = p * s_v * 2^10 for every row tile
      u4v bp[NRT][NG];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        softmax_update(rt, sc[0][rt], sc[1][rt]);
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
          float zs = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const unsigned s_lo = tl.sz[i * NG + gg];        // token 4gq+i
            const unsigned s_hi = tl.sz[(4 + i) * NG + gg];  // token 16+4gq+i
            bp[rt][gg][i] = pack2(sc[0][rt][i] * (h_lo(s_lo) * kPScale),
                                  sc[1][rt][i] * (h_lo(s_hi) * kPScale));
            zs += sc[0][rt][i] * h_hi(s_lo) + sc[1][rt][i] * h_hi(s_hi);
          }
          zacc[rt][gg] += zs;
        }
      }
      // ---- O^T += V^T P'^T, one 16-channel tile of exact codes at a time
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) {
        unsigned r[4];
        if constexpr (PATH == P_T8) {
          dec8(tl.vh[mt], tl.vl[mt], r);
#pragma unroll
          for (int j = 0; j < 4; ++j) r[j] = hadd2(r[j], kMinus1024);
        } else if constexpr (PATH == P_D4) {
          dec4(tl.vh[mt], r);
#pragma unroll
          for (int j = 0; j < 4; ++j) r[j] = hadd2(r[j], kMinusDraft);
        } else {
          constexpr int PER = 4 / C::W;   // channel tiles per dword
#pragma unroll
          for (int j = 0; j < 4; ++j)
            r[j] = declow<C::W>(tl.vh[mt / PER], 4 * (mt % PER) + j);
        }
        const u4v av = u4v{r[0], r[1], r[2], r[3]};
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
          acc[rt][mt] = mfma16(av, bp[rt][mt / (C::MT / NG)], acc[rt][mt]);
      }
    };

    if (t0 < t1) {
      QTile<C> ta, tb;
      load_tile(ta, t0);
      int64_t t = t0;
      while (true) {
        if (t + 1 < t1) load_tile(tb, t + 1);
        compute_tile(ta, t);
        if (++t >= t1) break;
        if (t + 1 < t1) load_tile(ta, t + 1);
        compute_tile(tb, t);
        if (++t >= t1) break;
      }
    }
  } else {
    // ================= fp16 residual ring ==================================
    const int64_t ti = (int64_t)(split - a.s_q) * NW + wave;
    const int64_t nrt = cdiv(a.n_r, kTile);
    if (ti < nrt) {
      const int64_t p0 = a.n_q + ti * kTile;           // first position
      const int64_t slot0 = p0 % g.ring;               // 32-aligned slot
      u4v bq[NRT][C::KS], bql[NRT][C::KS];   // q * c0 = hi + lo
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const __half* qr = s_q + (l16 + 16 * rt) * D + gq * (D / 4);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float xa = opaque(__half2float(qr[8 * ks + 2 * j]) * a.c0);
            const float xb =
                opaque(__half2float(qr[8 * ks + 2 * j + 1]) * a.c0);
            const unsigned hi = pack2(xa, xb);
            bq[rt][ks][j] = hi;
            bql[rt][ks][j] = pack2(xa - h_lo(hi), xb - h_hi(hi));
          }
      }
      const __half* kres = a.p.k_res + blk * g.res_block;
      f4v sc[2][NRT];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        unsigned kd[D / 8];
        ldg<D / 8>(kres + (slot0 + 16 * st + l16) * D + gq * (D / 4), kd);
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          f4v s = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < C::KS; ++ks) {
            const u4v ka = u4v{kd[4 * ks], kd[4 * ks + 1], kd[4 * ks + 2],
                               kd[4 * ks + 3]};
            s = mfma16(ka, bq[rt][ks], s);
            s = mfma16(ka, bql[rt][ks], s);
          }
          // causal / validity mask: row sees positions <= L - T + t(row)
          const int row = l16 + 16 * rt;
          const int64_t lim =
              row < a.rows ? L - a.T + row / a.gs : L - 1;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t pos = p0 + 16 * st + 4 * gq + i;
            s[i] = pos <= lim ? s[i] : -INFINITY;
          }
          sc[st][rt] = s;
        }
      }
      // V tile (token-permuted fp16), zero the slots past the context
      unsigned vd[D / 4];
      ldg<D / 4>(a.p.v_res + blk * g.res_block + (slot0 / kTile) * kTile * D +
                     lane * (D / 2),
                 vd);
      if (p0 + kTile > L) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const unsigned keep =
              (p0 + 4 * gq + i < L ? 0x0000FFFFu : 0u) |
              (p0 + 16 + 4 * gq + i < L ? 0xFFFF0000u : 0u);
#pragma unroll
          for (int mt = 0; mt < C::MT; ++mt) vd[4 * mt + i] &= keep;
        }
      }
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        softmax_update(rt, sc[0][rt], sc[1][rt]);
        u4v bp;
#pragma unroll
        for (int i = 0; i < 4; ++i) bp[i] = pack2(sc[0][rt][i], sc[1][rt][i]);
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
          acc[rt][mt] = mfma16(
              u4v{vd[4 * mt], vd[4 * mt + 1], vd[4 * mt + 2], vd[4 * mt + 3]},
              bp, acc[rt][mt]);
      }
    }
  }

  // ---- per-wave finish: full-row l, zero-point term folded into o
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    l_run[rt] = xor_sum(l_run[rt]);
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) zacc[rt][gg] = xor_sum(zacc[rt][gg]);
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
      acc[rt][mt] = acc[rt][mt] * oscale + zacc[rt][mt / (C::MT / NG)];
  }

  // ---- merge the 4 waves through LDS: (2,3) -> (0,1), then 1 -> 0
  auto put = [&](int slot) {
    float* o = s_slab + slot * RP * D;
    float* ml = s_ml + slot * 2 * RP;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const int row = l16 + 16 * rt;
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
        *(f4v*)(o + row * D + 16 * mt + 4 * gq) = acc[rt][mt];
      if (gq == 0) {
        ml[row] = m_run[rt];
        ml[RP + row] = l_run[rt];
      }
    }
  };
  auto take = [&](int slot) {
    const float* o = s_slab + slot * RP * D;
    const float* ml = s_ml + slot * 2 * RP;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const int row = l16 + 16 * rt;
      const float mo = ml[row], lo = ml[RP + row];
      const float M = fmaxf(m_run[rt], mo);
      const float fa = M == -INFINITY ? 0.f : fast_exp2(m_run[rt] - M);
      const float fb = M == -INFINITY ? 0.f : fast_exp2(mo - M);
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
        acc[rt][mt] = acc[rt][mt] * fa +
                      *(const f4v*)(o + row * D + 16 * mt + 4 * gq) * fb;
      l_run[rt] = l_run[rt] * fa + lo * fb;
      m_run[rt] = M;
    }
  };
  if (wave >= 2) put(wave - 2);
  __syncthreads();
  if (wave < 2) take(wave);
  __syncthreads();
  if (wave == 1) put(0);
  __syncthreads();
  if (wave == 0) take(0);

  // ---- workgroup partial: o[RP][D], m[RP], l[RP]
  const int64_t pstride = (int64_t)RP * (D + 2);
  float* pblk = a.ws + blk * a.s_alloc * pstride;
  if (wave == 0) {
    float* po = pblk + split * pstride;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const int row = l16 + 16 * rt;
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
        *(f4v*)(po + row * D + 16 * mt + 4 * gq) = acc[rt][mt];
      if (gq == 0) {
        po[RP * D + row] = m_run[rt];
        po[RP * D + RP + row] = l_run[rt];
      }
    }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = atomicAdd(&a.tickets[blk], 1u);
    s_flag = prev == (unsigned)(S - 1);
  }
  __syncthreads();
  if (!s_flag) return;
  __threadfence();

  // ---- last workgroup of the block: log-sum-exp merge of all partials
  float* wts = s_slab;   // [S][RP] weights, then M and sum per row
  for (int row = tid; row < a.rows; row += NT) {
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, pblk[s * pstride + RP * D + row]);
    float lsum = 0.f;
    for (int s = 0; s < S; ++s) {
      const float* ps = pblk + s * pstride + RP * D;
      const float e = ps[row] == -INFINITY ? 0.f : fast_exp2(ps[row] - M);
      wts[s * RP + row] = e;
      lsum += ps[RP + row] * e;
    }
    const float inv = 1.f / lsum;
    for (int s = 0; s < S; ++s) wts[s * RP + row] *= inv;
    if (a.lse) {
      const int t = row / a.gs, h = kvh * a.gs + row % a.gs;
      a.lse[((int64_t)b * a.Hq + h) * a.T + t] = (M + __log2f(lsum)) * kLn2;
    }
  }
  __syncthreads();
  for (int e = tid; e < a.rows * D; e += NT) {
    const int row = e / D, c = e % D;
    float o = 0.f;
    for (int s = 0; s < S; ++s)
      o += wts[s * RP + row] * pblk[s * pstride + row * D + c];
    const int t = row / a.gs, h = kvh * a.gs + row % a.gs;
    a.out[(((int64_t)b * a.T + t) * a.Hq + h) * D + c] = __float2half(o);
  }
  if (tid == 0) a.tickets[blk] = 0u;
}

template <int PATH, int D, int NRT, int NG>
hipError_t go(const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.s_q + a.s_r, a.g.Hkv, a.g.B);
  hipLaunchKernelGGL((attn_kernel<PATH, D, NRT, NG>), grid, dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <int PATH, int D, int NRT>
hipError_t by_ng(const AttnArgs& a, hipStream_t s) {
  switch (a.g.d / a.g.Gv) {
    case 1: return go<PATH, D, NRT, 1>(a, s);
    case 2: return go<PATH, D, NRT, 2>(a, s);
    case 4: return go<PATH, D, NRT, 4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int PATH, int D>
hipError_t by_rows(const AttnArgs& a, hipStream_t s) {
  return a.rows_pad == 16 ? by_ng<PATH, D, 1>(a, s) : by_ng<PATH, D, 2>(a, s);
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  const int bits = a.g.bits, d = a.g.d;
  if (bits == 8 && a.path == KVQ_DRAFT4)
    return d == 64 ? by_rows<P_D4, 64>(a, s) : by_rows<P_D4, 128>(a, s);
  if (bits == 8)
    return d == 64 ? by_rows<P_T8, 64>(a, s) : by_rows<P_T8, 128>(a, s);
  if (bits == 2)
    return d == 64 ? by_rows<P_L2, 64>(a, s) : by_rows<P_L2, 128>(a, s);
  if (bits == 1 && d == 128) return by_rows<P_L1, 128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace kvq
