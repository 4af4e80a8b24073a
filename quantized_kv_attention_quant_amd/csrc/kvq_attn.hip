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
//   * the 4 waves merge in registers through LDS and write one partial
//     (m, l, o) per workgroup.  A second launch, one workgroup per (block,
//     row), merges that row's partials by log-sum-exp in parallel (fp16
//     output, natural-log LSE); the kernel boundary makes the partials
//     visible, so the split kernel needs no device-scope fence or ticket.
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
constexpr float kPExp = 10.f;                  // P' = p * s * 2^10
constexpr float kPScale = 1024.f;
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

// Reductions over the four 16-lane groups of a wave (lanes l, l^16, l^32,
// l^48), with the ds_bpermute byte addresses computed once by the caller.
__device__ __forceinline__ float bperm(int addr, float v) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(v)));
}
__device__ __forceinline__ float xor_max(float v, int a16, int a32) {
  v = fmaxf(v, bperm(a16, v));
  return fmaxf(v, bperm(a32, v));
}
__device__ __forceinline__ float xor_sum(float v, int a16, int a32) {
  v += bperm(a16, v);
  return v + bperm(a32, v);
}

// Decode constants held in registers: gfx9 VOP3 forms (v_and_or_b32,
// v_bfi_b32, v_perm_b32) cannot encode literal constants, so with literals
// the compiler splits every and-or into two instructions.
struct DecK {
  unsigned magic;    // fp16 pair (1024, 1024), VGPR
  unsigned magic_b;  // 0x64 in every byte, VGPR (v_perm source)
  unsigned m_f0;     // 0x00F000F0
  unsigned m_hi;     // 0xF0F0F0F0
};

__device__ __forceinline__ unsigned vreg(unsigned x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ DecK dec_consts() {
  DecK k;
  k.magic = vreg(kMagic);
  k.magic_b = vreg(0x64646464u);
  k.m_f0 = __builtin_amdgcn_readfirstlane(vreg(0x00F000F0u));
  k.m_hi = __builtin_amdgcn_readfirstlane(vreg(0xF0F0F0F0u));
  return k;
}

// 8-bit codes split over a hi and a lo nibble dword (nibble n = channel or
// token n of the dword).  Pair j = nibbles (j, j+4) as fp16 (1024 + code):
// two bit-field inserts build the bytes hi<<4|lo of the even and odd
// nibbles, four byte permutes place them under the 0x64 exponent byte.
__device__ __forceinline__ void dec8(unsigned H, unsigned L, unsigned* r,
                                     const DecK& k) {
  const unsigned ce = (k.m_hi & (H << 4)) | (~k.m_hi & L);
  const unsigned co = (k.m_hi & H) | (~k.m_hi & (L >> 4));
  r[0] = __builtin_amdgcn_perm(k.magic_b, ce, 0x05020500u);
  r[1] = __builtin_amdgcn_perm(k.magic_b, co, 0x05020500u);
  r[2] = __builtin_amdgcn_perm(k.magic_b, ce, 0x05030501u);
  r[3] = __builtin_amdgcn_perm(k.magic_b, co, 0x05030501u);
}

// Upper nibbles only: pair j = nibbles (j, j+4) as fp16 (1024 + 16*hi).
__device__ __forceinline__ void dec4(unsigned H, unsigned* r, const DecK& k) {
  r[0] = ((H << 4) & k.m_f0) | k.magic;
  r[1] = (H & k.m_f0) | k.magic;
  r[2] = ((H >> 4) & k.m_f0) | k.magic;
  r[3] = ((H >> 8) & k.m_f0) | k.magic;
}

// W-bit codes: the pair at bits (W*i, 16 + W*i) as exact fp16 codes.
template <int W>
__device__ __forceinline__ unsigned declow(unsigned H, int i, const DecK& k) {
  constexpr unsigned mask = ((1u << W) - 1u) * 0x00010001u;
  return hadd2(((H >> (W * i)) & mask) | k.magic, kMinus1024);
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

// Merge kernel, one workgroup per (block, row): combines the row's S split
// partials by log-sum-exp with every thread busy: per-split (m, l) into LDS,
// wave reductions for the row max and sum, then the o rows summed by NT/D
// thread groups, each with 8 loads in flight.  Runs as a second launch so
// the partials are visible without device-scope fences in the split kernel.
template <int D, int RP>
__global__ void __launch_bounds__(NT) merge_kernel(const AttnArgs a) {
  constexpr int NPART = NT / D;          // thread groups over the splits
  __shared__ float lds[2 * 1024 + 8 + NT];
  const int S = a.s_q + a.s_r;
  const int64_t blk = blockIdx.x / a.rows;
  const int row = (int)(blockIdx.x % a.rows);
  const int tid = threadIdx.x, wave = tid / kWave;
  const int64_t pstride = (int64_t)RP * (D + 2);
  const float* pblk = a.ws + blk * a.s_alloc * pstride;
  float* sm = lds;              // [S] m, then weights
  float* sl = lds + S;          // [S] l
  float* red = lds + 2 * S;     // [8] wave partials
  float* part = red + 8;        // [NPART][D]
  for (int s = tid; s < S; s += NT) {
    sm[s] = pblk[s * pstride + RP * D + row];
    sl[s] = pblk[s * pstride + RP * D + RP + row];
  }
  __syncthreads();
  float M = -INFINITY;
  for (int s = tid; s < S; s += NT) M = fmaxf(M, sm[s]);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
  if ((tid & (kWave - 1)) == 0) red[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float ls = 0.f;
  for (int s = tid; s < S; s += NT) {
    const float e = sm[s] == -INFINITY ? 0.f : fast_exp2(sm[s] - M);
    sm[s] = e;
    ls += sl[s] * e;
  }
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) ls += __shfl_xor(ls, o);
  if ((tid & (kWave - 1)) == 0) red[4 + wave] = ls;
  __syncthreads();
  const float lsum = (red[4] + red[5]) + (red[6] + red[7]);
  const int c = tid % D, pg = tid / D;
  const float* src = pblk + row * D + c;
  float o = 0.f;
  int s = pg;
  for (; s + 7 * NPART < S; s += 8 * NPART) {
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = src[(s + k * NPART) * pstride];
#pragma unroll
    for (int k = 0; k < 8; ++k) o += sm[s + k * NPART] * x[k];
  }
  for (; s < S; s += NPART) o += sm[s] * src[s * pstride];
  part[pg * D + c] = o;
  __syncthreads();
  const int b = (int)(blk / a.g.Hkv), kvh = (int)(blk % a.g.Hkv);
  const int t = row / a.gs, h = kvh * a.gs + row % a.gs;
  if (pg == 0) {
    float tot = 0.f;
#pragma unroll
    for (int k = 0; k < NPART; ++k) tot += part[k * D + c];
    a.out[(((int64_t)b * a.T + t) * a.Hq + h) * D + c] = __float2half(tot / lsum);
  }
  if (tid == 0 && a.lse)
    a.lse[((int64_t)b * a.Hq + h) * a.T + t] = (M + __log2f(lsum)) * kLn2;
}

// Dynamic LDS of the split kernel (the host sizes it):
//   s_qc   float [RP][D]                       q * sm_scale * log2(e)
//   s_bq   u4v   [ngr][NRT][KS][2][64]         B operands Q' = hi + lo of the
//                                              ngr key groups of one round,
//                                              in MFMA lane order
//   s_bias float [ngr][RP]                     accumulator start per row
//   s_ksz  half2 [2][ngr][D]                   key scale/zero of the current
//                                              and the next round's groups
// After the tile loop the same bytes hold the wave-merge slabs
//   slab float [2][RP][D], ml float [2][2][RP].
template <int RP, int D, int NRT, int KS>
struct Lds {
  static size_t bytes(int ngr) {
    const size_t loop = (size_t)RP * D * 4 + (size_t)ngr * NRT * KS * 2 * 64 * 16 +
                        (size_t)ngr * RP * 4 + (size_t)2 * ngr * D * 4;
    const size_t merge = (size_t)2 * RP * D * 4 + 4 * RP * 4;
    return loop > merge ? loop : merge;
  }
};

template <int PATH, int D, int NRT, int NG>
__global__ void __launch_bounds__(NT) attn_kernel(const AttnArgs a) {
  using C = Cfg<PATH, D, NRT, NG>;
  constexpr int RP = C::RP, KS = C::KS, MT = C::MT;
  extern __shared__ __align__(16) unsigned char smem[];
  const int ngr = a.ngr;
  float* s_qc = (float*)smem;
  u4v* s_bq = (u4v*)(smem + RP * D * 4);
  float* s_bias = (float*)(smem + RP * D * 4 + (size_t)ngr * NRT * KS * 2 * 64 * 16);
  unsigned* s_ksz = (unsigned*)(s_bias + ngr * RP);

  const CacheGeom& g = a.g;
  const int S = a.s_q + a.s_r;
  const int64_t wg = blockIdx.x;
  const int64_t blk = wg / S;
  const int split = (int)(wg % S);
  const int b = (int)(blk / g.Hkv), kvh = (int)(blk % g.Hkv);
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int l16 = lane & 15, gq = lane >> 4;
  const int a16 = (lane ^ 16) << 2, a32 = (lane ^ 32) << 2;
  const int64_t L = a.n_q + a.n_r;

  // Cooperative B-operand build: Q' (or q * c0 when sz == nullptr) of
  // `slots` key groups, split into fp16 hi + lo, in the lane order of the
  // score MFMA; s_bias gets  sum_c qc*z - KBIAS * sum_c Q'  per row.  A
  // power-of-two run of consecutive threads shares a (slot, row) and reduces
  // with shuffles in a fixed order, so the result is deterministic.  `pk` is the code-pair stride of the
  // operand layout (PERK for quantized keys, 1 for fp16 keys).
  auto build_b = [&](const unsigned* sz, int slots, int pk, float kbias) {
    constexpr int COMBOS = 4 * KS;                 // (gq, ks) per row
    // threads per (slot, row): as many as keep all 256 busy, a power of two
    int tpr = NT / (slots * RP);
    tpr = tpr >= COMBOS ? COMBOS : tpr >= 16 ? 16 : tpr >= 8 ? 8 : tpr >= 4 ? 4
          : tpr >= 2 ? 2 : 1;
    const int cpt = COMBOS / tpr;                  // combos per thread
    for (int it = tid / tpr; it < slots * RP; it += NT / tpr) {
      const int slot = it / RP, row = it % RP, part = tid % tpr;
      const float* qr = s_qc + row * D;
      const unsigned* zs = sz ? sz + slot * D : nullptr;
      float sum_q = 0.f, sum_z = 0.f;
      for (int cc = 0; cc < cpt; ++cc) {
        const int combo = part * cpt + cc;
        const int cg = combo / KS, ks = combo % KS;
        unsigned hi4[4], lo4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int p = 4 * ks + j;
          int ca, cb;
          if (sz) {
            ca = cg * (D / 4) + (p / pk) * 2 * pk + p % pk;
            cb = ca + pk;
          } else {
            ca = cg * (D / 4) + 2 * p;
            cb = ca + 1;
          }
          float xa = qr[ca], xb = qr[cb];
          if (sz) {
            const unsigned pa = zs[ca], pb = zs[cb];
            sum_z += xa * h_hi(pa) + xb * h_hi(pb);
            xa *= h_lo(pa);
            xb *= h_lo(pb);
          }
          xa = opaque(xa);
          xb = opaque(xb);
          const unsigned h = pack2(xa, xb);
          const unsigned l = pack2(xa - h_lo(h), xb - h_hi(h));
          hi4[j] = h;
          lo4[j] = l;
          sum_q += (h_lo(h) + h_hi(h)) + (h_lo(l) + h_hi(l));
        }
        u4v* dst = s_bq + ((slot * NRT + row / 16) * KS + ks) * 128 + 16 * cg + row % 16;
        dst[0] = u4v{hi4[0], hi4[1], hi4[2], hi4[3]};
        dst[64] = u4v{lo4[0], lo4[1], lo4[2], lo4[3]};
      }
      for (int o = 1; o < tpr; o <<= 1) {
        sum_q += __shfl_xor(sum_q, o);
        sum_z += __shfl_xor(sum_z, o);
      }
      if (part == 0) s_bias[slot * RP + row] = sum_z - kbias * sum_q;
    }
  };

  float m_run[NRT], l_run[NRT];
  f4v acc[NRT][MT];
  float zacc[NRT][NG];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) zacc[rt][gg] = 0.f;
  }
  const bool residual = split >= a.s_q;
  float oscale = 1.f;

  // Online-softmax update of row tile rt from the S^T accumulators of the
  // two subtiles; returns the probabilities in place.
  // The probabilities come out scaled by 2^pexp (the exponent is shifted
  // by pexp), so l and the zero-point sums carry that factor too; it is
  // removed once per wave at the end.
  auto softmax_update = [&](int rt, f4v& s0, f4v& s1, float pexp) {
    float mx = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                     fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
    mx = xor_max(mx, a16, a32);
    const float mnew = fmaxf(m_run[rt], mx);
    const float mref = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = fast_exp2(m_run[rt] - mref);
    const float mshift = mref - pexp;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s0[i] = fast_exp2(s0[i] - mshift);
      s1[i] = fast_exp2(s1[i] - mshift);
    }
    const float ps = ((s0[0] + s1[0]) + (s0[1] + s1[1])) +
                     ((s0[2] + s1[2]) + (s0[3] + s1[3]));
    l_run[rt] = l_run[rt] * alpha + ps;
    m_run[rt] = mnew;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[rt][mt] *= alpha;
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) zacc[rt][gg] *= alpha;
    }
  };

  // S^T = K Q'^T for the two 16-token subtiles, B operands from LDS slot.
  auto scores = [&](f4v (&sc)[2][NRT], const u4v (&ak)[2][KS], int slot) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const float bias = s_bias[slot * RP + l16 + 16 * rt];
      sc[0][rt] = f4v{bias, bias, bias, bias};
      sc[1][rt] = sc[0][rt];
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const u4v* src = s_bq + ((slot * NRT + rt) * KS + ks) * 128 + lane;
        const u4v bh = src[0], bl = src[64];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          sc[st][rt] = mfma16(ak[st][ks], bh, sc[st][rt]);
          sc[st][rt] = mfma16(ak[st][ks], bl, sc[st][rt]);
        }
      }
    }
  };

  // Key scale/zero of groups [g0, g0 + slots) for the round starting at
  // tile tr: this thread's share of the ngr * D u32, loaded to registers
  // now and stored to LDS buffer `buf` later (after the round's compute).
  constexpr int KSZ_PER = 2;   // u32 per thread: ngr * D <= 512
  auto ksz_fetch = [&](const __half2* base, int64_t g0, int slots, unsigned* r) {
#pragma unroll
    for (int k = 0; k < KSZ_PER; ++k) {
      const int e = tid + k * NT;
      r[k] = e < slots * D ? ((const unsigned*)(base + g0 * D))[e] : 0u;
    }
  };
  auto ksz_park = [&](int buf, const unsigned* r) {
#pragma unroll
    for (int k = 0; k < KSZ_PER; ++k) {
      const int e = tid + k * NT;
      if (e < ngr * D) s_ksz[buf * ngr * D + e] = r[k];
    }
  };

  if (!residual) {
    // ================= quantized prefix ===================================
    oscale = 1.f / kPScale;
    const int64_t nqt = a.n_q / kTile;
    const int64_t T0 = (int64_t)split * NW * a.tpw;
    const int64_t T1 = T0 + (int64_t)NW * a.tpw < nqt ? T0 + (int64_t)NW * a.tpw : nqt;
    const uint8_t* kh_base = a.p.k_hi + blk * g.k_block_bytes;
    const uint8_t* kl_base = C::TWO ? a.p.k_lo + blk * g.k_block_bytes : nullptr;
    const uint8_t* vh_base = a.p.v_hi + blk * g.v_block_bytes;
    const uint8_t* vl_base = C::TWO ? a.p.v_lo + blk * g.v_block_bytes : nullptr;
    const __half2* vsz_base = a.p.v_sz + blk * g.vsz_block;
    const __half2* ksz_base = a.p.k_sz + blk * g.ksz_block;
    const int64_t krow = D * C::W / 8;
    const int kofs = gq * (D * C::W / 32);
    const int vofs = lane * (D * C::W / 16);
    const int64_t ngroups = a.n_q / g.G;

    // Load pointers of one tile for this lane; next() moves them NW tiles on.
    struct TP {
      const uint8_t *kh, *kl, *vh, *vl;
      const unsigned *s;
    };
    const int64_t kstep = (int64_t)kTile * krow;       // bytes per K tile
    auto tile_ptr = [&](int64_t t) {
      TP p;
      p.kh = kh_base + (t * kTile + l16) * krow + kofs;
      p.kl = C::TWO ? kl_base + (t * kTile + l16) * krow + kofs : nullptr;
      p.vh = vh_base + t * g.v_tile_bytes + vofs;
      p.vl = C::TWO ? vl_base + t * g.v_tile_bytes + vofs : nullptr;
      p.s = (const unsigned*)(vsz_base + t * g.vsz_tile) + gq * 4 * NG;
      return p;
    };
    auto next = [&](TP& p) {
      p.kh += NW * kstep;
      if constexpr (C::TWO) p.kl += NW * kstep;
      p.vh += NW * g.v_tile_bytes;
      if constexpr (C::TWO) p.vl += NW * g.v_tile_bytes;
      p.s += NW * g.vsz_tile;
    };
    auto load_tile = [&](QTile<C>& tl, const TP& p) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        ldg<C::NDK>(p.kh + st * 16 * krow, tl.kh[st]);
        if constexpr (C::TWO) ldg<C::NDK>(p.kl + st * 16 * krow, tl.kl[st]);
      }
      ldg<C::NDV>(p.vh, tl.vh);
      if constexpr (C::TWO) ldg<C::NDV>(p.vl, tl.vl);
      ldg<4 * NG>(p.s, tl.sz);                     // scale pairs
      ldg<4 * NG>(p.s + 16 * NG, tl.sz + 4 * NG);  // zero-point pairs
    };

    const DecK dk = dec_consts();
    auto compute_tile = [&](const QTile<C>& tl, int slot) {
      // ---- K operands: codes (or draft points) as fp16, both subtiles
      u4v ak[2][KS];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          unsigned r[4];
          if constexpr (PATH == P_T8) {
            dec8(tl.kh[st][ks], tl.kl[st][ks], r, dk);
          } else if constexpr (PATH == P_D4) {
            dec4(tl.kh[st][ks], r, dk);
          } else {
            constexpr int KPD = C::PERK / 4;   // k-steps per dword
#pragma unroll
            for (int j = 0; j < 4; ++j)
              r[j] = declow<C::W>(tl.kh[st][ks / KPD], 4 * (ks % KPD) + j, dk);
          }
          ak[st][ks] = u4v{r[0], r[1], r[2], r[3]};
        }
      f4v sc[2][NRT];
      scores(sc, ak, slot);
      // ---- softmax and P' = p * s_v * 2^10 for every row tile
      u4v bp[NRT][NG];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        softmax_update(rt, sc[0][rt], sc[1][rt], kPExp);
        // P' pair i (tokens 4gq+i, 16+4gq+i) = fp16(p) * scale pair
        unsigned pp[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pp[i] = pack2(sc[0][rt][i], sc[1][rt][i]);
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
          float zs = zacc[rt][gg];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const unsigned sp = tl.sz[i * NG + gg];            // scales
            const unsigned zp = tl.sz[(4 + i) * NG + gg];      // zero-points
            bp[rt][gg][i] = __builtin_bit_cast(
                unsigned, __builtin_bit_cast(h2v, pp[i]) * __builtin_bit_cast(h2v, sp));
            zs += sc[0][rt][i] * h_lo(zp);
            zs += sc[1][rt][i] * h_hi(zp);
          }
          zacc[rt][gg] = zs;
        }
      }
      // ---- O^T += V^T P'^T, one 16-channel tile of exact codes at a time
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        unsigned r[4];
        if constexpr (PATH == P_T8) {
          dec8(tl.vh[mt], tl.vl[mt], r, dk);
#pragma unroll
          for (int j = 0; j < 4; ++j) r[j] = hadd2(r[j], kMinus1024);
        } else if constexpr (PATH == P_D4) {
          dec4(tl.vh[mt], r, dk);
#pragma unroll
          for (int j = 0; j < 4; ++j) r[j] = hadd2(r[j], kMinusDraft);
        } else {
          constexpr int PER = 4 / C::W;   // channel tiles per dword
#pragma unroll
          for (int j = 0; j < 4; ++j)
            r[j] = declow<C::W>(tl.vh[mt / PER], 4 * (mt % PER) + j, dk);
        }
        const u4v av = u4v{r[0], r[1], r[2], r[3]};
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
          acc[rt][mt] = mfma16(av, bp[rt][mt / (MT / NG)], acc[rt][mt]);
      }
    };

    // Rounds of NW consecutive tiles, wave w on the w-th: the round's key
    // groups are built once for the workgroup.  Every wave runs every round
    // (and its barriers); the next round's tile is prefetched before the
    // current one is computed.
    auto slots_of = [&](int64_t g0) {
      return g0 + ngr > ngroups ? (int)(ngroups - g0) : ngr;
    };
    // Rounds of NW consecutive tiles, wave w on the w-th.  The groups a
    // round needs are built into B operands once for the workgroup (between
    // two barriers) from scales parked in LDS by the previous round, whose
    // loads were in flight during its compute.
    int64_t cur_g0 = -1, parked_g0 = -1;
    int buf = 0;
    unsigned kpre[KSZ_PER];
    TP np = tile_ptr(T0 + wave);          // next tile to load
    auto round = [&](int64_t tr, QTile<C>& cur, QTile<C>& nxt) {
      const int64_t t = tr + wave;
      const int64_t g0 = tr * kTile / g.G;
      if (g0 != cur_g0) {
        __syncthreads();                       // old B operands consumed,
        build_b(s_ksz + buf * ngr * D,         // parked scales visible
                slots_of(g0), C::PERK, C::KBIAS);
        __syncthreads();
        cur_g0 = g0;
      }
      if (t + NW < T1) {
        load_tile(nxt, np);
        next(np);
      }
      const int64_t gn = (tr + NW) * kTile / g.G;   // next round's groups
      const bool fetch = tr + NW < T1 && gn != g0 && gn != parked_g0;
      if (fetch) ksz_fetch(ksz_base, gn, slots_of(gn), kpre);
      if (t < T1) compute_tile(cur, (int)(t * kTile / g.G - g0));
      if (fetch) {
        buf ^= 1;
        ksz_park(buf, kpre);
        parked_g0 = gn;
      }
    };
    if (T0 < T1) {
      QTile<C> ta, tb;
      if (T0 + wave < T1) {
        load_tile(ta, np);
        next(np);
      }
      const int64_t g_first = T0 * kTile / g.G;
      ksz_fetch(ksz_base, g_first, slots_of(g_first), kpre);
  // ---- q * c0 of this block's rows (row = t * gs + head-in-group) as fp32 in
    // LDS: 16-byte loads, all issued before the first LDS store
    {
      constexpr int CH = RP * D / 8;                 // 8-half chunks
      constexpr int PER = (CH + NT - 1) / NT;
      uint4 v[PER];
  #pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int e = tid + k * NT;
        const int row = e / (D / 8), c8 = e % (D / 8);
        v[k] = make_uint4(0u, 0u, 0u, 0u);
        if (e < CH && row < a.rows) {
          const int t = row / a.gs, hl = row % a.gs;
          v[k] = *(const uint4*)(a.q + (((int64_t)b * a.T + t) * a.Hq +
                                        kvh * a.gs + hl) * D + 8 * c8);
        }
      }
  #pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int e = tid + k * NT;
        if (e < CH) {
          const unsigned w4[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
          f4v lo4, hi4;
  #pragma unroll
          for (int x = 0; x < 2; ++x) {
            lo4[2 * x] = h_lo(w4[x]) * a.c0;
            lo4[2 * x + 1] = h_hi(w4[x]) * a.c0;
            hi4[2 * x] = h_lo(w4[2 + x]) * a.c0;
            hi4[2 * x + 1] = h_hi(w4[2 + x]) * a.c0;
          }
          *(f4v*)(s_qc + 8 * e) = lo4;
          *(f4v*)(s_qc + 8 * e + 4) = hi4;
        }
      }
    }
    __syncthreads();
      ksz_park(buf, kpre);
      parked_g0 = g_first;
      __syncthreads();
      for (int64_t tr = T0; tr < T1; tr += 2 * NW) {
        round(tr, ta, tb);
        if (tr + NW < T1) round(tr + NW, tb, ta);
      }
    }
  } else {
    // ================= fp16 residual ring ==================================
  // ---- q * c0 of this block's rows (row = t * gs + head-in-group) as fp32 in
    // LDS: 16-byte loads, all issued before the first LDS store
    {
      constexpr int CH = RP * D / 8;                 // 8-half chunks
      constexpr int PER = (CH + NT - 1) / NT;
      uint4 v[PER];
  #pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int e = tid + k * NT;
        const int row = e / (D / 8), c8 = e % (D / 8);
        v[k] = make_uint4(0u, 0u, 0u, 0u);
        if (e < CH && row < a.rows) {
          const int t = row / a.gs, hl = row % a.gs;
          v[k] = *(const uint4*)(a.q + (((int64_t)b * a.T + t) * a.Hq +
                                        kvh * a.gs + hl) * D + 8 * c8);
        }
      }
  #pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int e = tid + k * NT;
        if (e < CH) {
          const unsigned w4[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
          f4v lo4, hi4;
  #pragma unroll
          for (int x = 0; x < 2; ++x) {
            lo4[2 * x] = h_lo(w4[x]) * a.c0;
            lo4[2 * x + 1] = h_hi(w4[x]) * a.c0;
            hi4[2 * x] = h_lo(w4[2 + x]) * a.c0;
            hi4[2 * x + 1] = h_hi(w4[2 + x]) * a.c0;
          }
          *(f4v*)(s_qc + 8 * e) = lo4;
          *(f4v*)(s_qc + 8 * e + 4) = hi4;
        }
      }
    }
    __syncthreads();
    build_b(nullptr, 1, 1, 0.f);   // q * c0 = hi + lo, natural channel pairs
    __syncthreads();
    const int64_t ti = (int64_t)(split - a.s_q) * NW + wave;
    const int64_t nrt = cdiv(a.n_r, kTile);
    if (ti < nrt) {
      const int64_t p0 = a.n_q + ti * kTile;           // first position
      const int64_t slot0 = p0 % g.ring;               // 32-aligned slot
      const __half* kres = a.p.k_res + blk * g.res_block;
      u4v ak[2][KS];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        unsigned kd[D / 8];
        ldg<D / 8>(kres + (slot0 + 16 * st + l16) * D + gq * (D / 4), kd);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          ak[st][ks] = u4v{kd[4 * ks], kd[4 * ks + 1], kd[4 * ks + 2], kd[4 * ks + 3]};
      }
      unsigned vd[D / 4];
      ldg<D / 4>(a.p.v_res + blk * g.res_block + (slot0 / kTile) * kTile * D +
                     lane * (D / 2),
                 vd);
      f4v sc[2][NRT];
      scores(sc, ak, 0);
      // causal / validity mask: row sees positions <= L - T + t(row)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const int row = l16 + 16 * rt;
        const int64_t lim = row < a.rows ? L - a.T + row / a.gs : L - 1;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t pos = p0 + 16 * st + 4 * gq + i;
            sc[st][rt][i] = pos <= lim ? sc[st][rt][i] : -INFINITY;
          }
      }
      // V tile (token-permuted fp16): zero the slots past the context
      if (p0 + kTile > L) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const unsigned keep =
              (p0 + 4 * gq + i < L ? 0x0000FFFFu : 0u) |
              (p0 + 16 + 4 * gq + i < L ? 0xFFFF0000u : 0u);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) vd[4 * mt + i] &= keep;
        }
      }
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        softmax_update(rt, sc[0][rt], sc[1][rt], 0.f);
        u4v bp;
#pragma unroll
        for (int i = 0; i < 4; ++i) bp[i] = pack2(sc[0][rt][i], sc[1][rt][i]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[rt][mt] = mfma16(
              u4v{vd[4 * mt], vd[4 * mt + 1], vd[4 * mt + 2], vd[4 * mt + 3]},
              bp, acc[rt][mt]);
      }
    }
  }

  // ---- per-wave finish: full-row l, zero-point term folded into o; the
  // quantized waves' sums carry the 2^10 of their probabilities (oscale)
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    l_run[rt] = xor_sum(l_run[rt], a16, a32) * oscale;
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) zacc[rt][gg] = xor_sum(zacc[rt][gg], a16, a32) * oscale;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      acc[rt][mt] = acc[rt][mt] * oscale + zacc[rt][mt / (MT / NG)];
  }

  // ---- merge the 4 waves through LDS: (2,3) -> (0,1), then 1 -> 0
  float* s_slab = (float*)smem;
  float* s_ml = s_slab + 2 * RP * D;
  auto put = [&](int slot) {
    float* o = s_slab + slot * RP * D;
    float* ml = s_ml + slot * 2 * RP;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const int row = l16 + 16 * rt;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
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
      for (int mt = 0; mt < MT; ++mt)
        acc[rt][mt] = acc[rt][mt] * fa +
                      *(const f4v*)(o + row * D + 16 * mt + 4 * gq) * fb;
      l_run[rt] = l_run[rt] * fa + lo * fb;
      m_run[rt] = M;
    }
  };
  __syncthreads();   // the loop's LDS (q, B operands) is reused below
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
      for (int mt = 0; mt < MT; ++mt)
        *(f4v*)(po + row * D + 16 * mt + 4 * gq) = acc[rt][mt];
      if (gq == 0) {
        po[RP * D + row] = m_run[rt];
        po[RP * D + RP + row] = l_run[rt];
      }
    }
  }
}

template <int PATH, int D, int NRT, int NG>
hipError_t go(const AttnArgs& a, hipStream_t s) {
  const int64_t nb = (int64_t)a.g.B * a.g.Hkv;
  using C = Cfg<PATH, D, NRT, NG>;
  const size_t lds = Lds<C::RP, D, NRT, C::KS>::bytes(a.ngr);
  if (lds > 64 * 1024) {
    static bool raised = false;   // once per instantiation
    if (!raised) {
      hipError_t e = hipFuncSetAttribute(
          (const void*)attn_kernel<PATH, D, NRT, NG>,
          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      raised = true;
    }
  }
  hipLaunchKernelGGL((attn_kernel<PATH, D, NRT, NG>),
                     dim3((unsigned)(nb * (a.s_q + a.s_r))), dim3(NT), lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((merge_kernel<D, 16 * NRT>), dim3((unsigned)(nb * a.rows)),
                     dim3(NT), 0, s, a);
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
