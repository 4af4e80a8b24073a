// Split-K decode/verify attention read directly from the quantized cache.
//
// QuantSpec page, Approach: the draft attends over the upper-4-bit codes, the
// target verifies gamma+1 tokens over the 8-bit codes plus the fp16 buffer of
// recent tokens; Experimental setup, "Builds on: FlashDecoding" (split the
// context across workgroups, merge partial softmax statistics by
// log-sum-exp).  SpeCache page, Approach: output + speculative token (T = 2)
// over a 1/2-bit KIVI copy.
//
// Work decomposition (grid = splits x Hkv x B, NW waves per workgroup):
//   * a block's work is a sequence of units: two per 32-slot tile of the fp16
//     ring (its K, then its V, 8 KB each at d = 128) followed by the
//     quantized prefix in units of TPU 32-token tiles (codes, value
//     scale/zero and the key scale/zero of the tile's group).  Every stream
//     of the grid owns one contiguous run of units (a ring tile's two units
//     never split); a stream is one wave (up to 16 rows) or two waves that
//     take one 16-row tile each.  No wave waits for another inside the loop.
//   * each wave loads its next unit into registers with plain coalesced
//     16-byte loads while it computes the current one, then writes it to its
//     own LDS stage (XOR-permuted 16-byte pieces, so the decode's strided
//     reads are free of bank conflicts) and reads the operands from there.
//   * per tile the wave computes S^T = K * Q'^T on MFMA (16x16x32 f16, two
//     16-token subtiles x one or two 16-row tiles), runs the online softmax
//     on the S^T accumulators in place and feeds P'^T straight back as the B
//     operand of O^T += V^T * P'^T: the accumulator layout of the score MFMA
//     (lane = row, 4 consecutive tokens) is the operand layout the PV MFMA
//     needs once V is stored token-permuted, so no data crosses lanes.  Rows
//     are query tokens x GQA heads (T * Hq/Hkv <= 32).
//   * codes become fp16 MFMA operands in registers with the "0x6400 | code"
//     trick (fp16 1024 + code).  Per-channel key scales are folded into
//     Q' = q * s * sm_scale * log2(e) once per key group, kept as two fp16
//     parts (hi + lo, two MFMAs) so the scores carry ~22 bits of Q'; the 1024
//     offset (an MFMA of a constant operand with Q') and the zero-points go
//     into the accumulator's initial value.  1/2-bit codes decode as
//     1 + code 2^-W instead (no subtract; the offset 1 leaves the fp32 sums
//     with no cancellation to speak of), and their caches (groups of 32
//     tokens) cut the per-group work: 1-bit codes carry their key scales
//     themselves (code s / 2 is exact), 2-bit groups rebuild Q' with packed
//     fp16 operations from fixed hi + lo parts of q * c0, and both take the
//     zero-point term as one MFMA.  Per-token value scales are
//     folded into P' = p * s * 2^7, value zero-points and the 1024 offset
//     into a per-row fp32 side sum (packed fp16 dot products).
//   * the softmax reference moves lazily: scores are taken relative to the
//     row's reference (folded into the accumulator's initial value) and the
//     reference is only raised when a score exceeds it by more than 2^3, so
//     the common tile needs no cross-lane reduction and no rescale.
//   * the streams of a workgroup merge through LDS and write one partial
//     (m, l, o) per workgroup.  A second launch, one workgroup per (block,
//     row), merges that row's partials by log-sum-exp (fp16 output, natural-
//     log LSE); the kernel boundary makes the partials visible.
#include <mutex>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef unsigned u4v __attribute__((ext_vector_type(4)));
typedef unsigned u2v __attribute__((ext_vector_type(2)));

constexpr unsigned kMagic = 0x64006400u;       // fp16 pair (1024, 1024)
constexpr unsigned kMinus1024 = 0xE400E400u;   // fp16 pair (-1024, -1024)
constexpr unsigned kMinusDraft = 0xE3F1E3F1u;  // fp16 pair (-1016.5, -1016.5)
// Probabilities are taken as 2^(s - m_ref + kPExp) with s <= m_ref + kTau
// between reference moves: p' <= 2^10, and P' = p' * s_v stays an fp16
// normal for value scales up to 64.
constexpr float kPExp = 7.f;
constexpr float kTau = 3.f;
constexpr float kOScale = 1.f / 128.f;         // 2^-kPExp
constexpr float kLn2 = 0.693147180559945309f;
constexpr int kLdsBytes = 160 * 1024;

enum Path { P_T8 = 0, P_D4 = 1, P_L2 = 2, P_L1 = 3 };

__device__ __forceinline__ f4v mfma16(u4v a, u4v b, f4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(
      __builtin_bit_cast(h8v, a), __builtin_bit_cast(h8v, b), c, 0, 0, 0);
}

__device__ __forceinline__ unsigned hadd2(unsigned x, unsigned y) {
  h2v r = __builtin_bit_cast(h2v, x) + __builtin_bit_cast(h2v, y);
  return __builtin_bit_cast(unsigned, r);
}

__device__ __forceinline__ unsigned hmul2(unsigned x, unsigned y) {
  h2v r = __builtin_bit_cast(h2v, x) * __builtin_bit_cast(h2v, y);
  return __builtin_bit_cast(unsigned, r);
}

// fp32 += x.lo * y.lo + x.hi * y.hi (fp16 pairs, products exact in fp32)
__device__ __forceinline__ float dot2(unsigned x, unsigned y, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2v, x),
                                __builtin_bit_cast(h2v, y), acc, false);
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
// fp16 element j of a pair of dwords (4 halves)
__device__ __forceinline__ float h_at(u2v x, int j) {
  return j < 2 ? (j == 0 ? h_lo(x[0]) : h_hi(x[0]))
               : (j == 2 ? h_lo(x[1]) : h_hi(x[1]));
}

// The fp32 value as materialised in a register.  Splitting x into fp16
// hi = fp16(x) and lo = fp16(x - hi) needs both parts to see the same x,
// but the compiler may fold a product feeding an fp16 conversion into one
// mixed-precision FMA (a single rounding of the exact product) for one use
// and round the fp32 product for the other; on an fp16 rounding midpoint
// the two differ and lo gets the wrong sign.
__device__ __forceinline__ float opaque(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// fp16 pair (RN16(a * s.lo), RN16(b * t.lo)) of exact fp32 x fp16 products,
// and the pair of what those leave, RN16(a * s.lo - hi.lo), RN16(b * t.lo -
// hi.hi): one v_fma_mix each, so hi + lo carries ~22 bits of each product.
__device__ __forceinline__ unsigned hsplit_hi(float a, unsigned s, float b,
                                              unsigned t) {
  h2v r;
  r[0] = (_Float16)__builtin_fmaf(a, h_lo(s), 0.f);
  r[1] = (_Float16)__builtin_fmaf(b, h_lo(t), 0.f);
  return __builtin_bit_cast(unsigned, r);
}
__device__ __forceinline__ unsigned hsplit_lo(float a, unsigned s, float b,
                                              unsigned t, unsigned hi) {
  h2v r;
  r[0] = (_Float16)__builtin_fmaf(a, h_lo(s), -h_lo(hi));
  r[1] = (_Float16)__builtin_fmaf(b, h_lo(t), -h_hi(hi));
  return __builtin_bit_cast(unsigned, r);
}

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS
// operations, not for its outstanding global loads (a full __syncthreads
// would also drain those).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Reductions over the four 16-lane rows of a wave (lanes l, l^16, l^32,
// l^48) with the lane-swap permutes: the operands are combined in the same
// order on every lane, so all four get bit-identical results.
__device__ __forceinline__ float max_x4(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v),
                                            __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v),
                                            __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float sum_x4(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v),
                                            __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v),
                                            __float_as_uint(v), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
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
// (m & a) | (~m & b) in one instruction; the compiler splits the pattern
// into an and plus an and-or.
__device__ __forceinline__ unsigned bfi(unsigned m, unsigned a, unsigned b) {
  unsigned r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(m), "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ void dec8(unsigned H, unsigned L, unsigned* r,
                                     const DecK& k) {
  const unsigned ce = bfi(k.m_hi, H << 4, L);
  const unsigned co = bfi(k.m_hi, H, L >> 4);
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

// W-bit codes under the fp16 exponent of 1.0: the pair at bits (W*i,
// 16 + W*i) becomes the top mantissa bits, x = 1 + code 2^-W (exact; the
// offset 1 is at most a few codes, so taking it out of an fp32 sum later
// costs no precision, unlike the 1024 of the 0x6400 form).  `one` is the
// fp16 pair (1, 1), `m` the code bits' mask at their place under it.
template <int W>
__device__ __forceinline__ unsigned lowx(unsigned H, int i, unsigned one,
                                         unsigned m) {
  const int sh = (10 - W) - W * i;   // a constant once the caller unrolls
  const unsigned x = sh >= 0 ? H << (sh & 31) : H >> (-sh & 31);
  return (x & m) | one;
}

// ... times their channels' key scales: fma(x, s, -s) = code s 2^-W with a
// single rounding (x s < 2 s: no overflow), exact for 1-bit codes.
template <int W>
__device__ __forceinline__ unsigned declow_ks(unsigned H, int i, unsigned s,
                                              unsigned one, unsigned m) {
  const h2v xv = __builtin_bit_cast(h2v, lowx<W>(H, i, one, m));
  const h2v sv = __builtin_bit_cast(h2v, s);
  return __builtin_bit_cast(unsigned, __builtin_elementwise_fma(xv, sv, -sv));
}

template <int N>
__device__ __forceinline__ void lds_read(const unsigned char* p, unsigned* o) {
  if constexpr (N == 1) {
    o[0] = *(const unsigned*)p;
  } else if constexpr (N == 2) {
    const u2v v = *(const u2v*)p;
    o[0] = v[0]; o[1] = v[1];
  } else {
    static_assert(N % 4 == 0, "dword count");
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
      const u4v v = ((const u4v*)p)[k];
      o[4 * k] = v[0]; o[4 * k + 1] = v[1]; o[4 * k + 2] = v[2]; o[4 * k + 3] = v[3];
    }
  }
}

// Units move in 1 KB chunks: the NH waves of a stream load each chunk into
// registers (16/NH bytes per lane, one coalesced load per wave) and write it
// to the unit's LDS stage; a partial last chunk of a piece is loaded by the
// lanes whose bytes fall inside it.
constexpr int chunks_of(int bytes) { return (bytes + 1023) / 1024; }

// Per-path geometry.  A wave owns NRT 16-row tiles of the block's rows.
// SOLO streams (every wave its own run of units) carry NRT = 1 or 2 row
// tiles per wave; PAIR streams (17..32 rows) let two waves share one run,
// wave h taking row tile h, so each wave's state is that of 16 rows.
template <int PATH, int D, int NG, int NRT, bool PAIR>
struct Cfg {
  static_assert(NRT == 1 || (NRT == 2 && !PAIR), "row tiles per wave");
  static constexpr int NH = PAIR ? 2 : 1;        // waves per stream
  static constexpr int RTT = NH * NRT;           // row tiles per stream
  static constexpr int RP = 16 * RTT;            // staged (padded) rows
  static constexpr int W = PATH == P_L2 ? 2 : PATH == P_L1 ? 1 : 4;
  static constexpr bool TWO = PATH == P_T8;      // hi + lo planes
  static constexpr bool LOW = PATH == P_L2 || PATH == P_L1;
  static constexpr int KS = D / 32;              // MFMA k-steps per subtile
  static constexpr int NDK = D * W / 128;        // K dwords / lane / plane / subtile
  static constexpr int NDV = D * W / 64;         // V dwords / lane / plane / tile
  static constexpr int MT = D / 16;              // 16-channel output tiles
  static constexpr float KBIAS =
      PATH == P_T8 ? 1024.f : PATH == P_D4 ? 1016.5f : 0.f;
  // code offset of the value decode: 1024 for the 0x6400 form, and for
  // 1/2-bit codes (decoded as 1 + code 2^-W, accumulated times 2^W) 2^W
  static constexpr unsigned NEG = PATH == P_D4   ? kMinusDraft
                                  : PATH == P_L2 ? 0xC400C400u    // (-4, -4)
                                  : PATH == P_L1 ? 0xC000C000u    // (-2, -2)
                                                 : kMinus1024;
  // stage layout of one quantized tile (bytes)
  static constexpr int PL = 4 * D * W;           // one code plane
  static constexpr int VSZB = 128 * NG;          // value scale/zero pairs
  static constexpr int KSZB = 4 * D;             // key scale/zero of a group
  static constexpr int O_KH = 0, O_KL = PL;
  static constexpr int O_VH = TWO ? 2 * PL : PL, O_VL = O_VH + PL;
  static constexpr int O_VSZ = TWO ? 4 * PL : 2 * PL;
  static constexpr int O_KSZ = O_VSZ + VSZB;
  static constexpr int TILE = O_KSZ + KSZB;
  static constexpr int RESU = 64 * D;            // fp16 K or V of a ring tile
  // 1 KB chunks: a ring unit, a quantized tile; tiles per unit so that a
  // unit has about as many chunks as a ring unit
  static constexpr int NIR = chunks_of(RESU);
  static constexpr int NI_TILE =
      (TWO ? 4 : 2) * chunks_of(PL) + chunks_of(VSZB) + chunks_of(KSZB);
  static constexpr int TPU = NIR / NI_TILE > 1 ? NIR / NI_TILE : 1;
  static constexpr int NIQ = TPU * NI_TILE;
  static constexpr int NI = NIQ > NIR ? NIQ : NIR;
  static constexpr int STAGE = TPU * TILE > RESU ? TPU * TILE : RESU;
  static constexpr int QB = RP * D * 2;          // staged q rows (fp16)
  // waves per workgroup: 8 (two per SIMD) unless a wave holds two row
  // tiles (its state then needs more than the 256 registers of two waves
  // per SIMD)
  static constexpr int NW = NRT == 1 ? 8 : 4;
  static constexpr int NS = NW / NH;             // unit streams per workgroup
  // one LDS stage per wave: a wave writes and reads its own stage, in order;
  // the stream-merge slabs reuse the stage and q area after the unit loop
  static constexpr int DP = D + 4;               // merge slab row (floats)
  static constexpr int MERGE = NS * RP * (DP + 2) * 4;   // o rows + (m, l)
  static constexpr int SAREA = NW * STAGE;
  static constexpr int LDS = SAREA + QB > MERGE ? SAREA + QB : MERGE;
  static_assert(LDS <= kLdsBytes, "LDS");
};

// Merge kernel, one workgroup per (block, row): combines the row's S split
// partials by log-sum-exp.  Thread (pg, cq) owns columns 4cq..4cq+3 of the
// splits pg, pg + NPART, ...  Every thread issues its (m, l) loads and then
// the 16-byte loads of its first PRE splits before it waits, so a row with
// up to NPART * PRE splits costs one round trip.  The row max and sum are
// wave reductions through LDS; the NPART column sums meet in LDS.
template <int D, int RP>
__global__ void __launch_bounds__(256) merge_kernel(const AttnArgs a) {
  constexpr int NT = 256, DQ = D / 4;
  constexpr int NPART = NT / DQ;         // thread groups over the splits
  constexpr int PRE = 8;                 // o quads loaded up front
  constexpr int MLR = kMaxSplits / NT;   // (m, l) pairs per thread
  __shared__ float sw[kMaxSplits];       // split weights 2^(m - M)
  __shared__ float red[8];               // wave max, then wave sums
  __shared__ f4v part[NPART][DQ];
  const int S = a.S;
  const int row = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int64_t blk = (int64_t)b * a.g.Hkv + kvh;
  const int tid = threadIdx.x, wave = tid / kWave;
  const int64_t pstride = (int64_t)RP * (D + 2);
  const float* pblk = a.ws + blk * a.s_alloc * pstride;
  const int cq = tid % DQ, pg = tid / DQ;
  const float* src = pblk + row * D + 4 * cq;
  float mr[MLR], lr[MLR];
#pragma unroll
  for (int j = 0; j < MLR; ++j) {
    const int sp = tid + j * NT;
    mr[j] = sp < S ? pblk[sp * pstride + RP * D + row] : -INFINITY;
    lr[j] = sp < S ? pblk[sp * pstride + RP * D + RP + row] : 0.f;
  }
  f4v x[PRE];
#pragma unroll
  for (int k = 0; k < PRE; ++k) {
    const int sp = pg + k * NPART;
    x[k] = sp < S ? *(const f4v*)(src + sp * pstride) : f4v{0.f, 0.f, 0.f, 0.f};
  }
  float M = -INFINITY;
#pragma unroll
  for (int j = 0; j < MLR; ++j) M = fmaxf(M, mr[j]);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
  if ((tid & (kWave - 1)) == 0) red[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float ls = 0.f;
#pragma unroll
  for (int j = 0; j < MLR; ++j) {
    const int sp = tid + j * NT;
    if (sp < S) {
      const float e = mr[j] == -INFINITY ? 0.f : fast_exp2(mr[j] - M);
      sw[sp] = e;
      ls += lr[j] * e;
    }
  }
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) ls += __shfl_xor(ls, o);
  if ((tid & (kWave - 1)) == 0) red[4 + wave] = ls;
  __syncthreads();
  const float lsum = (red[4] + red[5]) + (red[6] + red[7]);
  f4v o = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < PRE; ++k) {
    const int sp = pg + k * NPART;
    if (sp < S) o += x[k] * sw[sp];
  }
  for (int sp = pg + PRE * NPART; sp < S; sp += NPART)
    o += *(const f4v*)(src + sp * pstride) * sw[sp];
  part[pg][cq] = o;
  __syncthreads();
  const int t = row / a.hs, h = kvh * a.gs + a.h0 + row % a.hs;
  if (pg == 0) {
    f4v tot = part[0][cq];
#pragma unroll
    for (int k = 1; k < NPART; ++k) tot += part[k][cq];
    const __half2 o01 = __halves2half2(__float2half(tot[0] / lsum), __float2half(tot[1] / lsum));
    const __half2 o23 = __halves2half2(__float2half(tot[2] / lsum), __float2half(tot[3] / lsum));
    uint2 w;
    w.x = *(const unsigned*)&o01;
    w.y = *(const unsigned*)&o23;
    *(uint2*)(a.out + (((int64_t)b * a.T + t) * a.Hq + h) * D + 4 * cq) = w;
  }
  if (tid == 0 && a.lse)
    a.lse[((int64_t)b * a.Hq + h) * a.T + t] = (M + __log2f(lsum)) * kLn2;
}

// Exact substitution (SpeCache page, Approach: the fetched pairs are used
// in full precision for the output token), in two kernels around the split
// pass:
//   * mask_kernel, before it, one workgroup per block: the block's mask of
//     fetched positions, one bit per quantized token (word t covers tile t),
//     which the split pass reads to leave those positions out of query row
//     t_exact's attention.  It needs the positions only, not the fetched
//     rows, so their transfer can still be in flight.
//   * exact_kernel, after it, one workgroup per (group of up to HB GQA
//     heads, kv head, batch): the partial of the fetched tokens' exact terms
//     for row t_exact of each head, with logits se_j in the log2 domain from
//     the exact keys:
//       m = max_j se_j,  l = sum_j 2^(se_j - m),  o = sum_j 2^(se_j - m) v_j,
//     into the spare partial slot S of the block, so the log-sum-exp merge
//     of the S + 1 partials gives the row its attention with the fetched
//     positions reading the exact fp16 K/V.  The other query rows of those
//     heads get an empty partial (m = -inf, l = 0, o = 0).
// Positions outside [0, n_q) are skipped.  Leaving the positions out of the
// split pass, instead of subtracting their quantized terms afterwards, keeps
// the result accurate when a fetched token carried most of the quantized
// attention mass but little of the exact one (no cancellation).
// 512 threads, two workgroups per CU: each wave takes fetched tokens w,
// w + 8, ... with its lanes over the channels and loads the fp16 rows of UT
// tokens together (the positions are scattered); the heads of the kv group
// share the loaded rows.  Each wave keeps (m, l, o) per head with the usual
// rescaling, and the 8 wave states meet in LDS by log-sum-exp.  Skipped
// entries read stand-in row 0 and are never folded in.
__global__ void __launch_bounds__(256) mask_kernel(const AttnArgs a) {
  constexpr int NT = 256;
  const int64_t blk = (int64_t)blockIdx.y * a.g.Hkv + blockIdx.x;
  unsigned* mw = a.xmask + blk * (a.g.L_max / kTile);
  const int nw = (int)(a.n_q / kTile);
  for (int w = threadIdx.x; w < nw; w += NT) mw[w] = 0u;
  __syncthreads();
  const int32_t* idx = a.idx_exact + blk * a.n_exact;
  for (int i = threadIdx.x; i < a.n_exact; i += NT) {
    const int p = idx[i];
    if (p >= 0 && p < a.n_q) atomicOr(mw + (p >> 5), 1u << (p & 31));
  }
}

template <int D, int RP>
__global__ void __launch_bounds__(512, 2) exact_kernel(const AttnArgs a) {
  constexpr int NT = 512, HB = 4;                // heads per workgroup
  constexpr int NWV = NT / kWave, CPL = D / kWave;
  constexpr int UT = 4;                          // tokens a wave loads together
  __shared__ float s_q[HB][D];
  __shared__ int s_idx[kMaxExact];
  __shared__ float s_o[NWV][HB][D], s_m[NWV][HB], s_l[NWV][HB];
  const CacheGeom& g = a.g;
  const int hl0 = blockIdx.x * HB, kvh = blockIdx.y, b = blockIdx.z;
  const int nh = a.hs - hl0 < HB ? a.hs - hl0 : HB;   // heads of this workgroup
  const int64_t blk = (int64_t)b * g.Hkv + kvh;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int n = a.n_exact;
  const int64_t pstride = (int64_t)RP * (D + 2);
  float* po = a.ws + (blk * a.s_alloc + a.S) * pstride;
  const __half* ke = a.k_exact + blk * n * D;
  const __half* ve = a.v_exact + blk * n * D;

  for (int i = tid; i < n; i += NT) s_idx[i] = a.idx_exact[blk * n + i];
  // empty partials for these heads' other query rows
  for (int t = 0; t < a.T; ++t) {
    if (t == a.t_exact) continue;
    for (int hh = 0; hh < nh; ++hh) {
      const int r = t * a.hs + hl0 + hh;
      for (int c = tid; c < D; c += NT) po[r * D + c] = 0.f;
      if (tid == 0) {
        po[RP * D + r] = -INFINITY;
        po[RP * D + RP + r] = 0.f;
      }
    }
  }
  for (int e = tid; e < HB * D; e += NT) {
    const int hh = e / D, c = e % D;
    s_q[hh][c] = hh < nh ? __half2float(a.q[(((int64_t)b * a.T + a.t_exact) * a.Hq +
                                             kvh * a.gs + a.h0 + hl0 + hh) * D + c]) * a.c0
                         : 0.f;
  }
  __syncthreads();

  float m[HB], l[HB], o[HB][CPL];
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int k = 0; k < CPL; ++k) o[hh][k] = 0.f;
  }
  for (int i0 = wave; i0 < n; i0 += NWV * UT) {
    float kx[UT][CPL], vx[UT][CPL];
    bool ok[UT];
#pragma unroll
    for (int u = 0; u < UT; ++u) {               // every load of the UT tokens first
      const int i = i0 + u * NWV;
      const int p = i < n ? s_idx[i] : -1;
      ok[u] = p >= 0 && p < a.n_q;
      const int64_t is = ok[u] ? i : 0;          // stand-in: never folded in
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        const int c = lane + kWave * k;
        kx[u][k] = __half2float(ke[is * D + c]);
        vx[u][k] = __half2float(ve[is * D + c]);
      }
    }
#pragma unroll
    for (int u = 0; u < UT; ++u) {
      float de[HB];
#pragma unroll
      for (int hh = 0; hh < HB; ++hh) {
        de[hh] = 0.f;
#pragma unroll
        for (int k = 0; k < CPL; ++k) de[hh] += s_q[hh][lane + kWave * k] * kx[u][k];
#pragma unroll
        for (int sh = 1; sh < kWave; sh <<= 1) de[hh] += __shfl_xor(de[hh], sh);
      }
      if (ok[u]) {                              // wave-uniform: one token per wave
#pragma unroll
        for (int hh = 0; hh < HB; ++hh) {
          const float mn = fmaxf(m[hh], de[hh]);
          const float alpha = fast_exp2(m[hh] - mn);   // 0 while m = -inf
          const float we = fast_exp2(de[hh] - mn);
          l[hh] = l[hh] * alpha + we;
#pragma unroll
          for (int k = 0; k < CPL; ++k) o[hh][k] = o[hh][k] * alpha + we * vx[u][k];
          m[hh] = mn;
        }
      }
    }
  }
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
#pragma unroll
    for (int k = 0; k < CPL; ++k) s_o[wave][hh][lane + kWave * k] = o[hh][k];
    if (lane == 0) {
      s_m[wave][hh] = m[hh];
      s_l[wave][hh] = l[hh];
    }
  }
  __syncthreads();
  for (int e = tid; e < nh * D; e += NT) {
    const int hh = e / D, c = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWV; ++w) M = fmaxf(M, s_m[w][hh]);
    float ot = 0.f, lt = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const float mw = s_m[w][hh];
      const float sc = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
      ot += s_o[w][hh][c] * sc;
      lt += s_l[w][hh] * sc;
    }
    const int row = a.t_exact * a.hs + hl0 + hh;
    po[row * D + c] = ot;
    if (c == 0) {
      po[RP * D + row] = M;
      po[RP * D + RP + row] = lt;
    }
  }
}

// Dynamic LDS of the split kernel:
//   stages  [NW][STAGE]       each wave's unit stage
//   s_q     fp16 [RP][D]      this block's query rows (zero past `rows`)
// After the unit loop the same bytes hold the stream-merge slabs
//   slab float [NS][RP][D+4], ml float [NS][2][RP].
// XM: exact substitution (a.xmask set): query row t_exact leaves the
// fetched positions out (a separate instantiation, so the plain path keeps
// its registers).
template <int PATH, int D, int NG, int NRT, bool PAIR, bool XM>
__global__ void __launch_bounds__((Cfg<PATH, D, NG, NRT, PAIR>::NW * 64))
    attn_kernel(const AttnArgs a) {
  using C = Cfg<PATH, D, NG, NRT, PAIR>;
  constexpr int KS = C::KS, MT = C::MT, NS = C::NS, RTT = C::RTT;
  constexpr int RP = C::RP;
  constexpr int NT = C::NW * kWave;
  extern __shared__ __align__(16) unsigned char smem[];

  const CacheGeom& g = a.g;
  const int S = a.S;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int64_t blk = (int64_t)b * g.Hkv + kvh;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int strm = PAIR ? wave >> 1 : wave;      // stream in the workgroup
  const int h = PAIR ? wave & 1 : 0;             // row tile of this wave
  const int lane = tid % kWave, l16 = lane & 15, gq = lane >> 4;
  // this lane's row in row tile rt of the wave
  auto row_of = [&](int rt) __attribute__((always_inline)) {
    return l16 + 16 * (h * NRT + rt);
  };
  const int L = (int)(a.n_q + a.n_r);

  // ---- the stream's run of units (32-bit: L_max <= 2^24 tokens)
  const int nqt = (int)(a.n_q / kTile), nrt = (int)cdiv(a.n_r, kTile);
  const int nres = 2 * nrt;                      // ring units
  const int U = nres + (nqt + C::TPU - 1) / C::TPU;
  const int Wt = S * NS;
  // The runs split the work evenly, counted in half-units: a ring unit (the
  // K or the V of a fp16 tile) weighs one, a quantized unit two.  The
  // quotient floor(x W2 / Wt) is taken in fp64, which is exact here (x W2 <
  // 2^40, and a non-integral quotient is at least 1/Wt from an integer) and
  // far cheaper than a 64-bit integer division, which has no instruction.
  constexpr int RW = C::RESU / 256;
  constexpr int QW = C::TPU * ((C::TWO ? 4 : 2) * C::PL + C::VSZB) / 256;
  const double Wtot = (double)nres * RW + (double)(U - nres) * QW;
  auto bound = [&](int x) __attribute__((always_inline)) {
    const int64_t w = (int64_t)((double)x * Wtot / (double)Wt);
    int v;
    if (w <= (int64_t)nres * RW) {
      v = (int)((w + RW) / (2 * RW)) * 2;
    } else {
      v = nres + (int)((w - (int64_t)nres * RW + QW / 2) / QW);
    }
    return v < U ? v : U;
  };
  const int c0s = split * NS;
  // wave-uniform: keep them (and everything derived) in scalar registers
  const int u0 = __builtin_amdgcn_readfirstlane(bound(c0s + strm));
  const int u1 = __builtin_amdgcn_readfirstlane(bound(c0s + strm + 1));

  unsigned char* stages = smem + wave * C::STAGE;
  __half* s_q = (__half*)(smem + C::SAREA);

  const uint8_t* kh_base = a.p.k_hi + blk * g.k_block_bytes;
  const uint8_t* kl_base = C::TWO ? a.p.k_lo + blk * g.k_block_bytes : nullptr;
  const uint8_t* vh_base = a.p.v_hi + blk * g.v_block_bytes;
  const uint8_t* vl_base = C::TWO ? a.p.v_lo + blk * g.v_block_bytes : nullptr;
  const uint8_t* vsz_base = (const uint8_t*)(a.p.v_sz + blk * g.vsz_block);
  const uint8_t* ksz_base = (const uint8_t*)(a.p.k_sz + blk * g.ksz_block);
  const uint8_t* kres_base = (const uint8_t*)(a.p.k_res + blk * g.res_block);
  const uint8_t* vres_base = (const uint8_t*)(a.p.v_res + blk * g.res_block);
  const int nq_mod = a.nq_mod;
  const int tiles_per_group = g.G / kTile;
  // key group of quantized tile t
  auto group_of = [&](int t) __attribute__((always_inline)) {
    return a.grp_shift >= 0 ? t >> a.grp_shift : t / tiles_per_group;
  };

  // ---- staged loads of a unit: fetch loads the unit's chunks into stg
  // (16 bytes per lane, one coalesced instruction per 1 KB chunk), commit
  // writes them to this wave's stage (the compiler waits for the loads
  // there).  Every path of fetch loads every stg entry (lanes past a partial
  // chunk and chunks past a ring unit re-read valid bytes, at addresses no
  // other load uses): a register left unloaded on one path, or a load merged
  // with an identical one, would be filled by a copy, and the copy would
  // wait for the loads just issued.
  const unsigned lofs = 16u * lane;
  // Stage layout: within each 1 KB chunk, the 16-byte pieces of the code
  // planes and of the ring tiles are XOR-permuted so that the compute's
  // LDS reads (16 bytes per lane, rows of 64, 256 or 128 bytes apart) fall
  // in distinct banks; the writes of a chunk stay a permutation of it.
  // Piece p = 64 k + l of a chunk is written by lane l; *_pat is its
  // physical piece within the chunk (identity where the geometry differs).
  constexpr bool SWZ = D == 128 && C::W == 4;   // code planes: 64-byte rows
  constexpr bool SWZR = D == 128;               // ring tiles: 256-byte rows
  const unsigned kpat = SWZ ? (lane & ~3u) | ((lane ^ (lane >> 3)) & 3u) : lane;
  const unsigned vpat = SWZ ? (lane & ~1u) | ((lane ^ (lane >> 3)) & 1u) : lane;
  const unsigned rkpat0 = SWZR ? (lane & ~15u) | ((lane ^ (lane >> 4)) & 15u) : lane;
  const unsigned rkpat1 = SWZR ? (lane & ~15u) | ((lane ^ (4u + (lane >> 4))) & 15u) : lane;
  const unsigned rvpat = SWZR ? (lane & ~7u) | ((lane ^ (lane >> 3)) & 7u) : lane;
  // 4-bit planes at d = 128, one tile per unit: chunk k of a key plane is
  // subtile k (16 tokens x 64 bytes), and lane (l16, gq) loads the 16 bytes
  // it feeds to the score MFMA straight from memory (still one coalesced
  // 1 KB per instruction).  The key codes then skip the stage; the tile's
  // keys are decoded from the buffer before the next unit is fetched.
  constexpr bool DIRECTK = SWZ && C::TPU == 1;
  const unsigned kdir = 64u * (lane & 15u) + 16u * (lane >> 4);
  u4v stg[C::NI];
  // may_ring = false where u is known to be a quantized unit: one load
  // path, so the buffer registers need no merging copies
  // Quantized tile pieces: 0/1 key planes, 2/3 value planes, 4 value
  // scales, 5 key scales; stg index of the first chunk of each piece.
  constexpr int kBytes[6] = {C::PL, C::TWO ? C::PL : 0, C::PL, C::TWO ? C::PL : 0,
                             C::VSZB, C::KSZB};
  constexpr int kFirst[6] = {0, chunks_of(kBytes[0]),
                             chunks_of(kBytes[0]) + chunks_of(kBytes[1]),
                             chunks_of(kBytes[0]) + chunks_of(kBytes[1]) + chunks_of(kBytes[2]),
                             C::NI_TILE - chunks_of(C::VSZB) - chunks_of(C::KSZB),
                             C::NI_TILE - chunks_of(C::KSZB)};
  // parts: 1 = keys and scales, 2 = values (with DIRECTK the values too come
  // straight to the registers, lane l holding its 32 bytes of each plane)
  // XM: the fetched-position mask words of the unit being fetched (loaded
  // before its chunks, so waiting for them never waits for the unit) and of
  // the unit being computed (taken at its commit)
  unsigned xwp[C::TPU], xwc[C::TPU];
#pragma unroll
  for (int j = 0; j < C::TPU; ++j) xwp[j] = xwc[j] = 0u;
  const unsigned* xm_blk = XM ? a.xmask + blk * (g.L_max / kTile) : nullptr;
  auto fetch_quant = [&](int u, int parts) __attribute__((always_inline)) {
    const int t0 = (u - nres) * C::TPU;
    if constexpr (XM) {
      if (parts & 1) {
#pragma unroll
        for (int j = 0; j < C::TPU; ++j)
          xwp[j] = xm_blk[t0 + j < nqt ? t0 + j : nqt - 1];
      }
    }
#pragma unroll
    for (int j = 0; j < C::TPU; ++j) {
      int t = t0 + j < nqt ? t0 + j : nqt - 1;
      t = t > 0 ? t : 0;
      const unsigned po = (unsigned)t * C::PL;
      const uint8_t* src[6] = {kh_base + po, kl_base + po, vh_base + po, vl_base + po,
                               vsz_base + (unsigned)t * C::VSZB,
                               ksz_base + (unsigned)group_of(t) * C::KSZB};
      constexpr int order[6] = {0, 1, 4, 5, 2, 3};   // keys and scales first
#pragma unroll
      for (int oi = 0; oi < 6; ++oi) {
        const int pc = order[oi];
        if (!(parts & (pc == 2 || pc == 3 ? 2 : 1))) continue;
#pragma unroll
        for (int k = 0; k < chunks_of(kBytes[pc]); ++k) {
          const int i = j * C::NI_TILE + kFirst[pc] + k;
          const int rem = kBytes[pc] - 1024 * k;
          if (DIRECTK && (pc == 2 || pc == 3)) {
            stg[i] = *(const u4v*)(src[pc] + 32u * lane + 16 * k);
          } else {
            const unsigned o = DIRECTK && pc < 2 ? kdir
                               : rem >= 1024 || lofs < (unsigned)rem ? lofs : 0u;
            stg[i] = *(const u4v*)(src[pc] + 1024 * k + o);
          }
        }
      }
    }
  };
  auto fetch = [&](int u, bool may_ring) __attribute__((always_inline)) {
    u = __builtin_amdgcn_readfirstlane(u);          // keep the address math scalar
    if (may_ring && u < nres) {
      int slot0 = nq_mod + kTile * (u >> 1);
      slot0 = slot0 >= g.ring ? slot0 - g.ring : slot0;
      const uint8_t* src = ((u & 1) ? vres_base : kres_base) + (unsigned)slot0 * (D * 2);
#pragma unroll
      for (int i = 0; i < C::NI; ++i)   // past NIR: re-reads at distinct addresses
        stg[i] = *(const u4v*)(src + (i < C::NIR ? 1024 * i + lofs
                                                 : 1024 * (i - C::NIR) + lofs + 16));
    } else {
      fetch_quant(u, 3);
    }
  };
  auto commit = [&](int u) __attribute__((always_inline)) {
    if (u < nres) {
      const unsigned pk = 16u * ((u & 1) ? rvpat : rkpat0);
      const unsigned pk1 = 16u * ((u & 1) ? rvpat : rkpat1);
#pragma unroll
      for (int i = 0; i < C::NIR; ++i)
        *(u4v*)(stages + 1024 * i + ((i & 1) ? pk1 : pk)) = stg[i];
    } else {
      if constexpr (XM) {
#pragma unroll
        for (int j = 0; j < C::TPU; ++j) xwc[j] = __builtin_amdgcn_readfirstlane(xwp[j]);
      }
#pragma unroll
      for (int j = 0; j < C::TPU; ++j) {
        constexpr int bytes[6] = {C::PL, C::TWO ? C::PL : 0, C::PL, C::TWO ? C::PL : 0,
                                  C::VSZB, C::KSZB};
        constexpr int offs[6] = {C::O_KH, C::O_KL, C::O_VH, C::O_VL, C::O_VSZ, C::O_KSZ};
        int i = j * C::NI_TILE;
#pragma unroll
        for (int pc = 0; pc < 6; ++pc)
#pragma unroll
          for (int k = 0; k < chunks_of(bytes[pc]); ++k, ++i) {
            const int rem = bytes[pc] - 1024 * k;
            const unsigned o = pc < 2 ? 16u * kpat : pc < 4 ? 16u * vpat : lofs;
            if (!(DIRECTK && pc < 4) && (rem >= 1024 || lofs < (unsigned)rem))
              *(u4v*)(stages + j * C::TILE + offs[pc] + 1024 * k + o) = stg[i];
          }
      }
    }
  };

  // ---- stage the query rows (zero past `rows`); the loads go out before
  // the first unit's, so waiting for them leaves that unit in flight
  {
    constexpr int QPT = (RP * (D / 8) + NT - 1) / NT;   // 16-byte chunks per thread
    const int q_chunks = a.rows * (D / 8);
    u4v qv[QPT];
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int k = tid + i * NT;
      qv[i] = u4v{0u, 0u, 0u, 0u};
      if (k < q_chunks) {
        const int r = k / (D / 8), c8 = k % (D / 8);
        const int t = r / a.hs, hl = a.h0 + r % a.hs;
        qv[i] = *(const u4v*)(a.q + (((int64_t)b * a.T + t) * a.Hq + kvh * a.gs + hl) * D +
                              8 * c8);
      }
    }
    if (u0 < u1) fetch(u0, true);
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int k = tid + i * NT;
      if (k < RP * (D / 8)) *(u4v*)(s_q + 8 * k) = qv[i];
    }
    lds_barrier();
  }

  // ---- per-wave state (NRT 16-row tiles)
  float m_ref[NRT], sig[NRT], l_run[NRT], binit[NRT];
  f4v cinit[NRT];
  f4v acc[NRT][MT];
  float zacc[NRT][NG];
  u4v bqh[NRT][KS], bql[NRT][KS];      // B operands Q' = hi + lo
  u4v bpres[NRT];                      // ring tile: P' between its two units
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    m_ref[rt] = -INFINITY;
    sig[rt] = l_run[rt] = binit[rt] = 0.f;
    cinit[rt] = f4v{0.f, 0.f, 0.f, 0.f};
    bpres[rt] = u4v{0u, 0u, 0u, 0u};
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) zacc[rt][gg] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bqh[rt][ks] = bql[rt][ks] = u4v{0u, 0u, 0u, 0u};
  }
  int cur_grp = -2;                    // -1: ring operands, >= 0: key group
  // exact substitution: rows of query token t_exact (one per GQA head)
  const int xlo = a.t_exact * a.hs, xhi = xlo + a.hs;
  const DecK dk = dec_consts();
  const float c0 = a.c0;
  // channels this lane multiplies in key-group operands: (cA(ks) + j,
  // cA(ks) + DAB + j), j = 0..3
  auto chan_a = [&](int ks) __attribute__((always_inline)) {
    if constexpr (C::W == 4) return gq * (D / 4) + 8 * ks;
    else if constexpr (C::W == 2) return gq * (D / 4) + 16 * (ks / 2) + 4 * (ks % 2);
    else return gq * (D / 4) + 4 * ks;
  };
  constexpr int DAB = C::W == 4 ? 4 : C::W == 2 ? 8 : 16;   // cB - cA
  // With one row tile, q * c0 of those channels stays in registers for the
  // whole run (measured faster than re-reading it from LDS per key group);
  // with two it is re-read (registers).  1/2-bit codes carry their key
  // scales themselves and never rebuild Q'.
  constexpr bool QC = NRT == 1 && !C::LOW;
  float qcA[QC ? KS : 1][4], qcB[QC ? KS : 1][4];
  auto load_qc = [&](int rt, int ks, float* fa, float* fb)
      __attribute__((always_inline)) {
    const __half* qr = s_q + row_of(rt) * D;
    const u2v qa = *(const u2v*)(qr + chan_a(ks));
    const u2v qb = *(const u2v*)(qr + chan_a(ks) + DAB);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      fa[j] = h_at(qa, j) * c0;
      fb[j] = h_at(qb, j) * c0;
    }
  };
  if constexpr (QC) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) load_qc(0, ks, qcA[ks], qcB[ks]);
  }

  auto refresh = [&](int rt) __attribute__((always_inline)) {
    const float v = binit[rt] + sig[rt];
    cinit[rt] = f4v{v, v, v, v};
  };

  // B operands of the fp16 ring: q * c0 over natural channel pairs
  // (2j, 2j+1) of each 8-channel k-step slice.
  auto build_res = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const __half* qr = s_q + row_of(rt) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u4v q8 = *(const u4v*)(qr + gq * (D / 4) + 8 * ks);
        unsigned hi[4], lo[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float xa = opaque(h_lo(q8[j]) * c0);
          const float xb = opaque(h_hi(q8[j]) * c0);
          hi[j] = pack2(xa, xb);
          lo[j] = pack2(xa - h_lo(hi[j]), xb - h_hi(hi[j]));
        }
        bqh[rt][ks] = u4v{hi[0], hi[1], hi[2], hi[3]};
        bql[rt][ks] = u4v{lo[0], lo[1], lo[2], lo[3]};
      }
      binit[rt] = 0.f;
      refresh(rt);
    }
  };

  // B operands of one key group: Q' = q * c0 * s over the channel pairs the
  // code decoder produces for k-step ks; the accumulator start is
  // sum_c q c0 z - KBIAS * sum_c Q'  (the second sum by MFMA against a
  // constant operand, over the same fp16 parts).
  auto build_quant = [&](const unsigned char* ksz) __attribute__((always_inline)) {
    float zs[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) zs[rt] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cA = chan_a(ks);
      const u4v sA = *(const u4v*)(ksz + 4 * cA);          // {s, z} of cA .. cA+3
      const u4v sB = *(const u4v*)(ksz + 4 * (cA + DAB));
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        float fa[4], fb[4];
        if constexpr (QC) {
#pragma unroll
          for (int j = 0; j < 4; ++j) { fa[j] = qcA[ks][j]; fb[j] = qcB[ks][j]; }
        } else {
          load_qc(rt, ks, fa, fb);
        }
        unsigned hi[4], lo[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // Q' = q c0 s as fp16 hi + lo, each from the exact product by one
          // mixed-precision fma (the fp16 s enters unconverted): hi rounds
          // the product once, lo rounds what hi leaves
          hi[j] = hsplit_hi(fa[j], sA[j], fb[j], sB[j]);
          lo[j] = hsplit_lo(fa[j], sA[j], fb[j], sB[j], hi[j]);
          zs[rt] = __builtin_fmaf(fa[j], h_hi(sA[j]), zs[rt]);
          zs[rt] = __builtin_fmaf(fb[j], h_hi(sB[j]), zs[rt]);
        }
        bqh[rt][ks] = u4v{hi[0], hi[1], hi[2], hi[3]};
        bql[rt][ks] = u4v{lo[0], lo[1], lo[2], lo[3]};
      }
    }
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const float z = sum_x4(zs[rt]);
      f4v cc = f4v{z, z, z, z};
      if constexpr (C::KBIAS != 0.f) {
        const u4v kn = u4v{C::NEG, C::NEG, C::NEG, C::NEG};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          cc = mfma16(kn, bqh[rt][ks], cc);
          cc = mfma16(kn, bql[rt][ks], cc);
        }
      }
      binit[rt] = cc[0];
      refresh(rt);
    }
  };

  // 1/2-bit codes (key groups of one or a few tiles) cut the per-group
  // work.  Both decode codes as x = 1 + code 2^-W (lowx), start from fixed
  // fp16 hi + lo pairs of q * c0 * 2^W over the key-group channel pairs,
  // built once when the run leaves the ring, and take a group's start
  // sum_c q c0 z as an MFMA of its zero-point pairs (the same for all 16
  // tokens) against those pairs, times 2^-W.
  //   1-bit: the key scales go into the decoded codes (declow_ks: code s / 2
  //     is exact), so those pairs are Q' itself and a group only brings its
  //     scale pairs.
  //   2-bit: code s is not always an fp16 value, so Q4 = 4 q c0 s is
  //     rebuilt per group with packed fp16 operations from the fixed pairs:
  //     hi' = RN(qh s), lo' = RN(RN(qh s - hi') + ql s), where qh s - hi'
  //     is exact (the residual of a product of two 11-bit significands
  //     under its rounding fits 11 bits), so hi' + lo' carries ~22 bits.
  //     Q4 x = Q4 + Q' code, so the start also takes - sum_c 4 q c0 s, an
  //     MFMA of the scale pairs against the fixed pairs (it differs from
  //     the sum of the rebuilt parts by their own ~2^-22 rounding).
  constexpr bool KSC = C::LOW && C::W == 1;           // scales in the codes
  constexpr int KW = C::LOW ? C::W : 0;
  constexpr bool QH = C::LOW && !KSC && NRT == 1;     // fixed pairs kept
  constexpr unsigned LMASK = ((1u << C::W) - 1u) * (0x00010001u << (10 - C::W));
  const unsigned l_one = C::LOW ? vreg(0x3C003C00u) : 0u;         // fp16 (1, 1)
  const unsigned l_mask = C::LOW ? __builtin_amdgcn_readfirstlane(vreg(LMASK)) : 0u;
  unsigned ksp[KSC ? KS : 1][4];       // key scale pairs of the current group
  u4v qch[QH ? KS : 1], qcl[QH ? KS : 1];
  // hi + lo pairs of q * c0 * 2^KW of row tile rt over k-step ks's pairs
  auto qc_pairs = [&](int rt, int ks, u4v& h4, u4v& l4) __attribute__((always_inline)) {
    float fa[4], fb[4];
    load_qc(rt, ks, fa, fb);
    unsigned hi[4], lo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float xa = opaque(fa[j] * (float)(1 << KW));
      const float xb = opaque(fb[j] * (float)(1 << KW));
      hi[j] = pack2(xa, xb);
      lo[j] = pack2(xa - h_lo(hi[j]), xb - h_hi(hi[j]));
    }
    h4 = u4v{hi[0], hi[1], hi[2], hi[3]};
    l4 = u4v{lo[0], lo[1], lo[2], lo[3]};
  };
  auto build_lowq = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (KSC) {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) qc_pairs(rt, ks, bqh[rt][ks], bql[rt][ks]);
      } else if constexpr (QH) {
        qc_pairs(0, ks, qch[ks], qcl[ks]);
      }
    }
  };
  auto build_lowk = [&](const unsigned char* ksz) __attribute__((always_inline)) {
    f4v cc[NRT], co[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) cc[rt] = co[rt] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cA = chan_a(ks);
      const u4v sA = *(const u4v*)(ksz + 4 * cA);          // {s, z} of cA .. cA+3
      const u4v sB = *(const u4v*)(ksz + 4 * (cA + DAB));
      unsigned sp[4], zp[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sp[j] = __builtin_amdgcn_perm(sB[j], sA[j], 0x05040100u);
        zp[j] = __builtin_amdgcn_perm(sB[j], sA[j], 0x07060302u);
      }
      const u4v az = u4v{zp[0], zp[1], zp[2], zp[3]};
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        if constexpr (KSC) {
#pragma unroll
          for (int j = 0; j < 4; ++j) ksp[ks][j] = sp[j];
          cc[rt] = mfma16(az, bqh[rt][ks], cc[rt]);
          cc[rt] = mfma16(az, bql[rt][ks], cc[rt]);
        } else {
          u4v h4, l4;
          if constexpr (QH) {
            h4 = qch[ks];
            l4 = qcl[ks];
          } else {
            qc_pairs(rt, ks, h4, l4);
          }
          cc[rt] = mfma16(az, h4, cc[rt]);
          cc[rt] = mfma16(az, l4, cc[rt]);
          const u4v as = u4v{sp[0], sp[1], sp[2], sp[3]};
          co[rt] = mfma16(as, h4, co[rt]);
          co[rt] = mfma16(as, l4, co[rt]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
#pragma clang fp contract(off)        // hi must stay the rounded product
            // (vector elements go through scalars: a bit cast of h4[j]
            // itself reads element 0 whatever j is)
            const unsigned hw = h4[j], lw = l4[j], sw = sp[j];
            const h2v qh = __builtin_bit_cast(h2v, hw);
            const h2v ql = __builtin_bit_cast(h2v, lw);
            const h2v sv = __builtin_bit_cast(h2v, sw);
            const h2v hi = qh * sv;
            const h2v lo = __builtin_elementwise_fma(
                ql, sv, __builtin_elementwise_fma(qh, sv, -hi));
            bqh[rt][ks][j] = __builtin_bit_cast(unsigned, hi);
            bql[rt][ks][j] = __builtin_bit_cast(unsigned, lo);
          }
        }
      }
    }
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      binit[rt] = cc[rt][0] * (1.f / (float)(1 << KW)) - co[rt][0];
      refresh(rt);
    }
  };

  // S^T = K Q'^T for the two 16-token subtiles, started at cinit.
  auto scores = [&](f4v (&sc)[2][NRT], const u4v (&ak)[2][KS])
      __attribute__((always_inline)) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) sc[0][rt] = sc[1][rt] = cinit[rt];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          sc[st][rt] = mfma16(ak[st][ks], bqh[rt][ks], sc[st][rt]);
          sc[st][rt] = mfma16(ak[st][ks], bql[rt][ks], sc[st][rt]);
        }
  };

  // Online softmax over the 8 scores this lane holds for row tile rt
  // (taken relative to the row reference, + kPExp); returns p' in place.
  // Fast path: every score of the wave is within kTau of its reference.
  auto softmax = [&](int rt, f4v& s0, f4v& s1) __attribute__((always_inline)) {
    const float lm = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                           fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
    const bool fin = m_ref[rt] != -INFINITY;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(fin && lm <= kPExp + kTau)) == 0, 1)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s0[i] = fast_exp2(s0[i]);
        s1[i] = fast_exp2(s1[i]);
      }
    } else {
      const float mx = max_x4(lm);               // row max, shifted
      const bool trig = !fin || mx > kPExp + kTau;
      const float m_old = m_ref[rt];
      const float m_new = trig ? fmaxf(m_old, mx - sig[rt]) : m_old;
      const float mref = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_old - mref);   // 0 when m_old = -inf
      const float delta = sig[rt] + mref - kPExp;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s0[i] = fast_exp2(s0[i] - delta);
        s1[i] = fast_exp2(s1[i] - delta);
      }
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
        l_run[rt] *= alpha;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[rt][mt] *= alpha;
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) zacc[rt][gg] *= alpha;
      }
      m_ref[rt] = m_new;
      sig[rt] = m_new == -INFINITY ? 0.f : kPExp - m_new;
      refresh(rt);
    }
    l_run[rt] += ((s0[0] + s1[0]) + (s0[1] + s1[1])) +
                 ((s0[2] + s1[2]) + (s0[3] + s1[3]));
  };

  // ---- one quantized 32-token tile from LDS
  auto quant_tile = [&](const unsigned char* tb, int t, int j, bool may_build, int u, bool next)
      __attribute__((always_inline)) {
    if constexpr (C::LOW) {    // the decode below needs the group's scales
      const int grp = group_of(t);
      if (may_build && grp != cur_grp) {
        if (cur_grp < 0) build_lowq();
        build_lowk(tb + C::O_KSZ);
        cur_grp = grp;
      }
    }
    u4v ak[2][KS];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int ko = SWZ ? ((l16 + 16 * st) * 4 + (gq ^ ((l16 >> 1) & 3))) * 16
                         : (l16 + 16 * st) * (D * C::W / 8) + gq * (D * C::W / 32);
      unsigned kh[C::NDK], kl[C::TWO ? C::NDK : 1];
      if constexpr (DIRECTK) {
        static_assert(C::NDK == 4, "one dword quad per subtile");
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          kh[k] = stg[st][k];
          if constexpr (C::TWO) kl[k] = stg[2 + st][k];
        }
      } else {
        lds_read<C::NDK>(tb + C::O_KH + ko, kh);
        if constexpr (C::TWO) lds_read<C::NDK>(tb + C::O_KL + ko, kl);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        unsigned r[4];
        if constexpr (PATH == P_T8) {
          dec8(kh[ks], kl[ks], r, dk);
        } else if constexpr (PATH == P_D4) {
          dec4(kh[ks], r, dk);
        } else {
          constexpr int KPD = 16 / C::W / 4;   // k-steps per dword
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if constexpr (KSC)
              r[j] = declow_ks<C::W>(kh[ks / KPD], 4 * (ks % KPD) + j, ksp[ks][j],
                                     l_one, l_mask);
            else
              r[j] = lowx<C::W>(kh[ks / KPD], 4 * (ks % KPD) + j, l_one, l_mask);
          }
        }
        ak[st][ks] = u4v{r[0], r[1], r[2], r[3]};
      }
    }
    if constexpr (DIRECTK) {   // key and scale registers are free now
      if (next) fetch_quant(__builtin_amdgcn_readfirstlane(u + 1), 1);
    }
    if constexpr (!C::LOW) {
      const int grp = group_of(t);
      if (may_build && grp != cur_grp) {
        build_quant(tb + C::O_KSZ);
        cur_grp = grp;
      }
    }
    f4v sc[2][NRT];
    scores(sc, ak);
    if constexpr (XM) {          // row t_exact leaves fetched positions out
      const unsigned xw = xwc[j];
      if (xw) {                  // wave-uniform: most tiles have none
        const unsigned m4 = xw >> (4 * gq);
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          const int row = row_of(rt);
          if (row >= xlo && row < xhi) {
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if ((m4 >> (16 * st + i)) & 1u) sc[st][rt][i] = -INFINITY;
          }
        }
      }
    }
    // value scale pairs (tokens 4gq+i, 16+4gq+i; [i][group]) and zero pairs
    unsigned sz[8 * NG];
    lds_read<4 * NG>(tb + C::O_VSZ + 16 * NG * gq, sz);
    lds_read<4 * NG>(tb + C::O_VSZ + 16 * NG * gq + 64 * NG, sz + 4 * NG);
    u4v bp[NRT][NG];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      softmax(rt, sc[0][rt], sc[1][rt]);
      unsigned pp[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pp[i] = pack2(sc[0][rt][i], sc[1][rt][i]);
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) {
        float z = zacc[rt][gg];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const unsigned q = hmul2(pp[i], sz[i * NG + gg]);
          bp[rt][gg][i] = q;
          z = dot2(pp[i], sz[4 * NG + i * NG + gg], z);
          z = dot2(q, C::NEG, z);                           // code offset
        }
        zacc[rt][gg] = z;
      }
    }
    unsigned vh[C::NDV], vl[C::TWO ? C::NDV : 1];
    if constexpr (DIRECTK) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        vh[k] = stg[kFirst[2]][k];
        vh[4 + k] = stg[kFirst[2] + 1][k];
        if constexpr (C::TWO) {
          vl[k] = stg[kFirst[3]][k];
          vl[4 + k] = stg[kFirst[3] + 1][k];
        }
      }
    } else if constexpr (SWZ) {   // halves of lane l's 32 bytes, swapped when bit 2 of l is set
      const int s0 = (lane >> 2) & 1;
      const int v0 = (2 * lane + s0) * 16, v1 = (2 * lane + 1 - s0) * 16;
      lds_read<4>(tb + C::O_VH + v0, vh);
      lds_read<4>(tb + C::O_VH + v1, vh + 4);
      if constexpr (C::TWO) {
        lds_read<4>(tb + C::O_VL + v0, vl);
        lds_read<4>(tb + C::O_VL + v1, vl + 4);
      }
    } else {
      lds_read<C::NDV>(tb + C::O_VH + lane * (D * C::W / 16), vh);
      if constexpr (C::TWO) lds_read<C::NDV>(tb + C::O_VL + lane * (D * C::W / 16), vl);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      unsigned r[4];
      if constexpr (PATH == P_T8) {
        dec8(vh[mt], vl[mt], r, dk);
      } else if constexpr (PATH == P_D4) {
        dec4(vh[mt], r, dk);
      } else {
        constexpr int PER = 4 / C::W;   // channel tiles per dword
#pragma unroll
        for (int j = 0; j < 4; ++j)
          r[j] = lowx<C::W>(vh[mt / PER], 4 * (mt % PER) + j, l_one, l_mask);
      }
      const u4v av = u4v{r[0], r[1], r[2], r[3]};
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
        acc[rt][mt] = mfma16(av, bp[rt][mt / (MT / NG)], acc[rt][mt]);
    }
    if constexpr (DIRECTK) {   // value registers are free now
      if (next) fetch_quant(__builtin_amdgcn_readfirstlane(u + 1), 2);
    }
  };

  // ---- ring tile r, first unit: fp16 K -> scores, mask, softmax, P'
  auto ring_k = [&](const unsigned char* sb, int r) __attribute__((always_inline)) {
    if (cur_grp != -1) {
      build_res();
      cur_grp = -1;
    }
    u4v ak[2][KS];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      unsigned kd[D / 8];
      if constexpr (SWZR) {   // pieces gq*4 + j of row l16 + 16 st, XOR (row & 7)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          lds_read<4>(sb + ((l16 + 16 * st) * 16 + ((gq * 4 + j) ^ (l16 & 7))) * 16, kd + 4 * j);
      } else {
        lds_read<D / 8>(sb + ((l16 + 16 * st) * D + gq * (D / 4)) * 2, kd);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        ak[st][ks] = u4v{kd[4 * ks], kd[4 * ks + 1], kd[4 * ks + 2], kd[4 * ks + 3]};
    }
    f4v sc[2][NRT];
    scores(sc, ak);
    // causal / validity mask: row sees positions <= L - T + t(row)
    const int p0 = (int)a.n_q + kTile * r;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const int row = row_of(rt);
      const int lim = row < a.rows ? L - a.T + row / a.hs : L - 1;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pos = p0 + 16 * st + 4 * gq + i;
          sc[st][rt][i] = pos <= lim ? sc[st][rt][i] : -INFINITY;
        }
      softmax(rt, sc[0][rt], sc[1][rt]);
#pragma unroll
      for (int i = 0; i < 4; ++i)   // (times 2^-W: 1/2-bit sums are scaled by 2^W)
        bpres[rt][i] = pack2(sc[0][rt][i] * (1.f / (float)(1 << KW)),
                             sc[1][rt][i] * (1.f / (float)(1 << KW)));
    }
  };

  // ---- ring tile r, second unit: fp16 V (token-permuted) -> O
  auto ring_v = [&](const unsigned char* sb, int r) __attribute__((always_inline)) {
    unsigned vd[D / 4];
    if constexpr (SWZR) {     // pieces j of lane l's 128 bytes, XOR (l & 7)
#pragma unroll
      for (int j = 0; j < 8; ++j) lds_read<4>(sb + (8 * lane + (j ^ (lane & 7))) * 16, vd + 4 * j);
    } else {
      lds_read<D / 4>(sb + lane * D, vd);
    }
    const int p0 = (int)a.n_q + kTile * r;
    if (p0 + kTile > L) {              // zero the slots past the context
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const unsigned keep = (p0 + 4 * gq + i < L ? 0x0000FFFFu : 0u) |
                              (p0 + 16 + 4 * gq + i < L ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) vd[4 * mt + i] &= keep;
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const u4v av = u4v{vd[4 * mt], vd[4 * mt + 1], vd[4 * mt + 2], vd[4 * mt + 3]};
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
        acc[rt][mt] = mfma16(av, bpres[rt], acc[rt][mt]);
    }
  };

  // ---- the unit loop, ring tiles first (K and V unit pairs), then the
  // quantized prefix.  Per unit: its staged chunks go to the stage (the
  // previous unit's reads of it were issued earlier, and LDS runs a wave's
  // accesses in order), then the next unit is fetched while this one is
  // computed.  No wave waits for another: the two waves of a 17..32-row
  // stream each load the whole unit (the second read hits the cache).
  // The two waves on a SIMD have about the same work, but the older one
  // wins issue while both are ready: it would finish first and leave the
  // other running alone.  Issue priority from the units left (3 down to 0
  // over the last four) lets the wave behind catch up before the end.
  auto step = [&](int u, bool quant_next) __attribute__((always_inline)) {
    const int rem = u1 - u;
    if (rem >= 4) __builtin_amdgcn_s_setprio(3);
    else if (rem == 3) __builtin_amdgcn_s_setprio(2);
    else if (rem == 2) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
    commit(u);
    if (!(DIRECTK && u >= nres) && u + 1 < u1) fetch(u + 1, !quant_next);
  };
  // may_build = false when every tile of the unit is known to belong to
  // the current key group: the inner loop below then carries the B
  // operands unchanged, so they stay in place in registers.
  // next = false only at the run's last unit (a call site of its own, so
  // `next` is a constant and the loop keeps one load path): nothing is left
  // in flight after the loop.
  auto quant_unit = [&](int u, bool may_build, bool next) __attribute__((always_inline)) {
    const int t0 = (u - nres) * C::TPU;
#pragma unroll
    for (int j = 0; j < C::TPU; ++j)
      if (t0 + j < nqt) quant_tile(stages + j * C::TILE, t0 + j, j, may_build, u, next);
  };
  auto in_group = [&](int u) __attribute__((always_inline)) {
    const int t0 = (u - nres) * C::TPU;
    const int t1 = (t0 + C::TPU < nqt ? t0 + C::TPU : nqt) - 1;
    return group_of(t0) == cur_grp && group_of(t1) == cur_grp;
  };
  {
    int u = u0;
    const int ur = u1 < nres ? u1 : nres;
    for (; u < ur; u += 2) {
      step(u, false);
      ring_k(stages, u >> 1);
      step(u + 1, false);
      ring_v(stages, u >> 1);
    }
    const int ul = u1 - 1;
    while (u < ul) {
      step(u, true);
      quant_unit(u, true, true);
      ++u;
      for (; u < ul && in_group(u); ++u) {
        step(u, true);
        quant_unit(u, false, true);
      }
    }
    if (u < u1) {                      // the last unit, a quantized one
      step(u, true);
      quant_unit(u, true, false);
    }
  }

  // ---- per-wave finish: full-row l, zero-point term folded into o; all
  // sums carry the 2^kPExp of the probabilities
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    l_run[rt] = sum_x4(l_run[rt]) * kOScale;
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) zacc[rt][gg] = sum_x4(zacc[rt][gg]) * kOScale;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      acc[rt][mt] = acc[rt][mt] * (kOScale * (float)(1 << KW)) +
                    zacc[rt][mt / (MT / NG)];
  }

  // ---- merge the NS streams through LDS in one step: every stream writes
  // its (o, m, l) rows, then each thread of the workgroup combines the NS
  // states of one (row, 4 columns) item and writes it to the workgroup
  // partial o[RP][D], m[RP], l[RP]. Slab rows are padded by 4 floats, so
  // the 16 rows of a wave's write land in different banks. Rows past `rows`
  // are never read by the merge and are not written.
  constexpr int DP = C::DP;
  constexpr int SLAB = RP * DP;
  float* s_slab = (float*)smem;                  // [NS][RP][DP]
  float* s_ml = s_slab + NS * SLAB;              // [NS][m, l][RP]
  lds_barrier();                                 // every stage and q read done
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int row = row_of(rt);
    float* o = s_slab + strm * SLAB + row * DP;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) *(f4v*)(o + 16 * mt + 4 * gq) = acc[rt][mt];
    if (gq == 0) {
      s_ml[strm * 2 * RP + row] = m_ref[rt];
      s_ml[strm * 2 * RP + RP + row] = l_run[rt];
    }
  }
  lds_barrier();
  const int64_t pstride = (int64_t)RP * (D + 2);
  float* po = a.ws + (blk * a.s_alloc + split) * pstride;
  constexpr int DQ = D / 4;
  for (int it = tid; it < a.rows * DQ; it += NT) {
    const int row = it / DQ, c = 4 * (it % DQ);
    float M = -INFINITY;
#pragma unroll
    for (int st = 0; st < NS; ++st) M = fmaxf(M, s_ml[st * 2 * RP + row]);
    f4v o = f4v{0.f, 0.f, 0.f, 0.f};
    float l = 0.f;
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const float ms = s_ml[st * 2 * RP + row];
      const float w = ms == -INFINITY ? 0.f : fast_exp2(ms - M);
      o += *(const f4v*)(s_slab + st * SLAB + row * DP + c) * w;
      l += s_ml[st * 2 * RP + RP + row] * w;
    }
    *(f4v*)(po + row * D + c) = o;
    if (c == 0) {
      po[RP * D + row] = M;
      po[RP * D + RP + row] = l;
    }
  }
}

constexpr int kMaxDevices = 64;

// Device scratch for kv_attn_verify_noalloc: the split partials of callers
// that cannot allocate.  Every GPU the library runs on holds its own copy
// until the process ends; host code uses the per-device address from
// hipGetSymbolAddress, never the array's name (a host-side stand-in).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Workgroups of one instantiation resident per CU on `dev` (0 if unknown).
template <int PATH, int D, int NG, int NRT, bool PAIR, bool XM>
int occupancy(int dev) {
  using C = Cfg<PATH, D, NG, NRT, PAIR>;
  static int cache[kMaxDevices];   // 0 = not queried yet
  if (dev < 0 || dev >= kMaxDevices) return 0;
  if (cache[dev] == 0) {
    hipError_t e = hipFuncSetAttribute(
        (const void*)attn_kernel<PATH, D, NG, NRT, PAIR, XM>,
        hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    if (e != hipSuccess) return 0;
    int n = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &n, (const void*)attn_kernel<PATH, D, NG, NRT, PAIR, XM>, C::NW * kWave, C::LDS);
    if (e != hipSuccess || n < 1) return 0;
    cache[dev] = n;
  }
  return cache[dev];
}

template <int PATH, int D, int NG, int NRT, bool PAIR, bool XM>
hipError_t go(AttnArgs a, hipStream_t s) {
  using C = Cfg<PATH, D, NG, NRT, PAIR>;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int occ = occupancy<PATH, D, NG, NRT, PAIR, XM>(dev);
  if (occ < 1) return hipErrorInvalidConfiguration;
  const int64_t nb = (int64_t)a.g.B * a.g.Hkv;
  const int64_t units = 2 * cdiv(a.n_r, kTile) + cdiv(a.n_q / kTile, C::TPU);
  // the last partial slot of each block stays free for exact substitution
  a.S = plan_splits(nb, (int64_t)cus * occ, units, C::NS, a.s_alloc - 1);
  a.nq_mod = (int)(a.n_q % a.g.ring);
  const int tpg = a.g.G / kTile;
  a.grp_shift = -1;
  for (int k = 0; k < 31; ++k)
    if (tpg == 1 << k) a.grp_shift = k;
  // exact substitution: the mask of fetched positions first, for the split
  // pass to read
  if (a.n_exact >= 0) {
    hipLaunchKernelGGL(mask_kernel, dim3((unsigned)a.g.Hkv, (unsigned)a.g.B),
                       dim3(256), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // grid: splits x kv heads x batch; consecutive workgroups are consecutive
  // splits of one block
  hipLaunchKernelGGL((attn_kernel<PATH, D, NG, NRT, PAIR, XM>),
                     dim3((unsigned)a.S, (unsigned)a.g.Hkv, (unsigned)a.g.B),
                     dim3(C::NW * kWave), C::LDS, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // then the exact-term partial into the spare slot S, once the fetched
  // rows are there (rows_ready: an event recorded after their transfer)
  if (a.n_exact >= 0) {
    if (a.rows_ready) {
      e = hipStreamWaitEvent(s, (hipEvent_t)a.rows_ready, 0);
      if (e != hipSuccess) return e;
    }
    const dim3 xg((unsigned)cdiv(a.hs, 4), (unsigned)a.g.Hkv, (unsigned)a.g.B);
    hipLaunchKernelGGL((exact_kernel<D, C::RP>), xg, dim3(512), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    ++a.S;                       // the merge reads the substitution partial too
  }
  hipLaunchKernelGGL((merge_kernel<D, C::RP>),
                     dim3((unsigned)a.rows, (unsigned)a.g.Hkv, (unsigned)a.g.B),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int PATH, int D, int NRT, bool PAIR>
hipError_t by_ng(const AttnArgs& a, hipStream_t s) {
  switch (a.g.d / a.g.Gv) {
    case 1: return a.xmask ? go<PATH, D, 1, NRT, PAIR, true>(a, s)
                           : go<PATH, D, 1, NRT, PAIR, false>(a, s);
    case 2: return a.xmask ? go<PATH, D, 2, NRT, PAIR, true>(a, s)
                           : go<PATH, D, 2, NRT, PAIR, false>(a, s);
    case 4: return a.xmask ? go<PATH, D, 4, NRT, PAIR, true>(a, s)
                           : go<PATH, D, 4, NRT, PAIR, false>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// 17..32 rows: two waves share a stream, one row tile each (measured
// faster than one wave holding both row tiles at one wave per SIMD).
template <int PATH, int D>
hipError_t by_rows(const AttnArgs& a, hipStream_t s) {
  if (a.rows_pad == 16) return by_ng<PATH, D, 1, false>(a, s);
  return by_ng<PATH, D, 1, true>(a, s);
}

}  // namespace

// Splits per block: enough workgroups to fill every resident slot once,
// choosing among 1x..8x the minimum (up to cap) the count whose last
// dispatch wave is fullest (the smallest such count on ties); no more than
// one split per `streams` units.
int plan_splits(int64_t nb, int64_t slots, int64_t units, int streams, int cap) {
  const int64_t smin = cdiv(slots, nb);
  int64_t best = smin;
  double best_eff = -1.0;
  for (int64_t s = smin; s <= 8 * smin && s <= cap; ++s) {
    const int64_t wg = nb * s;
    const double eff = (double)wg / (double)(slots * cdiv(wg, slots));
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = s;
    }
  }
  const int64_t by_units = cdiv(units, streams);
  if (best > by_units) best = by_units;
  if (best > cap) best = cap;
  return best < 1 ? 1 : (int)best;
}

hipError_t attn_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {              // once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

namespace {
hipError_t launch_rows(const AttnArgs& a, hipStream_t s) {
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
}  // namespace

// Calls with more than 32 rows (T * Hq/Hkv) run as consecutive launches over
// subsets of each kv group's query heads, hs = 32 / T heads at a time: every
// launch reads the whole cache for its heads and writes their rows of out
// and lse; the partial slots are reused in stream order.
hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  if (a.rows <= 32) return launch_rows(a, s);
  const int hs = 32 / a.T;
  for (int h0 = 0; h0 < a.gs; h0 += hs) {
    AttnArgs b = a;
    b.h0 = h0;
    b.hs = a.gs - h0 < hs ? a.gs - h0 : hs;
    b.rows = a.T * b.hs;
    b.rows_pad = b.rows <= 16 ? 16 : 32;
    const hipError_t e = launch_rows(b, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kvq
