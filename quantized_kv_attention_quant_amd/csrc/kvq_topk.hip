// Per-kv-head top-k of the speculative token's scores over the low-bit cache.
//
// SpeCache page, Approach: a speculative token decoded next to the output
// token scores the low-bit KV copy, and its top-k KV pairs are the ones
// prefetched for the next step.  The key of quantized token j of block
// (b, kvh) is the canonical binary32 value documented in kvq.h:
//   k^_jc = z + code*s (code*s exact), logit_hj = sequential sum over c of
//   q_hc * k^_jc with each product and sum rounded separately, key_j = max
//   over the GQA heads of the group, -0 folded to +0.
// The key must match the binary32 definition bit for bit, so this file is
// built with -ffp-contract=off (and the pragma below): no product is fused
// into the following sum.
//
// Two launches:
//   score_kernel, grid chunks x Hkv x B, 256 threads: a workgroup scores a
//     chunk of 1024 tokens, 4 per thread, with q and the chunk's (s, z)
//     pairs staged in LDS; a token's sum runs over c = 0..d-1 in order.
//     Each key becomes a 64-bit composite (order-preserving key bits << 32 |
//     ~index), so one unsigned compare orders by key descending then index
//     ascending.  The chunk's best P (the power of two at or above k) are
//     selected by a bitonic top-P network over the 4 composites each thread
//     holds in registers (compare partners in the same thread or wave are
//     exchanged by lane shuffles; the halving levels pass the survivors
//     through LDS), and its best k go to the workspace, sorted descending.
//   merge_kernel, grid Hkv x B, 512 threads: the chunks' sorted candidate
//     lists enter the same top-P levels as runs, 2048 elements at a time,
//     and the best k are written.  The kernel boundary makes the candidates visible;
//     no fence or counter is needed.
#include "kvq_internal.h"

#pragma clang fp contract(off)

namespace kvq {
namespace {

constexpr int NT = 256;
constexpr int kChunk = 1024;          // tokens per scoring workgroup
constexpr int TPT = kChunk / NT;      // consecutive tokens per thread
static_assert(TPT == 4, "a thread holds 4 composites");

__device__ __forceinline__ unsigned long long composite(float key, int64_t j) {
  unsigned u = __float_as_uint(key);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (0xFFFFFFFFu - (unsigned)j);
}

__device__ __forceinline__ float key_of(unsigned long long c) {
  unsigned u = (unsigned)(c >> 32);
  u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(u);
}

__device__ __forceinline__ unsigned long long shfl_xor64(unsigned long long x,
                                                         int m) {
  const unsigned lo = __shfl_xor((unsigned)x, m);
  const unsigned hi = __shfl_xor((unsigned)(x >> 32), m);
  return ((unsigned long long)hi << 32) | lo;
}

// Descending bitonic sort of the workgroup's NTS * 4 composites, element
// 4 * tid + m in e[m].  Element i meets i ^ j at stage (k, j); the pair is
// put in descending order when (i & k) == 0, ascending otherwise, so the
// run of every stage k ends ordered and the last one sorts all elements.
// Runs of k_first / 2 elements that already stand in that order (even runs
// descending, odd runs ascending) may skip the stages below k_first.
// With k_last below NTS * 4, the network stops after the stages of k_last:
// runs of k_last elements, alternately descending and ascending.
template <int NTS>
__device__ void sort_regs_desc(unsigned long long (&e)[TPT],
                               unsigned long long* lds, int k_first = 2,
                               int k_last = NTS * TPT) {
  const int tid = threadIdx.x;
  for (int k = k_first; k <= k_last; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j < TPT) {                      // both elements in this thread
#pragma unroll
        for (int m = 0; m < TPT; ++m) {
          const int mp = m ^ j;
          if (mp > m) {
            const int i = TPT * tid + m;
            const bool desc = (i & k) == 0;
            const unsigned long long x = e[m], y = e[mp];
            if (desc ? (x < y) : (x > y)) {
              e[m] = y;
              e[mp] = x;
            }
          }
        }
        continue;
      }
      const int tj = j / TPT;             // partner thread: tid ^ tj
      const bool lower = (tid & tj) == 0; // this thread holds the lower index
      unsigned long long y[TPT];
      if (tj < kWave) {
#pragma unroll
        for (int m = 0; m < TPT; ++m) y[m] = shfl_xor64(e[m], tj);
      } else {
        __syncthreads();                  // earlier readers of lds are done
#pragma unroll
        for (int m = 0; m < TPT; ++m) lds[TPT * tid + m] = e[m];
        __syncthreads();
#pragma unroll
        for (int m = 0; m < TPT; ++m) y[m] = lds[TPT * (tid ^ tj) + m];
      }
#pragma unroll
      for (int m = 0; m < TPT; ++m) {
        const int i = TPT * tid + m;
        const bool desc = (i & k) == 0;   // same for both (j < k)
        // the lower index keeps the larger in a descending pair
        const bool keep_max = desc == lower;
        const unsigned long long x = e[m];
        e[m] = keep_max ? (x > y[m] ? x : y[m]) : (x < y[m] ? x : y[m]);
      }
    }
  }
}

// Workgroup barrier for LDS hand-offs only (no global loads are pending
// where it is used).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Levels of a bitonic top-P network: from `live` composites (element
// 4 * tid + m in e[m], runs of P alternately descending and ascending, P a
// power of two, 4 <= P <= live / 2) down to the best P, sorted descending
// in the first P / 4 threads.  Each level keeps the max of element i of a
// descending run and element i of the ascending run after it (the best P
// of the two, a bitonic sequence) and sorts it again in log2(P)
// compare-exchange stages, alternating the direction by run.  The
// survivors of each level move through LDS to the first threads, so the
// waves left without live elements drop out of the later levels.
template <int NTS>
__device__ void top_reduce(unsigned long long (&e)[TPT], unsigned long long* lds,
                           int P, int live) {
  const int tid = threadIdx.x;
  for (; live > P; live >>= 1) {
    lds_barrier();                              // earlier readers of lds done
    if (TPT * tid < live) {
#pragma unroll
      for (int m = 0; m < TPT; ++m) lds[TPT * tid + m] = e[m];
    }
    lds_barrier();
    const int half = live >> 1;
    if (TPT * tid < half) {
#pragma unroll
      for (int m = 0; m < TPT; ++m) {
        const int i = TPT * tid + m;
        const int r = i / P, o = i % P;         // survivor run r, offset o
        const unsigned long long x = lds[2 * r * P + o], y = lds[(2 * r + 1) * P + o];
        e[m] = x > y ? x : y;
      }
      for (int j = P >> 1; j > 0; j >>= 1) {    // sort each run: P / 2 .. 1
        if (j < TPT) {                          // both elements in this thread
#pragma unroll
          for (int m = 0; m < TPT; ++m) {
            const int mp = m ^ j;
            if (mp > m) {
              const int i = TPT * tid + m;
              const bool desc = ((i / P) & 1) == 0;
              const unsigned long long x = e[m], y = e[mp];
              if (desc ? (x < y) : (x > y)) {
                e[m] = y;
                e[mp] = x;
              }
            }
          }
          continue;
        }
        const int tj = j / TPT;                 // partner thread in the wave
        const bool lower = (tid & tj) == 0;
#pragma unroll
        for (int m = 0; m < TPT; ++m) {
          const unsigned long long y = shfl_xor64(e[m], tj);
          const int i = TPT * tid + m;
          const bool keep_max = (((i / P) & 1) == 0) == lower;
          const unsigned long long x = e[m];
          e[m] = keep_max ? (x > y ? x : y) : (x < y ? x : y);
        }
      }
    }
  }
}

// The best P of the workgroup's NT * 4 composites, sorted descending in the
// first P / 4 threads: runs of P sorted by the network's first stages, then
// the halving levels.
__device__ void chunk_top(unsigned long long (&e)[TPT], unsigned long long* lds,
                          int P) {
  sort_regs_desc<NT>(e, lds, 2, P);
  top_reduce<NT>(e, lds, P, NT * TPT);
}

// Code of channel cc of a 1/2-bit code dword as a float, from the dword
// masked to one code per byte: mw[r] = (h >> (W * r)) & (one code mask in
// each byte), so channel cc = (8 / W) * byte + r sits in byte cc / (8 / W)
// of mw[cc % (8 / W)] and converts with one byte-to-float instruction.
template <int W>
__device__ __forceinline__ float code_bytes(const unsigned (&mw)[8 / W], int cc) {
  return (float)((mw[cc % (8 / W)] >> (8 * (cc / (8 / W)))) & 0xFFu);
}

// Code of channel cc of a code dword (hi plane; lo plane for 8-bit), per
// path, as a float.
template <int BITS, int PATH>
__device__ __forceinline__ float code_of(unsigned h, unsigned l, int cc) {
  if constexpr (BITS == 8) {
    const unsigned hn = (h >> (4 * cc)) & 15u;
    if constexpr (PATH == KVQ_DRAFT4) {
      return (float)(16u * hn) + 7.5f;
    } else {
      return (float)(16u * hn + ((l >> (4 * cc)) & 15u));
    }
  } else if constexpr (BITS == 2) {
    return (float)((h >> (2 * cc)) & 3u);
  } else {
    return (float)((h >> cc) & 1u);
  }
}

template <int BITS, int PATH, int D, int GS>
__global__ void __launch_bounds__(NT) score_kernel(const TopkArgs a) {
  constexpr int NGC = kChunk / 32 + 1;           // key groups a chunk can touch
  constexpr int SZR = D + 1;                     // padded row: groups in distinct banks
  __shared__ float s_q[D][GS];                   // q of the group, channel-major
  __shared__ __half2 s_sz[NGC * SZR];            // (s, z) of the chunk's key groups
  // the selection's exchange buffer reuses the (s, z) rows: every LDS write
  // of the selection follows a barrier after the last scoring read
  static_assert(sizeof(__half2) * NGC * SZR >= sizeof(unsigned long long) * NT * TPT,
                "exchange buffer fits the staged scales");
  unsigned long long* s_x = (unsigned long long*)s_sz;
  const CacheGeom& g = a.g;
  const int b = blockIdx.z, kvh = blockIdx.y, chunk = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t blk = (int64_t)b * g.Hkv + kvh;

  // GS is a.gs rounded up to a power of two; the slots past a.gs repeat
  // the group's last head, whose logit the max already holds
  for (int e = tid; e < GS * D; e += NT) {
    const int h = e / D, c = e % D;
    const int hs = h < a.gs ? h : a.gs - 1;
    s_q[c][h] = __half2float(a.q[((int64_t)b * a.Hq + kvh * a.gs + hs) * D + c]);
  }
  // the key groups the chunk's tokens fall in (G is a multiple of 32, so a
  // chunk touches at most 1024/32 + 1); groups past n_q are not read
  const int64_t c0 = (int64_t)chunk * kChunk;
  const int64_t gi0 = c0 / g.G;
  const int ng = (int)((c0 + kChunk - 1) / g.G - gi0) + 1;
  const __half2* ksz = a.p.k_sz + blk * g.ksz_block;
  for (int e = tid; e < ng * D; e += NT) {
    const int gi = e / D, c = e % D;
    s_sz[gi * SZR + c] = (gi0 + gi) * g.G < a.n_q ? ksz[(gi0 + gi) * D + c]
                                                  : __floats2half2_rn(0.f, 0.f);
  }
  __syncthreads();

  constexpr int W = BITS == 8 ? 4 : BITS;
  constexpr int NDW = D * W / 32;                // code dwords per plane row
  constexpr int CPD = 32 / W;                    // channels per code dword
  constexpr bool LO = BITS == 8 && PATH != KVQ_DRAFT4;
  const uint8_t* kh = a.p.k_hi + blk * g.k_block_bytes;
  const uint8_t* kl = LO ? a.p.k_lo + blk * g.k_block_bytes : nullptr;

  unsigned long long comp[TPT];
  if constexpr (BITS != 8) {
    // 1/2-bit codes: thread t scores the 4 consecutive tokens 4t .. 4t + 3
    // of the chunk together.  They share one key group (G is a multiple of
    // 32), so each channel's q and (s, z) come out of LDS once for all four
    // tokens; every token's sum still runs over c = 0..d-1 in order.  n_q is
    // a multiple of G, so the four are valid together or not at all.
    const int64_t j0 = c0 + TPT * tid;
    if (j0 < a.n_q) {
      unsigned hw[TPT][NDW];
#pragma unroll
      for (int x = 0; x < NDW / 4; ++x)
#pragma unroll
        for (int m = 0; m < TPT; ++m) {
          const uint4 v = ((const uint4*)(kh + (j0 + m) * (NDW * 4)))[x];
          hw[m][4 * x] = v.x; hw[m][4 * x + 1] = v.y;
          hw[m][4 * x + 2] = v.z; hw[m][4 * x + 3] = v.w;
        }
      const __half2* sz = s_sz + (int)(j0 / g.G - gi0) * SZR;
      float acc[TPT][GS];
#pragma unroll
      for (int m = 0; m < TPT; ++m)
#pragma unroll
        for (int h = 0; h < GS; ++h) acc[m][h] = 0.f;
      // one code dword per token per iteration; the dwords move down a
      // register window so the loop stays rolled
#pragma unroll 1
      for (int x = 0; x < NDW; ++x) {
        unsigned h0[TPT];
#pragma unroll
        for (int m = 0; m < TPT; ++m) {
          h0[m] = hw[m][0];
#pragma unroll
          for (int i = 0; i + 1 < NDW; ++i) hw[m][i] = hw[m][i + 1];
        }
        constexpr unsigned BM = BITS == 2 ? 0x03030303u : 0x01010101u;
        unsigned mw[TPT][8 / BITS];
#pragma unroll
        for (int m = 0; m < TPT; ++m)
#pragma unroll
          for (int r = 0; r < 8 / BITS; ++r) {
            mw[m][r] = (h0[m] >> (BITS * r)) & BM;
            // opaque to the optimizer, which would otherwise fold the mask
            // back into one bit-field extract per channel
            asm("" : "+v"(mw[m][r]));
          }
#pragma unroll
        for (int cc = 0; cc < CPD; ++cc) {
          const int c = x * CPD + cc;
          const float2 p = __half22float2(sz[c]);   // (s, z)
          float qc[GS];
#pragma unroll
          for (int h = 0; h < GS; ++h) qc[h] = s_q[c][h];
#pragma unroll
          for (int m = 0; m < TPT; ++m) {
            // z + code * s with code * s exact (a code of <= 8 bits times
            // an fp16 scale fits binary32), so one fused op rounds the same
            const float kc = __builtin_fmaf(code_bytes<BITS>(mw[m], cc), p.x, p.y);
#pragma unroll
            for (int h = 0; h < GS; ++h) acc[m][h] = acc[m][h] + qc[h] * kc;
          }
        }
      }
#pragma unroll
      for (int m = 0; m < TPT; ++m) {
        float key = acc[m][0];
#pragma unroll
        for (int h = 1; h < GS; ++h) key = fmaxf(key, acc[m][h]);
        key = key + 0.f;
        comp[m] = composite(key, j0 + m);
      }
    } else {
#pragma unroll
      for (int m = 0; m < TPT; ++m) comp[m] = 0ull;   // below every real key
    }
  } else {
    // 8-bit codes: thread t scores tokens t, t + 256, t + 512, t + 768 of the
    // chunk one at a time (one code row load per wave is one contiguous span)
#pragma unroll 1
    for (int m = 0; m < TPT; ++m) {
      const int64_t j = c0 + m * NT + tid;
      unsigned long long cm = 0ull;                // below every real key
      if (j < a.n_q) {
        unsigned hw[NDW], lw[LO ? NDW : 1];
#pragma unroll
        for (int x = 0; x < NDW / 4; ++x) {
          const uint4 v = ((const uint4*)(kh + j * (NDW * 4)))[x];
          hw[4 * x] = v.x; hw[4 * x + 1] = v.y; hw[4 * x + 2] = v.z; hw[4 * x + 3] = v.w;
          if constexpr (LO) {
            const uint4 u = ((const uint4*)(kl + j * (NDW * 4)))[x];
            lw[4 * x] = u.x; lw[4 * x + 1] = u.y; lw[4 * x + 2] = u.z; lw[4 * x + 3] = u.w;
          }
        }
        const __half2* sz = s_sz + (int)(j / g.G - gi0) * SZR;
        float acc[GS];
#pragma unroll
        for (int h = 0; h < GS; ++h) acc[h] = 0.f;
        // channels in order, one code dword per iteration; the dwords move
        // down a register window so the loop stays rolled (unrolled, every
        // channel's LDS reads would be hoisted and hold the registers)
#pragma unroll 1
        for (int x = 0; x < NDW; ++x) {
          const unsigned h0 = hw[0], l0 = LO ? lw[0] : 0u;
#pragma unroll
          for (int i = 0; i + 1 < NDW; ++i) {
            hw[i] = hw[i + 1];
            if constexpr (LO) lw[i] = lw[i + 1];
          }
#pragma unroll
          for (int cc = 0; cc < CPD; ++cc) {
            const int c = x * CPD + cc;
            const float code = code_of<BITS, PATH>(h0, l0, cc);
            const float2 p = __half22float2(sz[c]);   // (s, z)
            // z + code * s, code * s exact: one fused op rounds the same
            const float kc = __builtin_fmaf(code, p.x, p.y);
#pragma unroll
            for (int h = 0; h < GS; ++h) acc[h] = acc[h] + s_q[c][h] * kc;
          }
        }
        float key = acc[0];
#pragma unroll
        for (int h = 1; h < GS; ++h) key = fmaxf(key, acc[h]);
        key = key + 0.f;
        cm = composite(key, j);
      }
      comp[m] = cm;
    }
  }

  // the chunk's best k, sorted descending: the top-P network for P the
  // power of two at or above k, a full sort when P would exceed half the
  // chunk
  int P = TPT;
  while (P < a.k) P <<= 1;
  if (P <= NT * TPT / 2) chunk_top(comp, s_x, P);
  else sort_regs_desc<NT>(comp, s_x);
  unsigned long long* cand = a.cand + (blk * a.chunks + chunk) * a.k;
#pragma unroll
  for (int m = 0; m < TPT; ++m)
    if (TPT * tid + m < a.k) cand[TPT * tid + m] = comp[m];
}

// One workgroup per block: the best k of the chunks' candidates.
constexpr int NTM = 512;                 // merge threads
__global__ void __launch_bounds__(NTM) merge_kernel(const TopkArgs a) {
  __shared__ unsigned long long s_x[NTM * TPT];
  constexpr int cap = NTM * TPT;
  const int b = blockIdx.y, kvh = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t blk = (int64_t)b * a.g.Hkv + kvh;
  const unsigned long long* all = a.cand + blk * a.chunks * a.k;
  unsigned long long e[TPT];
  // each chunk's k candidates are sorted descending: chunk list c becomes a
  // run of P (P the power of two at or above k; past k, zeros, below every
  // real key), odd runs reversed, which is the state the top-P levels
  // start from; cap / P runs per pass, the best run kept as run 0 of the
  // next pass
  int P = TPT;
  while (P < a.k) P <<= 1;
  const int R = cap / P;                        // runs per pass (>= 8)
  auto elem = [&](int r, int c, int o) {        // run r from chunk c, offset o
    const int x = (r & 1) ? P - 1 - o : o;
    return c < a.chunks && x < a.k ? all[(int64_t)c * a.k + x] : 0ull;
  };
#pragma unroll
  for (int m = 0; m < TPT; ++m) {
    const int i = TPT * tid + m;
    e[m] = elem(i / P, i / P, i % P);
  }
  top_reduce<NTM>(e, s_x, P, cap);
  for (int next = R; next < a.chunks; next += R - 1) {
#pragma unroll
    for (int m = 0; m < TPT; ++m) {
      const int i = TPT * tid + m;
      if (i >= P) e[m] = elem(i / P, next + i / P - 1, i % P);
    }
    top_reduce<NTM>(e, s_x, P, cap);
  }
  int32_t* idx = a.idx + blk * a.k;
  float* key = a.key ? a.key + blk * a.k : nullptr;
#pragma unroll
  for (int m = 0; m < TPT; ++m) {
    const int i = TPT * tid + m;
    if (i < a.k) {
      const unsigned long long c = e[m];
      const bool valid = c != 0ull;
      idx[i] = valid ? (int32_t)(0xFFFFFFFFu - (unsigned)(c & 0xFFFFFFFFu)) : -1;
      if (key) key[i] = valid ? key_of(c) : -INFINITY;
    }
  }
}

template <int BITS, int PATH, int D, int GS>
hipError_t go(const TopkArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((score_kernel<BITS, PATH, D, GS>),
                     dim3(a.chunks, a.g.Hkv, a.g.B), dim3(NT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_kernel, dim3(a.g.Hkv, a.g.B), dim3(NTM), 0, s, a);
  return hipGetLastError();
}

// Query heads per kv head, rounded up to a power of two (at most 8).
template <int BITS, int PATH, int D>
hipError_t by_gs(const TopkArgs& a, hipStream_t s) {
  if (a.gs == 1) return go<BITS, PATH, D, 1>(a, s);
  if (a.gs == 2) return go<BITS, PATH, D, 2>(a, s);
  if (a.gs <= 4) return go<BITS, PATH, D, 4>(a, s);
  if (a.gs <= 8) return go<BITS, PATH, D, 8>(a, s);
  return hipErrorInvalidValue;
}

template <int BITS, int PATH>
hipError_t by_d(const TopkArgs& a, hipStream_t s) {
  return a.g.d == 64 ? by_gs<BITS, PATH, 64>(a, s) : by_gs<BITS, PATH, 128>(a, s);
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  // the top-P levels exchange compare partners within a wave: P <= 256
  if (a.chunk != kChunk || a.k < 1 || a.k > 256) return hipErrorInvalidValue;
  if (a.g.bits == 8)
    return a.path == KVQ_DRAFT4 ? by_d<8, KVQ_DRAFT4>(a, s)
                                : by_d<8, KVQ_TARGET>(a, s);
  if (a.g.bits == 2) return by_d<2, KVQ_TARGET>(a, s);
  if (a.g.d == 128) return by_gs<1, KVQ_TARGET, 128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace kvq
