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
// Grid: chunks x Hkv x B, 256 threads; a workgroup scores a chunk of 1024
// tokens (4 per thread), turns each key into a 64-bit composite
// (order-preserving key bits << 32 | ~index) so that one unsigned compare
// orders by key descending then index ascending, sorts the chunk in LDS
// (bitonic) and writes its best k.  The last workgroup of the block (atomic
// ticket, self-resetting) merges the chunk candidates the same way.
#include "kvq_internal.h"

#pragma clang fp contract(off)

namespace kvq {
namespace {

constexpr int NT = 256;
constexpr int kChunk = 1024;

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

// Descending bitonic sort of n (power of two) composites in LDS.
__device__ void sort_desc(unsigned long long* v, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += NT) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const unsigned long long x = v[i], y = v[ixj];
          const bool up = (i & k) == 0;   // this run ends descending
          if (up ? (x < y) : (x > y)) {
            v[i] = y;
            v[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

template <int BITS, int PATH, int D, int GS>
__global__ void __launch_bounds__(NT) topk_kernel(const TopkArgs a) {
  __shared__ float s_q[GS * D];
  __shared__ unsigned long long s_c[2 * kChunk];
  __shared__ int s_flag;
  const CacheGeom& g = a.g;
  const int b = blockIdx.z, kvh = blockIdx.y, chunk = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t blk = (int64_t)b * g.Hkv + kvh;

  for (int e = tid; e < GS * D; e += NT)
    s_q[e] = __half2float(a.q[((int64_t)b * a.Hq + kvh * GS + e / D) * D + e % D]);
  __syncthreads();

  constexpr int W = BITS == 8 ? 4 : BITS;
  constexpr int ROW = D * W / 8;
  const uint8_t* kh = a.p.k_hi + blk * g.k_block_bytes;
  const uint8_t* kl = BITS == 8 ? a.p.k_lo + blk * g.k_block_bytes : nullptr;
  const __half2* ksz = a.p.k_sz + blk * g.ksz_block;

  for (int e = tid; e < kChunk; e += NT) {
    const int64_t j = (int64_t)chunk * kChunk + e;
    unsigned long long comp = 0ull;   // below every real key
    if (j < a.n_q) {
      constexpr int NDW = ROW / 4;
      unsigned hw[NDW], lw[BITS == 8 ? NDW : 1];
#pragma unroll
      for (int x = 0; x < NDW / 4; ++x) {
        const uint4 v = ((const uint4*)(kh + j * ROW))[x];
        hw[4 * x] = v.x; hw[4 * x + 1] = v.y; hw[4 * x + 2] = v.z; hw[4 * x + 3] = v.w;
        if constexpr (BITS == 8) {
          const uint4 u = ((const uint4*)(kl + j * ROW))[x];
          lw[4 * x] = u.x; lw[4 * x + 1] = u.y; lw[4 * x + 2] = u.z; lw[4 * x + 3] = u.w;
        }
      }
      const __half2* sz = ksz + (j / g.G) * D;
      float acc[GS];
#pragma unroll
      for (int h = 0; h < GS; ++h) acc[h] = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) {
        float code;
        if constexpr (BITS == 8) {
          const unsigned hn = (hw[c / 8] >> (4 * (c % 8))) & 15u;
          if constexpr (PATH == KVQ_DRAFT4) {
            code = (float)(16u * hn) + 7.5f;
          } else {
            const unsigned ln = (lw[c / 8] >> (4 * (c % 8))) & 15u;
            code = (float)(16u * hn + ln);
          }
        } else if constexpr (BITS == 2) {
          code = (float)((hw[c / 16] >> (2 * (c % 16))) & 3u);
        } else {
          code = (float)((hw[c / 32] >> (c % 32)) & 1u);
        }
        const float2 p = __half22float2(sz[c]);   // (s, z)
        const float kc = p.y + code * p.x;
#pragma unroll
        for (int h = 0; h < GS; ++h) acc[h] = acc[h] + s_q[h * D + c] * kc;
      }
      float key = acc[0];
#pragma unroll
      for (int h = 1; h < GS; ++h) key = fmaxf(key, acc[h]);
      key = key + 0.f;
      comp = composite(key, j);
    }
    s_c[e] = comp;
  }
  __syncthreads();
  sort_desc(s_c, kChunk);
  unsigned long long* cand = a.cand + (blk * a.chunks + chunk) * a.k;
  for (int i = tid; i < a.k; i += NT) cand[i] = s_c[i];

  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = atomicAdd(&a.tickets[blk], 1u);
    s_flag = prev == (unsigned)(a.chunks - 1);
  }
  __syncthreads();
  if (!s_flag) return;
  __threadfence();

  // Merge: keep the best k in s_c[0, k); refill the rest in batches.
  const unsigned long long* all = a.cand + blk * a.chunks * a.k;
  const int total = a.chunks * a.k;
  const int cap = 2 * kChunk;
  int taken = 0;
  for (int i = tid; i < cap; i += NT) s_c[i] = i < total ? all[i] : 0ull;
  taken = total < cap ? total : cap;
  __syncthreads();
  sort_desc(s_c, cap);
  while (taken < total) {
    const int room = cap - a.k;
    for (int i = tid; i < room; i += NT)
      s_c[a.k + i] = taken + i < total ? all[taken + i] : 0ull;
    taken += room;
    __syncthreads();
    sort_desc(s_c, cap);
  }
  int32_t* idx = a.idx + blk * a.k;
  float* key = a.key ? a.key + blk * a.k : nullptr;
  for (int i = tid; i < a.k; i += NT) {
    const unsigned long long c = s_c[i];
    const bool valid = c != 0ull;
    idx[i] = valid ? (int32_t)(0xFFFFFFFFu - (unsigned)(c & 0xFFFFFFFFu)) : -1;
    if (key) key[i] = valid ? key_of(c) : -INFINITY;
  }
  if (tid == 0) a.tickets[blk] = 0u;
}

template <int BITS, int PATH, int D, int GS>
hipError_t go(const TopkArgs& a, hipStream_t s) {
  dim3 grid(a.chunks, a.g.Hkv, a.g.B);
  hipLaunchKernelGGL((topk_kernel<BITS, PATH, D, GS>), grid, dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <int BITS, int PATH, int D>
hipError_t by_gs(const TopkArgs& a, hipStream_t s) {
  switch (a.gs) {
    case 1: return go<BITS, PATH, D, 1>(a, s);
    case 2: return go<BITS, PATH, D, 2>(a, s);
    case 4: return go<BITS, PATH, D, 4>(a, s);
    case 8: return go<BITS, PATH, D, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int BITS, int PATH>
hipError_t by_d(const TopkArgs& a, hipStream_t s) {
  return a.g.d == 64 ? by_gs<BITS, PATH, 64>(a, s) : by_gs<BITS, PATH, 128>(a, s);
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.g.bits == 8)
    return a.path == KVQ_DRAFT4 ? by_d<8, KVQ_DRAFT4>(a, s)
                                : by_d<8, KVQ_TARGET>(a, s);
  if (a.g.bits == 2) return by_d<2, KVQ_TARGET>(a, s);
  if (a.g.d == 128) return by_gs<1, KVQ_TARGET, 128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace kvq
