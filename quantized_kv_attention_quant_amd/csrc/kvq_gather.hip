// On-demand reconstruction of a token subset of the quantized cache.
//
// MSpecKV page, Abstract: offloaded KV stays in quantized form and only the
// subsets that are needed are rebuilt when asked for.  Here a request is a
// list of token positions per (b, kvh) block; each position's key and value
// rows are written out in fp16:
//   quantized tokens (p < n_q):  x^ = fp16_rne( f32(z + f32(code * s)) )
//     with code = q (KVQ_TARGET, every stored bit) or 16*hi + 7.5
//     (KVQ_DRAFT4, the upper nibble the QuantSpec draft reads), the same
//     binary32 sequence as the top-k keys (one multiply, one add, no fusion);
//   residual tokens (n_q <= p < n_q + n_r):  the fp16 values in the ring;
//   any other position:  fp16 NaN rows (nothing outside the cache is read).
//
// One wave per requested token: lane l owns channels l, l + 64, ...  Key
// codes are one byte (and bit field) per channel of the token's plane row;
// value codes sit in the 32-token tile layout, one bit field per channel in
// a dword shared with the tile's other tokens.
#include "kvq_internal.h"

// Bit-exact binary32 arithmetic: built with -ffp-contract=off as well.
#pragma clang fp contract(off)

namespace kvq {
namespace {

constexpr int kWavesPerGroup = 4;

__global__ void __launch_bounds__(kWavesPerGroup * kWave)
    gather_kernel(const GatherArgs a) {
  const CacheGeom& g = a.g;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int64_t blk = (int64_t)b * g.Hkv + kvh;
  const int i = blockIdx.x * kWavesPerGroup + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (i >= a.n) return;
  const int d = g.d;
  const int64_t p = a.idx[blk * a.n + i];
  __half* ko = a.k_out + (blk * a.n + i) * d;
  __half* vo = a.v_out + (blk * a.n + i) * d;
  const int64_t L = a.n_q + a.n_r;

  if (p < 0 || p >= L) {
    const __half nan = __ushort_as_half((unsigned short)0x7e00);
    for (int c = lane; c < d; c += kWave) {
      ko[c] = nan;
      vo[c] = nan;
    }
    return;
  }
  if (p >= a.n_q) {                       // residual: ring slot p % ring
    const int slot = (int)(p % g.ring);
    const __half* kr = a.p.k_res + blk * g.res_block + (int64_t)slot * d;
    const __half* vr = a.p.v_res + blk * g.res_block + (int64_t)(slot / kTile) * kTile * d;
    for (int c = lane; c < d; c += kWave) {
      ko[c] = kr[c];
      vo[c] = vr[vres_index(slot % kTile, c, d)];
    }
    return;
  }

  const bool draft = a.path == KVQ_DRAFT4;
  for (int c = lane; c < d; c += kWave) {
    const __half2 ksz = key_sz(g, a.p, blk, p, c);
    const float kx = __fadd_rn(__high2float(ksz),
                               __fmul_rn(key_code(g, a.p, blk, p, c, draft), __low2float(ksz)));
    ko[c] = __float2half_rn(kx);
    const float2 vsz = value_sz(g, a.p, blk, p, c);
    const float vx = __fadd_rn(vsz.y, __fmul_rn(value_code(g, a.p, blk, p, c, draft), vsz.x));
    vo[c] = __float2half_rn(vx);
  }
}

// Rows of the host-resident fp16 copy (SpeCache page, Approach: the KV
// pairs the speculative token selects are fetched), one request of n rows
// per block: it crosses the host link once, as 2 * n * d * 2 bytes per block
// (the buffers are device-accessible pinned allocations).  The transfer is
// bound by the host link, not the CUs, so a small fixed grid carries it:
// kFetchGroups workgroups, each wave keeping UR groups of rows in flight
// (lane piece p of a row moves bytes 16p..16p+15 of its K and V), and the
// CUs stay free for attention running concurrently on another stream.
constexpr int kFetchGroups = 8, kFetchWaves = 8;

template <int D>
__global__ void __launch_bounds__(kFetchWaves * kWave)
    fetch_kernel(const FetchArgs a) {
  constexpr int LPR = D / 8;                    // lanes per row (16 bytes each)
  constexpr int RPW = kWave / LPR;              // rows per wave per load
  constexpr int UR = 4;                         // row groups in flight
  const int64_t total = (int64_t)a.B * a.Hkv * a.n;
  const int lane = threadIdx.x % kWave, sub = lane / LPR, piece = lane % LPR;
  const int64_t wave = (int64_t)blockIdx.x * kFetchWaves + threadIdx.x / kWave;
  const int64_t step = (int64_t)gridDim.x * kFetchWaves * RPW * UR;
  const unsigned nan2 = 0x7e007e00u;
  for (int64_t r0 = wave * RPW * UR; r0 < total; r0 += step) {
    uint4 kx[UR], vx[UR];
#pragma unroll
    for (int u = 0; u < UR; ++u) {              // every load first
      const int64_t r = r0 + u * RPW + sub;     // row blk * n + i
      kx[u] = vx[u] = make_uint4(nan2, nan2, nan2, nan2);
      if (r < total) {
        const int64_t p = a.idx[r];
        if (p >= 0 && p < a.host_len) {
          const int64_t blk = r / a.n;
          const int64_t row = (blk * a.host_len + p) * D;
          kx[u] = ((const uint4*)(a.host_k + row))[piece];
          vx[u] = ((const uint4*)(a.host_v + row))[piece];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      const int64_t r = r0 + u * RPW + sub;
      if (r < total) {
        ((uint4*)(a.k_out + r * D))[piece] = kx[u];
        ((uint4*)(a.v_out + r * D))[piece] = vx[u];
      }
    }
  }
}

}  // namespace

hipError_t launch_fetch(const FetchArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  const int64_t rows = (int64_t)a.B * a.Hkv * a.n;
  const int per_group = kFetchWaves * (kWave / (a.d / 8)) * 4;
  const unsigned groups = (unsigned)(cdiv(rows, per_group) < kFetchGroups
                                         ? cdiv(rows, per_group) : kFetchGroups);
  if (a.d == 128)
    hipLaunchKernelGGL(fetch_kernel<128>, dim3(groups), dim3(kFetchWaves * kWave), 0, s, a);
  else
    hipLaunchKernelGGL(fetch_kernel<64>, dim3(groups), dim3(kFetchWaves * kWave), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_kernel,
                     dim3((unsigned)cdiv(a.n, kWavesPerGroup), (unsigned)a.g.Hkv,
                          (unsigned)a.g.B),
                     dim3(kWavesPerGroup * kWave), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
