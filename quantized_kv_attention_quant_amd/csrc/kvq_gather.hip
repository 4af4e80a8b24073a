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

// Rows of a full-precision copy of the cache kept in host memory (SpeCache
// page, Approach: the full KV stays off the GPU and the pairs the
// speculative token selects are fetched).  One wave per requested row; each
// lane moves 16 bytes of K and of V straight from host memory (the buffers
// are device-accessible pinned allocations), so a request of n rows per
// block crosses the host link once, as 2 * n * d * 2 bytes per block.
__global__ void __launch_bounds__(kWavesPerGroup * kWave)
    fetch_kernel(const FetchArgs a) {
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int64_t blk = (int64_t)b * a.Hkv + kvh;
  const int i = blockIdx.x * kWavesPerGroup + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (i >= a.n) return;
  const int d8 = a.d / 8;                       // 16-byte pieces per row
  const int64_t p = a.idx[blk * a.n + i];
  uint4* ko = (uint4*)(a.k_out + (blk * a.n + i) * a.d);
  uint4* vo = (uint4*)(a.v_out + (blk * a.n + i) * a.d);
  if (lane >= d8) return;
  if (p < 0 || p >= a.host_len) {
    const unsigned nan2 = 0x7e007e00u;
    ko[lane] = make_uint4(nan2, nan2, nan2, nan2);
    vo[lane] = make_uint4(nan2, nan2, nan2, nan2);
    return;
  }
  const int64_t row = (blk * a.host_len + p) * a.d;
  ko[lane] = ((const uint4*)(a.host_k + row))[lane];
  vo[lane] = ((const uint4*)(a.host_v + row))[lane];
}

}  // namespace

hipError_t launch_fetch(const FetchArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  hipLaunchKernelGGL(fetch_kernel,
                     dim3((unsigned)cdiv(a.n, kWavesPerGroup), (unsigned)a.Hkv,
                          (unsigned)a.B),
                     dim3(kWavesPerGroup * kWave), 0, s, a);
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
