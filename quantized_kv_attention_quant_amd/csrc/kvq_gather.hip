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

__device__ inline float dequant(unsigned hi, unsigned lo, bool two, bool draft,
                                float s, float z) {
  float code;
  if (draft) code = 16.f * (float)hi + 7.5f;
  else code = (float)(two ? (hi << 4) | lo : hi);
  return __fadd_rn(z, __fmul_rn(code, s));
}

__global__ void __launch_bounds__(kWavesPerGroup * kWave)
    gather_kernel(const GatherArgs a) {
  const CacheGeom& g = a.g;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int64_t blk = (int64_t)b * g.Hkv + kvh;
  const int i = blockIdx.x * kWavesPerGroup + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (i >= a.n) return;
  const int d = g.d, w = g.w;
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

  const bool two = g.bits == 8, draft = a.path == KVQ_DRAFT4;
  const unsigned mask = (1u << w) - 1u;
  // keys: plane row of token p; scale/zero of its group
  const uint8_t* krow_hi = a.p.k_hi + blk * g.k_block_bytes + p * g.k_row_bytes;
  const uint8_t* krow_lo = two ? a.p.k_lo + blk * g.k_block_bytes + p * g.k_row_bytes : nullptr;
  const __half2* ksz = a.p.k_sz + blk * g.ksz_block + (p / g.G) * d;
  // values: tile of token p and the token's place in it
  const int64_t t = p / kTile;
  const int j = (int)(p % kTile);
  const int jg = (j % 16) / 4, ji = j % 4, jh = j / 16;
  const uint32_t* vt_hi =
      (const uint32_t*)(a.p.v_hi + blk * g.v_block_bytes + t * g.v_tile_bytes);
  const uint32_t* vt_lo =
      two ? (const uint32_t*)(a.p.v_lo + blk * g.v_block_bytes + t * g.v_tile_bytes)
          : nullptr;
  const int ngv = d / g.Gv;
  const __half* vsz = (const __half*)(a.p.v_sz + blk * g.vsz_block + t * g.vsz_tile);
  const int per_byte = 8 / w, per = 4 / w;

  for (int c = lane; c < d; c += kWave) {
    // key code: byte c / (8/w) of the row, bits w * (c % (8/w))
    const int kb = c / per_byte, ksh = w * (c % per_byte);
    const unsigned khi = ((unsigned)krow_hi[kb] >> ksh) & mask;
    const unsigned klo = two ? ((unsigned)krow_lo[kb] >> ksh) & mask : 0u;
    const __half2 sz = ksz[c];
    const float kx = dequant(khi, klo, two, draft, __low2float(sz), __high2float(sz));
    ko[c] = __float2half_rn(kx);
    // value code: dword (16 g + r) * (d w / 64) + m / per, bit 16 h + w (4 (m % per) + i)
    const int r = c % 16, m = c / 16;
    const int dw = (16 * jg + r) * (d * w / 64) + m / per;
    const int vsh = 16 * jh + w * (4 * (m % per) + ji);
    const unsigned vhi = (vt_hi[dw] >> vsh) & mask;
    const unsigned vlo = two ? (vt_lo[dw] >> vsh) & mask : 0u;
    // scale / zero: [part][g][i][group][h] halves within the tile
    const int gg = c / g.Gv;
    const int so = ((0 * 4 + jg) * 4 + ji) * ngv * 2 + gg * 2 + jh;
    const int zo = ((1 * 4 + jg) * 4 + ji) * ngv * 2 + gg * 2 + jh;
    const float vx = dequant(vhi, vlo, two, draft, __half2float(vsz[so]),
                             __half2float(vsz[zo]));
    vo[c] = __float2half_rn(vx);
  }
}

}  // namespace

hipError_t launch_gather(const GatherArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_kernel,
                     dim3((unsigned)cdiv(a.n, kWavesPerGroup), (unsigned)a.g.Hkv,
                          (unsigned)a.g.B),
                     dim3(kWavesPerGroup * kWave), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
