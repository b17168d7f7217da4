// K/V bridge of the HySparse2 cross-decoder (gfx950): a cross-decoder full
// layer computes its K and V from a self-decoder layer's hidden state with its
// own projection (javabetter.cn "mimo-v3-hysparse2", KV Bridging paragraph;
// siami.tw "xiaomi-mimo-v3-hysparse-2", section one).
//
// y[t, c] = sum_r hidden[t, r] * w[r, c], bf16 inputs, fp32 accumulation,
// rounded to bf16 (RNE) and scattered into the cache: columns [0, Hkv*D) are
// K heads, [Hkv*D, 2*Hkv*D) are V heads.
#include "hs2_internal.hpp"

namespace hs2 {
namespace {

__device__ __forceinline__ float bf(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__global__ void __launch_bounds__(256) bridge_valu(const uint16_t* __restrict__ H, int T, int dm,
                                                   const uint16_t* __restrict__ W, int Hkv, int D,
                                                   uint16_t* kout, uint16_t* vout, int64_t sn, int64_t sh) {
  const int C = 2 * Hkv * D;
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int t = blockIdx.y;
  if (c >= C) return;
  const uint16_t* hrow = H + (int64_t)t * dm;
  float acc = 0.f;
  for (int r = 0; r < dm; ++r) acc = fmaf(bf(hrow[r]), bf(W[(int64_t)r * C + c]), acc);
  const int half = Hkv * D;
  const int cc = c < half ? c : c - half;
  const int hh = cc / D, d = cc - hh * D;
  uint16_t* dst = (c < half ? kout : vout) + (int64_t)hh * sh + (int64_t)t * sn + d;
  *dst = __builtin_bit_cast(uint16_t, (__bf16)acc);
}

}  // namespace

hipError_t launch_bridge(const uint16_t* hidden, int T, int dm, const uint16_t* w, int Hkv, int D,
                         uint16_t* k_out, uint16_t* v_out, int64_t sn, int64_t sh, hipStream_t s) {
  TimedLaunch tl("kv_bridge", s);
  const int C = 2 * Hkv * D;
  hipLaunchKernelGGL(bridge_valu, dim3((C + 255) / 256, T), dim3(256), 0, s, hidden, T, dm, w, Hkv, D, k_out,
                     v_out, sn, sh);
  return hipGetLastError();
}

}  // namespace hs2
