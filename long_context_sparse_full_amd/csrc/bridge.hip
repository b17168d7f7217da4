// K/V bridge of the HySparse2 cross-decoder (gfx950): a cross-decoder full
// layer computes its K and V from a self-decoder layer's hidden state with its
// own projection (javabetter.cn "mimo-v3-hysparse2", KV Bridging paragraph;
// siami.tw "xiaomi-mimo-v3-hysparse-2", section one).
//
// y[t, c] = sum_r hidden[t, r] * w[r, c], bf16 inputs, fp32 accumulation,
// scattered into the cache: columns [0, Hkv*D) are K heads, [Hkv*D, 2*Hkv*D)
// are V heads.  A bf16 cache receives y rounded to bf16 (RNE); an FP8 cache
// the OCP E4M3FN code of y / scale of its head, rounded to nearest even and
// saturated at +-448.  A dense contraction, so it runs on bf16 MFMA
// (16x16x32) tiles; the L layers of one call (each its own weights and cache,
// one hidden state) are the grid's third dimension.  With FP8 scale
// maintenance the contraction keeps y in fp32 and records each head's
// max |y|, and a second kernel grows the scales, re-encodes the older rows of
// a head whose scale grew and encodes the new rows.
#include "hs2_internal.hpp"

#include <algorithm>


namespace hs2 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

// MFMA form: a workgroup computes a BT (tokens) x 64 (columns) tile; wave w
// owns the (BT/2) x 32 quarter (w >> 1, w & 1) as RT x 2 tiles of 16 x 16
// (RT = BT / 32).  BT = 32 halves the work per workgroup so that a 512-token
// block still gives every CU a workgroup (measured: 24 us against 39 us for
// BT = 64 at 512 x 4096 x 1024; 16-token tiles re-read the weights too often).
// Stage = 64 of the d_model contraction: hidden rows go straight from global
// memory into the MFMA A layout (8 consecutive elements per lane); the w_kv
// tile [64 x 64] goes through LDS, where each lane gathers the 8 contraction
// elements of its column.  The global loads of a stage are issued kRing
// stages ahead (a register ring), so the contraction is not paced by one load
// latency per stage.
constexpr int kBC = 64, kKS = 64, kWPad = 8, kRing = 4;

// E4M3FN code of x, round to nearest even, magnitudes above 448 saturating
// to 448 (x finite): subnormal codes are multiples of 2^-9 below 2^-6, normal
// codes (exponent e + 7, 3 mantissa bits) above; a mantissa that rounds up to
// 8 carries into the exponent field.
__device__ __forceinline__ uint8_t e4m3fn_rne_sat(float x) {
  const uint32_t sign = x < 0.f ? 0x80u : 0u;
  const float a = fminf(fabsf(x), 448.f);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)rintf(a * 512.f);
  } else {
    const int e = ilogbf(a);
    code = (uint32_t)((e + 7) * 8) + (uint32_t)rintf((ldexpf(a, -e) - 1.f) * 8.f);
  }
  return (uint8_t)(sign | code);
}

// E4M3FN code -> fp32 value (exact): the code read as a bf16 number by the
// hardware conversion (every E4M3FN value is a bf16 value).
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float (&f)[4]) {
  const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  f[0] = __uint_as_float(lo << 16);
  f[1] = __uint_as_float(lo & 0xffff0000u);
  f[2] = __uint_as_float(hi << 16);
  f[3] = __uint_as_float(hi & 0xffff0000u);
}

// output modes of the contraction
enum { kOutBf16 = 0, kOutFp8 = 1, kOutF32Amax = 2 };

template <int RT>
struct BridgeStage {
  u32x4_t w[2];
  u32x4_t a[RT][2];
};

template <int BT, int MODE>
__global__ void __launch_bounds__(256) bridge_mfma(const uint16_t* __restrict__ H, int T, int dm,
                                                   const uint16_t* __restrict__ Wall, int Hkv, int D, BridgeLayers P) {
  static_assert(BT == 32 || BT == 64, "token tile");
  constexpr int RT = BT / 32, CT = 2;
  using Stage = BridgeStage<RT>;
  __shared__ uint16_t Ws[kKS][kBC + kWPad];
  const int C = 2 * Hkv * D;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int wr = wave >> 1, wc = wave & 1;
  const int t0 = blockIdx.y * BT, c0 = blockIdx.x * kBC;
  const int layer = blockIdx.z;
  const uint16_t* __restrict__ W = Wall + (int64_t)layer * dm * C;
  const BridgeOut& O = P.out[layer];
  // this thread's part of a w_kv stage: row tid/4 of the stage, 16 columns
  const int wrow = tid >> 2, wcol = (tid & 3) * 16;
  f32x4_t acc[RT][CT];
#pragma unroll
  for (int a = 0; a < RT; ++a)
#pragma unroll
    for (int b = 0; b < CT; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  int arow[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) arow[rt] = min(t0 + wr * 16 * RT + rt * 16 + r16, T - 1);

  auto load_stage = [&](int k0, Stage& S) {
    // stages past the end reload the last one (unused): the loads stay
    // unconditional, so the compiler's wait counts keep the ring in flight
    k0 = min(k0, dm - kKS);
    const uint16_t* wp = W + (int64_t)(k0 + wrow) * C + c0 + wcol;
    S.w[0] = *(const u32x4_t*)wp;
    S.w[1] = *(const u32x4_t*)(wp + 8);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) S.a[rt][ks] = *(const u32x4_t*)(H + (int64_t)arow[rt] * dm + k0 + ks * 32 + 8 * g4);
  };
  auto compute_stage = [&](const Stage& S) {
    __syncthreads();  // previous stage's LDS reads done
    *(u32x4_t*)&Ws[wrow][wcol] = S.w[0];
    *(u32x4_t*)&Ws[wrow][wcol + 8] = S.w[1];
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        // B operand (contraction index 8 g4 + 0..7 of column r16) by two
        // transposing 64-bit LDS reads: in each 16-lane group, source lane
        // 4 k4 + a4 names columns 4 a4 .. 4 a4 + 3 of contraction row
        // 8 g4 + 4 h + k4, and lane i receives column i of those four rows
        const int k4 = r16 >> 2, a4 = r16 & 3;
        u32x4_t bf;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const uint16_t* src = &Ws[ks * 32 + 8 * g4 + 4 * hh + k4][wc * 16 * CT + ct * 16 + 4 * a4];
          const s16x4_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)src);
          const u32x2_t w2 = __builtin_bit_cast(u32x2_t, t);
          bf[2 * hh] = w2.x;
          bf[2 * hh + 1] = w2.y;
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, S.a[rt][ks]),
                                                                __builtin_bit_cast(bf16x8_t, bf), acc[rt][ct], 0, 0, 0);
      }
    }
  };
  Stage R0, R1, R2, R3;
  load_stage(0, R0);
  load_stage(kKS, R1);
  load_stage(2 * kKS, R2);
  load_stage(3 * kKS, R3);
  // Stage s is computed from ring slot s % kRing, which then loads stage
  // s + kRing.  Whole groups of kRing stages run without branches (so each
  // refill stays right after its stage; the scheduling barriers keep the
  // compiler from batching the refills), the last d_model / 64 % kRing stages
  // after them.
  const int ns = dm / kKS, nfull = ns / kRing * kRing;
  int k0 = 0;
  for (; k0 < nfull * kKS; k0 += kRing * kKS) {
    compute_stage(R0);
    load_stage(k0 + kRing * kKS, R0);
    __builtin_amdgcn_sched_barrier(0);
    compute_stage(R1);
    load_stage(k0 + (kRing + 1) * kKS, R1);
    __builtin_amdgcn_sched_barrier(0);
    compute_stage(R2);
    load_stage(k0 + (kRing + 2) * kKS, R2);
    __builtin_amdgcn_sched_barrier(0);
    compute_stage(R3);
    load_stage(k0 + (kRing + 3) * kKS, R3);
    __builtin_amdgcn_sched_barrier(0);
  }
  const int rem = ns - nfull;  // 0..3 stages, in slots R0.. in order
  if (rem > 0) compute_stage(R0);
  if (rem > 1) compute_stage(R1);
  if (rem > 2) compute_stage(R2);
  // scatter: column c -> K or V cache, head c/D, element c%D; token t
  const int half = Hkv * D;
  float amax = 0.f;  // kOutF32Amax: this thread's max |y| (the tile lies in one head)
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + wr * 16 * RT + rt * 16 + 4 * g4 + i;
        const int c = c0 + wc * 16 * CT + ct * 16 + r16;
        if (t >= T) continue;
        const float yv = acc[rt][ct][i];
        if constexpr (MODE == kOutF32Amax) {
          P.y[((int64_t)layer * T + t) * C + c] = yv;
          amax = fmaxf(amax, fabsf(yv));
          continue;
        }
        const int cc = c < half ? c : c - half;
        const int hh = cc / D, d = cc - hh * D;
        const int64_t e = (int64_t)hh * O.sh + (int64_t)(P.pos0 + t) * O.sn + d;
        if constexpr (MODE == kOutFp8) {
          const float sc = (c < half ? O.k_scale : O.v_scale)[hh];
          ((uint8_t*)(c < half ? O.k : O.v))[e] = e4m3fn_rne_sat(yv / sc);
        } else {
          ((uint16_t*)(c < half ? O.k : O.v))[e] = __builtin_bit_cast(uint16_t, (__bf16)yv);
        }
      }
  if constexpr (MODE == kOutF32Amax) {
    // one (layer, K/V, head) per 64-column tile (D is 64 or 128): a workgroup
    // maximum, then one atomic (non-negative floats order as their bits)
    __shared__ float red[4];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    if (tid == 0) {
      const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
      const int part = c0 < half ? 0 : 1, hh = (c0 - part * half) / D;
      atomicMax(&P.amax[(layer * 2 + part) * Hkv + hh], __float_as_uint(m));
    }
  }
}

// Scale maintenance, set-up: each head's max |y| cleared and its scale on
// entry kept (the finishing kernel overwrites the cache's scales).
__global__ void __launch_bounds__(256) bridge_grow_prep(BridgeLayers P, int Hkv) {
  const int n = P.L * 2 * Hkv;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int l = i / (2 * Hkv), part = (i / Hkv) & 1, h = i % Hkv;
    P.amax[i] = 0u;
    P.old_scale[i] = (part ? P.out[l].v_scale : P.out[l].k_scale)[h];
  }
}

// Scale maintenance, finish: per (layer, K/V, head) s' = max(s, max|y| / 448);
// workgroup 0 stores s'.  When s' > s the head's rows [0, pos0) are
// re-encoded in place, code' = encode(fp32(decode(code) * s) / s'); the new
// rows [pos0, pos0 + T) get encode(y / s') (zero codes when s' = 0).  Every
// workgroup first stages all heads' (s, s') in LDS (one memory round trip).
// The grid's threads share each grown head's older rows 16 bytes at a time,
// and share the new rows of all heads at once (one 16-byte unit of one head
// per thread, so a one-token append encodes every head in one round trip); a
// workgroup with no new units leaves at once unless a scale grew.
constexpr int kGrowHeads = 1024;  // heads staged in LDS (the launcher checks L * 2 * Hkv)
__global__ void __launch_bounds__(256) bridge_grow_finish(BridgeLayers P, int T, int Hkv, int D) {
  __shared__ float s_old_l[kGrowHeads], s_new_l[kGrowHeads];
  __shared__ int any_grew;
  const int nh = P.L * 2 * Hkv, C = 2 * Hkv * D, u16 = D / 16;
  if (threadIdx.x == 0) any_grew = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < nh; i += 256) {
    const float so = P.old_scale[i];
    const float sn = fmaxf(so, __uint_as_float(P.amax[i]) / 448.f);
    s_old_l[i] = so;
    s_new_l[i] = sn;
    if (sn > so) any_grew = 1;
    if (blockIdx.x == 0) {
      const int l = i / (2 * Hkv), part = (i / Hkv) & 1, h = i % Hkv;
      (part ? P.out[l].v_scale : P.out[l].k_scale)[h] = sn;
    }
  }
  __syncthreads();
  const int64_t gtid = (int64_t)blockIdx.x * 256 + threadIdx.x, gstride = (int64_t)gridDim.x * 256;
  const int64_t head_units = (int64_t)T * u16, new_units = head_units * nh;
  if (!any_grew && (int64_t)blockIdx.x * 256 >= new_units) return;  // uniform
  if (any_grew) {
    for (int i = 0; i < nh; ++i) {
      const float s_old = s_old_l[i], s_new = s_new_l[i];
      if (!(s_new > s_old)) continue;  // uniform: re-encode the older rows at the new scale
      const int l = i / (2 * Hkv), part = (i / Hkv) & 1, h = i % Hkv;
      const BridgeOut& O = P.out[l];
      uint8_t* base = (uint8_t*)(part ? O.v : O.k) + (int64_t)h * O.sh;
      const int64_t units = (int64_t)P.pos0 * u16;
      for (int64_t u = gtid; u < units; u += gstride) {
        const int64_t row = u / u16;
        u32x4_t* p = (u32x4_t*)(base + row * O.sn + (u - row * u16) * 16);
        const u32x4_t w = *p;
        u32x4_t o;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float f[4];
          e4m3x4_to_f32(w[q], f);
          uint32_t word = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) word |= (uint32_t)e4m3fn_rne_sat((f[e] * s_old) / s_new) << (8 * e);
          o[q] = word;
        }
        *p = o;
      }
    }
  }
  for (int64_t u = gtid; u < new_units; u += gstride) {
    const int i = (int)(u / head_units);
    const int64_t r = u - i * head_units, t = r / u16;
    const int col = (int)(r - t * u16) * 16;
    const int l = i / (2 * Hkv), part = (i / Hkv) & 1, h = i % Hkv;
    const BridgeOut& O = P.out[l];
    const float s_new = s_new_l[i];
    const float* yp = P.y + ((int64_t)l * T + t) * C + part * Hkv * D + h * D + col;
    u32x4_t o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        word |= (uint32_t)(s_new > 0.f ? e4m3fn_rne_sat(yp[4 * q + e] / s_new) : 0u) << (8 * e);
      o[q] = word;
    }
    uint8_t* base = (uint8_t*)(part ? O.v : O.k) + (int64_t)h * O.sh;
    *(u32x4_t*)(base + (P.pos0 + t) * O.sn + col) = o;
  }
}

}  // namespace

hipError_t launch_bridge(const uint16_t* hidden, int T, int dm, const uint16_t* w, int Hkv, int D,
                         const BridgeLayers& out, hipStream_t s) {
  const int C = 2 * Hkv * D;
  // the entry point admits D in {64, 128} and d_model % 64 == 0, so C and d_model
  // divide into whole tiles; tokens are clamped/guarded inside the kernel
  if (C % kBC != 0 || dm % kKS != 0 || out.L < 1 || out.L > kMaxBridgeLayers) return hipErrorInvalidValue;
  if (out.y != nullptr && out.L * 2 * Hkv > kGrowHeads) return hipErrorInvalidValue;
  const int ctiles = C / kBC;
  const bool fp8 = out.out[0].k_scale != nullptr;
  const bool grow = fp8 && out.y != nullptr;
  hipError_t e;
  if (grow) {
    TimedLaunch tl("kv_bridge", s);
    hipLaunchKernelGGL(bridge_grow_prep, dim3(1), dim3(256), 0, s, out, Hkv);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  {
    TimedLaunch tl("kv_bridge", s);
    const int mode = grow ? kOutF32Amax : (fp8 ? kOutFp8 : kOutBf16);
    // 64-token tiles where they still give every CU a workgroup, else 32
#define HS2_BRIDGE(BT)                                                                                            \
  do {                                                                                                          \
    const dim3 grid(ctiles, (T + BT - 1) / BT, out.L);                                                          \
    if (mode == kOutF32Amax)                                                                                    \
      hipLaunchKernelGGL((bridge_mfma<BT, kOutF32Amax>), grid, dim3(256), 0, s, hidden, T, dm, w, Hkv, D, out); \
    else if (mode == kOutFp8)                                                                                   \
      hipLaunchKernelGGL((bridge_mfma<BT, kOutFp8>), grid, dim3(256), 0, s, hidden, T, dm, w, Hkv, D, out);     \
    else                                                                                                        \
      hipLaunchKernelGGL((bridge_mfma<BT, kOutBf16>), grid, dim3(256), 0, s, hidden, T, dm, w, Hkv, D, out);    \
  } while (0)
    if (ctiles * ((T + 63) / 64) * out.L >= 256)
      HS2_BRIDGE(64);
    else
      HS2_BRIDGE(32);
#undef HS2_BRIDGE
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (grow) {
    TimedLaunch tl("kv_bridge", s);
    // enough threads for the largest head region or all heads' new rows, 16
    // bytes each, at most 2048 workgroups
    const int64_t units = std::max<int64_t>((int64_t)out.pos0, (int64_t)T * out.L * 2 * Hkv) * (D / 16);
    const int blocks = (int)std::min<int64_t>(2048, std::max<int64_t>(1, (units + 255) / 256));
    hipLaunchKernelGGL(bridge_grow_finish, dim3(blocks), dim3(256), 0, s, out, T, Hkv, D);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace hs2
