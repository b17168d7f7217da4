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
// (16x16x32) tiles.
#include "hs2_internal.hpp"


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

template <int RT>
struct BridgeStage {
  u32x4_t w[2];
  u32x4_t a[RT][2];
};

template <int BT, bool FP8OUT>
__global__ void __launch_bounds__(256) bridge_mfma(const uint16_t* __restrict__ H, int T, int dm,
                                                   const uint16_t* __restrict__ W, int Hkv, int D, BridgeOut O) {
  static_assert(BT == 32 || BT == 64, "token tile");
  constexpr int RT = BT / 32, CT = 2;
  using Stage = BridgeStage<RT>;
  __shared__ uint16_t Ws[kKS][kBC + kWPad];
  const int C = 2 * Hkv * D;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int wr = wave >> 1, wc = wave & 1;
  const int t0 = blockIdx.y * BT, c0 = blockIdx.x * kBC;
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
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + wr * 16 * RT + rt * 16 + 4 * g4 + i;
        const int c = c0 + wc * 16 * CT + ct * 16 + r16;
        if (t >= T) continue;
        const int cc = c < half ? c : c - half;
        const int hh = cc / D, d = cc - hh * D;
        const int64_t e = (int64_t)hh * O.sh + (int64_t)t * O.sn + d;
        if constexpr (FP8OUT) {
          const float sc = (c < half ? O.k_scale : O.v_scale)[hh];
          ((uint8_t*)(c < half ? O.k : O.v))[e] = e4m3fn_rne_sat(acc[rt][ct][i] / sc);
        } else {
          ((uint16_t*)(c < half ? O.k : O.v))[e] = __builtin_bit_cast(uint16_t, (__bf16)acc[rt][ct][i]);
        }
      }
}

}  // namespace

hipError_t launch_bridge(const uint16_t* hidden, int T, int dm, const uint16_t* w, int Hkv, int D,
                         const BridgeOut& out, hipStream_t s) {
  TimedLaunch tl("kv_bridge", s);
  const int C = 2 * Hkv * D;
  // the entry point admits D in {64, 128} and d_model % 64 == 0, so C and d_model
  // divide into whole tiles; tokens are clamped/guarded inside the kernel
  if (C % kBC != 0 || dm % kKS != 0) return hipErrorInvalidValue;
  // 64-token tiles where they still give every CU a workgroup, else 32
  const int ctiles = C / kBC;
  const bool fp8 = out.k_scale != nullptr;
#define HS2_BRIDGE(BT)                                                                                         \
  do {                                                                                                       \
    const dim3 grid(ctiles, (T + BT - 1) / BT);                                                              \
    if (fp8)                                                                                                 \
      hipLaunchKernelGGL((bridge_mfma<BT, true>), grid, dim3(256), 0, s, hidden, T, dm, w, Hkv, D, out);     \
    else                                                                                                     \
      hipLaunchKernelGGL((bridge_mfma<BT, false>), grid, dim3(256), 0, s, hidden, T, dm, w, Hkv, D, out);    \
  } while (0)
  if (ctiles * ((T + 63) / 64) >= 256)
    HS2_BRIDGE(64);
  else
    HS2_BRIDGE(32);
#undef HS2_BRIDGE
  return hipGetLastError();
}

}  // namespace hs2
