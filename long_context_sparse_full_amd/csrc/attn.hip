// Attention kernels of the HySparse2 cross-decoder hot path (gfx950).
//
//  * scan_mfma   -- full layer (split over positions, writes per-head log2
//                   logits for the score pass) and sparse layer (gathered rows,
//                   one workgroup per (b, t, g), final output) for bf16 queries
//                   over bf16 or E4M3FN caches.  QK^T and PV run on
//                   v_mfma_f32_16x16x32_bf16 with positions on the MFMA M side
//                   and up to 16 query rows (the heads of one GQA group) on N.
//  * scan_f32    -- the same two roles for fp32 caches on the VALU (fp32 products
//                   and sums; its scores come from the same 16-bit logit codes).
//  * combine     -- merges the per-split (max, sum, output) partials.
//  * score       -- importance scores: per position, sum over the group's query
//                   heads of the softmax probability, from the stored logits.
//
// The full layer scans every cached position and its attention probabilities
// pick the tokens (javabetter.cn "mimo-v3-hysparse2", first of the two
// changes); the sparse layers attend only to the selected rows of the same
// cache (aitop.news item 35442; javabetter.cn, KV Reuse paragraph).
#include <math.h>

#include <algorithm>

#include <type_traits>

#include "hs2_internal.hpp"
#include "select_common.hpp"

namespace hs2 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
// lazy reference maximum of the online softmax in the multi-query chunk kernel
constexpr float kLazyMax = 8.f;
constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2_t v;
  v.x = (__bf16)a;
  v.y = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// four E4M3FN codes (bytes 0..3 of w) -> two dwords of bf16 pairs (exact)
// (one v_cvt_scalef32_pk_bf16_fp8 per pair, scale 1.0: every E4M3FN value is a bf16 value)
__device__ __forceinline__ void e4m3x4_to_bf16(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}

__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Lane pairs (l, l ^ 16) and (l, l ^ 32) through the gfx950 permlane swaps:
// VALU lane exchanges with no LDS round trip.  Each swap hands every lane the
// two values of its pair (in some order); max and sum are symmetric in them.
__device__ __forceinline__ float fmax2(float a, float b) { return a > b ? a : b; }
__device__ __forceinline__ float max_x16(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmax2(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_x32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmax2(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float sum_x16(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float sum_x32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// 16-bit code of a log2-domain logit x below its tile maximum m:
// round((m - x) * 2^12), saturated; 65535 stands for "at least 16 below m".
// Step 2^-12 bounds the relative error of 2^x by 2^-13 * ln 2 < 8.5e-5.  The
// score pass takes the term of a saturated code as zero only when it is
// provably negligible (the probability of the tile maximum below
// 2^kExactFloor, so the term is below 2^(kExactFloor - 16)); otherwise it
// recomputes that logit in fp32 from the query and the cache row.
constexpr float kCodeScale = 4096.f;
constexpr float kCodeInv = 1.f / 4096.f;
constexpr float kExactFloor = -24.f;
__device__ __forceinline__ uint32_t logit_code(float m, float x) {
  const float d = (m - x) * kCodeScale;  // >= 0; +inf when x = -inf
  return d < 65534.5f ? (uint32_t)__builtin_rintf(d) : 65535u;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Head-dim slice held by lane group g4 (= lane / 16) for QK MFMA number c:
// 8 consecutive elements starting here.  K and Q use the same map, so the dot
// product is unchanged; the map only decides which bytes one load fetches.
template <bool FP8, int D>
__device__ __forceinline__ int dmap(int c, int g4) {
  if constexpr (!FP8) {
    return 32 * c + 8 * g4;  // bf16: 16 B per MFMA, 4 lanes cover 64 B of a row
  } else if constexpr (D == 128) {
    return 64 * (c >> 1) + 16 * g4 + 8 * (c & 1);  // fp8: one 16 B load feeds two MFMAs
  } else {
    return 16 * g4 + 8 * c;
  }
}

// ---------------------------------------------------------------------------
// MFMA scan (bf16 query; bf16 or E4M3FN cache)
// ---------------------------------------------------------------------------
// Raw (undecoded) K/V bytes of one 32-position tile, as this lane loads them:
// K rows j0+16*hh+(lane%16) in the MFMA A layout, 16 bytes per load starting at
// byte 16*g4 (then +64 per further load); V rows j0+16*(kk>>2)+4*g4+(kk&3),
// VE elements from element VE*(lane%16).
template <bool FP8, int D>
struct RawTile {
  static constexpr int NC = D / 32;
  static constexpr int VE = D / 16;
  static constexpr int KW = FP8 ? NC / 2 : NC;      // 16-byte K loads per 16-position half
  static constexpr int VW = FP8 ? VE / 4 : VE / 2;  // dwords of one V row slice
  u32x4_t k[2][KW];
  uint32_t v[8][VW];
};

// One V row slice (T: 16, 8 or 4 bytes) into dwords.
template <typename T>
__device__ __forceinline__ void ldv(uint32_t* dst, const char* p) {
  if constexpr (sizeof(T) == 16) {
    const u32x4_t w = *(const u32x4_t*)p;
    dst[0] = w.x; dst[1] = w.y; dst[2] = w.z; dst[3] = w.w;
  } else if constexpr (sizeof(T) == 8) {
    const u32x2_t w = *(const u32x2_t*)p;
    dst[0] = w.x; dst[1] = w.y;
  } else {
    dst[0] = *(const uint32_t*)p;
  }
}

// Loads of one tile from per-lane row addresses: kptr[hh] / vptr[kk] point at
// this lane's first byte of the row.
template <bool FP8, int D>
__device__ __forceinline__ void load_tile(RawTile<FP8, D>& R, const char* const kptr[2], const char* const vptr[8]) {
  using RT = RawTile<FP8, D>;
  constexpr int VB = RT::VW * 4;  // bytes per V row slice
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int c = 0; c < RT::KW; ++c) R.k[hh][c] = *(const u32x4_t*)(kptr[hh] + 64 * c);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    if constexpr (VB == 16) ldv<u32x4_t>(R.v[kk], vptr[kk]);
    else if constexpr (VB == 8) ldv<u32x2_t>(R.v[kk], vptr[kk]);
    else ldv<uint32_t>(R.v[kk], vptr[kk]);
  }
}

// Online-softmax state of one wave: row r = lane % 16; the 4 lanes of a row
// (lane groups g4) agree on m and hold partial sums l and output slices.
template <int D>
struct WaveState {
  float m, l;
  f32x4_t o[D / 16];
};

// One 32-position tile: decode, QK^T, mask (only when the tile crosses the
// causal / range limit), logits, online softmax, PV.  Positions of this lane's
// logits: j0 + 16*hh + 4*g4 + ii.
template <bool FP8, int D, bool WRITE_LOGITS>
__device__ __forceinline__ void compute_tile(const RawTile<FP8, D>& R, const u32x4_t (&qf)[D / 32], float cs, int j0,
                                             int jlim, bool need_mask, int g4, uint16_t* lg, float* lgm,
                                             int lgm_stride, WaveState<D>& S) {
  constexpr int NC = D / 32, VE = D / 16;
  u32x4_t kf[2][NC];
  uint32_t vd[8][VE / 2];
  if constexpr (!FP8) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int c = 0; c < NC; ++c) kf[hh][c] = R.k[hh][c];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int w = 0; w < VE / 2; ++w) vd[kk][w] = R.v[kk][w];
  } else {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int ii = 0; ii < NC / 2; ++ii) {
        const u32x4_t raw = R.k[hh][ii];
        uint32_t a0, a1, a2, a3, b0, b1, b2, b3;
        e4m3x4_to_bf16(raw.x, a0, a1);
        e4m3x4_to_bf16(raw.y, a2, a3);
        e4m3x4_to_bf16(raw.z, b0, b1);
        e4m3x4_to_bf16(raw.w, b2, b3);
        kf[hh][2 * ii] = u32x4_t{a0, a1, a2, a3};
        kf[hh][2 * ii + 1] = u32x4_t{b0, b1, b2, b3};
      }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      e4m3x4_to_bf16(R.v[kk][0], vd[kk][0], vd[kk][1]);
      if constexpr (VE == 8) e4m3x4_to_bf16(R.v[kk][1], vd[kk][2], vd[kk][3]);
    }
  }

  // logits S^T[position][row]
  f32x4_t s[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    s[hh] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) s[hh] = mfma_bf16(kf[hh][c], qf[c], s[hh]);
  }
  float x[2][4];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) x[hh][ii] = s[hh][ii] * cs;
  if (need_mask) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        if (j0 + 16 * hh + 4 * g4 + ii > jlim) x[hh][ii] = kNegInf;
  }
  float tmax = kNegInf;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) tmax = fmaxf(tmax, x[hh][ii]);
  tmax = max_x16(tmax);
  tmax = max_x32(tmax);
  if constexpr (WRITE_LOGITS) {
    if (lg) {  // lg -> this row's code at position j0 + 4*g4; lgm -> this row's tile maxima
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint32_t c0 = logit_code(tmax, x[hh][0]), c1 = logit_code(tmax, x[hh][1]);
        const uint32_t c2 = logit_code(tmax, x[hh][2]), c3 = logit_code(tmax, x[hh][3]);
        *(u32x2_t*)(lg + 16 * hh) = u32x2_t{c0 | (c1 << 16), c2 | (c3 << 16)};
      }
      if (g4 == 0) lgm[(j0 >> 5) * lgm_stride] = tmax;
    }
  }
  // online softmax in the log2 domain
  const float m_new = fmaxf(S.m, tmax);
  const float alpha = (m_new == S.m) ? 1.f : exp2_fast(S.m - m_new);
  const float m_use = (m_new == kNegInf) ? 0.f : m_new;
  float pr[2][4];
  float psum = 0.f;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      pr[hh][ii] = exp2_fast(x[hh][ii] - m_use);
      psum += pr[hh][ii];
    }
  S.l = S.l * alpha + psum;
  if (__any(alpha != 1.f)) {
#pragma unroll
    for (int dt = 0; dt < VE; ++dt) S.o[dt] *= alpha;
  }
  S.m = m_new;

  // PV: O^T[d][row] += V^T[d][pos] P^T[pos][row]; k-slot kk of lane group g4
  // is position 16*(kk>>2) + 4*g4 + (kk&3), for P and V alike
  const u32x4_t pf = u32x4_t{pack_bf16(pr[0][0], pr[0][1]), pack_bf16(pr[0][2], pr[0][3]),
                             pack_bf16(pr[1][0], pr[1][1]), pack_bf16(pr[1][2], pr[1][3])};
#pragma unroll
  for (int dt = 0; dt < VE; ++dt) {
    const int w = dt >> 1;
    u32x4_t va;
#pragma unroll
    for (int q2 = 0; q2 < 4; ++q2) {
      const uint32_t e0 = vd[2 * q2][w], e1 = vd[2 * q2 + 1][w];
      va[q2] = (dt & 1) ? __builtin_amdgcn_perm(e1, e0, 0x07060302u) : __builtin_amdgcn_perm(e1, e0, 0x05040100u);
    }
    S.o[dt] = mfma_bf16(va, pf, S.o[dt]);
  }
}

// Device-coherent scalar accesses for the per-workgroup partials that another
// workgroup of the same launch merges (they bypass the non-coherent per-XCD
// caches).
__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge the waves of a workgroup through LDS and emit, per row, either the
// split partial (max, sum, output) or the final normalised output and LSE.
template <bool FP8, int D, bool GATHER, int WAVES, bool COHERENT = false>
__device__ __forceinline__ void merge_and_store(const ScanParams& P, WaveState<D>& S, int unit, int split, int b, int g,
                                                int wave, int r, int g4, float (*sm_m)[16], float (*sm_l)[16],
                                                float (*sm_o)[16][D + 1]) {
  constexpr int VE = D / 16;
  float l_run = S.l;
  l_run = sum_x16(l_run);
  l_run = sum_x32(l_run);
  __syncthreads();
  if (g4 == 0) {
    sm_m[wave][r] = S.m;
    sm_l[wave][r] = l_run;
  }
#pragma unroll
  for (int dt = 0; dt < VE; ++dt)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) sm_o[wave][r][VE * (4 * g4 + ii) + dt] = S.o[dt][ii];
  __syncthreads();
  for (int e = threadIdx.x; e < P.rows * D; e += WAVES * 64) {
    const int rr = e / D, d = e - rr * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, sm_m[w][rr]);
    const float Ms = (M == kNegInf) ? 0.f : M;
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const float f = exp2_fast(sm_m[w][rr] - Ms);
      L += sm_l[w][rr] * f;
      O += sm_o[w][rr][d] * f;
    }
    if constexpr (GATHER) {
      const int tt = (unit / P.Hkv) % P.Tq;  // unit = (b, t, g); rows = heads of token t
      const int hh = g * P.G + rr;
      float o = (L > 0.f) ? O / L : 0.f;
      if constexpr (FP8) o *= P.v_scale[b * P.Hkv + g];
      const int64_t orow = ((int64_t)b * P.Tq + tt) * P.Hq + hh;
      ((__bf16*)P.out)[orow * D + d] = (__bf16)o;
      if (d == 0 && P.lse) P.lse[orow] = (L > 0.f) ? (M + log2f(L)) * kLn2 : kNegInf;
    } else {
      const int64_t pbase = ((int64_t)unit * P.nsplit + split) * 16 + rr;
      if constexpr (COHERENT) {  // read by another workgroup of the same launch
        st_coherent(P.part_o + pbase * D + d, O);
        if (d == 0) {
          st_coherent(P.part_ml + pbase * 2, M);
          st_coherent(P.part_ml + pbase * 2 + 1, L);
        }
      } else {
        P.part_o[pbase * D + d] = O;
        if (d == 0) {
          P.part_ml[pbase * 2] = M;
          P.part_ml[pbase * 2 + 1] = L;
        }
      }
    }
  }
}

// wait until at most N vector-memory operations of this wave are in flight
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Query fragments (MFMA B operand of QK^T): row r, head-dim slice dmap(c, g4).
template <bool FP8, int D, bool WAIT = true>
__device__ __forceinline__ void load_q(u32x4_t (&qf)[D / 32], const ScanParams& P, int b, int t, int h, bool row_ok,
                                       int g4) {
  const uint16_t* qb = (const uint16_t*)P.q + (((int64_t)b * P.Tq + (row_ok ? t : 0)) * P.Hq + (row_ok ? h : 0)) * D;
#pragma unroll
  for (int c = 0; c < D / 32; ++c) qf[c] = row_ok ? *(const u32x4_t*)(qb + dmap<FP8, D>(c, g4)) : u32x4_t{0u, 0u, 0u, 0u};
  // The fragments arrive before any tile load is issued: left in flight, the
  // compiler's wait bookkeeping would count them as pending inside the tile
  // loops and drain the prefetched tile (a full vmcnt(0)) on every iteration.
  // (WAIT = false: the caller waits once for everything in flight.)
  if constexpr (WAIT) wait_vm<0>();
}

// Full layer: one workgroup per (position split, unit); waves take interleaved
// 32-position tiles and prefetch the next tile while computing this one.
// Tile bases are wave-uniform (scalar registers); each lane adds a fixed
// 32-bit offset, so interior tiles need no per-lane address arithmetic.
// PAGED: the cache is a paged pool (P.pages); a 32-aligned tile lies in one
// page, so a full tile's base is its first row's physical row.
template <bool FP8, int D, bool WRITE_LOGITS, int WAVES, bool PAGED = false>
__global__ void __launch_bounds__(WAVES * 64) scan_full(ScanParams P) {
  constexpr int VE = D / 16, NC = D / 32, EB = FP8 ? 1 : 2;
  constexpr int STEP = WAVES * 32;
  __shared__ float sm_m[WAVES][16];
  __shared__ float sm_l[WAVES][16];
  __shared__ float sm_o[WAVES][16][D + 1];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g4 = lane >> 4;
  const int unit = blockIdx.y, split = blockIdx.x;
  const int g = unit % P.Hkv;
  const int tp = (unit / P.Hkv) % P.n_tpacks;
  const int b = unit / (P.Hkv * P.n_tpacks);
  const int tl = r / P.G;
  const int t = tp * P.tpack + tl;
  const bool row_ok = (r < P.rows) && (t < P.Tq);
  const int h = g * P.G + (r - tl * P.G);

  const int q0 = qpos_of(P.qpos_b, P.q_pos0, b, P.N, P.Tq);
  const int p_max = q0 + min(tp * P.tpack + P.tpack, P.Tq) - 1;
  // workgroup tile w = STEP positions; this split owns tiles split, split+nsplit, ...
  // (all splits sweep the cache together)
  const int j_begin = split * STEP;
  const int j_end = p_max + 1;
  const int jstride = P.nsplit * STEP;
  const int jlim = min(row_ok ? q0 + t : -1, j_end - 1);
  // tiles ending at or before j_nomask need no masking for any valid row
  const int j_nomask = min(q0 + tp * P.tpack, j_end - 1);

  // PAGED: lane i holds the page of this wave's tile i (i < 64), loaded
  // with the query fragments; a tile reads its page back with one readlane
  int pg_lane = 0;
  if constexpr (PAGED) {
    const int jt = j_begin + wave * 32 + lane * jstride;
    if (jt <= p_max)
      pg_lane = min(max(P.pages.table[(int64_t)b * P.pages.per_seq + (jt >> P.pages.shift)], 0), P.pages.pool - 1);
  }
  u32x4_t qf[NC];
  load_q<FP8, D>(qf, P, b, t, h, row_ok, g4);
  const int64_t kvoff = ((int64_t)b * P.sb + (int64_t)g * P.sh) * EB;
  const char* kb = (const char*)P.k + kvoff;
  const char* vb = (const char*)P.v + kvoff;
  const int64_t snb = P.sn * EB;
  float cs = P.scale_log2;
  if constexpr (FP8) cs *= P.k_scale[b * P.Hkv + g];
  uint16_t* lg_row = nullptr;
  float* lgm_row = nullptr;
  if constexpr (WRITE_LOGITS) {
    if (row_ok) {
      lg_row = P.lg16 + ((int64_t)unit * P.rows + r) * P.npad + 4 * g4;
      lgm_row = P.lgmax + (int64_t)unit * (P.npad >> 5) * P.rows + r;  // [unit][tile][row]
    }
  }

  // per-lane offsets (bytes) of this lane's K and V rows relative to the tile base
  uint32_t koff[2], voff[8];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) koff[hh] = (uint32_t)((16 * hh + r) * snb) + 16u * g4;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    voff[kk] = (uint32_t)((16 * (kk >> 2) + 4 * g4 + (kk & 3)) * snb) + (uint32_t)(VE * r * EB);

  WaveState<D> S;
  S.m = kNegInf;
  S.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < VE; ++dt) S.o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // first cache row of this wave's tile ti (at position j0)
  auto tile_row0 = [&](int j0, int ti) -> int64_t {
    if constexpr (PAGED) {
      const int pg = ti < 64 ? __builtin_amdgcn_readlane(pg_lane, ti) : (phys_row(P.pages, b, j0) >> P.pages.shift);
      return ((int64_t)pg << P.pages.shift) | (j0 & ((1 << P.pages.shift) - 1));
    } else {
      return j0;
    }
  };
  // full tile (j0 + 31 <= p_max): scalar tile base plus the fixed lane offsets
  auto load_full = [&](RawTile<FP8, D>& R, int j0, int ti) {
    const char* kp[2];
    const char* vp[8];
    const int64_t row0 = tile_row0(j0, ti);
    const char* tk = kb + row0 * snb;
    const char* tv = vb + row0 * snb;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) kp[hh] = tk + koff[hh];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) vp[kk] = tv + voff[kk];
    load_tile<FP8, D>(R, kp, vp);
  };
  auto load = [&](RawTile<FP8, D>& R, int j0, int ti) {
    if (j0 + 31 <= p_max) {
      load_full(R, j0, ti);
    } else {  // tail tile: rows past the last position repeat it
      const char* kp[2];
      const char* vp[8];
      auto row = [&](int j) -> int64_t { return PAGED ? phys_row(P.pages, b, j) : j; };
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) kp[hh] = kb + row(min(j0 + 16 * hh + r, p_max)) * snb + 16 * g4;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        vp[kk] = vb + row(min(j0 + 16 * (kk >> 2) + 4 * g4 + (kk & 3), p_max)) * snb + VE * r * EB;
      load_tile<FP8, D>(R, kp, vp);
    }
  };
  auto compute = [&](const RawTile<FP8, D>& R, int j0) {
    compute_tile<FP8, D, WRITE_LOGITS>(R, qf, cs, j0, jlim, j0 + 31 > j_nomask, g4,
                                       WRITE_LOGITS && lg_row ? lg_row + j0 : nullptr, lgm_row, P.rows, S);
  };

  // This wave's tiles: j_first + i * jstride for i < n; only the last one can
  // run past p_max.  The steady-state loop issues its two prefetches without
  // conditions, so the wait before each compute covers exactly the older tile
  // (a conditional load makes the compiler's in-order wait counts drain the
  // prefetch as well); at most three tiles are left to the epilogue.
  const int j_first = j_begin + wave * 32;
  const int n = j_first < j_end ? (j_end - 1 - j_first) / jstride + 1 : 0;
  const int n_full = j_first + 31 <= p_max ? min(n, (p_max - 31 - j_first) / jstride + 1) : 0;
  RawTile<FP8, D> A, B;
  int i = 0;
  if (n > 0) load(A, j_first, 0);
  for (; i + 2 < n_full; i += 2) {
    const int j0 = j_first + i * jstride;
    load_full(B, j0 + jstride, i + 1);
    compute(A, j0);
    load_full(A, j0 + 2 * jstride, i + 2);
    compute(B, j0 + jstride);
  }
  // tail: A holds tile i; at most three tiles remain
  if (i < n) {
    const int j0 = j_first + i * jstride;
    if (i + 1 < n) load(B, j0 + jstride, i + 1);
    compute(A, j0);
    if (i + 1 < n) {
      if (i + 2 < n) load(A, j0 + 2 * jstride, i + 2);
      compute(B, j0 + jstride);
      if (i + 2 < n) compute(A, j0 + 2 * jstride);
    }
  }
  if (P.sel_state && split == 0)  // tpack = 1: unit = selection row (b, t, g), query position q0 + tp
    sel_init_row(P.sel_state + (int64_t)unit * ST_WORDS, P.sel_hist + (int64_t)unit * 3 * kHistBins, q0 + tp,
                 P.sel_k, P.sel_window, 1, threadIdx.x, WAVES * 64);
  merge_and_store<FP8, D, false, WAVES>(P, S, unit, split, b, g, wave, r, g4, sm_m, sm_l, sm_o);
}

// ---------------------------------------------------------------------------
// Multi-query chunk (many query tokens per kv head).  A workgroup of 4 waves
// covers 4 x kFlashRG groups of 16 query rows (tpack tokens x G heads each) of
// one (b, kv head) over a position split.  Every 32-position K/V tile is
// fetched once by the whole workgroup straight from global memory into an LDS
// ring (3 buffers in the full pass, 4 in the score pass; one barrier per
// tile); each wave reads its MFMA fragments from LDS for its own row groups:
// S^T = K Q^T and O^T += V^T P^T as in the decode scan.  Pass 1 writes the split partials of each 16-row group in the
// decode layout (unit = (b, pack, g)), merged by the combine kernel; pass 2
// recomputes the logits and writes the scores against the merged
// log-sum-exp, so no per-head scratch is stored.  Linear work index: split
// fastest, then kv head, so the workgroups that read the same K/V range
// (same head and split, all token blocks) share an XCD.
// ---------------------------------------------------------------------------
template <int D, int RG>
struct ChunkState {
  float m[RG], l[RG];
  f32x4_t o[RG][D / 16];
  float mu[RG], thr[RG];  // exponent offset (m, or 0 before a reference) and move threshold
};

struct ChunkItem {
  int b, blk, g, split;
};
__device__ __forceinline__ ChunkItem chunk_item(const ScanParams& P, int nblk) {
  ChunkItem c;
  int L = blockIdx.x;
  c.split = L % P.nsplit;
  L /= P.nsplit;
  c.g = L % P.Hkv;
  L /= P.Hkv;
  c.blk = L % nblk;
  c.b = L / nblk;
  return c;
}

// Per-lane row data of a chunk work item: the query token of row r in group rg
// and its causal limit (-1 for rows past Tq).
struct ChunkRows {
  int t, jlim;
  bool ok;
};
template <int RG>
__device__ __forceinline__ ChunkRows chunk_row(const ScanParams& P, int q0, int blk, int rg, int r) {
  ChunkRows c;
  const int tl = r / P.G;
  const int tp = blk * RG + rg;
  c.t = tp * P.tpack + tl;
  c.ok = (r < P.rows) && (c.t < P.Tq);
  c.jlim = c.ok ? q0 + c.t : -1;
  return c;
}

template <bool FP8, int D>
struct FlashGeom {
  static constexpr int EB = FP8 ? 1 : 2;
  static constexpr int ROWB = D * EB;          // bytes per cached row
  static constexpr int CH = ROWB / 16;         // 16-byte chunks per row
  static constexpr int HALF = 32 * ROWB;       // K (or V) part of a tile
  static constexpr int TILE = 2 * HALF;        // one LDS tile buffer
};

// LDS swizzle of a tile row: 16-byte chunk c of row `row` sits at chunk
// c ^ flash_swz(row).  Chosen by measured bank conflicts (SQ_LDS_BANK_CONFLICT):
// the 16-byte K fragment reads (16 consecutive rows, one chunk each) are
// conflict-free with row & (CH - 1); the transposing 8-byte V reads (4
// consecutive rows x 2 adjacent chunks per 16 lanes) are with
// 2 (row & 7) + bit 3 of the row on 256-byte rows.
template <int CH, bool VPART>
__device__ __forceinline__ int flash_swz(int row) {
  if constexpr (VPART && CH == 16) return 2 * (row & 7) + ((row >> 3) & 1);
  return row & (CH - 1);
}
template <bool FP8, int D, bool VPART = false>
__device__ __forceinline__ const char* flash_at(const char* base, int row, int byte) {
  using FG = FlashGeom<FP8, D>;
  return base + row * FG::ROWB + (((byte >> 4) ^ flash_swz<FG::CH, VPART>(row)) << 4) + (byte & 15);
}

// One 16-byte global -> LDS load per lane: lane l's 16 bytes at sbase + voff
// land at LDS byte address lds + 16 l (M0 holds lds).  Written as inline asm
// so the compiler does not treat it as an LDS store of unknown extent and
// stall every later LDS read until the newest tile has landed: the ring below
// orders these loads and the reads with explicit waits and barriers.
__device__ __forceinline__ void lds_dma16(const char* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// Tile loads straight from global memory into LDS (16 bytes per lane) for a
// 256-thread workgroup: load i of thread tid fills LDS slot s = 256 i + tid
// of the tile (PARTS = 1: K rows; 2: K rows then V rows, 32 rows x CH chunks
// each), a wave-contiguous 1 KiB per instruction.  Slot (row, c) holds chunk
// c ^ flash_swz(row) of the row (per part), the swizzle flash_at() undoes;
// rows past p_max are clamped to it.  Waves whose slots lie past the tile
// issue nothing.  Row offsets are 32-bit (32 rows x the row stride < 2 GiB,
// checked by the launcher).
template <bool FP8, int D, int PARTS>
struct TileLoader {
  using FG = FlashGeom<FP8, D>;
  static constexpr int SLOTS = PARTS * 32 * FG::CH;
  static constexpr int PER = (SLOTS + 255) / 256;  // loads per thread per tile
  static constexpr int BYTES = PARTS * FG::HALF;   // one LDS tile buffer
  int prow[PER];
  uint32_t coff[PER];  // byte offset of the chunk within its row
  const char* kb;
  const char* vb;
  int64_t snb;
  int wave;
  __device__ __forceinline__ TileLoader(const char* kb_, const char* vb_, int64_t snb_, int tid, int wave_)
      : kb(kb_), vb(vb_), snb(snb_), wave(wave_) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int s = min(256 * i + tid, SLOTS - 1);
      const int which = s / (32 * FG::CH), rem = s - which * 32 * FG::CH;
      const int row = rem / FG::CH, pos = rem - row * FG::CH;
      prow[i] = row;
      coff[i] = 16u * (uint32_t)(pos ^ (which ? flash_swz<FG::CH, true>(row) : flash_swz<FG::CH, false>(row)));
    }
  }
  __device__ __forceinline__ void issue(const char* dst, int j0, int p_max) const {
    const int lim = p_max - j0;  // rows past it repeat row p_max
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int s0 = 256 * i + 64 * wave;  // wave-uniform
      if (s0 >= SLOTS) continue;
      const bool vpart = s0 >= 32 * FG::CH;
      const char* base = (vpart ? vb : kb) + (int64_t)j0 * snb;
      const uint32_t voff = (uint32_t)(min(prow[i], lim) * (int)snb) + coff[i];
      lds_dma16(base, voff, lds_addr(dst + 16 * s0));
    }
  }
};

// Ring pipeline step n over LDS tile buffers (tile n in buffer n % NBUF):
// wait for this wave's loads of tile n (later tiles, up to NBUF - 2 of them,
// may stay in flight), then a workgroup barrier: tile n is visible to every
// wave and the buffer of tile n - 1 is free for tile n + NBUF - 1.
template <int NBUF, int PER>
__device__ __forceinline__ void ring_wait(int n, int ntile) {
  static_assert(NBUF == 3 || NBUF == 4, "ring of 3 or 4 buffers");
  const int ahead = min(NBUF - 2, ntile - 1 - n);  // tiles issued after tile n
  if (NBUF == 4 && ahead >= 2) wait_vm<2 * PER>();
  else if (ahead >= 1) wait_vm<PER>();
  else wait_vm<0>();
  __syncthreads();
}

// QK^T of one tile from LDS: s[rg][hh] = the S^T block of positions
// 16 hh + (0..15) and row group rg.
template <bool FP8, int D, int RG>
__device__ __forceinline__ void flash_qk(const char* kl, const u32x4_t (&qf)[RG][D / 32], int r, int g4,
                                         f32x4_t (&s)[RG][2]) {
  constexpr int NC = D / 32;
  using RT = RawTile<FP8, D>;
  // K fragments (A of S^T): row 16*hh + r, bytes 64*c + 16*g4 of the row
  u32x4_t kf[2][NC];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int row = 16 * hh + r;
    if constexpr (!FP8) {
#pragma unroll
      for (int c = 0; c < NC; ++c) kf[hh][c] = *(const u32x4_t*)flash_at<FP8, D>(kl, row, 64 * c + 16 * g4);
    } else {
#pragma unroll
      for (int ii = 0; ii < RT::KW; ++ii) {
        const u32x4_t raw = *(const u32x4_t*)flash_at<FP8, D>(kl, row, 64 * ii + 16 * g4);
        uint32_t a0, a1, a2, a3, b0, b1, b2, b3;
        e4m3x4_to_bf16(raw.x, a0, a1);
        e4m3x4_to_bf16(raw.y, a2, a3);
        e4m3x4_to_bf16(raw.z, b0, b1);
        e4m3x4_to_bf16(raw.w, b2, b3);
        kf[hh][2 * ii] = u32x4_t{a0, a1, a2, a3};
        kf[hh][2 * ii + 1] = u32x4_t{b0, b1, b2, b3};
      }
    }
  }
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) s[rg][hh] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) s[rg][hh] = mfma_bf16(kf[hh][c], qf[rg][c], s[rg][hh]);
}

// Softmax and PV of one tile whose logits s came from flash_qk.
template <bool FP8, int D, int RG, bool BAND>
__device__ __forceinline__ void flash_pv(const char* vl, f32x4_t (&s)[RG][2], float cs, int j0,
                                         const int (&jlim)[RG], const int (&jlo)[RG], bool need_mask, int r, int g4,
                                         ChunkState<D, RG>& S) {
  constexpr int VE = D / 16;
  // Online softmax against each row's reference S.m (mu = S.m, or 0 before
  // the row has one).  The exponents x = s cs - mu are formed first; only when
  // some lane's x exceeds thr (kLazyMax, or -inf for a row with no reference
  // yet) does the rare path take the row maximum across lanes and move the
  // reference, rescaling that row's accumulators.
  u32x4_t pf[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    if (need_mask) {
      // position j0 + 4 g4 + o with o = 16 hh + ii: compared through
      // o > jlim - j0 - 4 g4 (and o < jlo - j0 - 4 g4), constants on one side
      const int dhi = jlim[rg] - j0 - 4 * g4;
      const int dlo = BAND ? jlo[rg] - j0 - 4 * g4 : 0;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          if (16 * hh + ii > dhi || (BAND && 16 * hh + ii < dlo)) s[rg][hh][ii] = kNegInf;
    }
    float x[2][4];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) x[hh][ii] = __builtin_fmaf(s[rg][hh][ii], cs, -S.mu[rg]);
    // chained three-input maxima (four instructions for the eight exponents)
    const float xm = fmaxf(fmaxf(fmaxf(fmaxf(fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), x[0][2]), x[0][3]), x[1][0]),
                                       x[1][1]), x[1][2]), x[1][3]);
    if (__any(xm > S.thr[rg])) {
      const float rmax = max_x32(max_x16(xm));  // the row's largest exponent
      const bool move = rmax > S.thr[rg];       // uniform over the row's lanes
      const float m_new = move ? S.mu[rg] + rmax : S.m[rg];
      const float alpha = !move ? 1.f : (S.m[rg] == kNegInf) ? 0.f : exp2_fast(S.m[rg] - m_new);
      S.l[rg] *= alpha;
#pragma unroll
      for (int dt = 0; dt < VE; ++dt) S.o[rg][dt] *= alpha;
      S.m[rg] = m_new;
      S.mu[rg] = move ? m_new : S.mu[rg];
      S.thr[rg] = move ? kLazyMax : S.thr[rg];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) x[hh][ii] = __builtin_fmaf(s[rg][hh][ii], cs, -S.mu[rg]);
    }
    float pr[2][4];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) pr[hh][ii] = exp2_fast(x[hh][ii]);
    S.l[rg] += ((pr[0][0] + pr[0][1]) + (pr[0][2] + pr[0][3])) + ((pr[1][0] + pr[1][1]) + (pr[1][2] + pr[1][3]));
    pf[rg] = u32x4_t{pack_bf16(pr[0][0], pr[0][1]), pack_bf16(pr[0][2], pr[0][3]), pack_bf16(pr[1][0], pr[1][1]),
                     pack_bf16(pr[1][2], pr[1][3])};
  }
  if constexpr (!FP8) {
    // V^T operands straight from LDS with the transposing 64-bit read: in each
    // 16-lane group, source lane s = 4k + a names 4 consecutive head dims
    // (piece a) of one V row (position k of the group's four); lane i then
    // receives head dim 16 dt + i of those four positions.  Two reads give the
    // 8 positions 4 g4 + {0..3}, 16 + 4 g4 + {0..3} that match the P layout.
    // Accumulator row m of block dt is head dim 16 dt + m.
    const int k4 = (r >> 2), a4 = r & 3;
#pragma unroll
    for (int dt = 0; dt < VE; ++dt) {
      u32x4_t va;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const char* src = flash_at<FP8, D, true>(vl, 16 * c + 4 * g4 + k4, 32 * dt + 8 * a4);
        const s16x4_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)src);
        const u32x2_t w = __builtin_bit_cast(u32x2_t, t);
        va[2 * c] = w.x;
        va[2 * c + 1] = w.y;
      }
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) S.o[rg][dt] = mfma_bf16(va, pf[rg], S.o[rg][dt]);
    }
  } else {
    // FP8: each lane decodes VE-element slices of 8 V rows (positions
    // 16 (kk >> 2) + 4 g4 + (kk & 3), head dims VE r ..), and byte permutes
    // build the V^T operand of each block dt; accumulator row m of block dt is
    // head dim VE m + dt.
    uint32_t vd[8][VE / 2];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const char* a = flash_at<FP8, D, true>(vl, 16 * (kk >> 2) + 4 * g4 + (kk & 3), VE * r);
      if constexpr (VE == 8) {
        const u32x2_t w = *(const u32x2_t*)a;
        e4m3x4_to_bf16(w.x, vd[kk][0], vd[kk][1]);
        e4m3x4_to_bf16(w.y, vd[kk][2], vd[kk][3]);
      } else {
        e4m3x4_to_bf16(*(const uint32_t*)a, vd[kk][0], vd[kk][1]);
      }
    }
#pragma unroll
    for (int dt = 0; dt < VE; ++dt) {
      const int w = dt >> 1;
      u32x4_t va;
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        const uint32_t e0 = vd[2 * q2][w], e1 = vd[2 * q2 + 1][w];
        va[q2] = (dt & 1) ? __builtin_amdgcn_perm(e1, e0, 0x07060302u) : __builtin_amdgcn_perm(e1, e0, 0x05040100u);
      }
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) S.o[rg][dt] = mfma_bf16(va, pf[rg], S.o[rg][dt]);
    }
  }
}

// 3 waves per SIMD: 3 workgroups of 48 KiB LDS rings per CU (bf16 D = 128),
// at most 168 VGPRs per wave.  BAND: sliding-window attention (P.band rows
// ending at each query), one split, final outputs written here; a handful of
// tiles per workgroup, so 2 waves per SIMD (the row limits need registers).
template <bool FP8, int D, bool BAND>
__global__ void __launch_bounds__(256, BAND ? 2 : 3) chunk_flash(ScanParams P) {
  constexpr int RG = kFlashRG, VE = D / 16, NC = D / 32;
  constexpr int NBUF = 3;  // LDS tile ring: tile n in buffer n % NBUF, NBUF - 1 tiles in flight
  using FG = FlashGeom<FP8, D>;
  __shared__ __align__(16) char tiles[NBUF][TileLoader<FP8, D, 2>::BYTES];
  const int lane = threadIdx.x & 63, tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g4 = lane >> 4;
  const int nblk = (P.n_tpacks + 4 * RG - 1) / (4 * RG);
  const ChunkItem it = chunk_item(P, nblk);
  const int b = it.b, g = it.g;
  const int blk_w = it.blk * 4 + wave;  // this wave's block of RG packs
  const int q0 = qpos_of(P.qpos_b, P.q_pos0, b, P.N, P.Tq);

  u32x4_t qf[RG][NC];
  int jlim[RG], jlo[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const ChunkRows cr = chunk_row<RG>(P, q0, blk_w, rg, r);
    jlim[rg] = cr.jlim;
    jlo[rg] = BAND ? cr.jlim - P.band + 1 : 0;  // sliding window: the row's first position
  }
  const int t_first = it.blk * 4 * RG * P.tpack;  // first token of the workgroup
  const int t_last = min(t_first + 4 * RG * P.tpack, P.Tq) - 1;
  const int p_max = q0 + t_last;
  const int wt_first = blk_w * RG * P.tpack;  // first token of this wave
  const int wt_last = min(wt_first + RG * P.tpack, P.Tq) - 1;
  const int j_nomask = q0 + min(wt_first, P.Tq - 1);
  // sliding window (one split): from the window start of the workgroup's first
  // token, in whole tiles; tiles before the window start of this wave's last
  // token need the lower mask
  const int j_begin = BAND ? max(0, q0 + t_first - P.band + 1) & ~31 : it.split * P.split_len;
  const int j_end = BAND ? p_max + 1 : min(j_begin + P.split_len, p_max + 1);
  const int jlo_nomask = BAND ? q0 + max(wt_last, 0) - P.band + 1 : 0;
  const int ntile = j_end > j_begin ? (j_end - j_begin + 31) / 32 : 0;

  const int64_t kvoff = ((int64_t)b * P.sb + (int64_t)g * P.sh) * FG::EB;
  const char* kb = (const char*)P.k + kvoff;
  const char* vb = (const char*)P.v + kvoff;
  const int64_t snb = P.sn * FG::EB;
  float cs = P.scale_log2;
  if constexpr (FP8) cs *= P.k_scale[b * P.Hkv + g];

  const TileLoader<FP8, D, 2> ld(kb, vb, snb, tid, wave);
  auto issue = [&](int tile) {
    if (tile < ntile) ld.issue(tiles[tile % NBUF], j_begin + 32 * tile, p_max);
  };

  // the ring's first tiles go out before the query fragments, and one wait
  // covers both; after it the compiler's own wait bookkeeping has nothing
  // pending across the loop (the tile loads are invisible to it)
#pragma unroll
  for (int t = 0; t < NBUF - 1; ++t) issue(t);
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const ChunkRows cr = chunk_row<RG>(P, q0, blk_w, rg, r);
    load_q<FP8, D, false>(qf[rg], P, b, cr.ok ? cr.t : 0, g * P.G + (r % P.G), cr.ok, g4);
  }
  ChunkState<D, RG> S;
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    S.m[rg] = kNegInf;
    S.l[rg] = 0.f;
    S.mu[rg] = 0.f;
    S.thr[rg] = kNegInf;
#pragma unroll
    for (int dt = 0; dt < VE; ++dt) S.o[rg][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  wait_vm<0>();
  // step n (buffer n % NBUF known at compile time in the unrolled body, so
  // every LDS address is a per-lane constant plus an immediate offset)
  auto step = [&](auto buf, int n) {
    constexpr int B = decltype(buf)::value;
    ring_wait<NBUF, TileLoader<FP8, D, 2>::PER>(n, ntile);
    if (n + NBUF - 1 < ntile) ld.issue(tiles[(B + NBUF - 1) % NBUF], j_begin + 32 * (n + NBUF - 1), p_max);
    const int j0 = j_begin + 32 * n;
    f32x4_t sc[RG][2];
    flash_qk<FP8, D, RG>(tiles[B], qf, r, g4, sc);
    flash_pv<FP8, D, RG, BAND>(tiles[B] + FG::HALF, sc, cs, j0, jlim, jlo,
                               j0 + 31 > j_nomask || (BAND && j0 < jlo_nomask), r, g4, S);
  };
  static_assert(NBUF == 3 || NBUF == 4, "the unrolled ring below has 3 or 4 buffers");
  for (int n = 0; n < ntile; n += NBUF) {
    step(std::integral_constant<int, 0>{}, n);
    if (n + 1 >= ntile) break;
    step(std::integral_constant<int, 1>{}, n + 1);
    if (n + 2 >= ntile) break;
    step(std::integral_constant<int, 2>{}, n + 2);
    if constexpr (NBUF == 4) {
      if (n + 3 >= ntile) break;
      step(std::integral_constant<int, NBUF - 1>{}, n + 3);
    }
  }

  // partials of this wave's row groups (16 rows each)
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const int tp = blk_w * RG + rg;
    if (tp >= P.n_tpacks) continue;  // uniform per wave
    float l = S.l[rg];
    l = sum_x16(l);
    l = sum_x32(l);
    if (r >= P.rows) continue;
    if constexpr (BAND) {  // one split: this is the row's whole softmax
      const int t = tp * P.tpack + r / P.G;
      if (t >= P.Tq) continue;
      const int64_t orow = ((int64_t)b * P.Tq + t) * P.Hq + g * P.G + r % P.G;
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const float vsc = FP8 ? P.v_scale[b * P.Hkv + g] : 1.f;
      const float f = inv * vsc;
      uint16_t* orow_p = (uint16_t*)P.out + orow * D;
      if constexpr (FP8) {  // head dims VE (4 g4 + ii) + dt: VE consecutive per ii, one 2*VE-byte store
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          uint32_t w[VE / 2];
#pragma unroll
          for (int dt = 0; dt < VE; dt += 2) w[dt / 2] = pack_bf16(S.o[rg][dt][ii] * f, S.o[rg][dt + 1][ii] * f);
          if constexpr (VE == 8)
            *(u32x4_t*)(orow_p + VE * (4 * g4 + ii)) = u32x4_t{w[0], w[1], w[2], w[3]};
          else
            *(u32x2_t*)(orow_p + VE * (4 * g4 + ii)) = u32x2_t{w[0], w[1]};
        }
      } else {  // head dims 16 dt + 4 g4 + ii: four consecutive per dt, one 8-byte store
#pragma unroll
        for (int dt = 0; dt < VE; ++dt)
          *(u32x2_t*)(orow_p + 16 * dt + 4 * g4) =
              u32x2_t{pack_bf16(S.o[rg][dt][0] * f, S.o[rg][dt][1] * f), pack_bf16(S.o[rg][dt][2] * f, S.o[rg][dt][3] * f)};
      }
      if (g4 == 0 && P.lse) P.lse[orow] = l > 0.f ? (S.m[rg] + log2f(l)) * kLn2 : kNegInf;
      continue;
    }
    const int unit = (b * P.n_tpacks + tp) * P.Hkv + g;
    const int64_t pb = ((int64_t)unit * P.nsplit + it.split) * 16 + r;
#pragma unroll
    for (int dt = 0; dt < VE; ++dt)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int d = FP8 ? VE * (4 * g4 + ii) + dt : 16 * dt + 4 * g4 + ii;  // see flash_tile
        P.part_o[pb * D + d] = S.o[rg][dt][ii];
      }
    if (g4 == 0) {
      P.part_ml[pb * 2] = S.m[rg];
      P.part_ml[pb * 2 + 1] = l;
    }
  }
}

// Score pass of the chunk: S[b,t,g,j] = sum over the G heads of token t of
// 2^(x_hj - lse2_h) for j <= p_t, 0 beyond.  K only; tiles past the
// workgroup's last query position are zeros without loads.  Logits in the
// S = Q K^T orientation (G >= 4): lane l holds rows 4*(l/16)+i of position
// l%16, all of one token, so a token's head sum starts with three in-lane adds;
// for G >= 8 one permlane16 swap then pairs the row groups (0,1) and (2,3) of
// both 16-position halves at once (G = 16 adds a permlane32 swap).

// Score pass, LDS-staged form: the workgroup's 4 waves hold kFlashRG row
// groups each (4 * kFlashRG packs per workgroup) and share every K tile
// through the LDS ring; each wave stages its tokens' 32-position score rows
// in LDS and writes them with 16-byte stores.  Software-pipelined: a step
// issues the next tile's QK^T while it forms this tile's terms.
template <bool FP8, int D, int G>
__global__ void __launch_bounds__(256, 2) chunk_score_flash(ScanParams P) {
  static_assert(G == 4 || G == 8 || G == 16, "chunk score pass: G in {4, 8, 16}");
  constexpr int RG = kFlashRG, NC = D / 32, NBUF = 4;
  constexpr int TP = 16 / G;  // tokens per row group
  using FG = FlashGeom<FP8, D>;
  using TL = TileLoader<FP8, D, 1>;
  using RT = RawTile<FP8, D>;
  __shared__ __align__(16) char tiles[NBUF][TL::BYTES];
  __shared__ __align__(16) float stage[4][RG * TP * 32];
  const int lane = threadIdx.x & 63, tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g4 = lane >> 4;
  const int nblk = (P.n_tpacks + 4 * RG - 1) / (4 * RG);
  const ChunkItem it = chunk_item(P, nblk);
  const int b = it.b, g = it.g;
  const int blk_w = it.blk * 4 + wave;  // this wave's block of RG packs
  const int q0 = qpos_of(P.qpos_b, P.q_pos0, b, P.N, P.Tq);

  // query fragments (row r of each group), and the log2-sum-exp of this
  // lane's four S rows 4*g4 + ii.  Rows past Tq (or past the pack) have a zero
  // query, so their logits are 0; a log2-sum-exp of +inf turns them into
  // exact zeros with no extra test.  Positions past a token's own are zeroed
  // when the tile's scores are flushed.
  u32x4_t qf[RG][NC];
  float rl_l2[RG][4];  // (loaded after the ring's first tiles are issued, below)
  const int t_first = it.blk * 4 * RG * P.tpack;  // first token of the workgroup
  const int t_last = min(t_first + 4 * RG * P.tpack, P.Tq) - 1;
  const int p_max = q0 + t_last;
  const int wt_first = blk_w * RG * P.tpack;  // first token of this wave
  const int j_nomask = q0 + min(wt_first, P.Tq - 1);
  const int j_begin = it.split * P.split_len;
  const int j_end = min(j_begin + P.split_len, P.N);  // every position gets a score (0 past p)
  const int j_load = min(j_end, p_max + 1);           // tiles starting below it are computed
  const int ntile = j_load > j_begin ? (j_load - j_begin + 31) / 32 : 0;

  const int64_t kvoff = ((int64_t)b * P.sb + (int64_t)g * P.sh) * FG::EB;
  const char* kb = (const char*)P.k + kvoff;
  const int64_t snb = P.sn * FG::EB;
  float cs = P.scale_log2;
  if constexpr (FP8) cs *= P.k_scale[b * P.Hkv + g];
  const TL ld(kb, kb, snb, tid, wave);
  auto issue = [&](int tile) {
    if (tile < ntile) ld.issue(tiles[tile % NBUF], j_begin + 32 * tile, p_max);
  };

  float* st = stage[wave];
  auto stage_flush = [&](int j0) {
    for (int q = lane; q < RG * TP * 8; q += 64) {  // q: 4-float piece
      const int row = q >> 3, pos = (q & 7) * 4;
      const int rg = row / TP, tl = row - rg * TP;
      const int t = (blk_w * RG + rg) * TP + tl;
      f32x4_t v = *(const f32x4_t*)(st + row * 32 + pos);
      if (t >= P.Tq) continue;
      if (j0 + 31 > j_nomask) {  // positions past the token's own are zero
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j0 + pos + e > q0 + t) v[e] = 0.f;
      }
      float* dst = P.scores + (((int64_t)b * P.Tq + t) * P.Hkv + g) * P.N + j0 + pos;
      if ((P.N & 3) == 0 && j0 + pos + 3 < P.N) {
        *(f32x4_t*)dst = v;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j0 + pos + e < P.N) dst[e] = v[e];
      }
    }
  };
  // QK^T of the tile in LDS buffer kl into s
  auto qk = [&](const char* kl, f32x4_t (&s)[RG][2]) {
    u32x4_t kf[2][NC];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int row = 16 * hh + r;
      if constexpr (!FP8) {
#pragma unroll
        for (int c = 0; c < NC; ++c) kf[hh][c] = *(const u32x4_t*)flash_at<FP8, D>(kl, row, 64 * c + 16 * g4);
      } else {
#pragma unroll
        for (int ii = 0; ii < RT::KW; ++ii) {
          const u32x4_t raw = *(const u32x4_t*)flash_at<FP8, D>(kl, row, 64 * ii + 16 * g4);
          uint32_t a0, a1, a2, a3, b0, b1, b2, b3;
          e4m3x4_to_bf16(raw.x, a0, a1);
          e4m3x4_to_bf16(raw.y, a2, a3);
          e4m3x4_to_bf16(raw.z, b0, b1);
          e4m3x4_to_bf16(raw.w, b2, b3);
          kf[hh][2 * ii] = u32x4_t{a0, a1, a2, a3};
          kf[hh][2 * ii + 1] = u32x4_t{b0, b1, b2, b3};
        }
      }
    }
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) s[rg][hh] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) s[rg][hh] = mfma_bf16(qf[rg][c], kf[hh][c], s[rg][hh]);
  };
  // exponentials, head sums and LDS staging of one tile's scores (causal
  // zeros are applied by the flush)
  auto terms = [&](const f32x4_t (&s)[RG][2]) {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      float hs[2];  // in-lane head sums of the two 16-position halves
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float acc[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) acc[ii] = exp2_fast(__builtin_fmaf(s[rg][hh][ii], cs, -rl_l2[rg][ii]));
        hs[hh] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      }
      if constexpr (G == 4) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) st[(rg * TP + g4) * 32 + 16 * hh + r] = hs[hh];
      } else {
        const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(hs[0]), __float_as_uint(hs[1]), false, false);
        float v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
        if constexpr (G == 16) v = sum_x32(v);
        if (G == 8 || g4 < 2) st[(rg * TP + (G == 8 ? g4 >> 1 : 0)) * 32 + 16 * (g4 & 1) + r] = v;
      }
    }
  };
  // the ring's first tiles go out before the query and log-sum-exp loads,
  // and one wait covers all of them (the compiler's own wait bookkeeping then
  // has nothing pending across the loop)
#pragma unroll
  for (int t = 0; t < NBUF - 1; ++t) issue(t);
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const ChunkRows cr = chunk_row<RG>(P, q0, blk_w, rg, r);
    load_q<FP8, D, false>(qf[rg], P, b, cr.ok ? cr.t : 0, g * P.G + (r % P.G), cr.ok, g4);
    const int tp = blk_w * RG + rg;
    const int unit = (b * P.n_tpacks + min(tp, P.n_tpacks - 1)) * P.Hkv + g;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const ChunkRows crr = chunk_row<RG>(P, q0, blk_w, rg, 4 * g4 + ii);
      rl_l2[rg][ii] = crr.ok ? P.lse2_in[(int64_t)unit * P.rows + 4 * g4 + ii] : __builtin_inff();
    }
  }
  wait_vm<0>();
  // software pipeline: step n issues tile n+1's QK^T (from LDS) and forms
  // tile n's terms while those MFMAs run; its barrier makes tile n+1 visible
  // and frees tile n's buffer for tile n+4
  f32x4_t SA[RG][2], SB[RG][2];
  if (ntile > 0) {
    ring_wait<NBUF, TL::PER>(0, ntile);
    if (NBUF - 1 < ntile) ld.issue(tiles[NBUF - 1], j_begin + 32 * (NBUF - 1), p_max);
    qk(tiles[0], SA);
  }
  auto step = [&](auto buf, int n, const f32x4_t (&cur)[RG][2], f32x4_t (&nxt)[RG][2]) {
    constexpr int B = decltype(buf)::value;  // tile n's buffer
    ring_wait<NBUF, TL::PER>(n + 1, ntile);  // (past the last tile: an extra barrier, every wave alike)
    if (n + NBUF < ntile) ld.issue(tiles[B], j_begin + 32 * (n + NBUF), p_max);
    {
      qk(tiles[(B + 1) % NBUF], nxt);  // past the last tile: a stale buffer, result unused
      terms(cur);
      // schedule: the K fragment reads first, then each MFMA followed by
      // three vector instructions of the terms, so the matrix core works
      // while the wave issues them
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (FP8 ? RT::KW : NC), 0);  // LDS reads
#pragma unroll
      for (int i = 0; i < 2 * RG * NC; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // three VALU
      }
    }
    stage_flush(j_begin + 32 * n);
  };
  static_assert(NBUF == 4, "the unrolled pipeline below has 4 buffers");
  for (int n = 0; n < ntile; n += NBUF) {
    step(std::integral_constant<int, 0>{}, n, SA, SB);
    if (n + 1 >= ntile) break;
    step(std::integral_constant<int, 1>{}, n + 1, SB, SA);
    if (n + 2 >= ntile) break;
    step(std::integral_constant<int, 2>{}, n + 2, SA, SB);
    if (n + 3 >= ntile) break;
    step(std::integral_constant<int, 3>{}, n + 3, SB, SA);
  }
  // remaining tiles lie past every query position of the workgroup: zeros
  if (ntile * 32 + j_begin < j_end) {
    for (int q = lane; q < RG * TP * 32; q += 64) st[q] = 0.f;
    for (int j0 = j_begin + 32 * ntile; j0 < j_end; j0 += 32) stage_flush(j0);
  }
}

constexpr int kGatherIdxCap = 2048;  // index-list entries staged in LDS at a time

// Sparse layer: one workgroup per (b, t, g) over its whole index list (staged
// in LDS), final output written directly.
template <bool FP8, int D, int WAVES>
__global__ void __launch_bounds__(WAVES * 64, (FP8 || D == 64) ? 3 : 2) scan_gather(ScanParams P) {
  constexpr int VE = D / 16, NC = D / 32, EB = FP8 ? 1 : 2;
  constexpr int STEP = WAVES * 32;
  __shared__ float sm_m[WAVES][16];
  __shared__ float sm_l[WAVES][16];
  __shared__ float sm_o[WAVES][16][D + 1];
  __shared__ int s_idx[kGatherIdxCap];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g4 = lane >> 4;
  const int unit = blockIdx.y;  // (b, t, g)
  const int g = unit % P.Hkv;
  const int t = (unit / P.Hkv) % P.Tq;
  const int b = unit / (P.Hkv * P.Tq);
  const bool row_ok = r < P.G;
  const int h = g * P.G + r;
  // the unit's rows: its index list, or with a sliding window the contiguous
  // range [p - band + 1, p] (clipped at 0)
  const int32_t* list = P.idx + (int64_t)unit * P.max_sel;
  const int p_t = qpos_of(P.qpos_b, P.q_pos0, b, P.N, P.Tq) + t;
  const int n = P.band > 0 ? min(p_t + 1, P.band) : min(max(P.count[unit], 0), P.max_sel);
  const int lo = p_t - n + 1;

  u32x4_t qf[NC];
  load_q<FP8, D>(qf, P, b, t, h, row_ok, g4);
  const int64_t kvoff = ((int64_t)b * P.sb + (int64_t)g * P.sh) * EB;
  const char* kb = (const char*)P.k + kvoff + 16 * g4;
  const char* vb = (const char*)P.v + kvoff + VE * r * EB;
  const int64_t snb = P.sn * EB;
  float cs = P.scale_log2;
  if constexpr (FP8) cs *= P.k_scale[b * P.Hkv + g];

  WaveState<D> S;
  S.m = kNegInf;
  S.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < VE; ++dt) S.o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int base = 0; base < n; base += kGatherIdxCap) {
    const int nb = min(kGatherIdxCap, n - base);
    __syncthreads();
    for (int i = threadIdx.x; i < nb; i += WAVES * 64) {
      const int j = P.band > 0 ? lo + base + i : min(max(list[base + i], 0), P.N - 1);
      s_idx[i] = P.pages.table ? phys_row(P.pages, b, j) : j;  // the row's place in the cache
    }
    __syncthreads();
    const int jl = base + nb - 1;
    auto load = [&](RawTile<FP8, D>& R, int j0) {
      const char* kp[2];
      const char* vp[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) kp[hh] = kb + (int64_t)s_idx[min(j0 - base + 16 * hh + r, nb - 1)] * snb;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        vp[kk] = vb + (int64_t)s_idx[min(j0 - base + 16 * (kk >> 2) + 4 * g4 + (kk & 3), nb - 1)] * snb;
      load_tile<FP8, D>(R, kp, vp);
    };
    auto compute = [&](const RawTile<FP8, D>& R, int j0) {
      compute_tile<FP8, D, false>(R, qf, cs, j0, jl, j0 + 31 > jl, g4, nullptr, nullptr, 0, S);
    };
    // This wave's tiles j_first + i * STEP, i < nt, in a two-tile register
    // ring (one tile in flight while the other is computed).  Loads are
    // issued without conditions (tiles past the list reload its last row,
    // unused), so the compiler's in-order wait counts leave the prefetched
    // tile in flight; a conditional load would make every wait drain it.
    // Two tiles rather than three keep an FP8 wave within 168 registers, so
    // a SIMD holds three waves (measured at 256 lists of 1152 rows at 1M FP8:
    // 50.8 us against 56.1 us with three tiles at two waves per SIMD).
    const int jend = base + nb;
    const int j_first = base + wave * 32;
    const int nt = j_first < jend ? (jend - 1 - j_first) / STEP + 1 : 0;
    if (nt > 0) {
      RawTile<FP8, D> A, B;
      load(A, j_first);
      int i = 0;
      for (; i + 2 <= nt; i += 2) {
        const int j0 = j_first + i * STEP;
        load(B, j0 + STEP);
        compute(A, j0);
        load(A, j0 + 2 * STEP);
        compute(B, j0 + STEP);
      }
      if (i < nt) compute(A, j_first + i * STEP);
    }
  }
  merge_and_store<FP8, D, true, WAVES>(P, S, unit, 0, b, g, wave, r, g4, sm_m, sm_l, sm_o);
}

// Sparse layer, split form: the index list of each (b, t, g) is cut into
// gsplit slices of gslice slots; one workgroup per slice (one 32-row tile per
// wave when gslice = 128) writes a partial (max, sum, output); the workgroup
// that finishes last for its (b, t, g) -- a device-scope counter, fenced on
// both sides -- merges the partials, writes the output and re-arms the counter.
template <bool FP8, int D, int WAVES>
__global__ void __launch_bounds__(WAVES * 64) scan_gather_split(ScanParams P) {
  constexpr int VE = D / 16, NC = D / 32, EB = FP8 ? 1 : 2;
  constexpr int STEP = WAVES * 32;
  __shared__ float sm_m[WAVES][16];
  __shared__ float sm_l[WAVES][16];
  __shared__ float sm_o[WAVES][16][D + 1];
  __shared__ int s_idx[kGatherIdxCap];
  __shared__ int s_last;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g4 = lane >> 4;
  const int unit = blockIdx.y, split = blockIdx.x;  // unit = (b, t, g)
  const int g = unit % P.Hkv;
  const int t = (unit / P.Hkv) % P.Tq;
  const int b = unit / (P.Hkv * P.Tq);
  const bool row_ok = r < P.G;
  const int h = g * P.G + r;
  const int32_t* list = P.idx + (int64_t)unit * P.max_sel;
  const int lo = split * P.split_len;  // gslice
  // The slice's first WAVES*64 list slots are read together with the count and
  // the query (one memory round trip instead of two); slots past the count lie
  // inside the list buffer and are never used.
  const int nspec = min(P.split_len, P.max_sel - lo);
  const int e0 = (int)threadIdx.x < nspec ? list[lo + threadIdx.x] : 0;
  const int n = min(max(P.count[unit], 0), P.max_sel);
  const int hi = min(lo + P.split_len, n);

  u32x4_t qf[NC];
  load_q<FP8, D>(qf, P, b, t, h, row_ok, g4);
  const int64_t kvoff = ((int64_t)b * P.sb + (int64_t)g * P.sh) * EB;
  const char* kb = (const char*)P.k + kvoff + 16 * g4;
  const char* vb = (const char*)P.v + kvoff + VE * r * EB;
  const int64_t snb = P.sn * EB;
  float cs = P.scale_log2;
  if constexpr (FP8) cs *= P.k_scale[b * P.Hkv + g];

  WaveState<D> S;
  S.m = kNegInf;
  S.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < VE; ++dt) S.o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nb = max(0, hi - lo);  // <= gslice <= kGatherIdxCap
  // each entry's place in the cache (its physical row in a paged pool)
  auto place = [&](int e) {
    const int j = min(max(e, 0), P.N - 1);
    return P.pages.table ? phys_row(P.pages, b, j) : j;
  };
  if ((int)threadIdx.x < nb) s_idx[threadIdx.x] = place(e0);
  for (int i = threadIdx.x + WAVES * 64; i < nb; i += WAVES * 64) s_idx[i] = place(list[lo + i]);
  __syncthreads();
  if (nb > 0) {
    const int jl = lo + nb - 1;
    auto load = [&](RawTile<FP8, D>& R, int j0) {
      const char* kp[2];
      const char* vp[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) kp[hh] = kb + (int64_t)s_idx[min(j0 - lo + 16 * hh + r, nb - 1)] * snb;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        vp[kk] = vb + (int64_t)s_idx[min(j0 - lo + 16 * (kk >> 2) + 4 * g4 + (kk & 3), nb - 1)] * snb;
      load_tile<FP8, D>(R, kp, vp);
    };
    // this wave's tiles j_first + i * STEP, i < nt; unconditional loads as in
    // the one-workgroup form (tiles past the slice reload its last row, unused)
    const int j_first = lo + wave * 32;
    const int nt = j_first < hi ? (hi - 1 - j_first) / STEP + 1 : 0;
    if (nt > 0) {
      RawTile<FP8, D> A, B;
      load(A, j_first);
      int i = 0;
      for (; i + 2 <= nt; i += 2) {
        const int j0 = j_first + i * STEP;
        load(B, j0 + STEP);
        compute_tile<FP8, D, false>(A, qf, cs, j0, jl, j0 + 31 > jl, g4, nullptr, nullptr, 0, S);
        load(A, j0 + 2 * STEP);
        compute_tile<FP8, D, false>(B, qf, cs, j0 + STEP, jl, j0 + STEP + 31 > jl, g4, nullptr, nullptr, 0, S);
      }
      if (i < nt) {
        const int j0 = j_first + i * STEP;
        compute_tile<FP8, D, false>(A, qf, cs, j0, jl, j0 + 31 > jl, g4, nullptr, nullptr, 0, S);
      }
    }
  }
  // partial of this slice (rows = G heads), same layout as the full-layer
  // splits, stored device-coherent for the merging workgroup
  merge_and_store<FP8, D, false, WAVES, true>(P, S, unit, split, b, g, wave, r, g4, sm_m, sm_l, sm_o);

  // arrival: the workgroup barrier completes every wave's stores, one release
  // fence orders them before the counter update
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    s_last = (atomicAdd(&P.gcounter[unit], 1) == P.nsplit - 1);
  }
  __syncthreads();
  if (!s_last) return;
  // The last slice merges all partials (device-coherent loads).  Output
  // elements e0 + q * NT (q < EPT) of this thread take their slices in batches
  // of SB whose loads are all issued before any is used (slices past nsplit
  // reload the last one with no weight); the first batch goes out before the
  // slices' (max, sum) loads, so both arrive in one memory round trip.
  constexpr int NT = WAVES * 64, EPT = 4, SB = 16;
  const int GD = P.G * D;
  const int64_t sst = (int64_t)16 * D;
  const float* po[EPT];
  int rq[EPT];
  float vv[EPT][SB];
  auto setup = [&](int e0) {
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const int e = min(e0 + q * NT, GD - 1);
      rq[q] = e / D;
      po[q] = P.part_o + ((int64_t)unit * P.nsplit * 16 + rq[q]) * D + (e - rq[q] * D);
    }
  };
  auto load_batch = [&](int sp0) {
#pragma unroll
    for (int q = 0; q < EPT; ++q)
#pragma unroll
      for (int k = 0; k < SB; ++k) vv[q][k] = ld_coherent(po[q] + min(sp0 + k, P.nsplit - 1) * sst);
  };
  setup(threadIdx.x);
  load_batch(0);
  float* sw = &sm_o[0][0][0];  // [nsplit][16] maxima, then weights 2^(m_s - M), in the merge buffer
  float* sl = sw + P.nsplit * 16;  // [nsplit][16] sums (the host keeps 2 * nsplit * 16 within the buffer)
  for (int e = threadIdx.x; e < P.nsplit * 16; e += NT) {
    const int sp = e >> 4, rr = e & 15;
    const int64_t pb = ((int64_t)unit * P.nsplit + sp) * 16 + rr;
    const bool ok = rr < P.G;
    const float mv = ok ? ld_coherent(P.part_ml + pb * 2) : kNegInf;
    const float lv = ok ? ld_coherent(P.part_ml + pb * 2 + 1) : 0.f;
    sw[e] = mv;
    sl[e] = lv;
  }
  __syncthreads();
  if (threadIdx.x < P.G) {
    const int rr = threadIdx.x;
    float M = kNegInf;
    for (int sp = 0; sp < P.nsplit; ++sp) M = fmaxf(M, sw[sp * 16 + rr]);
    const float Ms = (M == kNegInf) ? 0.f : M;
    float L = 0.f;
    for (int sp = 0; sp < P.nsplit; ++sp) {
      const float w = exp2_fast(sw[sp * 16 + rr] - Ms);
      L += sl[sp * 16 + rr] * w;
      sw[sp * 16 + rr] = w;
    }
    sm_m[0][rr] = M;
    sm_l[0][rr] = L;
  }
  __syncthreads();
  for (int e0 = threadIdx.x; e0 < GD; e0 += EPT * NT) {
    if (e0 != (int)threadIdx.x) {
      setup(e0);
      load_batch(0);
    }
    float acc[EPT] = {};
    for (int sp0 = 0;;) {
#pragma unroll
      for (int q = 0; q < EPT; ++q)
#pragma unroll
        for (int k = 0; k < SB; ++k)
          if (sp0 + k < P.nsplit) acc[q] += sw[(sp0 + k) * 16 + rq[q]] * vv[q][k];
      sp0 += SB;
      if (sp0 >= P.nsplit) break;
      load_batch(sp0);
    }
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const int e = e0 + q * NT;
      if (e >= GD) break;
      const int rr = rq[q], d = e - rr * D;
      const float M = sm_m[0][rr], L = sm_l[0][rr];
      float o = (L > 0.f) ? acc[q] / L : 0.f;
      if constexpr (FP8) o *= P.v_scale[b * P.Hkv + g];
      const int64_t orow = ((int64_t)b * P.Tq + t) * P.Hq + g * P.G + rr;
      ((__bf16*)P.out)[orow * D + d] = (__bf16)o;
      if (d == 0 && P.lse) P.lse[orow] = (L > 0.f) ? (M + log2f(L)) * kLn2 : kNegInf;
    }
  }
  if (threadIdx.x == 0) P.gcounter[unit] = 0;  // re-armed for the next call
}

// ---------------------------------------------------------------------------
// fp32 VALU scan (fp32 query and cache; exact fp32 products and sums)
// ---------------------------------------------------------------------------
template <int D, bool GATHER, bool WRITE_LOGITS>
__global__ void __launch_bounds__(256) scan_f32(ScanParams P) {
  constexpr int TJ = 64;
  constexpr int NACC = 16 * D / 256;
  __shared__ float Ks[TJ][D + 1];
  __shared__ float Vs[TJ][D];
  __shared__ float Qs[16][D];
  __shared__ float Ps[16][TJ];
  __shared__ float s_alpha[16];
  __shared__ int s_rows[TJ];

  const int tid = threadIdx.x;
  const int unit = blockIdx.y, split = blockIdx.x;
  const int g = unit % P.Hkv;
  const int t = (unit / P.Hkv) % P.Tq;  // tpack == 1
  const int b = unit / (P.Hkv * P.Tq);
  const int R = P.G;
  const int p = qpos_of(P.qpos_b, P.q_pos0, b, P.N, P.Tq) + t;

  int j_begin, j_end;
  const int32_t* list = nullptr;
  int band_lo = 0;  // sliding window: rows band_lo + i
  if constexpr (GATHER) {
    list = P.idx + (int64_t)unit * P.max_sel;
    j_begin = 0;
    j_end = P.band > 0 ? min(p + 1, P.band) : min(max(P.count[unit], 0), P.max_sel);
    band_lo = p - j_end + 1;
  } else {
    j_begin = split * P.split_len;
    j_end = min(j_begin + P.split_len, p + 1);
  }

  for (int e = tid; e < 16 * D; e += 256) {
    const int rr = e / D, d = e - rr * D;
    Qs[rr][d] = (rr < R) ? ((const float*)P.q)[(((int64_t)b * P.Tq + t) * P.Hq + g * P.G + rr) * D + d] : 0.f;
  }
  const float* kb = (const float*)P.k + (int64_t)b * P.sb + (int64_t)g * P.sh;
  const float* vb = (const float*)P.v + (int64_t)b * P.sb + (int64_t)g * P.sh;

  const int r = tid >> 4, c = tid & 15;  // logits: row r, positions c + 16*s
  float m_run = kNegInf, l_run = 0.f;
  float acc[NACC];
#pragma unroll
  for (int s = 0; s < NACC; ++s) acc[s] = 0.f;

  for (int j0 = j_begin; j0 < j_end; j0 += TJ) {
    const int nt = min(TJ, j_end - j0);
    if (tid < TJ)
      s_rows[tid] = !GATHER       ? min(j0 + tid, j_end - 1)
                    : P.band > 0 ? band_lo + min(j0 + tid, j_end - 1)
                                 : min(max(list[min(j0 + tid, j_end - 1)], 0), P.N - 1);
    __syncthreads();
    for (int e = tid; e < TJ * D; e += 256) {
      const int jj = e / D, d = e - jj * D;
      const int64_t row = s_rows[jj];
      Ks[jj][d] = kb[row * P.sn + d];
      Vs[jj][d] = vb[row * P.sn + d];
    }
    __syncthreads();
    float x[4];
    float tmax = kNegInf;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int jj = c + 16 * s;
      float dot = 0.f;
#pragma unroll 16
      for (int d = 0; d < D; ++d) dot = fmaf(Qs[r][d], Ks[jj][d], dot);
      const bool ok = (jj < nt) && (r < R) && (GATHER || j0 + jj <= p);
      x[s] = ok ? dot * P.scale_log2 : kNegInf;
      tmax = fmaxf(tmax, x[s]);
    }
    if constexpr (WRITE_LOGITS) {
      // per aligned 32-position half: positions c, c+16 (half 0) and c+32, c+48 (half 1)
      float hm0 = fmaxf(x[0], x[1]), hm1 = fmaxf(x[2], x[3]);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        hm0 = fmaxf(hm0, __shfl_xor(hm0, o));
        hm1 = fmaxf(hm1, __shfl_xor(hm1, o));
      }
      if (r < R) {
        uint16_t* lg = P.lg16 + ((int64_t)unit * P.rows + r) * P.npad + j0;
        float* lgm = P.lgmax + ((int64_t)unit * (P.npad >> 5) + (j0 >> 5)) * P.rows + r;  // [unit][tile][row]
#pragma unroll
        for (int s = 0; s < 4; ++s)
          if (c + 16 * s < nt) lg[c + 16 * s] = (uint16_t)logit_code(s < 2 ? hm0 : hm1, x[s]);
        if (c == 0) {
          lgm[0] = hm0;
          if (nt > 32) lgm[P.rows] = hm1;
        }
      }
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_new == m_run) ? 1.f : exp2f(m_run - m_new);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    float psum = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float pv = exp2f(x[s] - m_use);
      Ps[r][c + 16 * s] = pv;
      psum += pv;
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (c == 0) s_alpha[r] = alpha;
    __syncthreads();
#pragma unroll
    for (int s = 0; s < NACC; ++s) {
      const int e = tid + 256 * s;
      const int rr = e / D, d = e - rr * D;
      float a = acc[s] * s_alpha[rr];
      for (int jj = 0; jj < TJ; ++jj) a = fmaf(Ps[rr][jj], Vs[jj][d], a);
      acc[s] = a;
    }
    __syncthreads();
  }

#pragma unroll
  for (int o = 1; o < 16; o <<= 1) l_run += __shfl_xor(l_run, o);
  if (c == 0) {
    Ps[r][0] = m_run;
    Ps[r][1] = l_run;
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < NACC; ++s) {
    const int e = tid + 256 * s;
    const int rr = e / D, d = e - rr * D;
    if (rr >= R) continue;
    const float M = Ps[rr][0], L = Ps[rr][1];
    if constexpr (GATHER) {
      const int64_t orow = ((int64_t)b * P.Tq + t) * P.Hq + g * P.G + rr;
      ((float*)P.out)[orow * D + d] = (L > 0.f) ? acc[s] / L : 0.f;
      if (d == 0 && P.lse) P.lse[orow] = (L > 0.f) ? (M + log2f(L)) * kLn2 : kNegInf;
    } else {
      const int64_t pbase = ((int64_t)unit * P.nsplit + split) * 16 + rr;
      P.part_o[pbase * D + d] = acc[s];
      if (d == 0) {
        P.part_ml[pbase * 2] = M;
        P.part_ml[pbase * 2 + 1] = L;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// combine split partials -> output, LSE (natural) and log2 LSE for scores
// ---------------------------------------------------------------------------
constexpr int kMaxSplits = 2048;

__device__ __forceinline__ float block_reduce_256(float v, float* red, bool is_max) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float y = __shfl_xor(v, o);
    v = is_max ? fmaxf(v, y) : v + y;
  }
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = red[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) t = is_max ? fmaxf(t, red[w]) : t + red[w];
  return t;
}

// The selection rows (b, t, g) of the unit's tokens set up as the selection's
// own initialisation would (one workgroup, 256 threads).
__device__ __forceinline__ void sel_init_unit_rows(const CombineParams& P, int b, int tp, int g, int tid) {
  for (int tl = 0; tl < P.tpack; ++tl) {
    const int t = tp * P.tpack + tl;
    if (t >= P.Tq) break;
    const int64_t u = ((int64_t)b * P.Tq + t) * P.Hkv + g;
    sel_init_row(P.sel_state + u * ST_WORDS, P.sel_hist + u * 3 * kHistBins,
                 qpos_of(P.qpos_b, P.q_pos0, b, P.N, P.Tq) + t, P.sel_k, P.sel_window, 1, tid, 256);
  }
}

// LDS of one merging workgroup: split weights and sums, reduction slots, the
// per-thread partial sums
struct CombineLds {
  float sw[kMaxSplits];
  float sl[kMaxSplits];
  float red[8];
  float part[256];
};

// Merge of row r, head dims [32 z, 32 z + 32) of a unit by one workgroup:
// the split weights 2^(m_s - M) into LDS, then 8 groups of 32 threads sum
// interleaved splits, each thread's loads issued 32 at a time.
__device__ __forceinline__ void combine_row(const CombineParams& P, int unit, int r, int z, CombineLds& L_) {
  float* sw = L_.sw;
  float* sl = L_.sl;
  float* red = L_.red;
  float* part = L_.part;
  const int tid = threadIdx.x;
  const int g = unit % P.Hkv;
  const int tp = (unit / P.Hkv) % P.n_tpacks;
  const int b = unit / (P.Hkv * P.n_tpacks);
  const int tl = r / P.G, i = r - tl * P.G;
  const int t = tp * P.tpack + tl;
  if (t >= P.Tq) return;
  const int h = g * P.G + i;
  const float* ml = P.part_ml + ((int64_t)unit * P.nsplit * 16 + r) * 2;
  const int dl = tid & 31, pp = tid >> 5;
  const int d = z * 32 + dl;
  const float* po = P.part_o + ((int64_t)unit * P.nsplit * 16 + r) * P.D + d;
  const int64_t sstride = (int64_t)16 * P.D;
  // This thread sums splits pp, pp + 8, ... in batches of CB whose loads are
  // all issued before any is used (splits past nsplit reload the last one
  // with no weight).  The first batch is issued before the (max, sum) loads,
  // so both arrive in one memory round trip.
  constexpr int CB = 32;
  float vv[CB];
  auto load_batch = [&](int s0) {
#pragma unroll
    for (int k = 0; k < CB; ++k) vv[k] = po[(int64_t)min(s0 + 8 * k, P.nsplit - 1) * sstride];
  };
  load_batch(pp);
  // each split's (max, sum) read once; the sums wait in LDS
  float m = kNegInf;
  for (int s = tid; s < P.nsplit; s += 256) {
    const float ms = ml[s * 32], ls = ml[s * 32 + 1];
    sw[s] = ms;
    sl[s] = ls;
    m = fmaxf(m, ms);
  }
  const float M = block_reduce_256(m, red, true);  // its barriers also publish sw, sl
  const float Ms = (M == kNegInf) ? 0.f : M;
  float l = 0.f;
  for (int s = tid; s < P.nsplit; s += 256) {
    const float w = exp2f(sw[s] - Ms);
    sw[s] = w;
    l += sl[s] * w;
  }
  const float L = block_reduce_256(l, red, false);  // its barriers also publish the weights
  float acc = 0.f;
  for (int s0 = pp;;) {
#pragma unroll
    for (int k = 0; k < CB; ++k)
      if (s0 + 8 * k < P.nsplit) acc += sw[s0 + 8 * k] * vv[k];
    s0 += 8 * CB;
    if (s0 >= P.nsplit) break;
    load_batch(s0);
  }
  part[tid] = acc;
  __syncthreads();
  if (pp != 0) return;
  float O = 0.f;
#pragma unroll
  for (int q = 0; q < 8; ++q) O += part[q * 32 + dl];
  float o = (L > 0.f) ? O / L : 0.f;
  if (P.v_scale) o *= P.v_scale[b * P.Hkv + g];
  const int64_t orow = ((int64_t)b * P.Tq + t) * P.Hq + h;
  if (P.out_bf16)
    ((__bf16*)P.out)[orow * P.D + d] = (__bf16)o;
  else
    ((float*)P.out)[orow * P.D + d] = o;
  if (d == 0) {
    const float l2 = (L > 0.f) ? M + log2f(L) : kNegInf;
    if (P.lse) P.lse[orow] = l2 * kLn2;
    P.lse2[(int64_t)unit * P.rows + r] = l2;
  }
}

// grid (unit, row, head-dim chunk of 32)
__global__ void __launch_bounds__(256) combine(CombineParams P) {
  __shared__ CombineLds L_;
  const int unit = blockIdx.x, r = blockIdx.y;
  if (P.sel_state && r == 0 && blockIdx.z == 0) {
    const int g = unit % P.Hkv;
    const int tp = (unit / P.Hkv) % P.n_tpacks;
    const int b = unit / (P.Hkv * P.n_tpacks);
    sel_init_unit_rows(P, b, tp, g, threadIdx.x);
  }
  combine_row(P, unit, r, blockIdx.z, L_);
}

// The same merge for many units with few splits each (the chunk path: a
// handful of splits per unit): one workgroup per unit.  Rows' (M, L) and split weights go to LDS first, then
// each thread forms whole outputs (row, head dim) from the splits' partials,
// which a wave reads as contiguous runs of the head dimension.
constexpr int kFewSplits = 32;
constexpr int kFewSplitsMinUnits = 512;  // fewer units: the per-(row, slice) grid fills the GPU better
__global__ void __launch_bounds__(256) combine_few(CombineParams P) {
  __shared__ float sw[16][kFewSplits];
  __shared__ float sM[16], sL[16];
  const int unit = blockIdx.x, tid = threadIdx.x;
  const int g = unit % P.Hkv;
  const int tp = (unit / P.Hkv) % P.n_tpacks;
  const int b = unit / (P.Hkv * P.n_tpacks);
  if (P.sel_state) sel_init_unit_rows(P, b, tp, g, tid);
  if (tid < P.rows) {
    const float* ml = P.part_ml + ((int64_t)unit * P.nsplit * 16 + tid) * 2;
    float m = kNegInf;
    for (int sp = 0; sp < P.nsplit; ++sp) m = fmaxf(m, ml[sp * 32]);
    const float Ms = (m == kNegInf) ? 0.f : m;
    float l = 0.f;
    for (int sp = 0; sp < P.nsplit; ++sp) {
      const float w = exp2f(ml[sp * 32] - Ms);
      sw[tid][sp] = w;
      l += ml[sp * 32 + 1] * w;
    }
    sM[tid] = m;
    sL[tid] = l;
  }
  __syncthreads();
  const int64_t sstride = (int64_t)16 * P.D;
  const float vsc = P.v_scale ? P.v_scale[b * P.Hkv + g] : 1.f;
  for (int e = tid; e < P.rows * P.D; e += 256) {
    const int r = e / P.D, d = e - r * P.D;
    const int tl = r / P.G, i = r - tl * P.G;
    const int t = tp * P.tpack + tl;
    if (t >= P.Tq) continue;
    const float* po = P.part_o + ((int64_t)unit * P.nsplit * 16 + r) * P.D + d;
    float O = 0.f;
    for (int sp = 0; sp < P.nsplit; ++sp) O += sw[r][sp] * po[sp * sstride];
    const float L = sL[r];
    float o = (L > 0.f) ? O / L : 0.f;
    o *= vsc;
    const int64_t orow = ((int64_t)b * P.Tq + t) * P.Hq + g * P.G + i;
    if (P.out_bf16)
      ((__bf16*)P.out)[orow * P.D + d] = (__bf16)o;
    else
      ((float*)P.out)[orow * P.D + d] = o;
    if (d == 0) {
      const float l2 = (L > 0.f) ? sM[r] + log2f(L) : kNegInf;
      if (P.lse) P.lse[orow] = l2 * kLn2;
      P.lse2[(int64_t)unit * P.rows + r] = l2;
    }
  }
}

// ---------------------------------------------------------------------------
// scores[b,t,g,j] = sum_{heads of g} 2^(x_hj - lse2_h) for j <= p, 0 beyond
// ---------------------------------------------------------------------------

// log2-domain logit of query row (b, t, head h) against cache row j of kv head
// g, recomputed in fp32 from the stored elements: the scan's expression, summed
// in another order.
__device__ __forceinline__ float recompute_logit(const ScoreParams& P, int b, int t, int h, int g, int j) {
  const int64_t jr = P.pages.table ? phys_row(P.pages, b, j) : j;  // the row's place in the cache
  const int64_t krow = (int64_t)b * P.sb + (int64_t)g * P.sh + jr * P.sn;
  const int64_t qrow = (((int64_t)b * P.Tq + t) * P.Hq + h) * P.D;
  float acc = 0.f;
  if (P.kv_dtype == HS2_F32) {
    const f32x4_t* k = (const f32x4_t*)((const float*)P.k + krow);
    const f32x4_t* q = (const f32x4_t*)((const float*)P.q + qrow);
    for (int c = 0; c < P.D / 4; ++c) {
      const f32x4_t kk = k[c], qq = q[c];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_fmaf(qq[e], kk[e], acc);
    }
    return acc * P.scale_log2;
  }
  const u32x4_t* q = (const u32x4_t*)((const uint16_t*)P.q + qrow);  // 8 bf16 elements per load
  float cs = P.scale_log2;
  for (int c = 0; c < P.D / 8; ++c) {
    u32x4_t kk;
    if (P.kv_dtype == HS2_BF16) {
      kk = ((const u32x4_t*)((const uint16_t*)P.k + krow))[c];
    } else {  // 8 E4M3FN codes -> 8 bf16 values (exact)
      const u32x2_t raw = ((const u32x2_t*)((const uint8_t*)P.k + krow))[c];
      uint32_t a0, a1, a2, a3;
      e4m3x4_to_bf16(raw.x, a0, a1);
      e4m3x4_to_bf16(raw.y, a2, a3);
      kk = u32x4_t{a0, a1, a2, a3};
    }
    const u32x4_t qq = q[c];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = __builtin_fmaf(bf16_bits_to_f32(qq[w] & 0xffffu), bf16_bits_to_f32(kk[w] & 0xffffu), acc);
      acc = __builtin_fmaf(bf16_bits_to_f32(qq[w] >> 16), bf16_bits_to_f32(kk[w] >> 16), acc);
    }
  }
  if (P.kv_dtype == HS2_FP8_E4M3FN) cs *= P.k_scale[b * P.Hkv + g];
  return acc * cs;
}

// The terms of position j (j <= p) whose codes saturated, for row group tl
// (token t) of a unit: exact where the probability of the code's tile maximum
// exceeds 2^kExactFloor, zero otherwise -- the terms the code-based sum took
// as zero.  l2u: the unit's rows' log2-domain LSE.
__device__ __forceinline__ float saturated_terms(const ScoreParams& P, int unit, int b, int t, int tl, int g, int j,
                                                 const float* l2u) {
  float add = 0.f;
  for (int i = 0; i < P.G; ++i) {
    const int rr = tl * P.G + i;
    const int64_t row = (int64_t)unit * P.rows + rr;
    if (P.lg16[row * P.npad + j] != 65535u) continue;
    const float l2 = l2u[rr];
    const float c = P.lgmax[((int64_t)unit * (P.npad >> 5) + (j >> 5)) * P.rows + rr] - l2;
    if (!(c > kExactFloor)) continue;
    add += exp2_fast(recompute_logit(P, b, t, g * P.G + i, g, j) - l2);
  }
  return add;
}

// One head's term from its code (c = tile maximum - lse2); `exact` is set when
// the code saturated and the term is not provably negligible.
__device__ __forceinline__ float code_term(uint32_t code, float c, bool& exact) {
  const bool sat = code == 65535u;
  exact |= sat && c > kExactFloor;
  return sat ? 0.f : exp2_fast(__builtin_fmaf((float)code, -kCodeInv, c));
}

__global__ void __launch_bounds__(256) score(ScoreParams P) {
  const int unit = blockIdx.y;
  const int j4 = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (j4 >= P.N) return;
  const int g = unit % P.Hkv;
  const int tp = (unit / P.Hkv) % P.n_tpacks;
  const int b = unit / (P.Hkv * P.n_tpacks);
  for (int tl = 0; tl < P.tpack; ++tl) {
    const int t = tp * P.tpack + tl;
    if (t >= P.Tq) break;
    const int p = qpos_of(P.qpos_b, P.q_pos0, b, P.N, P.Tq) + t;
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    if (j4 <= p) {
      bool exact = false;
      for (int i = 0; i < P.G; ++i) {
        const int64_t row = (int64_t)unit * P.rows + tl * P.G + i;
        const float c = P.lgmax[((int64_t)unit * (P.npad >> 5) + (j4 >> 5)) * P.rows + tl * P.G + i] - P.lse2[row];
        const u32x2_t w = *(const u32x2_t*)(P.lg16 + row * P.npad + j4);
        const uint32_t code[4] = {w.x & 0xffffu, w.x >> 16, w.y & 0xffffu, w.y >> 16};
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] += code_term(code[e], c, exact);
      }
      if (exact) {  // rare: a tile holding a dominant logit and terms 16+ log2 units below it
        for (int e = 0; e < 4; ++e)
          if (j4 + e <= p) s[e] += saturated_terms(P, unit, b, t, tl, g, j4 + e, P.lse2 + (int64_t)unit * P.rows);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j4 + e > p) s[e] = 0.f;
    }
    float* dst = P.scores + (((int64_t)b * P.Tq + t) * P.Hkv + g) * P.N + j4;
    if ((P.N & 3) == 0) {
      *(f32x4_t*)dst = f32x4_t{s[0], s[1], s[2], s[3]};
    } else {
      for (int e = 0; e < 4 && j4 + e < P.N; ++e) dst[e] = s[e];
    }
  }
}

// The log2-domain LSE of every row of a unit from the scan's split partials
// (max, sum), the quantity the merge computes (summed in another order): wave
// w takes rows w, w + 4, w + 8, w + 12, each lane every 64th split with an
// online (max, sum); the loads of four splits of all four rows are issued
// together.  Ends with a barrier that publishes s_l2[rows].
__device__ __forceinline__ void unit_lse2(const float* part_ml, int unit, int nsplit, int rows, float* s_l2) {
  constexpr int QS = 4;  // splits per lane per batch
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* ml0 = part_ml + (int64_t)unit * nsplit * 32;
  float m[4], l[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    m[k] = kNegInf;
    l[k] = 0.f;
  }
  for (int s0 = 0; s0 < nsplit; s0 += 64 * QS) {
    float mv[4][QS], lv[4][QS];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int q = 0; q < QS; ++q) {
        const int r = wave + 4 * k, sp = s0 + lane + 64 * q;
        const bool ok = r < rows && sp < nsplit;
        const float* e = ml0 + ((int64_t)sp * 16 + r) * 2;
        mv[k][q] = ok ? e[0] : kNegInf;
        lv[k][q] = ok ? e[1] : 0.f;
      }
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int q = 0; q < QS; ++q) {
        const float mn = fmaxf(m[k], mv[k][q]);
        if (mn != kNegInf) {
          l[k] = l[k] * exp2f(m[k] - mn) + lv[k][q] * exp2f(mv[k][q] - mn);
          m[k] = mn;
        }
      }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float M = m[k];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    float L = (M == kNegInf) ? 0.f : l[k] * exp2f(m[k] - M);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
    const int r = wave + 4 * k;
    if (lane == 0 && r < rows) s_l2[r] = (L > 0.f) ? M + log2f(L) : kNegInf;
  }
  __syncthreads();
}

// The score pass of a decode step whose selection follows (one query token
// per unit): the scores as above, R groups of 4 positions per thread (1024 R
// positions per workgroup), and the first radix digit of every candidate's
// score counted into the selection's pass-0 histogram (an LDS histogram per
// workgroup, flushed with one global atomic per non-empty digit).  Counts are
// integers, so the histogram equals the one the selection's own first pass
// would build from the stored scores.
// MERGE: the full layer's merge runs in the same launch.  The first
// rows * D/32 workgroups of each unit merge one (row, 32 head dims) each
// (outputs, LSE), and every score workgroup derives its rows' LSE from the
// split partials itself while its first code loads are in flight; the
// selection rows were set up by the scan.
template <int R, int GC, bool MERGE>
__global__ void __launch_bounds__(256) score_hist(ScoreParams P, CombineParams C) {
  __shared__ union {
    int32_t h[kHistBins];
    CombineLds c;
  } U;
  __shared__ float s_l2[16];
  int32_t* h = U.h;
  const int unit = blockIdx.y;
  int bx = blockIdx.x;
  if constexpr (MERGE) {
    const int ncomb = C.rows * (C.D / 32);
    if (bx < ncomb) {
      combine_row(C, unit, bx / (C.D / 32), bx % (C.D / 32), U.c);
      return;
    }
    bx -= ncomb;
  }
  const int g = unit % P.Hkv;
  const int t = (unit / P.Hkv) % P.n_tpacks;  // tpack = 1
  const int b = unit / (P.Hkv * P.n_tpacks);
  const int p = qpos_of(P.qpos_b, P.q_pos0, b, P.N, P.Tq) + t;
  const int base = bx * 1024 * R;
  const int ncand = sel_ncand(p, P.sel_window);
  const int take = sel_take(ncand, P.sel_k, 1);
  float* dst = P.scores + (((int64_t)b * P.Tq + t) * P.Hkv + g) * P.N;
  float s[R][4];
#pragma unroll
  for (int q = 0; q < R; ++q) s[q][0] = s[q][1] = s[q][2] = s[q][3] = 0.f;
  int jc[R];  // group starts clamped to p: groups past p are zeroed below
#pragma unroll
  for (int q = 0; q < R; ++q) jc[q] = min(base + 4 * (threadIdx.x + 256 * q), p);
  bool exact = false;
  auto add_head = [&](const u32x2_t (&w)[R], const float (&mx)[R], float l2) {
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const float c = mx[q] - l2;
      const uint32_t code[4] = {w[q].x & 0xffffu, w[q].x >> 16, w[q].y & 0xffffu, w[q].y >> 16};
#pragma unroll
      for (int e = 0; e < 4; ++e) s[q][e] += code_term(code[e], c, exact);
    }
  };
  // the unit's rows' LSE: from the merge, or derived here after the first
  // code loads have been issued
  auto row_lse = [&]() -> const float* {
    if constexpr (MERGE) {
      unit_lse2(C.part_ml, unit, C.nsplit, P.rows, s_l2);
      return s_l2;
    } else {
      return P.lse2 + (int64_t)unit * P.rows;
    }
  };
  const float* l2u;
  if constexpr (GC > 0) {
    // every head's loads issued before any is used: one memory round trip
    u32x2_t w[GC][R];
    float mx[GC][R];
#pragma unroll
    for (int i = 0; i < GC; ++i) {
      const int64_t row = (int64_t)unit * P.rows + i;
#pragma unroll
      for (int q = 0; q < R; ++q) {
        w[i][q] = *(const u32x2_t*)(P.lg16 + row * P.npad + (jc[q] & ~3));
        mx[i][q] = P.lgmax[((int64_t)unit * (P.npad >> 5) + (jc[q] >> 5)) * P.rows + i];
      }
    }
    l2u = row_lse();
#pragma unroll
    for (int i = 0; i < GC; ++i) add_head(w[i], mx[i], l2u[i]);
  } else {
    // head-outer, group-inner: each head's loads for all R groups together
    u32x2_t w[R];
    float mx[R];
    auto load_head = [&](int i) {
      const int64_t row = (int64_t)unit * P.rows + i;
#pragma unroll
      for (int q = 0; q < R; ++q) {
        w[q] = *(const u32x2_t*)(P.lg16 + row * P.npad + (jc[q] & ~3));
        mx[q] = P.lgmax[((int64_t)unit * (P.npad >> 5) + (jc[q] >> 5)) * P.rows + i];
      }
    };
    load_head(0);
    l2u = row_lse();
    for (int i = 0; i < P.G; ++i) {
      if (i > 0) load_head(i);
      add_head(w, mx, l2u[i]);
    }
  }
  if (exact) {  // rare: a tile holding a dominant logit and terms 16+ log2 units below it
    for (int q = 0; q < R; ++q) {
      const int j4 = base + 4 * (threadIdx.x + 256 * q);
      for (int e = 0; e < 4; ++e)
        if (j4 + e <= p) s[q][e] += saturated_terms(P, unit, b, t, 0, g, j4 + e, l2u);
    }
  }
  uint32_t key[4 * R];
  uint64_t valid = 0;
#pragma unroll
  for (int q = 0; q < R; ++q) {
    const int j4 = base + 4 * (threadIdx.x + 256 * q);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (j4 + e > p) s[q][e] = 0.f;
    if (j4 < P.N) {
      if ((P.N & 3) == 0) {
        *(f32x4_t*)(dst + j4) = f32x4_t{s[q][0], s[q][1], s[q][2], s[q][3]};
      } else {
        for (int e = 0; e < 4 && j4 + e < P.N; ++e) dst[j4 + e] = s[q][e];
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      key[4 * q + e] = score_key(s[q][e]);
      valid |= (uint64_t)(j4 + e < ncand) << (4 * q + e);
    }
  }
  // workgroup-uniform: rows that need no radix pass, chunks past the candidates
  if (!(take > 0 && take < ncand) || base >= ncand) return;
  for (int i = threadIdx.x; i < kHistBins; i += 256) h[i] = 0;
  __syncthreads();
  hist_digit0<4 * R>(key, valid, h);
  __syncthreads();
  int32_t* gh = P.sel_hist + (int64_t)unit * 3 * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += 256)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

// Streaming-read probe: every byte of buf read once with 16-byte non-temporal
// loads, grid-stride; one xor word per thread (out: blocks*256 words).
__global__ void __launch_bounds__(256) stream_read(const u32x4_t* __restrict__ buf, int64_t n16, uint32_t* out) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * 256 * 4;
  for (int64_t i = (int64_t)blockIdx.x * 1024 + threadIdx.x; i < n16; i += stride) {
    u32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = (i + 256 * u < n16) ? __builtin_nontemporal_load(buf + i + 256 * u) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

// Read-pattern probe of the decode scan: the launch, split mapping, per-lane
// row offsets and tile loads of scan_full, two tiles in flight per wave, with
// the attention arithmetic replaced by an xor of the loaded words.  With CODES
// every valid row lane also stores what the scan stores per tile (two 8-byte
// words of 16-bit codes in the row-major code buffer, and the tile maximum from
// lane group 0).  Its duration with and without CODES, beside the scan's,
// separates the cache read, the code writes and the arithmetic.  One xor word
// per thread goes to part_o (as words): units x nsplit x 256 of them.
template <bool FP8, int D, bool CODES, int WAVES>
__global__ void __launch_bounds__(WAVES * 64) scan_read_probe(ScanParams P) {
  constexpr int VE = D / 16, EB = FP8 ? 1 : 2;
  constexpr int STEP = WAVES * 32;
  using RT = RawTile<FP8, D>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g4 = lane >> 4;
  const int unit = blockIdx.y, split = blockIdx.x;
  const int g = unit % P.Hkv;
  const int tp = (unit / P.Hkv) % P.n_tpacks;
  const int b = unit / (P.Hkv * P.n_tpacks);
  const int t = tp * P.tpack + r / P.G;
  const bool row_ok = (r < P.rows) && (t < P.Tq);
  const int q0 = qpos_of(P.qpos_b, P.q_pos0, b, P.N, P.Tq);
  const int p_max = q0 + min(tp * P.tpack + P.tpack, P.Tq) - 1;
  const int j_begin = split * STEP;
  const int j_end = p_max + 1;
  const int jstride = P.nsplit * STEP;
  const int64_t kvoff = ((int64_t)b * P.sb + (int64_t)g * P.sh) * EB;
  const char* kb = (const char*)P.k + kvoff;
  const char* vb = (const char*)P.v + kvoff;
  const int64_t snb = P.sn * EB;
  uint16_t* lg_row = nullptr;
  float* lgm_row = nullptr;
  if (CODES && row_ok) {
    lg_row = P.lg16 + ((int64_t)unit * P.rows + r) * P.npad + 4 * g4;
    lgm_row = P.lgmax + (int64_t)unit * (P.npad >> 5) * P.rows + r;
  }
  uint32_t koff[2], voff[8];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) koff[hh] = (uint32_t)((16 * hh + r) * snb) + 16u * g4;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    voff[kk] = (uint32_t)((16 * (kk >> 2) + 4 * g4 + (kk & 3)) * snb) + (uint32_t)(VE * r * EB);
  auto load_full = [&](RT& R, int j0) {
    const char* kp[2];
    const char* vp[8];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) kp[hh] = kb + (int64_t)j0 * snb + koff[hh];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) vp[kk] = vb + (int64_t)j0 * snb + voff[kk];
    load_tile<FP8, D>(R, kp, vp);
  };
  auto load = [&](RT& R, int j0) {
    if (j0 + 31 <= p_max) {
      load_full(R, j0);
    } else {  // tail tile: rows past the last position repeat it
      const char* kp[2];
      const char* vp[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) kp[hh] = kb + (int64_t)min(j0 + 16 * hh + r, p_max) * snb + 16 * g4;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        vp[kk] = vb + (int64_t)min(j0 + 16 * (kk >> 2) + 4 * g4 + (kk & 3), p_max) * snb + VE * r * EB;
      load_tile<FP8, D>(R, kp, vp);
    }
  };
  uint32_t acc = 0;
  auto consume = [&](const RT& R, int j0) {
    uint32_t x = 0;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int c = 0; c < RT::KW; ++c) x ^= R.k[hh][c].x ^ R.k[hh][c].y ^ R.k[hh][c].z ^ R.k[hh][c].w;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int w = 0; w < RT::VW; ++w) x ^= R.v[kk][w];
    acc = acc * 3u + x;
    if (CODES && lg_row) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) *(u32x2_t*)(lg_row + j0 + 16 * hh) = u32x2_t{x, x + (uint32_t)hh};
      if (g4 == 0) lgm_row[(j0 >> 5) * P.rows] = __uint_as_float(x & 0x3f7fffffu);
    }
  };
  // the scan's tile loop: unconditional prefetches in the steady state, at
  // most three tiles in the epilogue
  const int j_first = j_begin + wave * 32;
  const int n = j_first < j_end ? (j_end - 1 - j_first) / jstride + 1 : 0;
  const int n_full = j_first + 31 <= p_max ? min(n, (p_max - 31 - j_first) / jstride + 1) : 0;
  RT A, B;
  int i = 0;
  if (n > 0) load(A, j_first);
  for (; i + 2 < n_full; i += 2) {
    const int j0 = j_first + i * jstride;
    load_full(B, j0 + jstride);
    consume(A, j0);
    load_full(A, j0 + 2 * jstride);
    consume(B, j0 + jstride);
  }
  if (i < n) {
    const int j0 = j_first + i * jstride;
    if (i + 1 < n) load(B, j0 + jstride);
    consume(A, j0);
    if (i + 1 < n) {
      if (i + 2 < n) load(A, j0 + 2 * jstride);
      consume(B, j0 + jstride);
      if (i + 2 < n) consume(A, j0 + 2 * jstride);
    }
  }
  ((uint32_t*)P.part_o)[((int64_t)unit * P.nsplit + split) * (WAVES * 64) + threadIdx.x] = acc;
}

__global__ void debug_e4m3fn(const uint8_t* codes, float* out, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i * 4 >= n) return;
  uint32_t w = 0;
  for (int e = 0; e < 4 && i * 4 + e < n; ++e) w |= (uint32_t)codes[i * 4 + e] << (8 * e);
  uint32_t lo, hi;
  e4m3x4_to_bf16(w, lo, hi);
  const float v[4] = {bf16_bits_to_f32(lo & 0xffffu), bf16_bits_to_f32(lo >> 16), bf16_bits_to_f32(hi & 0xffffu),
                      bf16_bits_to_f32(hi >> 16)};
  for (int e = 0; e < 4 && i * 4 + e < n; ++e) out[i * 4 + e] = v[e];
}

template <bool FP8, int D, bool WL, int WAVES>
hipError_t go_full(const ScanParams& p, dim3 grid, hipStream_t s) {
  TimedLaunch tl("full_scan", s);
  if (WL && p.pages.table)  // a paged pool (the host admits it only with the logits written)
    hipLaunchKernelGGL((scan_full<FP8, D, WL, WAVES, true>), grid, dim3(WAVES * 64), 0, s, p);
  else
    hipLaunchKernelGGL((scan_full<FP8, D, WL, WAVES>), grid, dim3(WAVES * 64), 0, s, p);
  return hipGetLastError();
}

template <bool FP8, int D, int WAVES>
hipError_t go_gather_split(const ScanParams& p, dim3 grid, hipStream_t s) {
  TimedLaunch tl("sparse_gather", s);
  hipLaunchKernelGGL((scan_gather_split<FP8, D, WAVES>), grid, dim3(WAVES * 64), 0, s, p);
  return hipGetLastError();
}

template <bool FP8, int D, int WAVES>
hipError_t go_gather(const ScanParams& p, dim3 grid, hipStream_t s) {
  TimedLaunch tl("sparse_gather", s);
  hipLaunchKernelGGL((scan_gather<FP8, D, WAVES>), grid, dim3(WAVES * 64), 0, s, p);
  return hipGetLastError();
}

template <int D, bool GATHER, bool WL>
hipError_t go_f32(const ScanParams& p, dim3 grid, hipStream_t s, const char* name) {
  TimedLaunch tl(name, s);
  hipLaunchKernelGGL((scan_f32<D, GATHER, WL>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

constexpr int kScanWaves = 4;
constexpr int kGatherWaves = 4;

hipError_t launch_scan(const ScanParams& p, int kv_dtype, bool gather, bool write_logits, hipStream_t s) {
  const int units = gather ? p.B * p.Tq * p.Hkv : p.B * p.n_tpacks * p.Hkv;
  const dim3 grid(gather ? 1 : p.nsplit, units);
  const char* name = gather ? "sparse_gather" : "full_scan";
  if (kv_dtype == HS2_F32) {
    if (p.D == 128) {
      if (gather) return go_f32<128, true, false>(p, grid, s, name);
      return write_logits ? go_f32<128, false, true>(p, grid, s, name) : go_f32<128, false, false>(p, grid, s, name);
    }
    if (gather) return go_f32<64, true, false>(p, grid, s, name);
    return write_logits ? go_f32<64, false, true>(p, grid, s, name) : go_f32<64, false, false>(p, grid, s, name);
  }
  const bool fp8 = kv_dtype == HS2_FP8_E4M3FN;
#define HS2_GO(F8, DD)                                                                  \
  do {                                                                                  \
    if (gather) return go_gather<F8, DD, kGatherWaves>(p, grid, s);                     \
    if (write_logits) return go_full<F8, DD, true, kScanWaves>(p, grid, s);             \
    return go_full<F8, DD, false, kScanWaves>(p, grid, s);                              \
  } while (0)
  if (fp8) {
    if (p.D == 128) HS2_GO(true, 128);
    HS2_GO(true, 64);
  }
  if (p.D == 128) HS2_GO(false, 128);
  HS2_GO(false, 64);
#undef HS2_GO
}

hipError_t launch_gather_split(const ScanParams& p, int kv_dtype, hipStream_t s) {
  const dim3 grid(p.nsplit, p.B * p.Tq * p.Hkv);
  if (kv_dtype == HS2_FP8_E4M3FN)
    return p.D == 128 ? go_gather_split<true, 128, 4>(p, grid, s) : go_gather_split<true, 64, 4>(p, grid, s);
  return p.D == 128 ? go_gather_split<false, 128, 4>(p, grid, s) : go_gather_split<false, 64, 4>(p, grid, s);
}

// LDS-staged chunk kernels address a tile's rows with 32-bit offsets
bool flash_rows_fit(const ScanParams& p, int kv_dtype) {
  const int64_t snb = p.sn * (kv_dtype == HS2_FP8_E4M3FN ? 1 : 2);
  return snb > 0 && snb < (int64_t(1) << 26);
}

hipError_t launch_chunk_full(const ScanParams& p, int kv_dtype, hipStream_t s) {
  TimedLaunch tl(p.band > 0 ? "swa_chunk" : "chunk_full", s);
  if (!flash_rows_fit(p, kv_dtype)) return hipErrorInvalidValue;
  const int nblk = (p.n_tpacks + kChunkPacks - 1) / kChunkPacks;
  const dim3 grid(p.B * nblk * p.Hkv * p.nsplit);
#define HS2_CF(F8, DD)                                                                         \
  do {                                                                                         \
    if (p.band > 0) hipLaunchKernelGGL((chunk_flash<F8, DD, true>), grid, dim3(256), 0, s, p); \
    else hipLaunchKernelGGL((chunk_flash<F8, DD, false>), grid, dim3(256), 0, s, p);           \
  } while (0)
  if (kv_dtype == HS2_FP8_E4M3FN) {
    if (p.D == 128) HS2_CF(true, 128);
    else HS2_CF(true, 64);
  } else {
    if (p.D == 128) HS2_CF(false, 128);
    else HS2_CF(false, 64);
  }
#undef HS2_CF
  return hipGetLastError();
}

template <bool FP8, int D>
void go_chunk_score(const ScanParams& p, dim3 grid, hipStream_t s) {
  switch (p.G) {
    case 4: hipLaunchKernelGGL((chunk_score_flash<FP8, D, 4>), grid, dim3(256), 0, s, p); break;
    case 8: hipLaunchKernelGGL((chunk_score_flash<FP8, D, 8>), grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((chunk_score_flash<FP8, D, 16>), grid, dim3(256), 0, s, p); break;
  }
}

hipError_t launch_chunk_score(const ScanParams& p, int kv_dtype, hipStream_t s) {
  if (p.G != 4 && p.G != 8 && p.G != 16) return hipErrorInvalidValue;
  if (!flash_rows_fit(p, kv_dtype)) return hipErrorInvalidValue;
  const int nblk = (p.n_tpacks + kChunkPacks - 1) / kChunkPacks;
  // the score pass needs no partials, so its position splits are its own:
  // whole 128-position pieces, about kChunkScoreTargetWgs work items
  ScanParams q = p;
  const int64_t items = (int64_t)p.B * nblk * p.Hkv;
  const int64_t per_item = std::max<int64_t>(1, kChunkScoreTargetWgs / items);
  q.split_len = (int)(((p.N + per_item - 1) / per_item + 127) / 128 * 128);
  q.nsplit = (p.N + q.split_len - 1) / q.split_len;
  const dim3 grid(p.B * nblk * p.Hkv * q.nsplit);
  TimedLaunch tl("chunk_score", s);
  if (kv_dtype == HS2_FP8_E4M3FN) {
    if (p.D == 128) go_chunk_score<true, 128>(q, grid, s);
    else go_chunk_score<true, 64>(q, grid, s);
  } else {
    if (p.D == 128) go_chunk_score<false, 128>(q, grid, s);
    else go_chunk_score<false, 64>(q, grid, s);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, int units, hipStream_t s) {
  TimedLaunch tl("combine", s);
  if (p.nsplit <= kFewSplits && units >= kFewSplitsMinUnits)
    hipLaunchKernelGGL(combine_few, dim3(units), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(combine, dim3(units, p.rows, p.D / 32), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_score(const ScoreParams& p, int units, hipStream_t s, const CombineParams* merge) {
  TimedLaunch tl("score", s);
  if (p.sel_hist) {
    if (p.tpack != 1) return hipErrorInvalidValue;
    // Large grids (the pass is near its memory bound): 4 position groups per
    // thread and one head's loads at a time.  Small grids (latency-bound,
    // fewer workgroups than CUs): 2 groups per thread and, for 8 heads per
    // group, every head's loads at once (measured at 1M: 24.0 against 25.6 us;
    // at 32K: 11.2 against 14.5 us).  With the merge folded in, its
    // rows * D/32 workgroups per unit come first.
    const CombineParams c = merge ? *merge : CombineParams{};
    const int ncomb = merge ? c.rows * (c.D / 32) : 0;
    if (merge && (c.D % 32 || c.nsplit > kMaxSplits)) return hipErrorInvalidValue;
    const int blocks4 = (p.N + 4095) / 4096;
    if ((int64_t)blocks4 * units >= 512 || p.G != 8) {
      if (merge) hipLaunchKernelGGL((score_hist<4, 0, true>), dim3(ncomb + blocks4, units), dim3(256), 0, s, p, c);
      else hipLaunchKernelGGL((score_hist<4, 0, false>), dim3(blocks4, units), dim3(256), 0, s, p, c);
    } else {
      const int blocks2 = (p.N + 2047) / 2048;
      if (merge) hipLaunchKernelGGL((score_hist<2, 8, true>), dim3(ncomb + blocks2, units), dim3(256), 0, s, p, c);
      else hipLaunchKernelGGL((score_hist<2, 8, false>), dim3(blocks2, units), dim3(256), 0, s, p, c);
    }
  } else {
    const int blocks = (p.N + 1023) / 1024;
    hipLaunchKernelGGL(score, dim3(blocks, units), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_scan_read_probe(const ScanParams& p, int kv_dtype, bool codes, hipStream_t s) {
  if (kv_dtype == HS2_F32) return hipErrorInvalidValue;
  const dim3 grid(p.nsplit, p.B * p.n_tpacks * p.Hkv);
  TimedLaunch tl(codes ? "scan_read_probe_codes" : "scan_read_probe", s);
#define HS2_PR(F8, DD)                                                                                  \
  do {                                                                                                  \
    if (codes) hipLaunchKernelGGL((scan_read_probe<F8, DD, true, kScanWaves>), grid, dim3(kScanWaves * 64), 0, s, p); \
    else hipLaunchKernelGGL((scan_read_probe<F8, DD, false, kScanWaves>), grid, dim3(kScanWaves * 64), 0, s, p);      \
  } while (0)
  if (kv_dtype == HS2_FP8_E4M3FN) {
    if (p.D == 128) HS2_PR(true, 128);
    else HS2_PR(true, 64);
  } else {
    if (p.D == 128) HS2_PR(false, 128);
    else HS2_PR(false, 64);
  }
#undef HS2_PR
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* out, int blocks, hipStream_t s) {
  TimedLaunch tl("stream_read", s);
  hipLaunchKernelGGL(stream_read, dim3(blocks), dim3(256), 0, s, (const u32x4_t*)buf, (int64_t)(bytes / 16), out);
  return hipGetLastError();
}

hipError_t launch_debug_e4m3fn(const uint8_t* codes, float* out, int n, hipStream_t s) {
  const int threads = (n + 3) / 4;
  hipLaunchKernelGGL(debug_e4m3fn, dim3((threads + 255) / 256), dim3(256), 0, s, codes, out, n);
  return hipGetLastError();
}

}  // namespace hs2
