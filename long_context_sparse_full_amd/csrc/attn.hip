// Attention kernels of the HySparse2 cross-decoder hot path (gfx950).
//
//  * scan_mfma   -- full layer (split over positions, writes per-head log2
//                   logits for the score pass) and sparse layer (gathered rows,
//                   one workgroup per (b, t, g), final output) for bf16 queries
//                   over bf16 or E4M3FN caches.  QK^T and PV run on
//                   v_mfma_f32_16x16x32_bf16 with positions on the MFMA M side
//                   and up to 16 query rows (the heads of one GQA group) on N.
//  * scan_f32    -- the same two roles for fp32 caches on the VALU (exact fp32).
//  * combine     -- merges the per-split (max, sum, output) partials.
//  * score       -- importance scores: per position, sum over the group's query
//                   heads of the softmax probability, from the stored logits.
//
// The full layer scans every cached position and its attention probabilities
// pick the tokens (javabetter.cn "mimo-v3-hysparse2", first of the two
// changes); the sparse layers attend only to the selected rows of the same
// cache (aitop.news item 35442; javabetter.cn, KV Reuse paragraph).
#include <math.h>

#include "hs2_internal.hpp"

namespace hs2 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2_t v;
  v.x = (__bf16)a;
  v.y = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// four E4M3FN codes (bytes 0..3 of w) -> two dwords of bf16 pairs (exact)
__device__ __forceinline__ void e4m3x4_to_bf16(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  lo = pack_bf16(a.x, a.y);
  hi = pack_bf16(b.x, b.y);
}

__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

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
template <bool FP8, int D, bool GATHER, bool WRITE_LOGITS, int WAVES>
__global__ void __launch_bounds__(WAVES * 64) scan_mfma(ScanParams P) {
  constexpr int NC = D / 32;  // QK MFMAs per 16-position half
  constexpr int VE = D / 16;  // V elements per lane per row = PV MFMA tiles
  __shared__ float sm_m[WAVES][16];
  __shared__ float sm_l[WAVES][16];
  __shared__ float sm_o[WAVES][16][D + 1];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;   // query row (MFMA N index) / V column group
  const int g4 = lane >> 4;  // lane group
  const int unit = blockIdx.y;
  const int split = blockIdx.x;
  const int g = unit % P.Hkv;
  const int tp = (unit / P.Hkv) % P.n_tpacks;
  const int b = unit / (P.Hkv * P.n_tpacks);
  const int tl = r / P.G;
  const int hi = r - tl * P.G;
  const int t = tp * P.tpack + tl;
  const bool row_ok = (r < P.rows) && (t < P.Tq);
  const int h = g * P.G + hi;

  int j_begin, j_end, p_row, p_max;
  const int32_t* list = nullptr;
  if constexpr (GATHER) {
    list = P.idx + (int64_t)unit * P.max_sel;
    j_begin = 0;
    j_end = min(max(P.count[unit], 0), P.max_sel);
    p_row = row_ok ? 0x7fffffff : -1;
    p_max = j_end - 1;
  } else {
    const int t_last = min(tp * P.tpack + P.tpack, P.Tq) - 1;
    p_max = P.q_pos0 + t_last;
    j_begin = split * P.split_len;
    j_end = min(j_begin + P.split_len, p_max + 1);
    p_row = row_ok ? P.q_pos0 + t : -1;
  }
  const int jlim = min(p_row, j_end - 1);

  // query fragments (MFMA B operand of QK^T): row r, head-dim slice dmap(c, g4)
  u32x4_t qf[NC];
  {
    const uint16_t* qb = (const uint16_t*)P.q + (((int64_t)b * P.Tq + (row_ok ? t : 0)) * P.Hq + (row_ok ? h : 0)) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qf[c] = row_ok ? *(const u32x4_t*)(qb + dmap<FP8, D>(c, g4)) : u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  const int64_t kvoff = (int64_t)b * P.sb + (int64_t)g * P.sh;
  float cs = P.scale_log2;
  if constexpr (FP8) cs *= P.k_scale[b * P.Hkv + g];

  float m_run = kNegInf, l_run = 0.f;
  f32x4_t oacc[VE];
#pragma unroll
  for (int dt = 0; dt < VE; ++dt) oacc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int j0 = j_begin + wave * 32; j0 < j_end; j0 += WAVES * 32) {
    // ---- cache rows touched by this lane
    int krow[2], vrow[8];
    if constexpr (GATHER) {
      const int myrow = min(max(list[min(j0 + (lane & 31), j_end - 1)], 0), P.N - 1);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) krow[hh] = __shfl(myrow, 16 * hh + r);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) vrow[kk] = __shfl(myrow, 16 * (kk >> 2) + 4 * g4 + (kk & 3));
    } else {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) krow[hh] = min(j0 + 16 * hh + r, p_max);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) vrow[kk] = min(j0 + 16 * (kk >> 2) + 4 * g4 + (kk & 3), p_max);
    }

    // ---- K rows in the MFMA A layout: row = position (lane % 16), 8 head-dim elements
    u32x4_t kf[2][NC];
    if constexpr (!FP8) {
      const uint16_t* kb = (const uint16_t*)P.k + kvoff;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int c = 0; c < NC; ++c)
          kf[hh][c] = *(const u32x4_t*)(kb + (int64_t)krow[hh] * P.sn + dmap<FP8, D>(c, g4));
    } else {
      const uint8_t* kb = (const uint8_t*)P.k + kvoff;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int ii = 0; ii < NC / 2; ++ii) {
          const u32x4_t raw = *(const u32x4_t*)(kb + (int64_t)krow[hh] * P.sn + 64 * ii + 16 * g4);
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

    // ---- V rows: lane holds VE consecutive head-dim elements (VE*r ..) of 8 rows
    uint32_t vd[8][VE / 2];
    if constexpr (!FP8) {
      const uint16_t* vb = (const uint16_t*)P.v + kvoff + VE * r;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        if constexpr (VE == 8) {
          const u32x4_t w = *(const u32x4_t*)(vb + (int64_t)vrow[kk] * P.sn);
          vd[kk][0] = w.x; vd[kk][1] = w.y; vd[kk][2] = w.z; vd[kk][3] = w.w;
        } else {
          const u32x2_t w = *(const u32x2_t*)(vb + (int64_t)vrow[kk] * P.sn);
          vd[kk][0] = w.x; vd[kk][1] = w.y;
        }
      }
    } else {
      const uint8_t* vb = (const uint8_t*)P.v + kvoff + VE * r;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        if constexpr (VE == 8) {
          const u32x2_t w = *(const u32x2_t*)(vb + (int64_t)vrow[kk] * P.sn);
          e4m3x4_to_bf16(w.x, vd[kk][0], vd[kk][1]);
          e4m3x4_to_bf16(w.y, vd[kk][2], vd[kk][3]);
        } else {
          const uint32_t w = *(const uint32_t*)(vb + (int64_t)vrow[kk] * P.sn);
          e4m3x4_to_bf16(w, vd[kk][0], vd[kk][1]);
        }
      }
    }

    // ---- logits S^T[position][row]: lane holds row r at positions j0+16hh+4g4+ii
    f32x4_t s[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      s[hh] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) s[hh] = mfma_bf16(kf[hh][c], qf[c], s[hh]);
    }
    float x[2][4];
    float tmax = kNegInf;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int j = j0 + 16 * hh + 4 * g4 + ii;
        const float xv = (j <= jlim) ? s[hh][ii] * cs : kNegInf;
        x[hh][ii] = xv;
        tmax = fmaxf(tmax, xv);
      }
    if constexpr (WRITE_LOGITS) {
      if (row_ok) {
        float* lg = P.logits + ((int64_t)unit * P.rows + r) * P.npad + j0 + 4 * g4;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          *(f32x4_t*)(lg + 16 * hh) = f32x4_t{x[hh][0], x[hh][1], x[hh][2], x[hh][3]};
      }
    }

    // ---- online softmax (log2 domain); the 4 lanes of one row agree on m
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_new == m_run) ? 1.f : exp2_fast(m_run - m_new);
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
    l_run = l_run * alpha + psum;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < VE; ++dt) oacc[dt] *= alpha;
    }
    m_run = m_new;

    // ---- PV: O^T[d][row] += V^T[d][pos] P^T[pos][row]
    // P^T operand: k-slot kk of lane group g4 <-> position 16*(kk>>2) + 4*g4 + (kk&3)
    const u32x4_t pf = u32x4_t{pack_bf16(pr[0][0], pr[0][1]), pack_bf16(pr[0][2], pr[0][3]),
                               pack_bf16(pr[1][0], pr[1][1]), pack_bf16(pr[1][2], pr[1][3])};
#pragma unroll
    for (int dt = 0; dt < VE; ++dt) {
      const int w = dt >> 1;
      u32x4_t va;
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        const uint32_t e0 = vd[2 * q2][w], e1 = vd[2 * q2 + 1][w];
        va[q2] = (dt & 1) ? ((e0 >> 16) | (e1 & 0xffff0000u)) : ((e0 & 0xffffu) | (e1 << 16));
      }
      oacc[dt] = mfma_bf16(va, pf, oacc[dt]);
    }
  }

  // ---- merge the waves of this workgroup
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (g4 == 0) {
    sm_m[wave][r] = m_run;
    sm_l[wave][r] = l_run;
  }
#pragma unroll
  for (int dt = 0; dt < VE; ++dt)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) sm_o[wave][r][VE * (4 * g4 + ii) + dt] = oacc[dt][ii];
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
      // unit = (b, t, g); rows = G heads of token t
      const int tt = (unit / P.Hkv) % P.Tq;
      const int hh = g * P.G + rr;
      float o = (L > 0.f) ? O / L : 0.f;
      if constexpr (FP8) o *= P.v_scale[b * P.Hkv + g];
      const int64_t orow = ((int64_t)b * P.Tq + tt) * P.Hq + hh;
      ((__bf16*)P.out)[orow * D + d] = (__bf16)o;
      if (d == 0 && P.lse) P.lse[orow] = (L > 0.f) ? (M + log2f(L)) * kLn2 : kNegInf;
    } else {
      const int64_t pbase = ((int64_t)unit * P.nsplit + split) * 16 + rr;
      P.part_o[pbase * D + d] = O;
      if (d == 0) {
        P.part_ml[pbase * 2] = M;
        P.part_ml[pbase * 2 + 1] = L;
      }
    }
  }
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
  const int p = P.q_pos0 + t;

  int j_begin, j_end;
  const int32_t* list = nullptr;
  if constexpr (GATHER) {
    list = P.idx + (int64_t)unit * P.max_sel;
    j_begin = 0;
    j_end = min(max(P.count[unit], 0), P.max_sel);
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
    if (tid < TJ) s_rows[tid] = GATHER ? min(max(list[min(j0 + tid, j_end - 1)], 0), P.N - 1) : min(j0 + tid, j_end - 1);
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
      if (r < R) {
        float* lg = P.logits + ((int64_t)unit * P.rows + r) * P.npad + j0;
#pragma unroll
        for (int s = 0; s < 4; ++s)
          if (c + 16 * s < nt) lg[c + 16 * s] = x[s];
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
__global__ void combine(CombineParams P) {
  const int unit = blockIdx.x, r = blockIdx.y, d = threadIdx.x;
  const int g = unit % P.Hkv;
  const int tp = (unit / P.Hkv) % P.n_tpacks;
  const int b = unit / (P.Hkv * P.n_tpacks);
  const int tl = r / P.G, i = r - tl * P.G;
  const int t = tp * P.tpack + tl;
  if (t >= P.Tq) return;
  const int h = g * P.G + i;
  const float* ml = P.part_ml + ((int64_t)unit * P.nsplit * 16 + r) * 2;
  const float* po = P.part_o + ((int64_t)unit * P.nsplit * 16 + r) * P.D + d;
  float M = kNegInf;
  for (int s = 0; s < P.nsplit; ++s) M = fmaxf(M, ml[s * 32]);
  const float Ms = (M == kNegInf) ? 0.f : M;
  float L = 0.f, O = 0.f;
  for (int s = 0; s < P.nsplit; ++s) {
    const float f = exp2f(ml[s * 32] - Ms);
    L += ml[s * 32 + 1] * f;
    O += po[(int64_t)s * 16 * P.D] * f;
  }
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

// ---------------------------------------------------------------------------
// scores[b,t,g,j] = sum_{heads of g} 2^(x_hj - lse2_h) for j <= p, 0 beyond
// ---------------------------------------------------------------------------
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
    const int p = P.q_pos0 + t;
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    if (j4 <= p) {
      for (int i = 0; i < P.G; ++i) {
        const int r = tl * P.G + i;
        const float l2 = P.lse2[(int64_t)unit * P.rows + r];
        const f32x4_t x = *(const f32x4_t*)(P.logits + ((int64_t)unit * P.rows + r) * P.npad + j4);
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] += exp2f(x[e] - l2);
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

template <bool FP8, int D, bool GATHER, bool WL, int WAVES>
hipError_t go_mfma(const ScanParams& p, dim3 grid, hipStream_t s, const char* name) {
  TimedLaunch tl(name, s);
  hipLaunchKernelGGL((scan_mfma<FP8, D, GATHER, WL, WAVES>), grid, dim3(WAVES * 64), 0, s, p);
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
constexpr int kGatherWaves = 8;

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
#define HS2_GO(F8, DD)                                                                         \
  do {                                                                                         \
    if (gather) return go_mfma<F8, DD, true, false, kGatherWaves>(p, grid, s, name);           \
    if (write_logits) return go_mfma<F8, DD, false, true, kScanWaves>(p, grid, s, name);       \
    return go_mfma<F8, DD, false, false, kScanWaves>(p, grid, s, name);                        \
  } while (0)
  if (fp8) {
    if (p.D == 128) HS2_GO(true, 128);
    HS2_GO(true, 64);
  }
  if (p.D == 128) HS2_GO(false, 128);
  HS2_GO(false, 64);
#undef HS2_GO
}

hipError_t launch_combine(const CombineParams& p, int units, hipStream_t s) {
  TimedLaunch tl("combine", s);
  hipLaunchKernelGGL(combine, dim3(units, p.rows), dim3(p.D), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_score(const ScoreParams& p, int units, hipStream_t s) {
  TimedLaunch tl("score", s);
  const int blocks = (p.N + 1023) / 1024;
  hipLaunchKernelGGL(score, dim3(blocks, units), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_debug_e4m3fn(const uint8_t* codes, float* out, int n, hipStream_t s) {
  const int threads = (n + 3) / 4;
  hipLaunchKernelGGL(debug_e4m3fn, dim3((threads + 255) / 256), dim3(256), 0, s, codes, out, n);
  return hipGetLastError();
}

}  // namespace hs2
