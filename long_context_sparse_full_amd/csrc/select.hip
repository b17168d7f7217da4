// Selection kernels of the HySparse2 cross-decoder hot path (gfx950).
//
// Token mode: the k highest-scoring positions of C = [0, p - window] (ties to
// the lower position) united with the forced window [p - window + 1, p], in
// ascending order (zgeo.com.cn "xiaomi-mimo-v3-hysparse2-long-context-geo",
// "core principle": 1024 global tokens plus the 128 most recent kept by force;
// javabetter.cn "mimo-v3-hysparse2", the two changes versus HySparse).
//
// The k-th largest score is found exactly by a radix select over the 32-bit
// patterns of the non-negative fp32 scores (their unsigned order is their
// numeric order): digits of 12, 12 and 8 bits, each pass a histogram of the
// keys that share the digits found so far.  Histograms use integer atomics
// only, so every count -- and therefore the selection -- is deterministic.
// The emit pass keeps every key above the threshold and the lowest-positioned
// keys equal to it, compacted in ascending position order.
//
// Block mode (block_size > 1) is the previous generation's 64-token block
// selection (zgeo.com.cn comparison table): block mass = fp64 sum of its
// scores over C in ascending position, heaviest blocks first, ties to the
// lower block.
#include "hs2_internal.hpp"

namespace hs2 {
namespace {

// per-unit state; each pass reads the slots of the previous kernel and writes
// its own, so no kernel reads a slot that a sibling workgroup is writing
enum { ST_MODE = 0, ST_NCAND = 1, ST_TAKE = 2, ST_P = 3, ST_PREFIX1 = 4, ST_NEED1 = 5,
       ST_PREFIX2 = 6, ST_NEED2 = 7, ST_WORDS = 16 };
enum { MODE_RADIX = 0, MODE_ALL = 1, MODE_NONE = 2 };

__device__ __forceinline__ uint32_t score_key(float s) {
  const uint32_t u = __float_as_uint(s);
  return u == 0x80000000u ? 0u : u;  // -0 orders as +0
}

template <typename T>
__device__ __forceinline__ T block_exclusive_scan(T v, T* sm, T& total) {
  // 256 threads; sm has >= 256 + 8 slots
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  T x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sm[256 + wave] = x;
  __syncthreads();
  T wbase = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const T s = sm[256 + w];
    if (w < wave) wbase += s;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return wbase + x - v;
}

__global__ void __launch_bounds__(256) sel_init(SelectParams P) {
  const int u = blockIdx.x;
  const int t = (u / P.Hkv) % P.Tq;
  const int p = P.q_pos0 + t;
  const int ncand = max(0, p - P.window + 1);
  int take;
  if (P.block_size == 1) {
    take = min(P.k, ncand);
  } else {
    const int nb = ncand > 0 ? (ncand - 1) / P.block_size + 1 : 0;
    take = min(P.k, nb);
  }
  if (threadIdx.x == 0) {
    int32_t* st = P.state + (int64_t)u * ST_WORDS;
    st[ST_MODE] = (take == 0) ? MODE_NONE : ((P.block_size == 1 && take == ncand) ? MODE_ALL : MODE_RADIX);
    st[ST_NCAND] = ncand;
    st[ST_TAKE] = take;
    st[ST_P] = p;
  }
  if (P.block_size == 1) {
    int32_t* h = P.hist + (int64_t)u * 3 * kHistBins;
    for (int i = threadIdx.x; i < 3 * kHistBins; i += 256) h[i] = 0;
  }
}

// digits: pass 0 = bits 31..20, pass 1 = bits 19..8, pass 2 = bits 7..0
template <int PASS>
struct Digit {
  static constexpr int SHIFT = PASS == 0 ? 20 : (PASS == 1 ? 8 : 0);
  static constexpr int BINS = PASS == 2 ? 256 : 4096;
  static constexpr uint32_t MATCH = PASS == 0 ? 0u : (PASS == 1 ? 0xFFF00000u : 0xFFFFFF00u);
};

// Whole-block search of a digit histogram (counts of the keys that share the
// digits found so far): the digit d* holding the need-th largest key, and the
// number of keys in higher digits.  Thread T owns the BINS/256 digits just
// below BINS - T*BINS/256, so a forward scan over threads runs from the top.
template <int PASS>
__device__ void find_digit(const int32_t* gh, int need, int32_t* sm, int& digit, int& above_out) {
  constexpr int BINS = Digit<PASS>::BINS, BPT = BINS / 256;
  __shared__ int32_t s_digit, s_above;
  const int T = threadIdx.x;
  const int hi_d = BINS - T * BPT - 1;
  int32_t c[BPT];
  int32_t mine = 0;
#pragma unroll
  for (int e = 0; e < BPT; ++e) {
    c[e] = gh[hi_d - e];
    mine += c[e];
  }
  int32_t total;
  const int32_t above = block_exclusive_scan<int32_t>(mine, sm, total);
  if (above < need && need <= above + mine) {
    int32_t a = above;
#pragma unroll
    for (int e = 0; e < BPT; ++e) {
      if (a < need && need <= a + c[e]) {
        s_digit = hi_d - e;
        s_above = a;
      }
      a += c[e];
    }
  }
  __syncthreads();
  digit = s_digit;
  above_out = s_above;
  __syncthreads();
}

// The 64 candidate keys of this thread in one chunk, all loads issued at once:
// positions base + 4*(tid + 256*i) + e, i < 16, e < 4 (coalesced 16-byte
// loads when the row allows them).  Keys of positions >= end are flagged.
constexpr int kKeysPerThread = kSelChunk / 256;
struct ChunkKeys {
  uint32_t key[kKeysPerThread];
  uint64_t valid;  // bit 4*i + e
};

__device__ __forceinline__ void load_keys(const float* s, int base, int end, bool vec_ok, ChunkKeys& K) {
  K.valid = 0;
#pragma unroll
  for (int i = 0; i < kKeysPerThread / 4; ++i) {
    const int j = base + 4 * (threadIdx.x + 256 * i);
    if (vec_ok && j + 3 < end) {
      const float4 v = *(const float4*)(s + j);
      K.key[4 * i] = score_key(v.x);
      K.key[4 * i + 1] = score_key(v.y);
      K.key[4 * i + 2] = score_key(v.z);
      K.key[4 * i + 3] = score_key(v.w);
      K.valid |= (uint64_t)0xF << (4 * i);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = j + e < end;
        K.key[4 * i + e] = ok ? score_key(s[j + e]) : 0u;
        K.valid |= (uint64_t)ok << (4 * i + e);
      }
    }
  }
}

// LDS histogram of one digit over the keys that match `prefix`.  PASS 0 keys
// cluster in a few bins (the scores of one row share exponent and leading
// mantissa bits), so each thread counts some bins in registers and sends only
// the other keys to the (contended) LDS atomics.  SHORT (grids that do not
// fill the GPU several times over, whose passes are latency-bound): the bin of
// the thread's first key, counted with no branches.  Otherwise (throughput-
// bound grids): the first two bins the thread meets, fewer LDS atomics for a
// longer dependent chain.
template <int PASS, bool SHORT>
__device__ __forceinline__ void hist_keys(const ChunkKeys& K, uint32_t prefix, int32_t* h) {
  using DG = Digit<PASS>;
  if constexpr (PASS == 0 && SHORT) {
    const uint32_t b1 = K.key[0] >> DG::SHIFT;  // (key 0 may be a padding 0: only register hits lost)
    int32_t c1 = 0;
#pragma unroll
    for (int i = 0; i < kKeysPerThread; ++i) {
      const bool v = K.valid >> i & 1;
      const uint32_t bin = K.key[i] >> DG::SHIFT;
      const bool hit = v && bin == b1;
      c1 += hit;
      if (v && !hit) atomicAdd(&h[bin], 1);
    }
    if (c1) atomicAdd(&h[b1], c1);
  } else if constexpr (PASS == 0) {
    uint32_t b1 = 0xffffffffu, b2 = 0xffffffffu;
    int32_t c1 = 0, c2 = 0;
#pragma unroll
    for (int i = 0; i < kKeysPerThread; ++i) {
      if (!(K.valid >> i & 1)) continue;
      const uint32_t bin = K.key[i] >> DG::SHIFT;
      if (bin == b1) {
        ++c1;
      } else if (bin == b2) {
        ++c2;
      } else if (c1 == 0) {
        b1 = bin;
        c1 = 1;
      } else if (c2 == 0) {
        b2 = bin;
        c2 = 1;
      } else {
        atomicAdd(&h[bin], 1);
      }
    }
    if (c1) atomicAdd(&h[b1], c1);
    if (c2) atomicAdd(&h[b2], c2);
  } else {
#pragma unroll
    for (int i = 0; i < kKeysPerThread; ++i)
      if ((K.valid >> i & 1) && (K.key[i] & DG::MATCH) == prefix) atomicAdd(&h[(K.key[i] >> DG::SHIFT) & (DG::BINS - 1)], 1);
  }
}

// PASS 0 histograms all candidates; PASS 1 and 2 first settle the previous
// digit (every workgroup computes it while its loads are in flight; chunk 0
// records it) and histogram the keys that share the digits found so far.
// PASS 2 also stores, per chunk, the count of keys above the 24-bit prefix and
// the suffix sums of its 256-bin histogram, from which the emit pass gets every
// chunk's counts above and equal to the final threshold.
template <int PASS, bool SHORT>
__global__ void __launch_bounds__(256) sel_hist(SelectParams P) {
  using DG = Digit<PASS>;
  __shared__ int32_t h[DG::BINS];
  __shared__ int32_t sm[264];
  const int u = blockIdx.y, chunk = blockIdx.x;
  int32_t* st = P.state + (int64_t)u * ST_WORDS;
  if (st[ST_MODE] != MODE_RADIX) return;
  const int ncand = st[ST_NCAND];
  const int base = chunk * kSelChunk;
  if (base >= ncand) return;
  const int end = min(base + kSelChunk, ncand);
  ChunkKeys K;
  load_keys(P.scores + (int64_t)u * P.N, base, end, (P.N & 3) == 0, K);
  int32_t* hist = P.hist + (int64_t)u * 3 * kHistBins;
  uint32_t prefix = 0;
  if constexpr (PASS > 0) {
    // the previous pass's digit; inputs are what the kernel before wrote
    const uint32_t prev = PASS == 1 ? 0u : (uint32_t)st[ST_PREFIX1];
    int need = PASS == 1 ? st[ST_TAKE] : st[ST_NEED1];
    int d, above;
    find_digit<PASS - 1>(hist + (PASS - 1) * kHistBins, need, sm, d, above);
    prefix = prev | ((uint32_t)d << Digit<PASS - 1>::SHIFT);
    need -= above;
    if (chunk == 0 && threadIdx.x == 0) {
      st[PASS == 1 ? ST_PREFIX1 : ST_PREFIX2] = (int32_t)prefix;
      st[PASS == 1 ? ST_NEED1 : ST_NEED2] = need;
    }
  }
  for (int i = threadIdx.x; i < DG::BINS; i += 256) h[i] = 0;
  __syncthreads();
  hist_keys<PASS, SHORT>(K, prefix, h);
  __syncthreads();
  int32_t* gh = hist + PASS * kHistBins;
  for (int i = threadIdx.x; i < DG::BINS; i += 256)
    if (h[i]) atomicAdd(&gh[i], h[i]);
  if constexpr (PASS == 2) {
    int32_t above24 = 0;
#pragma unroll
    for (int i = 0; i < kKeysPerThread; ++i) above24 += (K.valid >> i & 1) && (K.key[i] >> 8) > (prefix >> 8);
    int32_t tot;
    block_exclusive_scan<int32_t>(above24, sm, tot);
    // suffix sums: thread T holds digit 255 - T; scan from the top digit
    const int32_t cnt = h[255 - threadIdx.x];
    int32_t dummy;
    const int32_t suf_excl = block_exclusive_scan<int32_t>(cnt, sm, dummy);
    int32_t* cs = P.cnt + ((int64_t)u * P.nchunks + chunk) * 258;
    cs[1 + (255 - threadIdx.x)] = suf_excl + cnt;  // keys with digit >= 255-T
    if (threadIdx.x == 0) {
      cs[0] = tot;
      cs[257] = 0;  // suffix beyond the top digit
    }
  }
}

// Ascending compaction: every key above tau and the lowest-positioned keys
// equal to tau (tau and their number from the last digit's histogram), then
// (chunk 0) the forced window, the count and the padding.
__global__ void __launch_bounds__(256) sel_emit(SelectParams P) {
  __shared__ int32_t sm[264];
  const int u = blockIdx.y, chunk = blockIdx.x;
  const int32_t* st = P.state + (int64_t)u * ST_WORDS;
  const int mode = st[ST_MODE];
  const int ncand = st[ST_NCAND];
  const int take = st[ST_TAKE];
  const int p = st[ST_P];
  int32_t* out = P.idx + (int64_t)u * P.max_sel;

  if (chunk == 0) {
    const int wlo = max(0, p - P.window + 1);
    const int nw = p - wlo + 1;
    for (int i = threadIdx.x; i < nw; i += 256) out[take + i] = wlo + i;
    for (int i = take + nw + threadIdx.x; i < P.max_sel; i += 256) out[i] = -1;
    if (threadIdx.x == 0) P.count[u] = take + nw;
  }
  if (mode == MODE_NONE) return;
  const int base = chunk * kSelChunk;
  if (base >= ncand) return;
  const int end = min(base + kSelChunk, ncand);
  if (mode == MODE_ALL) {
    for (int j = base + threadIdx.x; j < end; j += 256) out[j] = j;
    return;
  }
  // this chunk's keys, 16 consecutive positions per thread per round of 4096
  const float* s = P.scores + (int64_t)u * P.N;
  const bool vec_ok = (P.N & 3) == 0;
  uint32_t keys[kKeysPerThread];
#pragma unroll
  for (int rnd = 0; rnd < 4; ++rnd) {
    const int j0 = base + rnd * 4096 + threadIdx.x * 16;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = j0 + 4 * q;
      if (vec_ok && j + 3 < end) {
        const float4 v = *(const float4*)(s + j);
        keys[rnd * 16 + 4 * q] = score_key(v.x);
        keys[rnd * 16 + 4 * q + 1] = score_key(v.y);
        keys[rnd * 16 + 4 * q + 2] = score_key(v.z);
        keys[rnd * 16 + 4 * q + 3] = score_key(v.w);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) keys[rnd * 16 + 4 * q + e] = (j + e < end) ? score_key(s[j + e]) : 0u;
      }
    }
  }
  // final digit, threshold tau and how many keys equal to it are taken
  int d, above;
  find_digit<2>(P.hist + ((int64_t)u * 3 + 2) * kHistBins, st[ST_NEED2], sm, d, above);
  const uint32_t tau = (uint32_t)st[ST_PREFIX2] | (uint32_t)d;
  const int need = st[ST_NEED2] - above;
  // counts of all earlier chunks: above tau = above the 24-bit prefix + digits > d
  int32_t eq_before = 0, sel_before = 0;
  for (int c0 = 0; c0 < chunk; c0 += 256) {
    const int c = c0 + threadIdx.x;
    int32_t gt = 0, eq = 0;
    if (c < chunk) {
      const int32_t* cs = P.cnt + ((int64_t)u * P.nchunks + c) * 258;
      const int32_t suf_d = cs[1 + d], suf_d1 = cs[2 + d];
      gt = cs[0] + suf_d1;
      eq = suf_d - suf_d1;
    }
    int32_t eq_tot;
    const int32_t eqb = eq_before + block_exclusive_scan<int32_t>(eq, sm, eq_tot);
    const int32_t sel = gt + max(0, min(need - eqb, eq));
    int32_t sel_tot;
    block_exclusive_scan<int32_t>(sel, sm, sel_tot);
    eq_before += eq_tot;
    sel_before += sel_tot;
  }
  int32_t eq_rank = eq_before, slot = sel_before;
#pragma unroll
  for (int rnd = 0; rnd < 4; ++rnd) {
    const int j0 = base + rnd * 4096 + threadIdx.x * 16;
    int32_t my_eq = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) my_eq += (j0 + e < end) && keys[rnd * 16 + e] == tau;
    int32_t teq;
    int32_t r_eq = eq_rank + block_exclusive_scan<int32_t>(my_eq, sm, teq);
    uint32_t selmask = 0;
    int32_t my_sel = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t key = keys[rnd * 16 + e];
      bool take_it = false;
      if (j0 + e < end) {
        if (key > tau) {
          take_it = true;
        } else if (key == tau) {
          take_it = r_eq < need;
          ++r_eq;
        }
      }
      selmask |= (uint32_t)take_it << e;
      my_sel += take_it;
    }
    int32_t tsel;
    int32_t sl = slot + block_exclusive_scan<int32_t>(my_sel, sm, tsel);
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (selmask >> e & 1u) {
        if (sl < take) out[sl] = j0 + e;  // never past this unit's budget
        ++sl;
      }
    eq_rank += teq;
    slot += tsel;
  }
}

// ---------------------------------------------------------------------------
// block baseline
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) sel_block_mass(SelectParams P) {
  const int u = blockIdx.y;
  const int beta = blockIdx.x * 256 + threadIdx.x;
  const int32_t* st = P.state + (int64_t)u * ST_WORDS;
  const int ncand = st[ST_NCAND];
  const int nb = ncand > 0 ? (ncand - 1) / P.block_size + 1 : 0;
  if (beta >= nb) return;
  const float* s = P.scores + (int64_t)u * P.N;
  const int lo = beta * P.block_size;
  const int hi = min(lo + P.block_size, ncand);
  // ascending-position fp64 sum; loads issued 16 at a time
  double m = 0.0;
  int j = lo;
  for (; j + 16 <= hi; j += 16) {
    float v[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = s[j + e];
#pragma unroll
    for (int e = 0; e < 16; ++e) m += (double)v[e];
  }
  for (; j < hi; ++j) m += (double)s[j];
  P.bmass[(int64_t)u * P.nblocks_max + beta] = m;
}

__global__ void __launch_bounds__(256) sel_block_pick(SelectParams P) {
  __shared__ double s_m[256];
  __shared__ int s_b[256];
  __shared__ int32_t sm[264];
  const int u = blockIdx.x;
  const int32_t* st = P.state + (int64_t)u * ST_WORDS;
  const int ncand = st[ST_NCAND];
  const int take = st[ST_TAKE];
  const int p = st[ST_P];
  const int nb = ncand > 0 ? (ncand - 1) / P.block_size + 1 : 0;
  double* bm = P.bmass + (int64_t)u * P.nblocks_max;
  int32_t* out = P.idx + (int64_t)u * P.max_sel;
  // take rounds of (mass desc, block asc) argmax; a taken block's mass becomes -1
  for (int round = 0; round < take; ++round) {
    double best = -1.0;
    int bb = 0x7fffffff;
    for (int beta = threadIdx.x; beta < nb; beta += 256) {
      const double m = bm[beta];
      if (m > best || (m == best && beta < bb)) {
        best = m;
        bb = beta;
      }
    }
    s_m[threadIdx.x] = best;
    s_b[threadIdx.x] = bb;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (threadIdx.x < o) {
        const double m2 = s_m[threadIdx.x + o];
        const int b2 = s_b[threadIdx.x + o];
        if (m2 > s_m[threadIdx.x] || (m2 == s_m[threadIdx.x] && b2 < s_b[threadIdx.x])) {
          s_m[threadIdx.x] = m2;
          s_b[threadIdx.x] = b2;
        }
      }
      __syncthreads();
    }
    if (threadIdx.x == 0) bm[s_b[0]] = -1.0;
    __syncthreads();
  }
  // ascending emit of the taken blocks' candidate positions
  int32_t written = 0;
  for (int b0 = 0; b0 < nb; b0 += 256) {
    const int beta = b0 + threadIdx.x;
    int32_t n = 0;
    if (beta < nb && bm[beta] == -1.0) n = min(beta * P.block_size + P.block_size, ncand) - beta * P.block_size;
    int32_t tot;
    const int32_t off = written + block_exclusive_scan<int32_t>(n, sm, tot);
    for (int e = 0; e < n && off + e < P.max_sel; ++e) out[off + e] = beta * P.block_size + e;
    written += tot;
  }
  const int wlo = max(0, p - P.window + 1);
  const int nw = p - wlo + 1;
  for (int i = threadIdx.x; i < nw && written + i < P.max_sel; i += 256) out[written + i] = wlo + i;
  for (int i = written + nw + threadIdx.x; i < P.max_sel; i += 256) out[i] = -1;
  if (threadIdx.x == 0) P.count[u] = written + nw;
}

}  // namespace

hipError_t launch_select(const SelectParams& p, hipStream_t s) {
  const dim3 grid_c(p.nchunks, p.units);
  hipError_t e;
#define HS2_L(name, kern, grid)                                   \
  do {                                                            \
    TimedLaunch tl_(name, s);                                     \
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, p);           \
    if ((e = hipGetLastError()) != hipSuccess) return e;          \
  } while (0)
  HS2_L("select_init", sel_init, dim3(p.units));
  if (p.block_size == 1) {
    if (p.units * p.nchunks < 2048) {  // latency-bound passes
      HS2_L("select_hist", (sel_hist<0, true>), grid_c);
    } else {
      HS2_L("select_hist", (sel_hist<0, false>), grid_c);
    }
    HS2_L("select_hist", (sel_hist<1, false>), grid_c);
    HS2_L("select_hist", (sel_hist<2, false>), grid_c);
    HS2_L("select_emit", sel_emit, grid_c);
  } else {
    HS2_L("select_block_mass", sel_block_mass, dim3((p.nblocks_max + 255) / 256, p.units));
    HS2_L("select_block_pick", sel_block_pick, dim3(p.units));
  }
#undef HS2_L
  return hipSuccess;
}

}  // namespace hs2
