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
// Bracketed path (grids of many rows, where the passes are throughput-bound):
// a fixed sample of each row -- every SR-th run of 64 positions, at most
// 16384 keys -- gives the sample's keys of ranks r -/+ m around the expected
// rank r of the k-th key (m = 4 sqrt(r) + 8), to 24 bits by a two-digit radix
// on chip.  One pass over the scores then collects the keys above the upper
// bound (all taken) and the keys between the bounds, with exact counts, and
// one workgroup per row finds the k-th key among the latter by a radix select
// on chip and writes the taken positions in ascending order.  The
// counts show whether the bracket holds the k-th key; a row where it does not
// (an unrepresentative sample, heavy ties, k above the lists' size) is done
// by one workgroup running the plain radix select over that row alone.  Every
// row's result is the exact selection either way; the sample only decides
// which of the two exact routes a row takes.
//
// Block mode (block_size > 1) is the previous generation's 64-token block
// selection (zgeo.com.cn comparison table): block mass = fp64 sum of its
// scores over C in ascending position, heaviest blocks first, ties to the
// lower block.
#include <type_traits>

#include "hs2_internal.hpp"
#include "select_common.hpp"

namespace hs2 {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Inclusive prefix sum over the 64 lanes of a wave by DPP moves: shifts of
// 1, 2, 4 and 8 lanes within each row of 16 (lanes shifted in from outside the
// row add 0), then the last lane of row 0 / row 2 added to rows 1 / 3 and the
// last lane of row 1 added to rows 2 and 3.
__device__ __forceinline__ int32_t wave_inclusive_scan(int32_t x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// Exclusive prefix sums over the 256 threads of a workgroup of N values per
// thread at once (one pair of barriers); total[k] = sum of v[k] over the
// workgroup.  sm has >= 256 + 4 * N slots.
template <int N>
__device__ __forceinline__ void block_exclusive_scan_n(int32_t (&v)[N], int32_t* sm, int32_t (&total)[N]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t x[N];
#pragma unroll
  for (int k = 0; k < N; ++k) x[k] = wave_inclusive_scan(v[k]);
  if (lane == 63) {
#pragma unroll
    for (int k = 0; k < N; ++k) sm[256 + 4 * k + wave] = x[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < N; ++k) {
    int32_t wbase = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int32_t s = sm[256 + 4 * k + w];
      if (w < wave) wbase += s;
      tot += s;
    }
    total[k] = tot;
    v[k] = wbase + x[k] - v[k];
  }
  __syncthreads();
}

template <typename T>
__device__ __forceinline__ T block_exclusive_scan(T v, T* sm, T& total) {
  static_assert(sizeof(T) == 4, "32-bit scan");
  int32_t a[1] = {(int32_t)v}, t[1];
  block_exclusive_scan_n<1>(a, (int32_t*)sm, t);
  total = (T)t[0];
  return (T)a[0];
}

// Query position of selection row u = (b, t, g).
__device__ __forceinline__ int row_pos(const SelectParams& P, int u) {
  return qpos_of(P.qpos_b, P.q_pos0, u / (P.Hkv * P.Tq), P.N, P.Tq) + (u / P.Hkv) % P.Tq;
}

__global__ void __launch_bounds__(256) sel_init(SelectParams P) {
  const int u = blockIdx.x;
  const int t = (u / P.Hkv) % P.Tq;
  sel_init_row(P.state + (int64_t)u * ST_WORDS, P.block_size == 1 ? P.hist + (int64_t)u * 3 * kHistBins : nullptr,
               qpos_of(P.qpos_b, P.q_pos0, u / (P.Hkv * P.Tq), P.N, P.Tq) + t, P.k, P.cand_window, P.block_size,
               threadIdx.x, 256);
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
__device__ void find_digit(const int32_t* gh, int need, int32_t* sm, int& digit, int& above_out,
                           int* count_out = nullptr) {
  constexpr int BINS = Digit<PASS>::BINS, BPT = BINS / 256;
  __shared__ int32_t s_digit, s_above, s_count;
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
        s_count = c[e];
      }
      a += c[e];
    }
  }
  __syncthreads();
  digit = s_digit;
  above_out = s_above;
  if (count_out) *count_out = s_count;
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

__device__ __forceinline__ void load_keys_first(const float* s, int base, int end, bool vec_ok, ChunkKeys& K) {
  // Every load is issued before any key is formed (a conversion right after
  // its own load makes each load wait for the previous one): measured faster
  // for the collecting pass, and for the histogram passes on small grids.
  float4 v[kKeysPerThread / 4];
  if (vec_ok && end - base == kSelChunk) {  // whole chunk (workgroup-uniform): unguarded 16-byte loads
#pragma unroll
    for (int i = 0; i < kKeysPerThread / 4; ++i) v[i] = *(const float4*)(s + base + 4 * (threadIdx.x + 256 * i));
    K.valid = ~0ull;
  } else {
    K.valid = 0;
#pragma unroll
    for (int i = 0; i < kKeysPerThread / 4; ++i) {
      const int j = base + 4 * (threadIdx.x + 256 * i);
      v[i].x = j < end ? s[j] : 0.f;
      v[i].y = j + 1 < end ? s[j + 1] : 0.f;
      v[i].z = j + 2 < end ? s[j + 2] : 0.f;
      v[i].w = j + 3 < end ? s[j + 3] : 0.f;
      const uint64_t nv = (uint64_t)min(max(end - j, 0), 4);
      K.valid |= ((1ull << nv) - 1) << (4 * i);
    }
  }
#pragma unroll
  for (int i = 0; i < kKeysPerThread / 4; ++i) {
    K.key[4 * i] = score_key(v[i].x);
    K.key[4 * i + 1] = score_key(v[i].y);
    K.key[4 * i + 2] = score_key(v[i].z);
    K.key[4 * i + 3] = score_key(v[i].w);
  }
}

// Keys converted as their loads return: measured faster for the histogram
// passes on large grids (by 10% at 2048 rows x 128K scores).
__device__ __forceinline__ void load_keys_inline(const float* s, int base, int end, bool vec_ok, ChunkKeys& K) {
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

// The chunk's keys in runs of 16 consecutive positions: key 16*r + e at
// position base + 4096*r + 16*threadIdx.x + e (r < 4), so the thread order is
// the position order within each quarter of the chunk.
__device__ __forceinline__ void load_keys_runs(const float* s, int base, int end, bool vec_ok, ChunkKeys& K) {
  K.valid = 0;
#pragma unroll
  for (int rnd = 0; rnd < 4; ++rnd) {
    const int j0 = base + rnd * 4096 + threadIdx.x * 16;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = j0 + 4 * q, i = rnd * 16 + 4 * q;
      if (vec_ok && j + 3 < end) {
        const float4 v = *(const float4*)(s + j);
        K.key[i] = score_key(v.x);
        K.key[i + 1] = score_key(v.y);
        K.key[i + 2] = score_key(v.z);
        K.key[i + 3] = score_key(v.w);
        K.valid |= (uint64_t)0xF << i;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = j + e < end;
          K.key[i + e] = ok ? score_key(s[j + e]) : 0u;
          K.valid |= (uint64_t)ok << (i + e);
        }
      }
    }
  }
}

// LDS histogram of one digit over the keys that match `prefix` (pass 0: all
// keys, by the windowed register counts of hist_digit0).
template <int PASS>
__device__ __forceinline__ void hist_keys(const ChunkKeys& K, uint32_t prefix, int32_t* h) {
  using DG = Digit<PASS>;
  if constexpr (PASS == 0) {
    hist_digit0<kKeysPerThread>(K.key, K.valid, h);
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
// FIRST: all score loads issued before any key is formed (measured faster on
// grids of up to about two workgroups per CU, slower on large ones).
template <int PASS, bool FIRST>
__global__ void __launch_bounds__(256) sel_hist(SelectParams P) {
  using DG = Digit<PASS>;
  __shared__ int32_t h[DG::BINS];
  __shared__ int32_t sm[264];
  const int u = blockIdx.y, chunk = blockIdx.x;
  int32_t* st = P.state + (int64_t)u * ST_WORDS;
  // the row's mode and candidate count follow from its position (the same
  // values the set-up stored), so the score loads need not wait for a state read
  const int ncand = sel_ncand(row_pos(P, u), P.cand_window);
  const int take = sel_take(ncand, P.k, 1);
  if (sel_mode(take, ncand, 1) != MODE_RADIX) return;
  const int base = chunk * kSelChunk;
  if (base >= ncand) return;
  const int end = min(base + kSelChunk, ncand);
  ChunkKeys K;
  if constexpr (FIRST)
    load_keys_first(P.scores + (int64_t)u * P.N, base, end, (P.N & 3) == 0, K);
  else
    load_keys_inline(P.scores + (int64_t)u * P.N, base, end, (P.N & 3) == 0, K);
  int32_t* hist = P.hist + (int64_t)u * 3 * kHistBins;
  uint32_t prefix = 0;
  if constexpr (PASS > 0) {
    // the previous pass's digit; inputs are what the kernel before wrote
    const uint32_t prev = PASS == 1 ? 0u : (uint32_t)st[ST_PREFIX1];
    int need = PASS == 1 ? take : st[ST_NEED1];
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
  hist_keys<PASS>(K, prefix, h);
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

// Forced window after the `take` selected positions, then the count and the
// -1 padding of the row's list.  When the window competes, sel_window_merge
// writes these instead (some selected positions may lie in the window).
__device__ __forceinline__ void write_window(const SelectParams& P, int u, int take, int p, int32_t* out) {
  if (P.competes) return;
  const int wlo = max(0, p - P.window + 1);
  const int nw = p - wlo + 1;
  for (int i = threadIdx.x; i < nw; i += 256) out[take + i] = wlo + i;
  for (int i = take + nw + threadIdx.x; i < P.max_sel; i += 256) out[i] = -1;
  if (threadIdx.x == 0) P.count[u] = take + nw;
}

// Bracketed path, first step: one workgroup per row sets the row's state up
// and brackets its k-th key from a sample.  Runs i * SR of 64 positions
// (i < nsr <= kBracketRuns) of the candidates are read, 32 keys per thread
// per half of the sample, once per digit; the sample's keys of ranks r_hi = r - m and r_lo =
// r + m (0 = largest) are found to 24 bits -- the first digit for both from
// one histogram, the second from one histogram each -- and stored as the
// prefixes P_hi >= P_lo.  Rows of up to kBracketRuns runs are sampled whole
// (SR = 1), and then both ranks are the k-th key itself.  A rank below 0
// leaves nothing above the bracket (P_hi = 2^24 - 1); one past the sample
// leaves nothing below it (P_lo = 0).
struct BracketRow {
  const float* row;
  int ncand, SR, nsr;
  bool vec_ok;
};
constexpr int kBracketKeys = kKeysPerThread / 2;  // keys per thread per half of the sample

// half h: float4 slot q = tid + 256 * m (m in [8h, 8h + 8)) is the (q & 15)-th
// of sampled run q >> 4, so a wave reads four whole runs
__device__ __forceinline__ void bracket_load(const BracketRow& R, int h, uint32_t (&key)[kBracketKeys],
                                             uint64_t& valid) {
  valid = 0;
#pragma unroll
  for (int mm = 0; mm < kBracketKeys / 4; ++mm) {
    const int q = threadIdx.x + 256 * (h * (kBracketKeys / 4) + mm), run = q >> 4;
    const int j = run * R.SR * 64 + (q & 15) * 4;
    float4 v = {0.f, 0.f, 0.f, 0.f};
    int nv = 0;
    if (run < R.nsr) {
      nv = min(max(R.ncand - j, 0), 4);
      if (R.vec_ok && nv == 4) {
        v = *(const float4*)(R.row + j);
      } else {
        v.x = nv > 0 ? R.row[j] : 0.f;
        v.y = nv > 1 ? R.row[j + 1] : 0.f;
        v.z = nv > 2 ? R.row[j + 2] : 0.f;
        v.w = nv > 3 ? R.row[j + 3] : 0.f;
      }
    }
    key[4 * mm] = score_key(v.x);
    key[4 * mm + 1] = score_key(v.y);
    key[4 * mm + 2] = score_key(v.z);
    key[4 * mm + 3] = score_key(v.w);
    valid |= (uint64_t)((1u << nv) - 1) << (4 * mm);
  }
}

// The two ranks' 24-bit prefixes from a sample of HALVES halves, read once
// per digit (64 KiB per row at most, from the caches the second time: keeping
// the keys in registers instead would take three times the registers).  h0
// and h1 are cleared on entry.
template <int HALVES>
__device__ __forceinline__ void bracket_prefixes(const BracketRow& R, int r_hi, int r_lo, int nsamp, int32_t* h0,
                                                 int32_t* h1, int32_t* sm, uint32_t& p_hi, uint32_t& p_lo) {
  uint32_t key[kBracketKeys];
  uint64_t valid;
#pragma unroll 1
  for (int h = 0; h < HALVES; ++h) {
    bracket_load(R, h, key, valid);
    hist_digit0<kBracketKeys>(key, valid, h0);
  }
  __syncthreads();
  // first digits of the two ranks (uniform conditions around the block-wide searches)
  const bool want_hi = r_hi >= 0, want_lo = r_lo < nsamp;
  int d_hi = 0, a_hi = 0, d_lo = 0, a_lo = 0;
  if (want_hi) find_digit<0>(h0, r_hi + 1, sm, d_hi, a_hi);
  if (want_lo) find_digit<0>(h0, r_lo + 1, sm, d_lo, a_lo);
  // second digits: h1 for the upper rank, h0 (cleared) for the lower one
  for (int i = threadIdx.x; i < kHistBins; i += 256) h0[i] = 0;
  __syncthreads();
#pragma unroll 1
  for (int h = 0; h < HALVES; ++h) {
    bracket_load(R, h, key, valid);
#pragma unroll
    for (int i = 0; i < kBracketKeys; ++i) {
      if (!(valid >> i & 1)) continue;
      const uint32_t d = key[i] >> 20, d2 = (key[i] >> 8) & 0xFFFu;
      if (want_hi && d == (uint32_t)d_hi) atomicAdd(&h1[d2], 1);
      if (want_lo && d == (uint32_t)d_lo) atomicAdd(&h0[d2], 1);
    }
  }
  __syncthreads();
  p_hi = 0xFFFFFFu;
  p_lo = 0u;
  if (want_hi) {
    int d2, a2;
    find_digit<1>(h1, r_hi + 1 - a_hi, sm, d2, a2);
    p_hi = ((uint32_t)d_hi << 12) | (uint32_t)d2;
  }
  if (want_lo) {
    int d2, a2;
    find_digit<1>(h0, r_lo + 1 - a_lo, sm, d2, a2);
    p_lo = ((uint32_t)d_lo << 12) | (uint32_t)d2;
  }
}

__global__ void __launch_bounds__(256) sel_bracket(SelectParams P) {
  __shared__ int32_t h0[kHistBins], h1[kHistBins];
  __shared__ int32_t sm[264];
  const int u = blockIdx.x, tid = threadIdx.x;
  int32_t* st = P.state + (int64_t)u * ST_WORDS;
  const int p = row_pos(P, u);
  const int ncand = sel_ncand(p, P.cand_window), take = sel_take(ncand, P.k, 1);
  const int mode = sel_mode(take, ncand, 1);
  if (tid == 0) {
    st[ST_MODE] = mode;
    st[ST_NCAND] = ncand;
    st[ST_TAKE] = take;
    st[ST_P] = p;
    st[ST_DONE] = 0;
  }
  if (mode != MODE_RADIX) return;  // (uniform) the per-row kernel writes these rows
  BracketRow R;
  R.row = P.scores + (int64_t)u * P.N;
  R.ncand = ncand;
  R.vec_ok = (P.N & 3) == 0;
  const int nruns = (ncand + 63) >> 6;
  R.SR = nruns <= kBracketRuns ? 1 : max(kBracketStride, (nruns + kBracketRuns - 1) / kBracketRuns);
  R.nsr = (nruns + R.SR - 1) / R.SR;
  const int last = (R.nsr - 1) * R.SR * 64;  // first position of the last sampled run (< ncand)
  const int nsamp = (R.nsr - 1) * 64 + min(64, ncand - last);
  int r_hi, r_lo;
  if (R.SR == 1) {
    r_hi = r_lo = take - 1;
  } else {
    const float r = (float)take * (float)nsamp / (float)ncand;
    const float m = 4.f * sqrtf(r) + 8.f;
    r_hi = (int)floorf(r - m);
    r_lo = min((int)ceilf(r + m), nsamp);
  }
  for (int i = tid; i < kHistBins; i += 256) {
    h0[i] = 0;
    h1[i] = 0;
  }
  __syncthreads();
  uint32_t p_hi, p_lo;
  if (R.nsr > kBracketRuns / 2)
    bracket_prefixes<2>(R, r_hi, r_lo, nsamp, h0, h1, sm, p_hi, p_lo);
  else
    bracket_prefixes<1>(R, r_hi, r_lo, nsamp, h0, h1, sm, p_hi, p_lo);
  if (tid == 0) {
    st[ST_PHI] = (int32_t)p_hi;
    st[ST_PLO] = (int32_t)p_lo;
  }
}

// Bracketed path, second step (one workgroup per chunk of a row): the
// positions of the chunk's keys whose 24-bit prefix lies above P_hi, and the
// positions and keys of those between P_lo and P_hi, go to lists the chunk
// owns, a quarter of them per wave (kWaveTake and kWaveBin entries), and each
// wave stores its two list lengths.  The bounds are compared as floats (for
// non-negative scores and -0 the same order as the keys; the bound of an
// empty upper side is a NaN, above which nothing lies).  Each key slot's
// compare gives the wave's ballot of hits, an empty ballot costs a scalar
// branch, and a hit goes at the wave's running count plus its rank in the
// ballot into the wave's own lists in LDS; the wave then copies its lists out
// with whole-row stores (hits are spread thinly over the row, so writing them
// at once would cost one narrow global store per ballot).  One pass, no
// atomics, no barrier.  A wave with more hits than its quarter holds
// (clustered scores) leaves its row to the per-row kernel.
constexpr int kWaveTake = kCompactTake / 4, kWaveBin = kCompactBin / 4;
struct CollectLds {
  int32_t la[4][kWaveTake], lb[4][kWaveBin], lk[4][kWaveBin];
};
template <bool VEC>
__device__ __forceinline__ void collect_chunk(const SelectParams& P, int u, int chunk, int base, int end,
                                              CollectLds& L) {
  constexpr int NV = kKeysPerThread / 4;  // float4 loads per thread
  // element 4 i + e at position base + 4 (tid + 256 i) + e; positions past the
  // chunk read as NaN, which no bound test accepts
  const float* s = P.scores + (int64_t)u * P.N;
  const float nan = __int_as_float(0x7fc00000);
  float4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j = base + 4 * (threadIdx.x + 256 * i);
    if constexpr (VEC) {
      // N a multiple of 4: a group that starts before the chunk's end lies in
      // the row; one past it loads the chunk's first group and is masked
      v[i] = *(const float4*)(s + (j < end ? j : base));
    } else {
      v[i].x = j < end ? s[j] : nan;
      v[i].y = j + 1 < end ? s[j + 1] : nan;
      v[i].z = j + 2 < end ? s[j + 2] : nan;
      v[i].w = j + 3 < end ? s[j + 3] : nan;
    }
  }
  const int32_t* stw = P.state + (int64_t)u * ST_WORDS;
  const float hi = __uint_as_float(((uint32_t)stw[ST_PHI] << 8) | 0xFFu);
  const float lo = __uint_as_float((uint32_t)stw[ST_PLO] << 8);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t below = (1ull << lane) - 1;  // lanes ranked before this one
  int oa = 0, ob = 0;  // wave-uniform running counts
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j = base + 4 * (threadIdx.x + 256 * i);
    float x[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    if constexpr (VEC) {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = j + e < end ? x[e] : nan;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // above: x > hi; inside: lo <= x and not above (NaN fails both, -0 >= +0 holds)
      const bool ha = x[e] > hi, hb = x[e] >= lo && !(x[e] > hi);
      const uint64_t ba = __ballot(ha), bb = __ballot(hb);
      if (ba) {  // uniform
        const int o = oa + __popcll(ba & below);
        if (ha && o < kWaveTake) L.la[wave][o] = j + e;
        oa += __popcll(ba);
      }
      if (bb) {  // uniform
        const int o = ob + __popcll(bb & below);
        if (hb && o < kWaveBin) {
          L.lb[wave][o] = j + e;
          L.lk[wave][o] = (int32_t)score_key(x[e]);
        }
        ob += __popcll(bb);
      }
    }
  }
  const int64_t cw = ((int64_t)u * P.nchunks + chunk) * 4 + wave;
  int32_t* cand = P.cand + ((int64_t)u * P.nchunks + chunk) * kCandWords;
  int32_t* la = cand + wave * kWaveTake;                              // above: positions
  int32_t* lb = cand + kCompactTake + wave * kWaveBin;                // inside: positions
  int32_t* lk = cand + kCompactTake + kCompactBin + wave * kWaveBin;  // inside: keys
  const int na = min(oa, kWaveTake), nb = min(ob, kWaveBin);
  for (int i = lane; i < na; i += 64) la[i] = L.la[wave][i];
  for (int i = lane; i < nb; i += 64) {
    lb[i] = L.lb[wave][i];
    lk[i] = L.lk[wave][i];
  }
  if (lane == 0) {
    P.cnt[2 * cw] = oa;
    P.cnt[2 * cw + 1] = ob;
  }
}

// VEC: rows of a multiple of 4 scores (16-byte loads); else scalar loads
template <bool VEC>
__global__ void __launch_bounds__(256) sel_collect(SelectParams P) {
  const int u = blockIdx.y, chunk = blockIdx.x;
  // the row's mode and candidates follow from its position, so the score
  // loads go out before the bracket is read
  const int ncand = sel_ncand(row_pos(P, u), P.cand_window);
  const int take = sel_take(ncand, P.k, 1);
  if (sel_mode(take, ncand, 1) != MODE_RADIX) return;
  const int base = chunk * kSelChunk;
  if (base >= ncand) return;
  const int end = min(base + kSelChunk, ncand);
  __shared__ CollectLds L;
  collect_chunk<VEC>(P, u, chunk, base, end, L);
}

// Ascending bitonic sort of n (a power of two) LDS elements by the workgroup.
template <typename T>
__device__ void lds_bitonic_sort(T* a, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += 256) {
        const int l = i ^ j;
        if (l > i) {
          const T x = a[i], y = a[l];
          if ((x > y) == ((i & k) == 0)) {
            a[i] = y;
            a[l] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int pow2_at_least(int n) {
  int m = 1;
  while (m < n) m <<= 1;
  return m;
}

// Output order of the finishing kernel: a bitmap over the row's candidates
// in LDS (16-byte groups of 128 positions; group q at slot q + q/32, so the
// runs of 16 consecutive threads start on distinct banks) for rows of up to
// kBitmapMaxCand candidates, a sort of the taken positions beyond.
__host__ __device__ __forceinline__ int bm_slot4(int q) { return q + (q >> 5); }
constexpr int kBitmapMaxCand = 1 << 18;
inline size_t finish_lds_bytes(int N) {
  const int nq = (min(N, kBitmapMaxCand) + 127) >> 7;
  return ((size_t)bm_slot4(nq - 1) + 1) * 16;
}

// Bracketed path, third step: one workgroup per row.  The (chunk, wave) list
// lengths give the row's na keys above the bracket and nb inside it; the
// bracket holds the k-th key when na < take <= na + nb, and with every list
// within its room the row is settled here, else left to the per-row kernel.  The bin's keys (16 per thread in registers) give the need = take -
// na highest by a radix select on chip (digits of 12, 12 and 8 bits): every
// key above the threshold tau and, of the keys equal to tau, the lowest
// positions (found by sorting the tied positions, when not all of them are
// taken).  Those and the na positions above the bracket are the row's
// selection, written in ascending order from a prefix count of their bitmap
// (or a sort of them), then the window.
__global__ void __launch_bounds__(256) sel_finish(SelectParams P) {
  constexpr int BPT = kCompactBin / 256, APT = kCompactTake / 256;
  extern __shared__ __align__(16) u32x4_t bm4[];  // finish_lds_bytes(N)
  __shared__ int32_t h[kHistBins];               // digit histograms, then tied positions or the taken list
  __shared__ int32_t s_pa[4 * kFinishMaxChunks], s_pb[4 * kFinishMaxChunks];  // list starts per (chunk, wave)
  __shared__ int32_t sm[264];
  __shared__ int32_t s_n;
  int32_t* st = P.state + (int64_t)blockIdx.x * ST_WORDS;
  if (st[ST_MODE] != MODE_RADIX) return;
  const int u = blockIdx.x, take = st[ST_TAKE], p = st[ST_P], ncand = st[ST_NCAND];
  const int tid = threadIdx.x;
  // the (chunk, wave) regions' list lengths, their exclusive prefix sums and
  // the totals; a region over its quarter lost entries, and a length outside
  // [0, room] can only be corrupt: either sends the row to the per-row kernel
  const int nch = (ncand + kSelChunk - 1) / kSelChunk;
  if (nch > kFinishMaxChunks) return;  // (uniform) left to the per-row kernel
  const int nreg = 4 * nch;
  const int32_t* cnt = P.cnt + (int64_t)u * P.nchunks * 8;
  int na = 0, nb = 0, over = 0;
  for (int r0 = 0; r0 < nreg; r0 += 256) {
    const int r = r0 + tid;
    const int ca = r < nreg ? cnt[2 * r] : 0, cb = r < nreg ? cnt[2 * r + 1] : 0;
    int32_t v[3] = {ca, cb, (ca < 0) | (cb < 0) | (ca > kWaveTake) | (cb > kWaveBin)}, t[3];
    block_exclusive_scan_n<3>(v, sm, t);
    if (r < nreg) {
      s_pa[r] = na + v[0];
      s_pb[r] = nb + v[1];
    }
    na += t[0];
    nb += t[1];
    over += t[2];
  }
  if (over || !(na < take && take <= na + nb && take <= kCompactTake && nb <= kCompactBin)) return;
  __syncthreads();
  // entry i of a list lies in the last region whose start is <= i
  auto region_of = [&](const int32_t* starts, int i) {
    int lo = 0, hi = nreg - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (starts[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };
  // region r = 4 c + w: chunk c's lists, wave w's quarter
  const int32_t* cand = P.cand + (int64_t)u * P.nchunks * kCandWords;
  uint32_t bk[BPT];
  int32_t bp[BPT], ap[APT];
  uint64_t bvalid = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int i = tid + 256 * j;
    const bool ok = i < nb;
    bp[j] = -1;
    bk[j] = 0u;
    if (ok) {
      const int r = region_of(s_pb, i);
      const int32_t* cc = cand + (int64_t)(r >> 2) * kCandWords + kCompactTake + (r & 3) * kWaveBin + (i - s_pb[r]);
      bp[j] = cc[0];
      bk[j] = (uint32_t)cc[kCompactBin];
    }
    bvalid |= (uint64_t)ok << j;
  }
#pragma unroll
  for (int r_ = 0; r_ < APT; ++r_) {
    const int i = tid + 256 * r_;
    ap[r_] = -1;
    if (i < na) {
      const int r = region_of(s_pa, i);
      ap[r_] = cand[(int64_t)(r >> 2) * kCandWords + (r & 3) * kWaveTake + (i - s_pa[r])];
    }
  }
  // radix select of the need-th largest bin key
  int need = take - na, d, above, n_eq = 0;
  for (int i = tid; i < kHistBins; i += 256) h[i] = 0;
  __syncthreads();
  hist_digit0<BPT>(bk, bvalid, h);
  __syncthreads();
  find_digit<0>(h, need, sm, d, above);
  uint32_t tau = (uint32_t)d << 20;
  need -= above;
  for (int i = tid; i < kHistBins; i += 256) h[i] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < BPT; ++j)
    if ((bvalid >> j & 1) && (bk[j] & 0xFFF00000u) == tau) atomicAdd(&h[(bk[j] >> 8) & 0xFFFu], 1);
  __syncthreads();
  find_digit<1>(h, need, sm, d, above);
  tau |= (uint32_t)d << 8;
  need -= above;
  for (int i = tid; i < 256; i += 256) h[i] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < BPT; ++j)
    if ((bvalid >> j & 1) && (bk[j] & 0xFFFFFF00u) == tau) atomicAdd(&h[bk[j] & 0xFFu], 1);
  __syncthreads();
  find_digit<2>(h, need, sm, d, above, &n_eq);
  tau |= (uint32_t)d;
  need -= above;  // keys equal to tau that are taken: 1 <= need <= n_eq
  // ties: the need lowest positions among the n_eq keys equal to tau
  int32_t cut = INT32_MAX;
  if (need < n_eq) {  // uniform
    if (tid == 0) s_n = 0;
    const int np = pow2_at_least(n_eq);
    for (int i = n_eq + tid; i < np; i += 256) h[i] = INT32_MAX;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < BPT; ++j)
      if ((bvalid >> j & 1) && bk[j] == tau) h[atomicAdd(&s_n, 1)] = bp[j];
    __syncthreads();
    lds_bitonic_sort(h, np);
    cut = h[need - 1];
    __syncthreads();
  }
  uint32_t bsel = 0;  // bin entries taken
#pragma unroll
  for (int j = 0; j < BPT; ++j)
    bsel |= (uint32_t)((bvalid >> j & 1) && (bk[j] > tau || (bk[j] == tau && bp[j] <= cut))) << j;
  int32_t* out = P.idx + (int64_t)u * P.max_sel;
  if (ncand <= kBitmapMaxCand) {  // uniform
    const int nq = (ncand + 127) >> 7;  // 128-position groups
    const int nslots = bm_slot4(nq - 1) + 1;
    for (int i = tid; i < nslots; i += 256) bm4[i] = u32x4_t{0u, 0u, 0u, 0u};
    __syncthreads();
    uint32_t* bm = (uint32_t*)bm4;
    // (positions come from the collecting pass, always in [0, ncand); the test
    // keeps every LDS access inside the bitmap whatever the lists hold)
    auto mark = [&](int pos) {
      if ((unsigned)pos < (unsigned)ncand) atomicOr(&bm[4 * bm_slot4(pos >> 7) + ((pos >> 5) & 3)], 1u << (pos & 31));
    };
#pragma unroll
    for (int r = 0; r < APT; ++r)
      if (ap[r] >= 0) mark(ap[r]);
#pragma unroll
    for (int j = 0; j < BPT; ++j)
      if (bsel >> j & 1) mark(bp[j]);
    __syncthreads();
    // at most 8 groups per thread (kBitmapMaxCand / 128 / 256); the mask of
    // the non-empty ones lets the output loop visit only those
    const int per = (nq + 255) >> 8;
    const int q0 = min(tid * per, nq), q1 = min(q0 + per, nq);
    int32_t cnt = 0;
    uint32_t nz = 0;
    for (int q = q0; q < q1; ++q) {
      const u32x4_t v = bm4[bm_slot4(q)];
      const int c = __popc(v.x) + __popc(v.y) + __popc(v.z) + __popc(v.w);
      cnt += c;
      nz |= (uint32_t)(c != 0) << (q - q0);
    }
    int32_t tot;
    int32_t o = block_exclusive_scan<int32_t>(cnt, sm, tot);
    while (nz) {
      const int q = q0 + __builtin_ctz(nz);
      nz &= nz - 1;
      const u32x4_t v = bm4[bm_slot4(q)];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t bits = v[c];
        while (bits) {
          if (o < take) out[o] = (q << 7) + (c << 5) + __builtin_ctz(bits);
          ++o;
          bits &= bits - 1;
        }
      }
    }
  } else {  // long rows: the taken positions sorted
    if (tid == 0) s_n = 0;
    const int ntp = pow2_at_least(take);
    for (int i = take + tid; i < ntp; i += 256) h[i] = INT32_MAX;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < APT; ++r)
      if (ap[r] >= 0) h[atomicAdd(&s_n, 1)] = ap[r];
#pragma unroll
    for (int j = 0; j < BPT; ++j)
      if (bsel >> j & 1) h[atomicAdd(&s_n, 1)] = bp[j];
    __syncthreads();
    lds_bitonic_sort(h, ntp);
    for (int i = tid; i < take; i += 256) out[i] = h[i];
  }
  write_window(P, u, take, p, out);
  if (tid == 0) st[ST_DONE] = 1;
}

// Ordered compaction of one chunk's keys (load_keys_runs layout): every key
// above tau, and of the keys equal to tau those whose rank among the row's
// equal keys (eq_before of them in earlier chunks) is below need, into the
// slots from sel_before on (keys taken in earlier chunks), never past take.
// The four quarters' counts go through two packed scans (16 bits per quarter;
// a quarter holds at most 4096 keys): first the keys equal to tau, whose rank
// decides which of them are taken, then the taken keys, whose prefix is the
// output slot.  eq_tot / sel_tot: this chunk's equal and taken keys.
__device__ __forceinline__ void emit_chunk(const ChunkKeys& K, int base, uint32_t tau, int need, int32_t eq_before,
                                           int32_t sel_before, int take, int32_t* out, int32_t* sm, int32_t& eq_tot,
                                           int32_t& sel_tot) {
  int32_t eqc[4];
#pragma unroll
  for (int rnd = 0; rnd < 4; ++rnd) {
    int32_t c = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) c += (K.valid >> (rnd * 16 + e) & 1) && K.key[rnd * 16 + e] == tau;
    eqc[rnd] = c;
  }
  int32_t pe[2] = {eqc[0] | (eqc[1] << 16), eqc[2] | (eqc[3] << 16)}, te[2];
  block_exclusive_scan_n<2>(pe, sm, te);
  uint32_t selmask[4];
  int32_t selc[4];
  int32_t rbase = eq_before;
#pragma unroll
  for (int rnd = 0; rnd < 4; ++rnd) {
    const int f = (rnd & 1) * 16, w = rnd >> 1;
    int32_t r_eq = rbase + ((pe[w] >> f) & 0xffff);
    rbase += (te[w] >> f) & 0xffff;
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t key = K.key[rnd * 16 + e];
      bool take_it = false;
      if (K.valid >> (rnd * 16 + e) & 1) {
        if (key > tau) {
          take_it = true;
        } else if (key == tau) {
          take_it = r_eq < need;
          ++r_eq;
        }
      }
      m |= (uint32_t)take_it << e;
    }
    selmask[rnd] = m;
    selc[rnd] = __builtin_popcount(m);
  }
  eq_tot = rbase - eq_before;
  int32_t ps[2] = {selc[0] | (selc[1] << 16), selc[2] | (selc[3] << 16)}, ts[2];
  block_exclusive_scan_n<2>(ps, sm, ts);
  int32_t sbase = sel_before;
#pragma unroll
  for (int rnd = 0; rnd < 4; ++rnd) {
    const int j0 = base + rnd * 4096 + threadIdx.x * 16;
    const int f = (rnd & 1) * 16, w = rnd >> 1;
    int32_t sl = sbase + ((ps[w] >> f) & 0xffff);
    sbase += (ts[w] >> f) & 0xffff;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (selmask[rnd] >> e & 1u) {
        if ((uint32_t)sl < (uint32_t)take) out[sl] = j0 + e;  // never past this unit's budget
        ++sl;
      }
  }
  sel_tot = sbase - sel_before;
}

// Ascending compaction: every key above tau and the lowest-positioned keys
// equal to tau (tau and their number from the last digit's histogram), then
// (chunk 0) the forced window, the count and the padding.
__global__ void __launch_bounds__(256) sel_emit(SelectParams P) {
  __shared__ int32_t sm[264];
  const int u = blockIdx.y, chunk = blockIdx.x;
  const int32_t* st = P.state + (int64_t)u * ST_WORDS;
  const int p = row_pos(P, u);  // as stored by the set-up
  const int ncand = sel_ncand(p, P.cand_window);
  const int take = sel_take(ncand, P.k, 1);
  const int mode = sel_mode(take, ncand, 1);
  int32_t* out = P.idx + (int64_t)u * P.max_sel;

  if (chunk == 0) write_window(P, u, take, p, out);
  if (mode == MODE_NONE) return;
  const int base = chunk * kSelChunk;
  if (base >= ncand) return;
  const int end = min(base + kSelChunk, ncand);
  if (mode == MODE_ALL) {
    for (int j = base + threadIdx.x; j < end; j += 256) out[j] = j;
    return;
  }
  ChunkKeys K;
  load_keys_runs(P.scores + (int64_t)u * P.N, base, end, (P.N & 3) == 0, K);
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
  int32_t eq_c, sel_c;
  emit_chunk(K, base, tau, need, eq_before, sel_before, take, out, sm, eq_c, sel_c);
}

// A row the bracketed path did not settle -- and every row that takes all or
// none of its candidates -- done by one workgroup: the three radix digits
// over the row's candidates (each pass reads the row once; digits of 12, 12
// and 8 bits as in the multi-workgroup passes), then the ordered compaction
// chunk by chunk with running counts, then the window.
__global__ void __launch_bounds__(256) sel_row_exact(SelectParams P) {
  __shared__ int32_t h[kHistBins];
  __shared__ int32_t sm[264];
  const int u = blockIdx.x;
  if (P.state[(int64_t)u * ST_WORDS + ST_DONE]) return;
  const int p = row_pos(P, u);
  const int ncand = sel_ncand(p, P.cand_window), take = sel_take(ncand, P.k, 1);
  const int mode = sel_mode(take, ncand, 1);
  int32_t* out = P.idx + (int64_t)u * P.max_sel;
  if (mode == MODE_ALL) {
    for (int j = threadIdx.x; j < ncand; j += 256) out[j] = j;
  } else if (mode == MODE_RADIX) {
    const float* row = P.scores + (int64_t)u * P.N;
    const bool vec_ok = (P.N & 3) == 0;
    int need = take;
    uint32_t prefix = 0;
    // one pass per digit: the LDS histogram of the keys sharing the digits so far
    auto count = [&](auto pass_tag) {
      constexpr int PASS = decltype(pass_tag)::value;
      for (int i = threadIdx.x; i < kHistBins; i += 256) h[i] = 0;
      __syncthreads();
#pragma unroll 1
      for (int base = 0; base < ncand; base += kSelChunk) {
        ChunkKeys K;
        load_keys_runs(row, base, min(base + kSelChunk, ncand), vec_ok, K);
        hist_keys<PASS>(K, prefix, h);
      }
      __syncthreads();
      int d, above;
      find_digit<PASS>(h, need, sm, d, above);
      prefix |= (uint32_t)d << Digit<PASS>::SHIFT;
      need -= above;
    };
    count(std::integral_constant<int, 0>());
    count(std::integral_constant<int, 1>());
    count(std::integral_constant<int, 2>());
    // prefix is now the k-th key tau; need of the keys equal to it are taken
    int32_t eq_before = 0, sel_before = 0;
#pragma unroll 1
    for (int base = 0; base < ncand; base += kSelChunk) {
      ChunkKeys K;
      load_keys_runs(row, base, min(base + kSelChunk, ncand), vec_ok, K);
      int32_t eq_c, sel_c;
      emit_chunk(K, base, prefix, need, eq_before, sel_before, take, out, sm, eq_c, sel_c);
      eq_before += eq_c;
      sel_before += sel_c;
    }
  }
  write_window(P, u, take, p, out);
}

// The window competes (candidates [0, p]): the emit wrote the `take`
// selected positions in ascending order, some of them possibly inside the
// window [p - window + 1, p], which are then its last entries.  One workgroup
// per row counts them, and the window follows the selected positions below it
// (so the list is the ascending union, each position once), then the count
// and the -1 padding.
__global__ void __launch_bounds__(256) sel_window_merge(SelectParams P) {
  __shared__ int32_t sm[264];
  const int u = blockIdx.x;
  const int p = row_pos(P, u);
  const int take = sel_take(sel_ncand(p, P.cand_window), P.k, 1);
  const int wlo = max(0, p - P.window + 1);
  const int nw = p - wlo + 1;
  int32_t* out = P.idx + (int64_t)u * P.max_sel;
  // the last min(take, nw) selected entries hold every selected window position
  const int first = take - min(take, nw);
  int32_t c = 0;
  for (int i = first + threadIdx.x; i < take; i += 256) c += out[i] >= wlo;
  int32_t in_window;
  block_exclusive_scan<int32_t>(c, sm, in_window);  // its barriers also order the reads before the writes
  const int below = take - in_window;
  for (int i = threadIdx.x; i < nw; i += 256) out[below + i] = wlo + i;
  for (int i = below + nw + threadIdx.x; i < P.max_sel; i += 256) out[i] = -1;
  if (threadIdx.x == 0) P.count[u] = below + nw;
}

// ---------------------------------------------------------------------------
// block baseline
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) sel_block_mass(SelectParams P) {
  const int u = blockIdx.y;
  const int beta = blockIdx.x * 256 + threadIdx.x;
  const int ncand = sel_ncand(row_pos(P, u), P.window);  // as stored by the set-up
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

// Block masses with coalesced loads: a workgroup stages 4096 consecutive
// scores (64 threads x 16 floats per wave row) in LDS, then one thread per
// block adds its block's scores in ascending position, as the plain kernel
// does.  Power-of-two block sizes up to 256; a block's BS scores sit at LDS
// slot t (BS + 4): 16-byte writes and reads, and the 16 lanes of a 16-byte
// read phase start 4 banks apart, so neither side conflicts.
constexpr int kMassTile = 4096;
template <int BS>
__global__ void __launch_bounds__(256) sel_block_mass_tiled(SelectParams P) {
  __shared__ __align__(16) float sv[kMassTile + 4 * (kMassTile / BS)];
  const int u = blockIdx.y;
  const int ncand = sel_ncand(row_pos(P, u), P.window);  // as stored by the set-up
  const int lo = blockIdx.x * kMassTile;
  if (lo >= ncand) return;
  const float* s = P.scores + (int64_t)u * P.N;
  const bool vec_ok = (P.N & 3) == 0;
#pragma unroll
  for (int r = 0; r < kMassTile / 1024; ++r) {
    const int i = 4 * threadIdx.x + 1024 * r;  // tile offset of this float4
    const int j = lo + i;
    float4 v;
    if (vec_ok && j + 3 < ncand) {
      v = *(const float4*)(s + j);
    } else {
      v.x = j < ncand ? s[j] : 0.f;
      v.y = j + 1 < ncand ? s[j + 1] : 0.f;
      v.z = j + 2 < ncand ? s[j + 2] : 0.f;
      v.w = j + 3 < ncand ? s[j + 3] : 0.f;
    }
    *(float4*)(sv + i + 4 * (i / BS)) = v;  // 4 | BS, so the float4 stays inside one block
  }
  __syncthreads();
  constexpr int NB = kMassTile / BS;
  for (int t = threadIdx.x; t < NB; t += 256) {
    const int beta = blockIdx.x * NB + t;
    if (beta * BS >= ncand) break;
    const int n = min(BS, ncand - beta * BS);
    const float* b = sv + t * (BS + 4);
    double m = 0.0;
    int e = 0;
    for (; e + 4 <= n; e += 4) {
      const float4 x = *(const float4*)(b + e);
      m += (double)x.x;
      m += (double)x.y;
      m += (double)x.z;
      m += (double)x.w;
    }
    for (; e < n; ++e) m += (double)b[e];
    P.bmass[(int64_t)u * P.nblocks_max + beta] = m;
  }
}

// (mass desc, block asc) order: true when (m, b) comes before (bm, bb)
__device__ __forceinline__ bool mass_before(double m, int b, double bm, int bb) {
  return m > bm || (m == bm && b < bb);
}

// Better of two (mass, block) candidates in (mass desc, block asc) order.
__device__ __forceinline__ void pick_better(double& m, int& b, double m2, int b2) {
  if (mass_before(m2, b2, m, b)) {
    m = m2;
    b = b2;
  }
}
__device__ __forceinline__ double dbl_of(uint32_t lo, uint32_t hi) {
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// DPP step: candidate of the lane given by dpp_ctrl (within its row of 16)
template <int CTRL>
__device__ __forceinline__ void argmax_dpp(double& m, int& b) {
  const uint64_t u = (uint64_t)__double_as_longlong(m);
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)u, CTRL, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  const int b2 = __builtin_amdgcn_update_dpp(0, b, CTRL, 0xF, 0xF, false);
  pick_better(m, b, dbl_of(lo, hi), b2);
}
// Wave-wide best (mass desc, block asc); every lane returns it.  Quad swaps,
// the 8- and 16-lane mirrors, then the gfx950 permlane swaps of 16-lane rows
// and 32-lane halves: each step merges two groups that already agree.
__device__ __forceinline__ void wave_argmax(double& m, int& b) {
  argmax_dpp<0xB1>(m, b);   // quad_perm [1,0,3,2]
  argmax_dpp<0x4E>(m, b);   // quad_perm [2,3,0,1]
  argmax_dpp<0x141>(m, b);  // row_half_mirror
  argmax_dpp<0x140>(m, b);  // row_mirror
  {
    const uint64_t u = (uint64_t)__double_as_longlong(m);
    const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
    const auto bb = __builtin_amdgcn_permlane16_swap((uint32_t)b, (uint32_t)b, false, false);
    m = dbl_of(lo[0], hi[0]);
    b = (int)bb[0];
    pick_better(m, b, dbl_of(lo[1], hi[1]), (int)bb[1]);
  }
  {
    const uint64_t u = (uint64_t)__double_as_longlong(m);
    const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
    const auto bb = __builtin_amdgcn_permlane32_swap((uint32_t)b, (uint32_t)b, false, false);
    m = dbl_of(lo[0], hi[0]);
    b = (int)bb[0];
    pick_better(m, b, dbl_of(lo[1], hi[1]), (int)bb[1]);
  }
}

// Heaviest blocks, one wave per row, masses in LDS (rows of up to
// kPickLdsBlocks blocks: at most 64 KiB).  Each lane keeps the best of its
// strided blocks; a round takes the wave's best (no barriers) and only its
// owner lane rescans.  Same order and ties as the plain kernel.  The ascending
// emit then walks the blocks 64 at a time: a ballot gives each taken block its
// rank, and the wave writes a taken block's positions with coalesced stores.
constexpr int kPickLdsBlocks = 8192;
__global__ void __launch_bounds__(64) sel_block_pick_wave(SelectParams P) {
  extern __shared__ double s_mass[];  // [nblocks_max]
  const int u = blockIdx.x;
  const int lane = threadIdx.x;
  const int32_t* st = P.state + (int64_t)u * ST_WORDS;
  const int ncand = st[ST_NCAND];
  const int take = st[ST_TAKE];
  const int p = st[ST_P];
  const int bs = P.block_size;
  const int nb = ncand > 0 ? (ncand - 1) / bs + 1 : 0;
  const double* bm = P.bmass + (int64_t)u * P.nblocks_max;
  // each lane's four best blocks, best first; (-1, INT_MAX) marks an empty slot
  constexpr int L = 4;
  double cm[L];
  int cb[L];
  auto clear = [&]() {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      cm[i] = -1.0;
      cb[i] = 0x7fffffff;
    }
  };
  auto insert = [&](double x, int beta) {
    if (!mass_before(x, beta, cm[L - 1], cb[L - 1])) return;
    cm[L - 1] = x;
    cb[L - 1] = beta;
#pragma unroll
    for (int i = L - 1; i > 0; --i)
      if (mass_before(cm[i], cb[i], cm[i - 1], cb[i - 1])) {
        const double tm = cm[i];
        const int tb = cb[i];
        cm[i] = cm[i - 1];
        cb[i] = cb[i - 1];
        cm[i - 1] = tm;
        cb[i - 1] = tb;
      }
  };
  clear();
  constexpr int R = 16;  // loads in flight per lane
  for (int b0 = 0; b0 < nb; b0 += 64 * R) {
    double x[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int beta = b0 + lane + 64 * r;
      x[r] = beta < nb ? bm[beta] : -1.0;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int beta = b0 + lane + 64 * r;
      if (beta < nb) {
        s_mass[beta] = x[r];
        insert(x[r], beta);
      }
    }
  }
  int left = L;  // entries of the list not taken yet
  for (int round = 0; round < take; ++round) {
    double m = cm[0];
    int b = cb[0];
    wave_argmax(m, b);
    if (cb[0] == b) {  // the owner lane takes its head
      s_mass[b] = -1.0;
#pragma unroll
      for (int i = 0; i < L - 1; ++i) {
        cm[i] = cm[i + 1];
        cb[i] = cb[i + 1];
      }
      cm[L - 1] = -1.0;
      cb[L - 1] = 0x7fffffff;
      if (--left == 0) {  // list used up: rebuild it from the untaken blocks
        clear();
#pragma unroll 4
        for (int beta = lane; beta < nb; beta += 64) {
          const double x = s_mass[beta];
          if (x >= 0.0) insert(x, beta);
        }
        left = L;
      }
    }
  }
  int32_t* out = P.idx + (int64_t)u * P.max_sel;
  int32_t written = 0;
  for (int b0 = 0; b0 < nb; b0 += 64) {
    const int beta = b0 + lane;
    const uint64_t tk = __ballot(beta < nb && s_mass[beta] == -1.0);
    uint64_t rest = tk;
    int32_t off = written;
    while (rest) {  // wave-uniform: one taken block at a time, in ascending order
      const int lb2 = __builtin_ctzll(rest);
      rest &= rest - 1;
      const int blk = b0 + lb2;
      const int n = min(blk * bs + bs, ncand) - blk * bs;
      for (int e = lane; e < n; e += 64)
        if (off + e < P.max_sel) out[off + e] = blk * bs + e;
      off += n;
    }
    written = off;
  }
  const int wlo = max(0, p - P.window + 1);
  const int nw = p - wlo + 1;
  for (int i = lane; i < nw && written + i < P.max_sel; i += 64) out[written + i] = wlo + i;
  for (int i = written + nw + lane; i < P.max_sel; i += 64) out[i] = -1;
  if (lane == 0) P.count[u] = written + nw;
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

hipError_t launch_select(const SelectParams& p_in, hipStream_t s) {
  const SelectParams& p = p_in;
  const dim3 grid_c(p.nchunks, p.units);
  hipError_t e;
#define HS2_L(name, kern, grid)                                   \
  do {                                                            \
    TimedLaunch tl_(name, s);                                     \
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, p);           \
    if ((e = hipGetLastError()) != hipSuccess) return e;          \
  } while (0)
  if (p.block_size == 1 && sel_bracketed(p.units, p.nchunks)) {
    // many rows: bracket from a sample, one collecting pass, finish on chip,
    // unsettled rows by the per-row kernel (the set-up is the bracket's)
    HS2_L("select_bracket", sel_bracket, dim3(p.units));
    if ((p.N & 3) == 0)
      HS2_L("select_collect", sel_collect<true>, grid_c);
    else
      HS2_L("select_collect", sel_collect<false>, grid_c);
    {
      TimedLaunch tl_("select_finish", s);
      hipLaunchKernelGGL(sel_finish, dim3(p.units), dim3(256), finish_lds_bytes(p.N), s, p);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    HS2_L("select_exact", sel_row_exact, dim3(p.units));
    if (p.competes) HS2_L("select_window", sel_window_merge, dim3(p.units));
    return hipSuccess;
  }
  if (!(p.pre_hist0 && p.block_size == 1)) HS2_L("select_init", sel_init, dim3(p.units));
  if (p.block_size == 1) {
    const bool small = p.units * p.nchunks <= 512;  // up to about two workgroups per CU: latency-bound passes
    if (!p.pre_hist0) {
      if (small) HS2_L("select_hist", (sel_hist<0, true>), grid_c);
      else HS2_L("select_hist", (sel_hist<0, false>), grid_c);
    }
    if (small) HS2_L("select_hist", (sel_hist<1, true>), grid_c);
    else HS2_L("select_hist", (sel_hist<1, false>), grid_c);
    if (small) HS2_L("select_hist", (sel_hist<2, true>), grid_c);
    else HS2_L("select_hist", (sel_hist<2, false>), grid_c);
    HS2_L("select_emit", sel_emit, grid_c);
    if (p.competes) HS2_L("select_window", sel_window_merge, dim3(p.units));
  } else {
    const dim3 grid_t((p.N + kMassTile - 1) / kMassTile, p.units);
    switch (p.block_size) {
      case 4: HS2_L("select_block_mass", sel_block_mass_tiled<4>, grid_t); break;
      case 8: HS2_L("select_block_mass", sel_block_mass_tiled<8>, grid_t); break;
      case 16: HS2_L("select_block_mass", sel_block_mass_tiled<16>, grid_t); break;
      case 32: HS2_L("select_block_mass", sel_block_mass_tiled<32>, grid_t); break;
      case 64: HS2_L("select_block_mass", sel_block_mass_tiled<64>, grid_t); break;
      case 128: HS2_L("select_block_mass", sel_block_mass_tiled<128>, grid_t); break;
      case 256: HS2_L("select_block_mass", sel_block_mass_tiled<256>, grid_t); break;
      default: HS2_L("select_block_mass", sel_block_mass, dim3((p.nblocks_max + 255) / 256, p.units));
    }
    if (p.nblocks_max <= kPickLdsBlocks) {
      const size_t lds = (size_t)max(p.nblocks_max, 1) * sizeof(double);
      TimedLaunch tl_("select_block_pick", s);
      hipLaunchKernelGGL(sel_block_pick_wave, dim3(p.units), dim3(64), lds, s, p);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    } else {
      HS2_L("select_block_pick", sel_block_pick, dim3(p.units));
    }
  }
#undef HS2_L
  return hipSuccess;
}

}  // namespace hs2
