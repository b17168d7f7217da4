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
// Collected path: the keys that share the 24-bit prefix found by the first two
// passes are few (a handful on attention scores: the third digit only splits
// near-equal values).  Where that bin and k are small enough, one pass
// collects the keys above the prefix (all selected) and the bin's keys, and
// one workgroup per row finishes the selection on chip: the bin's keys in
// (score desc, position asc) order, then every taken position sorted
// ascending.  That replaces the third histogram pass and the emit pass, each a
// full read of the scores; rows whose bin is too large take those two passes.
//
// Block mode (block_size > 1) is the previous generation's 64-token block
// selection (zgeo.com.cn comparison table): block mass = fp64 sum of its
// scores over C in ascending position, heaviest blocks first, ties to the
// lower block.
#include <atomic>

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
  if (PASS == 2 && P.collected && st[ST_COMPACT]) return;  // finished by the collected path
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

// Collected path, first step (after the second histogram pass): settle the
// second digit, decide whether the row is collected (k <= kCompactTake and at
// most kCompactBin keys share the 24-bit prefix -- both known exactly from the
// histograms), and if so append this chunk's keys above the prefix (positions)
// and in its bin (key, position) to the row's lists.  Offsets come from one
// atomic per list and workgroup, so list order varies between runs; the
// finishing kernel sorts, which makes the result deterministic.
__global__ void __launch_bounds__(256) sel_collect(SelectParams P) {
  __shared__ int32_t sm[264];
  __shared__ int32_t s_base[2];
  const int u = blockIdx.y, chunk = blockIdx.x;
  int32_t* st = P.state + (int64_t)u * ST_WORDS;
  if (st[ST_MODE] != MODE_RADIX) return;
  const int ncand = st[ST_NCAND];
  const int base = chunk * kSelChunk;
  if (base >= ncand) return;
  const int end = min(base + kSelChunk, ncand);
  ChunkKeys K;
  load_keys_first(P.scores + (int64_t)u * P.N, base, end, (P.N & 3) == 0, K);
  const int32_t* hist = P.hist + (int64_t)u * 3 * kHistBins;
  int need = st[ST_NEED1];
  int d, above, nbin;
  find_digit<1>(hist + kHistBins, need, sm, d, above, &nbin);
  const uint32_t prefix = (uint32_t)st[ST_PREFIX1] | ((uint32_t)d << Digit<1>::SHIFT);
  need -= above;
  const bool compact = st[ST_TAKE] <= kCompactTake && nbin <= kCompactBin && ncand <= kCompactMaxCand;
  if (chunk == 0 && threadIdx.x == 0) {
    st[ST_PREFIX2] = (int32_t)prefix;
    st[ST_NEED2] = need;
    st[ST_COMPACT] = compact;
  }
  if (!compact) return;
  const uint32_t p24 = prefix >> 8;
  uint64_t hit_a = 0, hit_b = 0;  // keys above the prefix / in its bin
#pragma unroll
  for (int i = 0; i < kKeysPerThread; ++i) {
    const uint32_t hk = K.key[i] >> 8;
    hit_a |= (uint64_t)(hk > p24) << i;
    hit_b |= (uint64_t)(hk == p24) << i;
  }
  hit_a &= K.valid;
  hit_b &= K.valid;
  const int32_t na = __popcll(hit_a), nb = __popcll(hit_b);
  // both counts in one scan: at most kSelChunk each, so the halves never carry
  int32_t tot;
  const int32_t off = block_exclusive_scan<int32_t>((na << 16) | nb, sm, tot);
  if (threadIdx.x == 0) {
    s_base[0] = atomicAdd(&st[ST_NABOVE], tot >> 16);
    s_base[1] = atomicAdd(&st[ST_NBIN], tot & 0xffff);
  }
  __syncthreads();
  int32_t* cand = P.cand + (int64_t)u * kCandWords;
  int oa = s_base[0] + (off >> 16), ob = s_base[1] + (off & 0xffff);
  if (hit_a | hit_b) {
#pragma unroll
    for (int i = 0; i < kKeysPerThread; ++i) {
      const int pos = base + 4 * (threadIdx.x + 256 * (i >> 2)) + (i & 3);
      if (hit_a >> i & 1) {
        if (oa < kCompactTake) cand[oa] = pos;
        ++oa;
      } else if (hit_b >> i & 1) {
        if (ob < kCompactBin) {
          cand[kCompactTake + ob] = (int32_t)K.key[i];
          cand[kCompactTake + kCompactBin + ob] = pos;
        }
        ++ob;
      }
    }
  }
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

// Collected path, second step: one workgroup per collected row.  The bin's
// keys sorted by (score desc, position asc) give the need2 highest keys with
// ties to the lower position.  Those and the keys above the prefix are the
// row's `take` positions: marked in an LDS bitmap over the candidates, they
// come out in ascending order from a prefix count of the bitmap, followed by
// the window.  Each thread counts a run of 16-byte bitmap groups; group q sits
// at q + q/32, so the runs of 16 consecutive threads start on distinct banks.
__host__ __device__ __forceinline__ int bm_slot4(int q) { return q + (q >> 5); }

// dynamic LDS of the finishing kernel for rows of up to min(N, kCompactMaxCand) candidates
inline size_t finish_lds_bytes(int N) {
  const int nq = (min(N, kCompactMaxCand) + 127) >> 7;
  return ((size_t)bm_slot4(nq - 1) + 1) * 16;
}

__global__ void __launch_bounds__(256) sel_finish(SelectParams P) {
  extern __shared__ __align__(16) u32x4_t bm4[];  // finish_lds_bytes(N)
  __shared__ uint64_t s_bin[kCompactBin];
  __shared__ int32_t sm[264];
  const int u = blockIdx.x;
  const int32_t* st = P.state + (int64_t)u * ST_WORDS;
  if (st[ST_MODE] != MODE_RADIX || !st[ST_COMPACT]) return;
  const int take = st[ST_TAKE], p = st[ST_P], ncand = st[ST_NCAND];
  // the histograms make these exact (na + need = take, need <= nb); the clamps
  // only keep LDS accesses inside their arrays
  const int na = min(st[ST_NABOVE], kCompactTake);
  const int nb = min(st[ST_NBIN], kCompactBin);
  const int need = min(max(st[ST_NEED2], 0), nb);
  const int32_t* cand = P.cand + (int64_t)u * kCandWords;
  // every list load issued at once: positions above the prefix, then the bin
  constexpr int kAbovePerThread = kCompactTake / 256;
  int32_t apos[kAbovePerThread];
#pragma unroll
  for (int r = 0; r < kAbovePerThread; ++r) {
    const int i = threadIdx.x + 256 * r;
    apos[r] = i < na ? cand[i] : -1;
  }
  const int nbp = pow2_at_least(nb);
  for (int i = threadIdx.x; i < nbp; i += 256)
    s_bin[i] = i < nb ? ((uint64_t)(~(uint32_t)cand[kCompactTake + i]) << 32) |
                            (uint32_t)cand[kCompactTake + kCompactBin + i]
                      : ~0ull;
  const int nq = (ncand + 127) >> 7;  // 128-position groups
  const int nslots = bm_slot4(nq - 1) + 1;
  for (int i = threadIdx.x; i < nslots; i += 256) bm4[i] = u32x4_t{0u, 0u, 0u, 0u};
  __syncthreads();
  lds_bitonic_sort(s_bin, nbp);
  uint32_t* bm = (uint32_t*)bm4;
  auto mark = [&](int pos) {
    if (pos >= 0 && pos < ncand) atomicOr(&bm[4 * bm_slot4(pos >> 7) + ((pos >> 5) & 3)], 1u << (pos & 31));
  };
#pragma unroll
  for (int r = 0; r < kAbovePerThread; ++r) mark(apos[r]);
  for (int i = threadIdx.x; i < need; i += 256) mark((int)(uint32_t)s_bin[i]);
  __syncthreads();
  // at most 32 groups per thread (kCompactMaxCand / 128 / 256); the mask of
  // the non-empty ones lets the output loop visit only those
  const int per = (nq + 255) >> 8;
  const int q0 = min((int)threadIdx.x * per, nq), q1 = min(q0 + per, nq);
  int32_t cnt = 0;
  uint32_t nz = 0;
#pragma unroll 4
  for (int q = q0; q < q1; ++q) {
    const u32x4_t v = bm4[bm_slot4(q)];
    const int c = __popc(v.x) + __popc(v.y) + __popc(v.z) + __popc(v.w);
    cnt += c;
    nz |= (uint32_t)(c != 0) << (q - q0);
  }
  int32_t tot;
  int32_t o = block_exclusive_scan<int32_t>(cnt, sm, tot);
  int32_t* out = P.idx + (int64_t)u * P.max_sel;
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
  write_window(P, u, take, p, out);
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

  if (mode == MODE_RADIX && P.collected && st[ST_COMPACT]) return;  // written by the collected path
  if (chunk == 0) write_window(P, u, take, p, out);
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
  // The four rounds' counts go through two packed scans (16 bits per round;
  // a round holds at most 4096 keys): first the keys equal to tau, whose rank
  // decides which of them are taken, then the taken keys, whose prefix is the
  // output slot.  Positions are ordered by (round, thread, element).
  int32_t eqc[4];
#pragma unroll
  for (int rnd = 0; rnd < 4; ++rnd) {
    const int j0 = base + rnd * 4096 + threadIdx.x * 16;
    int32_t c = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) c += (j0 + e < end) && keys[rnd * 16 + e] == tau;
    eqc[rnd] = c;
  }
  int32_t pe[2] = {eqc[0] | (eqc[1] << 16), eqc[2] | (eqc[3] << 16)}, te[2];
  block_exclusive_scan_n<2>(pe, sm, te);
  uint32_t selmask[4];
  int32_t selc[4];
  int32_t rbase = eq_before;
#pragma unroll
  for (int rnd = 0; rnd < 4; ++rnd) {
    const int j0 = base + rnd * 4096 + threadIdx.x * 16;
    const int f = (rnd & 1) * 16, w = rnd >> 1;
    int32_t r_eq = rbase + ((pe[w] >> f) & 0xffff);
    rbase += (te[w] >> f) & 0xffff;
    uint32_t m = 0;
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
      m |= (uint32_t)take_it << e;
    }
    selmask[rnd] = m;
    selc[rnd] = __builtin_popcount(m);
  }
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
// does.  Power-of-two block sizes up to 256; LDS slot i + i / BS keeps the
// threads' sequential reads on distinct banks.
constexpr int kMassTile = 4096;
template <int BS>
__global__ void __launch_bounds__(256) sel_block_mass_tiled(SelectParams P) {
  __shared__ float sv[kMassTile + kMassTile / BS];
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
    const int base = i + i / BS;  // 4 | BS, so the float4 stays inside one block
    sv[base] = v.x;
    sv[base + 1] = v.y;
    sv[base + 2] = v.z;
    sv[base + 3] = v.w;
  }
  __syncthreads();
  constexpr int NB = kMassTile / BS;
  for (int t = threadIdx.x; t < NB; t += 256) {
    const int beta = blockIdx.x * NB + t;
    if (beta * BS >= ncand) break;
    const int n = min(BS, ncand - beta * BS);
    const float* b = sv + t * (BS + 1);
    double m = 0.0;
    for (int e = 0; e < n; ++e) m += (double)b[e];
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
  SelectParams p = p_in;
  p.collected = p.block_size == 1 && p.units * p.nchunks >= kSelMinWorkgroups;
  const dim3 grid_c(p.nchunks, p.units);
  hipError_t e;
#define HS2_L(name, kern, grid)                                   \
  do {                                                            \
    TimedLaunch tl_(name, s);                                     \
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, p);           \
    if ((e = hipGetLastError()) != hipSuccess) return e;          \
  } while (0)
  if (!(p.pre_hist0 && p.block_size == 1)) HS2_L("select_init", sel_init, dim3(p.units));
  if (p.block_size == 1) {
    const bool small = p.units * p.nchunks <= 512;  // up to about two workgroups per CU: latency-bound passes
    if (!p.pre_hist0) {
      if (small) HS2_L("select_hist", (sel_hist<0, true>), grid_c);
      else HS2_L("select_hist", (sel_hist<0, false>), grid_c);
    }
    if (small) HS2_L("select_hist", (sel_hist<1, true>), grid_c);
    else HS2_L("select_hist", (sel_hist<1, false>), grid_c);
    // The collected path saves two full reads of the scores but adds two
    // launches: taken where the passes are throughput-bound.
    if (p.collected) {
      HS2_L("select_collect", sel_collect, grid_c);
      // the LDS attribute is set once per device, for the largest bitmap
      static std::atomic<uint64_t> attr_done{0};
      int dev = 0;
      if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
      const uint64_t bit = 1ull << (dev & 63);
      if (!(attr_done.load() & bit)) {
        if ((e = hipFuncSetAttribute((const void*)sel_finish, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)finish_lds_bytes(kCompactMaxCand))) != hipSuccess)
          return e;
        attr_done.fetch_or(bit);
      }
      const size_t lds = finish_lds_bytes(p.N);
      TimedLaunch tl_("select_finish", s);
      hipLaunchKernelGGL(sel_finish, dim3(p.units), dim3(256), lds, s, p);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
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
