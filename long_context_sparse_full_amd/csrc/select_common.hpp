// Device pieces of the token selection that other kernels run as well: the
// per-row selection state, its initialisation, the order-preserving key of a
// score and the first radix digit's histogram.  The full-layer kernels use
// them to set a row's selection up and to count its first digit while they
// write the scores (the top-k with forced window of the HySparse2 cross
// decoder: zgeo.com.cn "xiaomi-mimo-v3-hysparse2-long-context-geo", "core
// principle"; javabetter.cn "mimo-v3-hysparse2", changes versus HySparse).
#pragma once

#include "hs2_internal.hpp"

namespace hs2 {

// per-row state words; each selection kernel reads the slots written by the
// kernels before it and writes its own
// (ST_DONE, ST_PLO, ST_PHI: the bracketed path's settled flag and bracket)
enum { ST_MODE = 0, ST_NCAND = 1, ST_TAKE = 2, ST_P = 3, ST_PREFIX1 = 4, ST_NEED1 = 5,
       ST_PREFIX2 = 6, ST_NEED2 = 7, ST_DONE = 8, ST_PLO = 9, ST_PHI = 10, ST_WORDS = 16 };
enum { MODE_RADIX = 0, MODE_ALL = 1, MODE_NONE = 2 };

// Candidates of a query at position p: [0, p - window], so ncand of them; the
// selection takes min(k, ncand) of them (token mode) or min(k, blocks).
__device__ __forceinline__ int sel_ncand(int p, int window) { return max(0, p - window + 1); }
__device__ __forceinline__ int sel_take(int ncand, int k, int block_size) {
  if (block_size == 1) return min(k, ncand);
  const int nb = ncand > 0 ? (ncand - 1) / block_size + 1 : 0;
  return min(k, nb);
}
__device__ __forceinline__ int sel_mode(int take, int ncand, int block_size) {
  return (take == 0) ? MODE_NONE : ((block_size == 1 && take == ncand) ? MODE_ALL : MODE_RADIX);
}

// State of row u and, in token mode, its three digit histograms cleared; run
// by one whole workgroup of nthreads threads (thread tid).
__device__ __forceinline__ void sel_init_row(int32_t* st, int32_t* hist3, int p, int k, int window, int block_size,
                                             int tid, int nthreads) {
  const int ncand = sel_ncand(p, window);
  const int take = sel_take(ncand, k, block_size);
  if (tid == 0) {
    st[ST_MODE] = sel_mode(take, ncand, block_size);
    st[ST_NCAND] = ncand;
    st[ST_TAKE] = take;
    st[ST_P] = p;
    st[ST_DONE] = 0;
  }
  if (block_size == 1)
    for (int i = tid; i < 3 * kHistBins; i += nthreads) hist3[i] = 0;
}

// Radix key of a non-negative score: its bit pattern, whose unsigned order is
// the numeric order (-0 counts as +0).
__device__ __forceinline__ uint32_t score_key(float s) {
  const uint32_t u = __float_as_uint(s);
  return u == 0x80000000u ? 0u : u;
}

// First digit (key bits 31..20) of NK keys per thread added to the LDS
// histogram h[kHistBins] (valid: bit i = key i counts).  A row's keys cluster
// in a few neighbouring digits (they share exponent and leading mantissa
// bits), which would serialise LDS atomics on a few addresses.  So each thread
// counts the keys of an 8-digit window, from three digits below the digit of
// the wave's first key, in 8-bit fields of one 64-bit word (NK <= 255: no
// field overflows); keys outside the window use LDS atomics.  The window
// counts are summed over the wave in 16-bit fields (64 * NK < 65536) and
// added by one lane.
template <int NK>
__device__ __forceinline__ void hist_digit0(const uint32_t (&key)[NK], uint64_t valid, int32_t* h) {
  static_assert(NK <= 64 && NK * 64 < 65536, "field widths");
  const uint32_t first = __builtin_amdgcn_readfirstlane(key[0] >> 20);
  const uint32_t wbase = first >= 3 ? first - 3 : 0;
  uint64_t acc = 0;
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const bool v = valid >> i & 1;
    const uint32_t bin = key[i] >> 20;
    const uint32_t off = bin - wbase;
    const bool in = off < 8u;
    acc += (v && in) ? 1ull << (8 * off) : 0ull;
    if (v && !in) atomicAdd(&h[bin], 1);
  }
  // fields 0-3 and 4-7 widened to 16 bits, then summed over the wave
  uint64_t lo = 0, hi = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    lo |= ((acc >> (8 * j)) & 0xFFull) << (16 * j);
    hi |= ((acc >> (8 * j + 32)) & 0xFFull) << (16 * j);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lo += __shfl_xor(lo, o);
    hi += __shfl_xor(hi, o);
  }
  if ((threadIdx.x & 63) == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int32_t c0 = (int32_t)((lo >> (16 * j)) & 0xFFFFull), c1 = (int32_t)((hi >> (16 * j)) & 0xFFFFull);
      if (c0 && wbase + j < (uint32_t)kHistBins) atomicAdd(&h[wbase + j], c0);
      if (c1 && wbase + 4 + j < (uint32_t)kHistBins) atomicAdd(&h[wbase + 4 + j], c1);
    }
  }
}

}  // namespace hs2
