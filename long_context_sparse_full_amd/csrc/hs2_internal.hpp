// Internal declarations shared by the C-ABI shim and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hs2.h"

namespace hs2 {

// Position of query token 0 of batch entry b: the per-batch array when the
// caller gave one (clamped into [0, N - Tq] so that every access stays inside
// the cache), else the call's q_pos0.
__host__ __device__ inline int qpos_of(const int32_t* qpos_b, int q_pos0, int b, int N, int Tq) {
  if (!qpos_b) return q_pos0;
  const int v = qpos_b[b];
  return v < 0 ? 0 : (v > N - Tq ? N - Tq : v);
}

// ---------------------------------------------------------------------------
// full / sparse attention "scan" launches
// ---------------------------------------------------------------------------
// A unit is (b, token-pack, kv group g).  Its rows are the query heads of the
// group for `tpack` consecutive tokens: row r = tl*G + i <-> token
// t = tp*tpack + tl, head h = g*G + i.  Rows never exceed 16 (one MFMA tile).
// A paged cache's row map: logical row j of sequence b is physical row
// (page << shift) | (j & (2^shift - 1)) of the pool, page = the table entry
// [b * per_seq + (j >> shift)] clamped to [0, pool).  Pages hold 2^shift >= 32
// rows, so an aligned 32-row tile never straddles two pages.
struct PageMap {
  const int32_t* table;  // nullptr = contiguous cache
  int shift, per_seq, pool;
};
__device__ __forceinline__ int phys_row(const PageMap& M, int b, int j) {
  const int pg = min(max(M.table[(int64_t)b * M.per_seq + (j >> M.shift)], 0), M.pool - 1);
  return (pg << M.shift) | (j & ((1 << M.shift) - 1));
}

struct ScanParams {
  const void* k;
  const void* v;
  int64_t sb, sh, sn;  // K/V strides, elements
  const float* k_scale;
  const float* v_scale;
  int B, Hkv, N, D, G;
  const void* q;
  int Tq, Hq, q_pos0;
  const int32_t* qpos_b;  // per-batch q_pos0 [B] (device), or nullptr
  float scale_log2;  // softmax_scale * log2(e)
  int tpack;         // tokens per unit
  int n_tpacks;      // ceil(Tq / tpack)
  int rows;          // tpack * G
  int nsplit;        // position splits per unit
  int split_len;     // positions per split (multiple of 256)
  float* part_ml;    // [units][nsplit][16][2]   (max, sum) in log2 units
  float* part_o;     // [units][nsplit][16][D]   unnormalised output
  // per-head logits for the score pass, 16-bit log-domain code relative to the
  // row's maximum over each aligned 32-position tile (see the score kernel)
  uint16_t* lg16;    // [units][rows][npad]  code = round((tile max - x) * 4096), 65535 = below range
  float* lgmax;      // [units][npad/32][rows] tile maxima (log2 domain)
  int64_t npad;
  // gather (sparse layer) mode: one unit per (b, t, g), tpack = 1
  const int32_t* idx;
  const int32_t* count;
  int max_sel;
  void* out;         // [B, Tq, Hq, D] in q's element type
  float* lse;        // [B, Tq, Hq] natural log (nullable)
  int32_t* gcounter; // split gather: per-(b, t, g) arrival counters (zero between calls)
  // multi-query chunk score pass: scores [B, Tq, Hkv, N]
  float* scores;
  // sliding-window attention: query t attends to [p - band + 1, p] (0 = no
  // lower limit).  Gathers then read that contiguous range instead of a list
  // (idx unused), and the chunk pass, with one split, writes out / lse itself.
  int band;
  // multi-query chunk path: log2-domain LSE per (unit, row) from the merge,
  // read by the score pass
  const float* lse2_in;
  // full layer with the token selection after it, one query token per unit
  // (tpack = 1): the scan's first split of each unit sets the unit's
  // selection row up (state words, digit histograms cleared) as the
  // selection's own set-up would; sel_state nullptr = none
  int32_t* sel_state;
  int32_t* sel_hist;
  int sel_k, sel_window;
  // paged cache (full layer with one query token per unit, and the gathers):
  // row j of sequence b lies at physical row phys_row(b, j) of a pool shared
  // by the sequences (stride_b 0); ptab nullptr = contiguous rows
  PageMap pages;
};

// Multi-query chunk path: a workgroup of 4 waves, each holding kFlashRG
// groups of 16 query rows (tpack tokens x G heads), so kChunkPacks packs per
// workgroup share every K/V tile through LDS.  The planner takes it when there
// are at least kChunkMinPacks packs per (b, kv head).
constexpr int kFlashRG = 2;
constexpr int kChunkPacks = 4 * kFlashRG;
constexpr int kChunkMinPacks = 4;
// Chunk position splits.  The full pass holds three workgroups per CU (48 KiB
// LDS rings), so about 768 work items fill the 256 CUs in one round (1024
// left a second round a third full: 5% slower); the score pass holds four per
// CU and splits the positions on its own, about 1024 work items in all.
constexpr int64_t kChunkTargetWgs = 768;
constexpr int64_t kChunkScoreTargetWgs = 1024;

constexpr int kSelChunk = 16384;  // candidates per workgroup in the select passes
constexpr int kHistBins = 4096;  // 12-bit digits
// Workgroups per selection pass (units x chunks) from which a grid takes the
// bracketed path: one pass over the scores instead of four.
constexpr int kSelMinWorkgroups = 2048;
// bracketed path: largest k it settles, largest bin between the bracket's
// bounds, and the list words of each chunk (positions above the bin, then the
// bin's positions and keys)
constexpr int kCompactTake = 2048;
constexpr int kCompactBin = 4096;
constexpr int kCandWords = kCompactTake + 2 * kCompactBin;
// sample of a row for its bracket: every SR-th run of 64 positions, SR at
// least kBracketStride (rows of more than kBracketRuns runs), at most
// kBracketRuns runs
constexpr int kBracketRuns = 256;
constexpr int kBracketStride = 16;
// chunks per row the bracketed path's finishing step gathers from (rows of
// up to 4M candidates; longer rows take the per-row kernel)
constexpr int kFinishMaxChunks = 256;
__host__ __device__ inline bool sel_bracketed(int units, int nchunks) {
  return (int64_t)units * nchunks >= kSelMinWorkgroups;
}

struct CombineParams {
  const float* part_ml;
  const float* part_o;
  int nsplit, rows, tpack, n_tpacks, G, Hkv, Hq, Tq, D;
  const float* v_scale;  // FP8 only, [B*Hkv]
  int out_bf16;
  void* out;
  float* lse;    // natural log, nullable
  float* lse2;   // [units][rows] log2-domain, for the score pass
  // token selection prepared by the merge (one query token per unit): the
  // state words and digit histograms of row `unit` at sel_state + unit * 16
  // and sel_hist + unit * 3 * kHistBins are initialised as the selection's
  // own set-up would (candidates [0, p - sel_window]: the selection's
  // candidate window); sel_state nullptr = no selection
  int32_t* sel_state;
  int32_t* sel_hist;
  int sel_k, sel_window, q_pos0, N;
  const int32_t* qpos_b;  // per-batch q_pos0 [B] (device), or nullptr
};

struct ScoreParams {
  const uint16_t* lg16;
  const float* lgmax;
  const float* lse2;
  int64_t npad;
  int rows, tpack, n_tpacks, G, Hkv, Tq, N, q_pos0;
  const int32_t* qpos_b;  // per-batch q_pos0 [B] (device), or nullptr
  float* scores;  // [B, Tq, Hkv, N]
  // one query token per unit: also count the first radix digit of every
  // candidate's score (positions [0, p - sel_window], sel_window being the
  // selection's candidate window) into the selection's
  // pass-0 histogram sel_hist + unit * 3 * kHistBins, cleared beforehand by the
  // merge; rows whose selection needs no radix pass are skipped.  nullptr = none
  int32_t* sel_hist;
  int sel_k, sel_window;
  // The query and cache, for the exact terms of saturated codes (the score
  // pass recomputes such a logit from q and the cache row).
  const void* q;
  int Hq, D, kv_dtype;
  const void* k;
  int64_t sb, sh, sn;     // cache strides, elements
  const float* k_scale;   // FP8 only
  float scale_log2;       // softmax_scale * log2(e)
  PageMap pages;          // paged cache (see ScanParams)
};

// ---------------------------------------------------------------------------
// selection
// ---------------------------------------------------------------------------

struct SelectParams {
  const float* scores;  // [units][N]
  int units, Tq, Hkv, N, q_pos0, k, window, block_size, max_sel, nchunks;
  const int32_t* qpos_b;  // per-batch q_pos0 [B] (device), or nullptr
  // candidates of a query at p: [0, p - cand_window]; cand_window = window,
  // or 0 when the window competes (then a last kernel places the window after
  // the selected positions below it)
  int cand_window, competes;
  int32_t* idx;
  int32_t* count;
  int32_t* state;   // [units][16]
  int32_t* hist;    // [units][3][4096] digit histograms of the three passes
  int32_t* cnt;     // radix path: [units][nchunks][258]: keys above the 24-bit prefix, suffix sums of the
                    // last digit; bracketed path: [units][nchunks][4 waves][2] list lengths
  int32_t* cand;    // bracketed path: [units][nchunks][kCandWords] each chunk's lists, a quarter per wave
  double* bmass;    // [units][nblocks_max] (block mode)
  int nblocks_max;
  int pre_hist0;    // token mode: state and pass-0 histogram already built (merge + score pass)
};

// launchers (return hipError_t of the launch)
hipError_t launch_scan(const ScanParams& p, int kv_dtype, bool gather, bool write_logits, hipStream_t s);
hipError_t launch_gather_split(const ScanParams& p, int kv_dtype, hipStream_t s);
// Multi-query chunk full layer: MFMA pass writing split partials (then
// launch_combine), and the score pass recomputing QK^T against the merged LSE.
hipError_t launch_chunk_full(const ScanParams& p, int kv_dtype, hipStream_t s);
hipError_t launch_chunk_score(const ScanParams& p, int kv_dtype, hipStream_t s);
hipError_t launch_combine(const CombineParams& p, int units, hipStream_t s);
// merge != nullptr (selection with one query token per unit, bf16/FP8): the
// full layer's merge runs inside the score launch.
hipError_t launch_score(const ScoreParams& p, int units, hipStream_t s, const CombineParams* merge = nullptr);
hipError_t launch_select(const SelectParams& p, hipStream_t s);
// K/V bridge outputs: per layer, the cache of one batch entry (row n of head
// h at k/v + h*sh + n*sn), new rows from pos0 on; FP8 caches pass that batch
// entry's per-head scales (Hkv each), bf16 caches nullptr.
struct BridgeOut {
  void* k;
  void* v;
  int64_t sn, sh;
  float* k_scale;
  float* v_scale;
};
constexpr int kMaxBridgeLayers = 16;
struct BridgeLayers {
  int L, pos0;
  BridgeOut out[kMaxBridgeLayers];
  // FP8 scale maintenance (nullptr y: the projection is encoded at once with
  // the scales as they are): the fp32 projections [L][T][2 Hkv D], and per
  // (layer, K/V, head) the bit pattern of max |y| and the scale on entry
  float* y;
  uint32_t* amax;
  float* old_scale;
};
hipError_t launch_bridge(const uint16_t* hidden, int T, int dm, const uint16_t* w, int Hkv, int D,
                         const BridgeLayers& out, hipStream_t s);
hipError_t launch_debug_e4m3fn(const uint8_t* codes, float* out, int n, hipStream_t s);
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* out, int blocks, hipStream_t s);
// Read-pattern probe of the decode scan (same plan and grid as launch_scan
// over the full cache); `codes` adds the scan's code stores.
hipError_t launch_scan_read_probe(const ScanParams& p, int kv_dtype, bool codes, hipStream_t s);

// timing hooks used by the launchers
struct TimedLaunch {
  TimedLaunch(const char* name, hipStream_t s);
  ~TimedLaunch();
  const char* name_;
  hipStream_t s_;
  void* ev0_;
  void* ev1_;
};

}  // namespace hs2
