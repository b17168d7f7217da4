// Internal declarations shared by the C-ABI shim and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hs2.h"

namespace hs2 {

// ---------------------------------------------------------------------------
// full / sparse attention "scan" launches
// ---------------------------------------------------------------------------
// A unit is (b, token-pack, kv group g).  Its rows are the query heads of the
// group for `tpack` consecutive tokens: row r = tl*G + i <-> token
// t = tp*tpack + tl, head h = g*G + i.  Rows never exceed 16 (one MFMA tile).
struct ScanParams {
  const void* k;
  const void* v;
  int64_t sb, sh, sn;  // K/V strides, elements
  const float* k_scale;
  const float* v_scale;
  int B, Hkv, N, D, G;
  const void* q;
  int Tq, Hq, q_pos0;
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
  // fused full layer (one cooperative launch): nsplit workgroups per unit
  float* scores;       // [B, Tq, Hkv, N]
  int lds_slots;       // tiles per workgroup whose codes stay in LDS; later tiles use lg16/lgmax
  uint64_t* flags;     // [units * nsplit] grid-barrier arrival words
  uint64_t epoch;      // this launch's arrival value (unique per launch)
  // multi-query chunk path: log2-domain LSE per (unit, row) from the merge,
  // read by the score pass
  const float* lse2_in;
  // fused full layer + token selection (tpack = 1): top-k of C = [0, p - window]
  // with the window appended; output idx/count/max_sel above.  sel_hist:
  // [units][3][kHistBins] radix histograms; sel_stepcnt: [units][nsteps][2]
  // (above-threshold, equal-to-threshold) counts per workgroup step.  nullptr
  // sel_hist = no selection.
  int sel_k, sel_window, sel_nsteps;
  int32_t* sel_hist;
  int32_t* sel_stepcnt;
};

// Multi-query chunk path: a workgroup of 4 waves, each holding kFlashRG
// groups of 16 query rows (tpack tokens x G heads), so kChunkPacks packs per
// workgroup share every K/V tile through LDS.  The planner takes it when there
// are at least kChunkMinPacks packs per (b, kv head).
constexpr int kFlashRG = 2;
constexpr int kChunkPacks = 4 * kFlashRG;
constexpr int kChunkMinPacks = 4;
// Chunk position splits: about this many full-pass work items in all.
#ifndef HS2_CHUNK_TARGET_WGS
#define HS2_CHUNK_TARGET_WGS 1024
#endif

constexpr int kSelChunk = 16384;  // candidates per workgroup in the select passes
constexpr int kHistBins = 4096;  // 12-bit digits
// Workgroups per selection pass from which the passes are throughput-bound
// (larger grids take the collected path).
constexpr int kSelMinWorkgroups = 2048;
// collected selection path: largest k, largest 24-bit threshold bin, and the
// per-row list words (positions above the bin, then the bin's keys and positions)
constexpr int kCompactTake = 2048;
constexpr int kCompactBin = 1024;
constexpr int kCandWords = kCompactTake + 2 * kCompactBin;
// candidates per row of the collected path (its finishing step keeps a bitmap
// of them in LDS: 128 KiB at this size)
constexpr int kCompactMaxCand = 1 << 20;

// Fused decode full layer: workgroup shape and LDS plan shared by the launcher
// and the host planner.
// 8 waves (2 per SIMD) per workgroup; 4 for the bf16 D=128 scan, whose two
// in-flight 16 KiB tiles per wave need the whole register file of a SIMD.
#ifndef HS2_FUSED_FP8_WAVES
#define HS2_FUSED_FP8_WAVES 8
#endif
__host__ __device__ constexpr int fused_waves(int kv_dtype, int D) {
  return (kv_dtype == HS2_BF16 && D == 128) ? 4 : (kv_dtype == HS2_FP8_E4M3FN ? HS2_FUSED_FP8_WAVES : 8);
}
constexpr int kFusedLdsBytes = 160 * 1024;
__host__ __device__ inline int fused_merge_bytes(int rows, int D) { return 4 * rows * (D + 4) * 4; }
// fused selection: LDS histogram, scan scratch and up to kFusedSelMaxSteps step
// prefixes per workgroup; grid barriers: 1 (layer) + 4 (selection)
constexpr int kFusedSelMaxSteps = 64;
constexpr int kFusedSelectLds = (kHistBins + 16 + 2 * kFusedSelMaxSteps) * 4;
constexpr int kFusedBarriers = 5;
__host__ __device__ inline int fused_slot_bytes(int rows) { return rows * (32 * 2 + 4); }

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
  // own set-up would; sel_state nullptr = no selection
  int32_t* sel_state;
  int32_t* sel_hist;
  int sel_k, sel_window, q_pos0;
};

struct ScoreParams {
  const uint16_t* lg16;
  const float* lgmax;
  const float* lse2;
  int64_t npad;
  int rows, tpack, n_tpacks, G, Hkv, Tq, N, q_pos0;
  float* scores;  // [B, Tq, Hkv, N]
  // one query token per unit: also count the first radix digit of every
  // candidate's score (positions [0, p - sel_window]) into the selection's
  // pass-0 histogram sel_hist + unit * 3 * kHistBins, cleared beforehand by the
  // merge; rows whose selection needs no radix pass are skipped.  nullptr = none
  int32_t* sel_hist;
  int sel_k, sel_window;
};

// ---------------------------------------------------------------------------
// selection
// ---------------------------------------------------------------------------

struct SelectParams {
  const float* scores;  // [units][N]
  int units, Tq, Hkv, N, q_pos0, k, window, block_size, max_sel, nchunks;
  int32_t* idx;
  int32_t* count;
  int32_t* state;   // [units][16]
  int32_t* hist;    // [units][3][4096] digit histograms of the three passes
  int32_t* cnt;     // [units][nchunks][258]: keys above the 24-bit prefix, suffix sums of the last digit
  int32_t* cand;    // [units][kCandWords]: the collected path's lists
  double* bmass;    // [units][nblocks_max] (block mode)
  int nblocks_max;
  int pre_hist0;    // token mode: state and pass-0 histogram already built (merge + score pass)
  int collected;    // set by the launcher: the collected path runs (rows may finish there)
};

// launchers (return hipError_t of the launch)
hipError_t launch_scan(const ScanParams& p, int kv_dtype, bool gather, bool write_logits, hipStream_t s);
hipError_t launch_gather_split(const ScanParams& p, int kv_dtype, hipStream_t s);
// Cooperative launch of the fused full layer (scan, grid barrier, combine,
// scores).  Returns hipErrorNotSupported when the device cannot co-schedule
// the grid; the caller then uses the multi-kernel path.
hipError_t launch_scan_fused(const ScanParams& p, int kv_dtype, int units, hipStream_t s);
int fused_max_workgroups(int kv_dtype, int D);  // co-resident workgroups, 0 if unavailable
// Multi-query chunk full layer: MFMA pass writing split partials (then
// launch_combine), and the score pass recomputing QK^T against the merged LSE.
hipError_t launch_chunk_full(const ScanParams& p, int kv_dtype, hipStream_t s);
hipError_t launch_chunk_score(const ScanParams& p, int kv_dtype, hipStream_t s);
hipError_t launch_combine(const CombineParams& p, int units, hipStream_t s);
hipError_t launch_score(const ScoreParams& p, int units, hipStream_t s);
hipError_t launch_select(const SelectParams& p, hipStream_t s);
// K/V bridge output: the cache rows of one batch entry from the first new
// position on (element (h, t, d) at h*sh + t*sn + d); FP8 caches pass that
// batch entry's per-head scales (Hkv each), bf16 caches nullptr.
struct BridgeOut {
  void* k;
  void* v;
  int64_t sn, sh;
  const float* k_scale;
  const float* v_scale;
};
hipError_t launch_bridge(const uint16_t* hidden, int T, int dm, const uint16_t* w, int Hkv, int D,
                         const BridgeOut& out, hipStream_t s);
hipError_t launch_debug_e4m3fn(const uint8_t* codes, float* out, int n, hipStream_t s);
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* out, int blocks, hipStream_t s);

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
