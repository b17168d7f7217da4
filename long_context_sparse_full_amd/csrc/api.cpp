// C-ABI shim of the HySparse2 cross-decoder hot path: argument validation,
// workspace planning, dispatch to the gfx950 kernels, per-kernel event timing.
// Validation never touches the GPU, so every error path runs without a device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <ctime>
#include <mutex>
#include <string>
#include <vector>

#include "hs2_internal.hpp"

namespace {

thread_local std::string t_err;

int fail(int status, const std::string& msg) {
  t_err = msg;
  return status;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t rup(int64_t a, int64_t b) { return cdiv(a, b) * b; }
size_t a256(size_t x) { return (x + 255) & ~size_t(255); }
bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int esize(int dt) { return dt == HS2_F32 ? 4 : (dt == HS2_BF16 ? 2 : 1); }

int check_kv(const hs2_kv_desc* kv, const char* what) {
  const std::string w(what);
  if (!kv) return fail(HS2_ERR_INVALID_ARG, w + ": kv descriptor is NULL");
  if (!kv->k || !kv->v) return fail(HS2_ERR_INVALID_ARG, w + ": k or v pointer is NULL");
  if (kv->B <= 0 || kv->Hkv <= 0 || kv->N <= 0 || kv->D <= 0)
    return fail(HS2_ERR_INVALID_ARG, w + ": B, Hkv, N and D must be positive");
  if (kv->dtype != HS2_F32 && kv->dtype != HS2_BF16 && kv->dtype != HS2_FP8_E4M3FN)
    return fail(HS2_ERR_UNSUPPORTED, w + ": unknown kv dtype " + std::to_string(kv->dtype));
  if (kv->D != 64 && kv->D != 128)
    return fail(HS2_ERR_UNSUPPORTED, w + ": head_dim " + std::to_string(kv->D) + " (supported: 64, 128)");
  if (kv->stride_n < kv->D || kv->stride_h < 0 || kv->stride_b < 0)
    return fail(HS2_ERR_INVALID_ARG, w + ": strides must satisfy stride_n >= D, stride_h >= 0, stride_b >= 0");
  const int es = esize(kv->dtype);
  if (!al16(kv->k) || !al16(kv->v)) return fail(HS2_ERR_INVALID_ARG, w + ": k/v base pointers must be 16-byte aligned");
  if ((kv->stride_n * es) % 16 || (kv->stride_h * es) % 16 || (kv->stride_b * es) % 16)
    return fail(HS2_ERR_INVALID_ARG, w + ": k/v strides must be multiples of 16 bytes");
  if (kv->stride_n * es > (int64_t(1) << 24))
    return fail(HS2_ERR_UNSUPPORTED, w + ": k/v row stride above 16 MiB");
  if (kv->dtype == HS2_FP8_E4M3FN && (!kv->k_scale || !kv->v_scale))
    return fail(HS2_ERR_UNSUPPORTED, w + ": FP8_E4M3FN cache needs k_scale and v_scale");
  return HS2_OK;
}

int check_q(const hs2_kv_desc* kv, const void* q, int q_dtype, int Tq, int Hq, const char* what) {
  const std::string w(what);
  if (!q) return fail(HS2_ERR_INVALID_ARG, w + ": q is NULL");
  if (Tq <= 0 || Hq <= 0) return fail(HS2_ERR_INVALID_ARG, w + ": Tq and Hq must be positive");
  if (Hq % kv->Hkv) return fail(HS2_ERR_INVALID_ARG, w + ": Hq must be a multiple of Hkv");
  if (Hq / kv->Hkv > 16) return fail(HS2_ERR_UNSUPPORTED, w + ": more than 16 query heads per kv head");
  const bool ok = (q_dtype == HS2_F32 && kv->dtype == HS2_F32) || (q_dtype == HS2_BF16 && kv->dtype == HS2_BF16) ||
                  (q_dtype == HS2_BF16 && kv->dtype == HS2_FP8_E4M3FN);
  if (!ok) return fail(HS2_ERR_UNSUPPORTED, w + ": (q, kv) dtype pair not supported");
  if (!al16(q)) return fail(HS2_ERR_INVALID_ARG, w + ": q must be 16-byte aligned");
  return HS2_OK;
}

struct FullPlan {
  bool chunk;  // multi-query chunk kernels (MFMA pass + merge + score recompute)
  int tpack, n_tpacks, rows, units, nsplit, split_len;
  int64_t npad;
  size_t off_ml, off_o, off_lse2, off_lg16, off_lgmax, off_flags, total;
};

// Position splits: about HS2_SCAN_TARGET_WGS workgroups in total (4 per CU on
// 256 CUs; 8 for a bf16 cache, whose scan measured 2-3% faster with the finer
// splits while the FP8 scan measured slower), split lengths a multiple of 256
// positions (64 on the fp32 path).
#ifndef HS2_SCAN_TARGET_WGS
#define HS2_SCAN_TARGET_WGS 1024
#endif
#ifndef HS2_SCAN_TARGET_WGS_BF16
#define HS2_SCAN_TARGET_WGS_BF16 2048
#endif
FullPlan plan_full(const hs2_kv_desc* kv, int Tq, int Hq) {
  FullPlan p{};
  const int G = Hq / kv->Hkv;
  const bool f32 = kv->dtype == HS2_F32;
  p.tpack = f32 ? 1 : std::max(1, std::min(Tq, 16 / G));
  p.n_tpacks = (int)cdiv(Tq, p.tpack);
  p.rows = p.tpack * G;
  p.units = kv->B * p.n_tpacks * kv->Hkv;
  const bool g_pow2 = G == 4 || G == 8 || G == 16;  // the chunk score pass sums heads in 4-row lane groups
  p.chunk = !f32 && g_pow2 && p.n_tpacks >= hs2::kChunkMinPacks;
  if (p.chunk) {  // work items (b, block of packs, g) x position splits, HS2_CHUNK_TARGET_WGS in all
    const int64_t items = (int64_t)kv->B * cdiv(p.n_tpacks, hs2::kChunkPacks) * kv->Hkv;
    const int64_t per_item = std::max<int64_t>(1, HS2_CHUNK_TARGET_WGS / items);
    p.split_len = (int)rup(cdiv(kv->N, per_item), 128);  // whole 32-position tiles
  } else {
    const int64_t target = kv->dtype == HS2_BF16 ? HS2_SCAN_TARGET_WGS_BF16 : HS2_SCAN_TARGET_WGS;
    const int64_t per_unit = std::max<int64_t>(1, target / p.units);
    const int64_t quantum = f32 ? 64 : 256;
    p.split_len = (int)rup(cdiv(kv->N, per_unit), quantum);
  }
  p.nsplit = (int)cdiv(kv->N, p.split_len);
  p.npad = rup(kv->N, 64);
  size_t off = 0;
  p.off_ml = off;
  off = a256(off + (size_t)p.units * p.nsplit * 16 * 2 * sizeof(float));
  p.off_o = off;
  off = a256(off + (size_t)p.units * p.nsplit * 16 * kv->D * sizeof(float));
  p.off_lse2 = off;
  off = a256(off + (size_t)p.units * p.rows * sizeof(float));
  const size_t code_units = p.chunk ? 0 : (size_t)p.units;  // the chunk path stores no logit codes
  p.off_lg16 = off;
  off = a256(off + code_units * p.rows * (size_t)p.npad * sizeof(uint16_t));
  p.off_lgmax = off;
  off = a256(off + code_units * p.rows * (size_t)(p.npad / 32) * sizeof(float));
  p.off_flags = off;  // fused path: per grid barrier one word per workgroup (<= units * nsplit)
  off = a256(off + (size_t)hs2::kFusedBarriers * p.units * p.nsplit * sizeof(uint64_t));
  p.total = off;
  return p;
}

// Full-layer path selection (process-wide):
//   0 = automatic: the scan + combine + score kernels, then (for
//       hs2_full_attn_topk) the select kernels -- the fastest form measured at
//       1M context, where the cooperative launch and the selection's grid
//       barriers cost more than the scratch traffic they save;
//   1 = the fused cooperative kernel wherever the device can co-schedule it;
//   2 = as 1 with LDS code storage cut to one tile per workgroup (every later
//       tile takes the global-buffer route; exercises it at small sizes);
//   3 = never fused.
std::atomic<int> g_full_mode{0};

// Grid-barrier epochs: unique per fused launch in this process, never 0.
uint64_t next_epoch() {
  static std::atomic<uint64_t> ctr{((uint64_t)(uintptr_t)&ctr << 16) ^ ((uint64_t)time(nullptr) << 40) ^
                                   0x9e3779b97f4a7c15ull};
  uint64_t e;
  do {
    e = ctr.fetch_add(1, std::memory_order_relaxed) + 1;
  } while (e == 0);
  return e;
}

struct SelPlan {
  int units, nchunks, nblocks_max;
  size_t off_state, off_hist, off_cnt, off_cand, off_bmass, total;
};

SelPlan plan_select(int B, int Tq, int Hkv, int N, int block_size) {
  SelPlan p{};
  p.units = B * Tq * Hkv;
  p.nchunks = (int)cdiv(N, hs2::kSelChunk);
  p.nblocks_max = block_size > 1 ? (int)cdiv(N, block_size) : 0;
  size_t off = 0;
  p.off_state = off;
  off = a256(off + (size_t)p.units * 16 * sizeof(int32_t));
  if (block_size == 1) {
    p.off_hist = off;
    off = a256(off + (size_t)p.units * 3 * hs2::kHistBins * sizeof(int32_t));
    p.off_cnt = off;
    off = a256(off + (size_t)p.units * p.nchunks * 258 * sizeof(int32_t));
    p.off_cand = off;
    off = a256(off + (size_t)p.units * hs2::kCandWords * sizeof(int32_t));
  } else {
    p.off_bmass = off;
    off = a256(off + (size_t)p.units * p.nblocks_max * sizeof(double));
  }
  p.total = off;
  return p;
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

int hip_fail(hipError_t e, const char* what) {
  return fail(HS2_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// ---------------------------------------------------------------------------
// event timing
// ---------------------------------------------------------------------------
const char* const kKernelNames[] = {"full_scan",   "combine",     "score",        "select_init",
                                    "select_hist", "select_collect", "select_finish", "select_emit",
                                    "select_block_mass", "select_block_pick", "sparse_gather", "kv_bridge", "stream_read",
                                    "chunk_full",  "chunk_score", nullptr};

std::mutex g_tmu;
bool g_timing = false;
struct TimingRec {
  const char* name;
  hipEvent_t a, b;
};
std::vector<TimingRec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

namespace hs2 {
TimedLaunch::TimedLaunch(const char* name, hipStream_t s) : name_(name), s_(s), ev0_(nullptr), ev1_(nullptr) {
  if (!g_timing) return;
  std::lock_guard<std::mutex> lk(g_tmu);
  hipEvent_t a = take_event(), b = take_event();
  if (!a || !b) return;
  ev0_ = a;
  ev1_ = b;
  hipEventRecord(a, s);
}
TimedLaunch::~TimedLaunch() {
  if (!ev0_) return;
  std::lock_guard<std::mutex> lk(g_tmu);
  hipEventRecord((hipEvent_t)ev1_, s_);
  g_recs.push_back(TimingRec{name_, (hipEvent_t)ev0_, (hipEvent_t)ev1_});
}
}  // namespace hs2

extern "C" {

int hs2_abi_version(void) { return HS2_ABI_VERSION; }

int hs2_full_attn_set_mode(int mode) {
  if (mode < 0 || mode > 3) return fail(HS2_ERR_INVALID_ARG, "hs2_full_attn_set_mode: mode must be 0..3");
  g_full_mode.store(mode, std::memory_order_relaxed);
  return HS2_OK;
}

const char* hs2_status_string(int status) {
  switch (status) {
    case HS2_OK: return "ok";
    case HS2_ERR_INVALID_ARG: return "invalid argument";
    case HS2_ERR_UNSUPPORTED: return "unsupported";
    case HS2_ERR_WORKSPACE: return "workspace too small";
    case HS2_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* hs2_last_error(void) { return t_err.c_str(); }

size_t hs2_full_attn_scores_workspace(const hs2_kv_desc* kv, int32_t Tq, int32_t Hq) {
  if (!kv || kv->B <= 0 || kv->Hkv <= 0 || kv->N <= 0 || kv->D <= 0 || Tq <= 0 || Hq <= 0 || Hq % kv->Hkv) return 0;
  return plan_full(kv, Tq, Hq).total;
}

}  // extern "C"

namespace {
// Selection folded into the fused full layer (hs2_full_attn_topk).
struct SelFuse {
  int32_t k, window, max_sel;
  int32_t* idx;
  int32_t* count;
  void* ws;  // fused-selection region: histograms, then step counts
  bool done = false;
  // kernel sequence: the merge set the selection up and the score pass built
  // its first histogram (layout of plan_select over ws)
  bool hist0_done = false;
};

size_t sel_fuse_hist_bytes(int units) { return a256((size_t)units * 3 * hs2::kHistBins * sizeof(int32_t)); }
int sel_fuse_nsteps(int N) { return (int)cdiv(N, 128); }  // the smallest workgroup step (4 waves)
size_t sel_fuse_bytes(int units, int N) {
  return sel_fuse_hist_bytes(units) + a256((size_t)units * sel_fuse_nsteps(N) * 2 * sizeof(int32_t));
}

int full_layer(const hs2_kv_desc* kv, const void* q, hs2_dtype q_dtype, int32_t Tq, int32_t Hq, int32_t q_pos0,
               float softmax_scale, void* out, float* lse, float* scores, void* workspace, size_t workspace_bytes,
               hipStream_t stream, SelFuse* sel);
// hs2_select_topk_window; pre_hist0: the row state and first histogram are
// already built (full layer's merge and score pass)
int select_impl(const float* scores, int32_t B, int32_t Tq, int32_t Hkv, int32_t N, int32_t q_pos0, int32_t k,
                int32_t window, int32_t block_size, int32_t* idx, int32_t* count, int32_t max_sel, void* workspace,
                size_t workspace_bytes, hipStream_t stream, bool pre_hist0);
}  // namespace

extern "C" {

int hs2_full_attn_scores(const hs2_kv_desc* kv, const void* q, hs2_dtype q_dtype, int32_t Tq, int32_t Hq,
                         int32_t q_pos0, float softmax_scale, void* out, float* lse, float* scores, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  return full_layer(kv, q, q_dtype, Tq, Hq, q_pos0, softmax_scale, out, lse, scores, workspace, workspace_bytes,
                    stream, nullptr);
}

}  // extern "C"

namespace {
int full_layer(const hs2_kv_desc* kv, const void* q, hs2_dtype q_dtype, int32_t Tq, int32_t Hq, int32_t q_pos0,
               float softmax_scale, void* out, float* lse, float* scores, void* workspace, size_t workspace_bytes,
               hipStream_t stream, SelFuse* sel) {
  int st = check_kv(kv, "hs2_full_attn_scores");
  if (st) return st;
  if ((st = check_q(kv, q, q_dtype, Tq, Hq, "hs2_full_attn_scores"))) return st;
  if (q_pos0 < 0 || (int64_t)q_pos0 + Tq > kv->N)
    return fail(HS2_ERR_INVALID_ARG, "hs2_full_attn_scores: need 0 <= q_pos0 and q_pos0 + Tq <= N");
  if (!out || !scores) return fail(HS2_ERR_INVALID_ARG, "hs2_full_attn_scores: out and scores must not be NULL");
  if (!al16(out) || !al16(scores) || (lse && ((uintptr_t)lse & 3)))
    return fail(HS2_ERR_INVALID_ARG, "hs2_full_attn_scores: out/scores must be 16-byte aligned, lse 4-byte");
  if (!std::isfinite(softmax_scale)) return fail(HS2_ERR_INVALID_ARG, "hs2_full_attn_scores: softmax_scale not finite");
  const FullPlan pl = plan_full(kv, Tq, Hq);
  if (!workspace || workspace_bytes < pl.total)
    return fail(HS2_ERR_WORKSPACE, "hs2_full_attn_scores: workspace needs " + std::to_string(pl.total) + " bytes");
  if ((uintptr_t)workspace & 255) return fail(HS2_ERR_INVALID_ARG, "hs2_full_attn_scores: workspace must be 256-byte aligned");

  hs2::ScanParams p{};
  p.k = kv->k;
  p.v = kv->v;
  p.sb = kv->stride_b;
  p.sh = kv->stride_h;
  p.sn = kv->stride_n;
  p.k_scale = kv->k_scale;
  p.v_scale = kv->v_scale;
  p.B = kv->B;
  p.Hkv = kv->Hkv;
  p.N = kv->N;
  p.D = kv->D;
  p.G = Hq / kv->Hkv;
  p.q = q;
  p.Tq = Tq;
  p.Hq = Hq;
  p.q_pos0 = q_pos0;
  p.scale_log2 = softmax_scale * 1.44269504088896340736f;
  p.tpack = pl.tpack;
  p.n_tpacks = pl.n_tpacks;
  p.rows = pl.rows;
  p.nsplit = pl.nsplit;
  p.split_len = pl.split_len;
  p.part_ml = at<float>(workspace, pl.off_ml);
  p.part_o = at<float>(workspace, pl.off_o);
  p.lg16 = at<uint16_t>(workspace, pl.off_lg16);
  p.lgmax = at<float>(workspace, pl.off_lgmax);
  p.npad = pl.npad;
  hipError_t e;

  // fused path: one workgroup per CU slot, nsplit of them per unit
  if (pl.chunk) {  // many query tokens: MFMA pass -> merge -> score recompute
    hs2::CombineParams c{};
    c.part_ml = p.part_ml;
    c.part_o = p.part_o;
    c.nsplit = pl.nsplit;
    c.rows = pl.rows;
    c.tpack = pl.tpack;
    c.n_tpacks = pl.n_tpacks;
    c.G = p.G;
    c.Hkv = kv->Hkv;
    c.Hq = Hq;
    c.Tq = Tq;
    c.D = kv->D;
    c.v_scale = kv->dtype == HS2_FP8_E4M3FN ? kv->v_scale : nullptr;
    c.out_bf16 = q_dtype == HS2_BF16;
    c.out = out;
    c.lse = lse;
    c.lse2 = at<float>(workspace, pl.off_lse2);
    if ((e = hs2::launch_chunk_full(p, kv->dtype, stream)) != hipSuccess) return hip_fail(e, "chunk_full launch");
    if ((e = hs2::launch_combine(c, pl.units, stream)) != hipSuccess) return hip_fail(e, "combine launch");
    p.lse2_in = c.lse2;
    p.scores = scores;
    if ((e = hs2::launch_chunk_score(p, kv->dtype, stream)) != hipSuccess) return hip_fail(e, "chunk_score launch");
    return HS2_OK;
  }

  const int mode = g_full_mode.load(std::memory_order_relaxed);
  const bool want_fused = mode == 1 || mode == 2;
  const int nwg = want_fused ? hs2::fused_max_workgroups(kv->dtype, kv->D) : 0;
  if (nwg >= pl.units) {
    const int W = hs2::fused_waves(kv->dtype, kv->D);
    const int64_t step = 32 * W;
    const int64_t su = std::max<int64_t>(1, std::min<int64_t>({nwg / pl.units, pl.nsplit, cdiv(kv->N, step)}));
    const int64_t scan_steps = cdiv((int64_t)q_pos0 + Tq, step);  // steps covering [0, last query position]
    const int64_t need = cdiv(scan_steps, su) * W;                 // tiles of the busiest workgroup
    const int64_t fit = (hs2::kFusedLdsBytes - hs2::fused_merge_bytes(pl.rows, kv->D) - 256) /
                        hs2::fused_slot_bytes(pl.rows);
    // the selection keeps every score of a workgroup in registers: 4 octets per
    // thread, i.e. at most kFusedSelMaxSteps steps per workgroup over [0, N)
    const int64_t my_steps = cdiv(cdiv(kv->N, step), su);
    const bool fuse_sel = sel != nullptr && pl.tpack == 1 && p.G <= 8 && my_steps <= hs2::kFusedSelMaxSteps;
    hs2::ScanParams f = p;
    f.nsplit = (int)su;
    f.lds_slots = (int)std::min(need, mode == 2 ? (int64_t)1 : fit);
    f.scores = scores;
    f.out = out;
    f.lse = lse;
    f.flags = at<uint64_t>(workspace, pl.off_flags);
    f.epoch = next_epoch();
    if (fuse_sel) {
      f.sel_k = sel->k;
      f.sel_window = sel->window;
      f.sel_nsteps = (int)cdiv(kv->N, step);
      f.sel_hist = static_cast<int32_t*>(sel->ws);
      f.sel_stepcnt = at<int32_t>(sel->ws, sel_fuse_hist_bytes(pl.units));
      f.idx = sel->idx;
      f.count = sel->count;
      f.max_sel = sel->max_sel;
    }
    if (sel == nullptr || fuse_sel) {
      e = hs2::launch_scan_fused(f, kv->dtype, pl.units, stream);
      if (e == hipSuccess) {
        if (sel) sel->done = fuse_sel;
        return HS2_OK;
      }
      if (e != hipErrorNotSupported && e != hipErrorCooperativeLaunchTooLarge)
        return hip_fail(e, "fused full layer launch");
      (void)hipGetLastError();  // the device declined the cooperative grid: use the kernel sequence
    }
  }

  e = hs2::launch_scan(p, kv->dtype, false, true, stream);
  if (e != hipSuccess) return hip_fail(e, "full_scan launch");

  hs2::CombineParams c{};
  c.part_ml = p.part_ml;
  c.part_o = p.part_o;
  c.nsplit = pl.nsplit;
  c.rows = pl.rows;
  c.tpack = pl.tpack;
  c.n_tpacks = pl.n_tpacks;
  c.G = p.G;
  c.Hkv = kv->Hkv;
  c.Hq = Hq;
  c.Tq = Tq;
  c.D = kv->D;
  c.v_scale = kv->dtype == HS2_FP8_E4M3FN ? kv->v_scale : nullptr;
  c.out_bf16 = q_dtype == HS2_BF16;
  c.out = out;
  c.lse = lse;
  c.lse2 = at<float>(workspace, pl.off_lse2);
  // one query token per unit: the merge sets the selection's rows up and the
  // score pass counts their first digit, which saves the selection two passes
  const bool pre_sel = sel != nullptr && pl.tpack == 1;
  int32_t* sel_hist = nullptr;
  if (pre_sel) {
    const SelPlan sp = plan_select(kv->B, Tq, kv->Hkv, kv->N, 1);
    c.sel_state = at<int32_t>(sel->ws, sp.off_state);
    c.sel_hist = sel_hist = at<int32_t>(sel->ws, sp.off_hist);
    c.sel_k = sel->k;
    c.sel_window = sel->window;
    c.q_pos0 = q_pos0;
  }
  if ((e = hs2::launch_combine(c, pl.units, stream)) != hipSuccess) return hip_fail(e, "combine launch");

  hs2::ScoreParams s{};
  s.lg16 = p.lg16;
  s.lgmax = p.lgmax;
  s.lse2 = c.lse2;
  s.npad = pl.npad;
  s.rows = pl.rows;
  s.tpack = pl.tpack;
  s.n_tpacks = pl.n_tpacks;
  s.G = p.G;
  s.Hkv = kv->Hkv;
  s.Tq = Tq;
  s.N = kv->N;
  s.q_pos0 = q_pos0;
  s.scores = scores;
  s.sel_hist = sel_hist;
  s.sel_k = pre_sel ? sel->k : 0;
  s.sel_window = pre_sel ? sel->window : 0;
  if ((e = hs2::launch_score(s, pl.units, stream)) != hipSuccess) return hip_fail(e, "score launch");
  if (pre_sel) sel->hist0_done = true;
  return HS2_OK;
}
}  // namespace

extern "C" {

size_t hs2_full_attn_topk_workspace(const hs2_kv_desc* kv, int32_t Tq, int32_t Hq) {
  if (!kv || kv->B <= 0 || kv->Hkv <= 0 || kv->N <= 0 || kv->D <= 0 || Tq <= 0 || Hq <= 0 || Hq % kv->Hkv) return 0;
  const FullPlan pl = plan_full(kv, Tq, Hq);
  const size_t sel = plan_select(kv->B, Tq, kv->Hkv, kv->N, 1).total;
  return pl.total + std::max(sel, sel_fuse_bytes(kv->B * Tq * kv->Hkv, kv->N));
}

int hs2_full_attn_topk(const hs2_kv_desc* kv, const void* q, hs2_dtype q_dtype, int32_t Tq, int32_t Hq,
                       int32_t q_pos0, float softmax_scale, void* out, float* lse, float* scores, int32_t k,
                       int32_t window, int32_t* idx, int32_t* count, int32_t max_sel, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  int st = check_kv(kv, "hs2_full_attn_topk");
  if (st) return st;
  if (!idx || !count) return fail(HS2_ERR_INVALID_ARG, "hs2_full_attn_topk: NULL idx/count");
  if (k < 0 || window < 0) return fail(HS2_ERR_INVALID_ARG, "hs2_full_attn_topk: need k >= 0 and window >= 0");
  const int64_t need_sel = std::min<int64_t>((int64_t)k + window, kv->N);
  if (max_sel < need_sel)
    return fail(HS2_ERR_INVALID_ARG, "hs2_full_attn_topk: max_sel must be >= min(k + window, N) = " +
                                         std::to_string(need_sel));
  if (((uintptr_t)idx & 3) || ((uintptr_t)count & 3))
    return fail(HS2_ERR_INVALID_ARG, "hs2_full_attn_topk: idx/count must be 4-byte aligned");
  if (Tq <= 0 || Hq <= 0 || Hq % kv->Hkv) return check_q(kv, q, q_dtype, Tq, Hq, "hs2_full_attn_topk");
  const size_t need_ws = hs2_full_attn_topk_workspace(kv, Tq, Hq);
  if (!workspace || workspace_bytes < need_ws)
    return fail(HS2_ERR_WORKSPACE, "hs2_full_attn_topk: workspace needs " + std::to_string(need_ws) + " bytes");
  const size_t full_bytes = plan_full(kv, Tq, Hq).total;
  void* rest = static_cast<char*>(workspace) + full_bytes;
  SelFuse sel{k, window, max_sel, idx, count, rest};
  st = full_layer(kv, q, q_dtype, Tq, Hq, q_pos0, softmax_scale, out, lse, scores, workspace, full_bytes, stream,
                  &sel);
  if (st || sel.done) return st;
  return select_impl(scores, kv->B, Tq, kv->Hkv, kv->N, q_pos0, k, window, 1, idx, count, max_sel, rest,
                     workspace_bytes - full_bytes, stream, sel.hist0_done);
}

size_t hs2_select_workspace(int32_t B, int32_t Tq, int32_t Hkv, int32_t N) {
  if (B <= 0 || Tq <= 0 || Hkv <= 0 || N <= 0) return 0;
  return std::max(plan_select(B, Tq, Hkv, N, 1).total, plan_select(B, Tq, Hkv, N, 2).total);
}

size_t hs2_select_workspace_for(int32_t B, int32_t Tq, int32_t Hkv, int32_t N, int32_t block_size) {
  if (B <= 0 || Tq <= 0 || Hkv <= 0 || N <= 0 || block_size < 1) return 0;
  return plan_select(B, Tq, Hkv, N, block_size).total;
}

int hs2_select_topk_window(const float* scores, int32_t B, int32_t Tq, int32_t Hkv, int32_t N, int32_t q_pos0,
                           int32_t k, int32_t window, int32_t block_size, int32_t* idx, int32_t* count,
                           int32_t max_sel, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return select_impl(scores, B, Tq, Hkv, N, q_pos0, k, window, block_size, idx, count, max_sel, workspace,
                     workspace_bytes, stream, false);
}

}  // extern "C"

namespace {
int select_impl(const float* scores, int32_t B, int32_t Tq, int32_t Hkv, int32_t N, int32_t q_pos0, int32_t k,
                int32_t window, int32_t block_size, int32_t* idx, int32_t* count, int32_t max_sel, void* workspace,
                size_t workspace_bytes, hipStream_t stream, bool pre_hist0) {
  if (!scores || !idx || !count) return fail(HS2_ERR_INVALID_ARG, "hs2_select_topk_window: NULL scores/idx/count");
  if (B <= 0 || Tq <= 0 || Hkv <= 0 || N <= 0)
    return fail(HS2_ERR_INVALID_ARG, "hs2_select_topk_window: B, Tq, Hkv, N must be positive");
  if (q_pos0 < 0 || (int64_t)q_pos0 + Tq > N)
    return fail(HS2_ERR_INVALID_ARG, "hs2_select_topk_window: need 0 <= q_pos0 and q_pos0 + Tq <= N");
  if (k < 0 || window < 0 || block_size < 1)
    return fail(HS2_ERR_INVALID_ARG, "hs2_select_topk_window: need k >= 0, window >= 0, block_size >= 1");
  const int64_t need_sel = std::min<int64_t>((int64_t)k * block_size + window, N);
  if (max_sel < need_sel)
    return fail(HS2_ERR_INVALID_ARG, "hs2_select_topk_window: max_sel must be >= min(k*block_size + window, N) = " +
                                         std::to_string(need_sel));
  if (!al16(scores) || ((uintptr_t)idx & 3) || ((uintptr_t)count & 3))
    return fail(HS2_ERR_INVALID_ARG, "hs2_select_topk_window: scores must be 16-byte aligned, idx/count 4-byte");
  const SelPlan pl = plan_select(B, Tq, Hkv, N, block_size);
  if (!workspace || workspace_bytes < pl.total)
    return fail(HS2_ERR_WORKSPACE, "hs2_select_topk_window: workspace needs " + std::to_string(pl.total) + " bytes");
  if ((uintptr_t)workspace & 255)
    return fail(HS2_ERR_INVALID_ARG, "hs2_select_topk_window: workspace must be 256-byte aligned");
  hs2::SelectParams p{};
  p.scores = scores;
  p.units = pl.units;
  p.Tq = Tq;
  p.Hkv = Hkv;
  p.N = N;
  p.q_pos0 = q_pos0;
  p.k = k;
  p.window = window;
  p.block_size = block_size;
  p.max_sel = max_sel;
  p.nchunks = pl.nchunks;
  p.idx = idx;
  p.count = count;
  p.state = at<int32_t>(workspace, pl.off_state);
  p.hist = block_size == 1 ? at<int32_t>(workspace, pl.off_hist) : nullptr;
  p.cnt = block_size == 1 ? at<int32_t>(workspace, pl.off_cnt) : nullptr;
  p.cand = block_size == 1 ? at<int32_t>(workspace, pl.off_cand) : nullptr;
  p.bmass = block_size > 1 ? at<double>(workspace, pl.off_bmass) : nullptr;
  p.nblocks_max = pl.nblocks_max;
  p.pre_hist0 = pre_hist0 ? 1 : 0;
  const hipError_t e = hs2::launch_select(p, stream);
  if (e != hipSuccess) return hip_fail(e, "select launch");
  return HS2_OK;
}
}  // namespace

extern "C" {

int hs2_sparse_attn_gather(const hs2_kv_desc* kv, const void* q, hs2_dtype q_dtype, int32_t Tq, int32_t Hq,
                           float softmax_scale, const int32_t* idx, const int32_t* count, int32_t max_sel, void* out,
                           float* lse, hipStream_t stream) {
  int st = check_kv(kv, "hs2_sparse_attn_gather");
  if (st) return st;
  if ((st = check_q(kv, q, q_dtype, Tq, Hq, "hs2_sparse_attn_gather"))) return st;
  if (!idx || !count || !out) return fail(HS2_ERR_INVALID_ARG, "hs2_sparse_attn_gather: NULL idx/count/out");
  if (max_sel <= 0) return fail(HS2_ERR_INVALID_ARG, "hs2_sparse_attn_gather: max_sel must be positive");
  if (!al16(out) || ((uintptr_t)idx & 3) || ((uintptr_t)count & 3) || (lse && ((uintptr_t)lse & 3)))
    return fail(HS2_ERR_INVALID_ARG, "hs2_sparse_attn_gather: out must be 16-byte aligned, idx/count/lse 4-byte");
  if (!std::isfinite(softmax_scale)) return fail(HS2_ERR_INVALID_ARG, "hs2_sparse_attn_gather: softmax_scale not finite");
  hs2::ScanParams p{};
  p.k = kv->k;
  p.v = kv->v;
  p.sb = kv->stride_b;
  p.sh = kv->stride_h;
  p.sn = kv->stride_n;
  p.k_scale = kv->k_scale;
  p.v_scale = kv->v_scale;
  p.B = kv->B;
  p.Hkv = kv->Hkv;
  p.N = kv->N;
  p.D = kv->D;
  p.G = Hq / kv->Hkv;
  p.q = q;
  p.Tq = Tq;
  p.Hq = Hq;
  p.q_pos0 = 0;
  p.scale_log2 = softmax_scale * 1.44269504088896340736f;
  p.tpack = 1;
  p.n_tpacks = Tq;
  p.rows = p.G;
  p.nsplit = 1;
  p.idx = idx;
  p.count = count;
  p.max_sel = max_sel;
  p.out = out;
  p.lse = lse;
  const hipError_t e = hs2::launch_scan(p, kv->dtype, true, false, stream);
  if (e != hipSuccess) return hip_fail(e, "sparse_gather launch");
  return HS2_OK;
}

namespace {
struct GatherPlan {
  int nsplit, slice;
  size_t off_ml, off_o, off_cnt, total;
};
// slices of 128 list slots (one 32-row tile per wave of a 4-wave workgroup)
constexpr int kSplitGatherMaxUnits = 64;

GatherPlan plan_gather(int units, int max_sel, int D) {
  GatherPlan g{};
  g.slice = 128;
  g.nsplit = (int)cdiv(max_sel, g.slice);
  if (g.nsplit > 32) {  // long lists: about 32 slices of a multiple of 128 slots, at most 2048
    g.slice = (int)std::min<int64_t>(rup(cdiv(max_sel, 32), 128), 2048);
    g.nsplit = (int)cdiv(max_sel, g.slice);
  }
  size_t off = 0;
  g.off_cnt = off;
  off = a256(off + (size_t)units * sizeof(int32_t));
  g.off_ml = off;
  off = a256(off + (size_t)units * g.nsplit * 16 * 2 * sizeof(float));
  g.off_o = off;
  off = a256(off + (size_t)units * g.nsplit * 16 * D * sizeof(float));
  g.total = off;
  return g;
}
}  // namespace

size_t hs2_sparse_attn_workspace(int32_t B, int32_t Tq, int32_t Hkv, int32_t D, int32_t max_sel) {
  if (B <= 0 || Tq <= 0 || Hkv <= 0 || D <= 0 || max_sel <= 0) return 0;
  return plan_gather(B * Tq * Hkv, max_sel, D).total;
}

int hs2_sparse_attn_gather_ws(const hs2_kv_desc* kv, const void* q, hs2_dtype q_dtype, int32_t Tq, int32_t Hq,
                              float softmax_scale, const int32_t* idx, const int32_t* count, int32_t max_sel,
                              void* out, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_kv(kv, "hs2_sparse_attn_gather_ws");
  if (st) return st;
  if ((st = check_q(kv, q, q_dtype, Tq, Hq, "hs2_sparse_attn_gather_ws"))) return st;
  if (!idx || !count || !out) return fail(HS2_ERR_INVALID_ARG, "hs2_sparse_attn_gather_ws: NULL idx/count/out");
  if (max_sel <= 0) return fail(HS2_ERR_INVALID_ARG, "hs2_sparse_attn_gather_ws: max_sel must be positive");
  if (!al16(out) || ((uintptr_t)idx & 3) || ((uintptr_t)count & 3) || (lse && ((uintptr_t)lse & 3)))
    return fail(HS2_ERR_INVALID_ARG, "hs2_sparse_attn_gather_ws: out must be 16-byte aligned, idx/count/lse 4-byte");
  if (!std::isfinite(softmax_scale))
    return fail(HS2_ERR_INVALID_ARG, "hs2_sparse_attn_gather_ws: softmax_scale not finite");
  if (kv->dtype == HS2_F32)  // the fp32 path has no split form; it needs no workspace
    return hs2_sparse_attn_gather(kv, q, q_dtype, Tq, Hq, softmax_scale, idx, count, max_sel, out, lse, stream);
  const int units = kv->B * Tq * kv->Hkv;
  const GatherPlan gp = plan_gather(units, max_sel, kv->D);
  if (!workspace || workspace_bytes < gp.total)
    return fail(HS2_ERR_WORKSPACE, "hs2_sparse_attn_gather_ws: workspace needs " + std::to_string(gp.total) + " bytes");
  // The split form pays off only while one workgroup per (b, t, g) leaves the
  // GPU mostly idle; from 64 units on, the one-workgroup kernel is used (it
  // needs no workspace).  Also the merging workgroup keeps a maximum (then
  // weight) and a sum per (slice, row) in its 4-wave merge buffer
  // (4 * 16 * (D + 1) floats), so longer lists take the one-workgroup kernel too.
  if (units >= kSplitGatherMaxUnits || (int64_t)2 * gp.nsplit * 16 > 4 * 16 * (kv->D + 1))
    return hs2_sparse_attn_gather(kv, q, q_dtype, Tq, Hq, softmax_scale, idx, count, max_sel, out, lse, stream);
  if ((uintptr_t)workspace & 255)
    return fail(HS2_ERR_INVALID_ARG, "hs2_sparse_attn_gather_ws: workspace must be 256-byte aligned");
  hs2::ScanParams p{};
  p.k = kv->k;
  p.v = kv->v;
  p.sb = kv->stride_b;
  p.sh = kv->stride_h;
  p.sn = kv->stride_n;
  p.k_scale = kv->k_scale;
  p.v_scale = kv->v_scale;
  p.B = kv->B;
  p.Hkv = kv->Hkv;
  p.N = kv->N;
  p.D = kv->D;
  p.G = Hq / kv->Hkv;
  p.q = q;
  p.Tq = Tq;
  p.Hq = Hq;
  p.scale_log2 = softmax_scale * 1.44269504088896340736f;
  p.tpack = 1;
  p.n_tpacks = Tq;
  p.rows = p.G;
  p.nsplit = gp.nsplit;
  p.split_len = gp.slice;
  p.part_ml = at<float>(workspace, gp.off_ml);
  p.part_o = at<float>(workspace, gp.off_o);
  p.gcounter = at<int32_t>(workspace, gp.off_cnt);
  p.idx = idx;
  p.count = count;
  p.max_sel = max_sel;
  p.out = out;
  p.lse = lse;
  const hipError_t e = hs2::launch_gather_split(p, kv->dtype, stream);
  if (e != hipSuccess) return hip_fail(e, "sparse_gather launch");
  return HS2_OK;
}

int hs2_kv_bridge(const void* hidden, int32_t T, int32_t d_model, const void* w_kv, const hs2_kv_desc* kv_out,
                  int32_t batch_index, int32_t pos0, hipStream_t stream) {
  int st = check_kv(kv_out, "hs2_kv_bridge");
  if (st) return st;
  if (kv_out->dtype != HS2_BF16 && kv_out->dtype != HS2_FP8_E4M3FN)
    return fail(HS2_ERR_UNSUPPORTED, "hs2_kv_bridge: output cache must be BF16 or FP8_E4M3FN");
  if (!hidden || !w_kv) return fail(HS2_ERR_INVALID_ARG, "hs2_kv_bridge: NULL hidden or w_kv");
  if (T <= 0 || d_model <= 0) return fail(HS2_ERR_INVALID_ARG, "hs2_kv_bridge: T and d_model must be positive");
  if (d_model % 64) return fail(HS2_ERR_UNSUPPORTED, "hs2_kv_bridge: d_model must be a multiple of 64");
  if (batch_index < 0 || batch_index >= kv_out->B)
    return fail(HS2_ERR_INVALID_ARG, "hs2_kv_bridge: batch_index out of range");
  if (pos0 < 0 || (int64_t)pos0 + T > kv_out->N)
    return fail(HS2_ERR_INVALID_ARG, "hs2_kv_bridge: need 0 <= pos0 and pos0 + T <= N");
  if (!al16(hidden) || !al16(w_kv)) return fail(HS2_ERR_INVALID_ARG, "hs2_kv_bridge: hidden/w_kv must be 16-byte aligned");
  const int64_t off = (int64_t)batch_index * kv_out->stride_b + (int64_t)pos0 * kv_out->stride_n;
  const bool fp8 = kv_out->dtype == HS2_FP8_E4M3FN;
  const size_t esz = fp8 ? 1 : 2;
  hs2::BridgeOut o{};
  o.k = static_cast<char*>(const_cast<void*>(kv_out->k)) + off * esz;
  o.v = static_cast<char*>(const_cast<void*>(kv_out->v)) + off * esz;
  o.sn = kv_out->stride_n;
  o.sh = kv_out->stride_h;
  o.k_scale = fp8 ? kv_out->k_scale + (int64_t)batch_index * kv_out->Hkv : nullptr;
  o.v_scale = fp8 ? kv_out->v_scale + (int64_t)batch_index * kv_out->Hkv : nullptr;
  const hipError_t e = hs2::launch_bridge(static_cast<const uint16_t*>(hidden), T, d_model,
                                          static_cast<const uint16_t*>(w_kv), kv_out->Hkv, kv_out->D, o, stream);
  if (e != hipSuccess) return hip_fail(e, "kv_bridge launch");
  return HS2_OK;
}

int hs2_debug_e4m3fn_to_f32(const uint8_t* codes, float* out, int32_t n, hipStream_t stream) {
  if (!codes || !out || n <= 0) return fail(HS2_ERR_INVALID_ARG, "hs2_debug_e4m3fn_to_f32: bad arguments");
  const hipError_t e = hs2::launch_debug_e4m3fn(codes, out, n, stream);
  if (e != hipSuccess) return hip_fail(e, "debug_e4m3fn launch");
  return HS2_OK;
}

int hs2_debug_stream_read(const void* buf, size_t bytes, uint32_t* out, int32_t blocks, hipStream_t stream) {
  if (!buf || !out || bytes < 16 || blocks <= 0 || !al16(buf))
    return fail(HS2_ERR_INVALID_ARG, "hs2_debug_stream_read: bad arguments");
  const hipError_t e = hs2::launch_stream_read(buf, bytes, out, blocks, stream);
  if (e != hipSuccess) return hip_fail(e, "stream_read launch");
  return HS2_OK;
}

int hs2_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_timing = on != 0;
  return HS2_OK;
}

int hs2_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_tmu);
  for (auto& r : g_recs) {
    hipEventSynchronize(r.b);
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
  return HS2_OK;
}

int hs2_timing_collect(const char* kernel_name, double* total_ms, int32_t* launches) {
  if (!kernel_name || !total_ms || !launches) return fail(HS2_ERR_INVALID_ARG, "hs2_timing_collect: NULL argument");
  std::lock_guard<std::mutex> lk(g_tmu);
  double tot = 0.0;
  int32_t n = 0;
  for (auto& r : g_recs) {
    if (std::strcmp(r.name, kernel_name) != 0) continue;
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return hip_fail(e, "hs2_timing_collect");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return hip_fail(e, "hs2_timing_collect");
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return HS2_OK;
}

const char* hs2_timing_kernel_name(int32_t i) {
  const int32_t n = (int32_t)(sizeof(kKernelNames) / sizeof(kKernelNames[0])) - 1;
  return (i >= 0 && i < n) ? kKernelNames[i] : nullptr;
}

}  // extern "C"
