// C-ABI shim of the HySparse2 cross-decoder hot path: argument validation,
// workspace planning, dispatch to the gfx950 kernels, per-kernel event timing.
// Validation never touches the GPU, so every error path runs without a device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
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

// A paged cache's table against the rules in hs2.h (bf16/FP8 only; the pool
// is shared, so stride_b is 0).
int check_pages(const hs2_kv_desc* kv, const hs2_page_table* pt, const char* what) {
  const std::string w(what);
  if (kv->dtype == HS2_F32) return fail(HS2_ERR_UNSUPPORTED, w + ": paged caches are bf16 or FP8_E4M3FN");
  if (!pt || !pt->table) return fail(HS2_ERR_INVALID_ARG, w + ": page table is NULL");
  if ((uintptr_t)pt->table & 3) return fail(HS2_ERR_INVALID_ARG, w + ": page table must be 4-byte aligned");
  const int32_t pr = pt->page_rows;
  if (pr < 32 || pr > (1 << 24) || (pr & (pr - 1)))
    return fail(HS2_ERR_INVALID_ARG, w + ": page_rows must be a power of two from 32 to 2^24");
  if (pt->pages_per_seq <= 0 || (int64_t)pt->pages_per_seq * pr < kv->N)
    return fail(HS2_ERR_INVALID_ARG, w + ": pages_per_seq * page_rows must cover N");
  if (pt->pool_pages <= 0 || (int64_t)pt->pool_pages * pr > INT32_MAX)
    return fail(HS2_ERR_INVALID_ARG, w + ": need 0 < pool_pages and pool_pages * page_rows < 2^31");
  if (kv->stride_b != 0) return fail(HS2_ERR_INVALID_ARG, w + ": a paged pool is shared by the sequences (stride_b = 0)");
  return HS2_OK;
}

hs2::PageMap page_map(const hs2_page_table* pt) {
  hs2::PageMap m{};
  if (!pt) return m;
  m.table = pt->table;
  while ((1 << m.shift) < pt->page_rows) ++m.shift;
  m.per_seq = pt->pages_per_seq;
  m.pool = pt->pool_pages;
  return m;
}

// The read-only view of a writable cache descriptor (for validation).
hs2_kv_desc as_read_desc(const hs2_kv_out_desc& o) {
  hs2_kv_desc d{};
  d.k = o.k;
  d.v = o.v;
  d.dtype = o.dtype;
  d.stride_b = o.stride_b;
  d.stride_h = o.stride_h;
  d.stride_n = o.stride_n;
  d.k_scale = o.k_scale;
  d.v_scale = o.v_scale;
  d.B = o.B;
  d.Hkv = o.Hkv;
  d.N = o.N;
  d.D = o.D;
  return d;
}

struct FullPlan {
  bool chunk;  // multi-query chunk kernels (MFMA pass + merge + score recompute)
  int tpack, n_tpacks, rows, units, nsplit, split_len;
  int64_t npad;
  size_t off_ml, off_o, off_lse2, off_lg16, off_lgmax, total;
};

// Position splits: about kScanTargetWgs workgroups in total (4 per CU on 256
// CUs; 8 for a bf16 cache, whose scan measured 2-3% faster with the finer
// splits while the FP8 scan measured slower), split lengths a multiple of 256
// positions (64 on the fp32 path).
constexpr int64_t kScanTargetWgs = 1024, kScanTargetWgsBf16 = 2048;
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
  if (p.chunk) {  // work items (b, block of packs, g) x position splits, kChunkTargetWgs in all
    const int64_t items = (int64_t)kv->B * cdiv(p.n_tpacks, hs2::kChunkPacks) * kv->Hkv;
    const int64_t per_item = std::max<int64_t>(1, hs2::kChunkTargetWgs / items);
    p.split_len = (int)rup(cdiv(kv->N, per_item), 128);  // whole 32-position tiles
  } else {
    const int64_t target = kv->dtype == HS2_BF16 ? kScanTargetWgsBf16 : kScanTargetWgs;
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
  p.total = off;
  return p;
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
  if (block_size == 1 && !hs2::sel_bracketed(p.units, p.nchunks)) {  // digit histograms and per-chunk counts
    p.off_hist = off;
    off = a256(off + (size_t)p.units * 3 * hs2::kHistBins * sizeof(int32_t));
    p.off_cnt = off;
    off = a256(off + (size_t)p.units * p.nchunks * 258 * sizeof(int32_t));
    p.off_cand = off;
  } else if (block_size == 1) {  // bracketed: each chunk's per-wave list lengths and lists
    p.off_hist = off;
    p.off_cnt = off;
    off = a256(off + (size_t)p.units * p.nchunks * 8 * sizeof(int32_t));
    p.off_cand = off;
    off = a256(off + (size_t)p.units * p.nchunks * hs2::kCandWords * sizeof(int32_t));
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
const char* const kKernelNames[] = {"full_scan",      "combine",        "score",         "select_init",
                                    "select_hist",    "select_bracket", "select_collect", "select_finish",
                                    "select_exact",   "select_emit",    "select_window",  "select_block_mass",
                                    "select_block_pick", "sparse_gather", "kv_bridge",    "stream_read",
                                    "chunk_full",     "chunk_score",    "swa_chunk",      "scan_read_probe",
                                    "scan_read_probe_codes", nullptr};

// Timing state (only while hs2_timing_enable(1) is in force): the event pairs
// of the launches since the last reset.  Events are created per launch and
// destroyed by hs2_timing_reset, so none outlives the caller's reset.
std::mutex g_tmu;
std::atomic<bool> g_timing{false};
struct TimingRec {
  const char* name;
  hipEvent_t a, b;
};
std::vector<TimingRec> g_recs;

}  // namespace

namespace hs2 {
TimedLaunch::TimedLaunch(const char* name, hipStream_t s) : name_(name), s_(s), ev0_(nullptr), ev1_(nullptr) {
  if (!g_timing.load(std::memory_order_acquire)) return;
  hipEvent_t a = nullptr, b = nullptr;
  if (hipEventCreate(&a) != hipSuccess) return;
  if (hipEventCreate(&b) != hipSuccess) {
    (void)hipEventDestroy(a);
    return;
  }
  ev0_ = a;
  ev1_ = b;
  (void)hipEventRecord(a, s);
}
TimedLaunch::~TimedLaunch() {
  if (!ev0_) return;
  (void)hipEventRecord((hipEvent_t)ev1_, s_);
  std::lock_guard<std::mutex> lk(g_tmu);
  g_recs.push_back(TimingRec{name_, (hipEvent_t)ev0_, (hipEvent_t)ev1_});
}
}  // namespace hs2

extern "C" {

int hs2_abi_version(void) { return HS2_ABI_VERSION; }

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
// Token selection prepared by the full layer (hs2_full_attn_topk): with one
// query token per unit, the merge sets the selection rows up and the score
// pass builds the first radix histogram (layout of plan_select over ws).
struct SelPrep {
  int32_t k, window;
  int32_t cand_window;  // window, or 0 when the window competes
  void* ws;
  bool hist0_done = false;
};

int full_layer(const hs2_kv_desc* kv, const void* q, hs2_dtype q_dtype, int32_t Tq, int32_t Hq, int32_t q_pos0,
               const int32_t* q_pos0_b, float softmax_scale, void* out, float* lse, float* scores, void* workspace,
               size_t workspace_bytes, hipStream_t stream, SelPrep* sel, const hs2_page_table* pages = nullptr);
// the one-workgroup gather on checked arguments (pages nullptr: contiguous)
int gather_single(const hs2_kv_desc* kv, const hs2_page_table* pages, const void* q, int32_t Tq, int32_t Hq,
                  float softmax_scale, const int32_t* idx, const int32_t* count, int32_t max_sel, void* out,
                  float* lse, hipStream_t stream);
// hs2_full_attn_topk, on a contiguous (pages nullptr) or paged cache
int full_attn_topk_impl(const char* name, const hs2_kv_desc* kv, const hs2_page_table* pages, const void* q,
                        hs2_dtype q_dtype, int32_t Tq, int32_t Hq, int32_t q_pos0, const int32_t* q_pos0_b,
                        float softmax_scale, void* out, float* lse, float* scores, int32_t k, int32_t window,
                        int32_t flags, int32_t* idx, int32_t* count, int32_t max_sel, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);
// hs2_select_topk_window; pre_hist0: the row state and first histogram are
// already built (full layer's merge and score pass)
int select_impl(const float* scores, int32_t B, int32_t Tq, int32_t Hkv, int32_t N, int32_t q_pos0,
                const int32_t* q_pos0_b, int32_t k, int32_t window, int32_t block_size, int32_t flags, int32_t* idx,
                int32_t* count, int32_t max_sel, void* workspace, size_t workspace_bytes, hipStream_t stream,
                bool pre_hist0);
}  // namespace

extern "C" {

int hs2_full_attn_scores(const hs2_kv_desc* kv, const void* q, hs2_dtype q_dtype, int32_t Tq, int32_t Hq,
                         int32_t q_pos0, const int32_t* q_pos0_b, float softmax_scale, void* out, float* lse,
                         float* scores, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return full_layer(kv, q, q_dtype, Tq, Hq, q_pos0, q_pos0_b, softmax_scale, out, lse, scores, workspace,
                    workspace_bytes, stream, nullptr);
}

}  // extern "C"

namespace {
int full_layer(const hs2_kv_desc* kv, const void* q, hs2_dtype q_dtype, int32_t Tq, int32_t Hq, int32_t q_pos0,
               const int32_t* q_pos0_b, float softmax_scale, void* out, float* lse, float* scores, void* workspace,
               size_t workspace_bytes, hipStream_t stream, SelPrep* sel, const hs2_page_table* pages) {
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
  if ((uintptr_t)q_pos0_b & 3) return fail(HS2_ERR_INVALID_ARG, "hs2_full_attn_scores: q_pos0_b must be 4-byte aligned");
  if (pages && pl.chunk)
    return fail(HS2_ERR_UNSUPPORTED, "hs2_full_attn_topk_paged: many query tokens per kv head (the chunk path) "
                                     "on a paged cache");

  hs2::ScanParams p{};
  p.pages = page_map(pages);
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
  p.qpos_b = q_pos0_b;
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

  // one query token per unit: the selection's rows are set up before the
  // score pass, which counts their first digit -- this saves the selection two
  // passes (grids of many rows take the bracketed selection, which needs
  // neither).  bf16/FP8 caches: the scan sets the rows up and the merge runs
  // inside the score launch; fp32: the merge kernel does both.
  const bool pre_sel = sel != nullptr && pl.tpack == 1 &&
                       !hs2::sel_bracketed(pl.units, (int)cdiv(kv->N, hs2::kSelChunk));
  const bool fused_merge = pre_sel && kv->dtype != HS2_F32;
  int32_t* sel_hist = nullptr;
  int32_t* sel_state = nullptr;
  if (pre_sel) {
    const SelPlan sp = plan_select(kv->B, Tq, kv->Hkv, kv->N, 1);
    sel_state = at<int32_t>(sel->ws, sp.off_state);
    sel_hist = at<int32_t>(sel->ws, sp.off_hist);
  }
  if (fused_merge) {
    p.sel_state = sel_state;
    p.sel_hist = sel_hist;
    p.sel_k = sel->k;
    p.sel_window = sel->cand_window;
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
  if (pre_sel && !fused_merge) {
    c.sel_state = sel_state;
    c.sel_hist = sel_hist;
    c.sel_k = sel->k;
    c.sel_window = sel->cand_window;
    c.q_pos0 = q_pos0;
    c.N = kv->N;
    c.qpos_b = q_pos0_b;
  }
  if (!fused_merge && (e = hs2::launch_combine(c, pl.units, stream)) != hipSuccess)
    return hip_fail(e, "combine launch");

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
  s.qpos_b = q_pos0_b;
  s.scores = scores;
  s.sel_hist = sel_hist;
  s.sel_k = pre_sel ? sel->k : 0;
  s.sel_window = pre_sel ? sel->cand_window : 0;
  s.q = q;
  s.Hq = Hq;
  s.D = kv->D;
  s.kv_dtype = kv->dtype;
  s.k = kv->k;
  s.sb = kv->stride_b;
  s.sh = kv->stride_h;
  s.sn = kv->stride_n;
  s.k_scale = kv->k_scale;
  s.scale_log2 = p.scale_log2;
  s.pages = p.pages;
  if ((e = hs2::launch_score(s, pl.units, stream, fused_merge ? &c : nullptr)) != hipSuccess)
    return hip_fail(e, "score launch");
  if (pre_sel) sel->hist0_done = true;
  return HS2_OK;
}
}  // namespace

extern "C" {

size_t hs2_full_attn_topk_workspace(const hs2_kv_desc* kv, int32_t Tq, int32_t Hq) {
  if (!kv || kv->B <= 0 || kv->Hkv <= 0 || kv->N <= 0 || kv->D <= 0 || Tq <= 0 || Hq <= 0 || Hq % kv->Hkv) return 0;
  const FullPlan pl = plan_full(kv, Tq, Hq);
  const size_t sel = plan_select(kv->B, Tq, kv->Hkv, kv->N, 1).total;
  return pl.total + sel;
}

int hs2_full_attn_topk(const hs2_kv_desc* kv, const void* q, hs2_dtype q_dtype, int32_t Tq, int32_t Hq,
                       int32_t q_pos0, const int32_t* q_pos0_b, float softmax_scale, void* out, float* lse,
                       float* scores, int32_t k, int32_t window, int32_t flags, int32_t* idx, int32_t* count,
                       int32_t max_sel, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return full_attn_topk_impl("hs2_full_attn_topk", kv, nullptr, q, q_dtype, Tq, Hq, q_pos0, q_pos0_b, softmax_scale,
                             out, lse, scores, k, window, flags, idx, count, max_sel, workspace, workspace_bytes,
                             stream);
}

int hs2_full_attn_topk_paged(const hs2_kv_desc* kv, const hs2_page_table* pages, const void* q, hs2_dtype q_dtype,
                             int32_t Tq, int32_t Hq, int32_t q_pos0, const int32_t* q_pos0_b, float softmax_scale,
                             void* out, float* lse, float* scores, int32_t k, int32_t window, int32_t flags,
                             int32_t* idx, int32_t* count, int32_t max_sel, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  const char* name = "hs2_full_attn_topk_paged";
  int st = check_kv(kv, name);
  if (st) return st;
  if ((st = check_pages(kv, pages, name))) return st;
  return full_attn_topk_impl(name, kv, pages, q, q_dtype, Tq, Hq, q_pos0, q_pos0_b, softmax_scale, out, lse, scores,
                             k, window, flags, idx, count, max_sel, workspace, workspace_bytes, stream);
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
                           const int32_t* q_pos0_b, int32_t k, int32_t window, int32_t block_size, int32_t flags,
                           int32_t* idx, int32_t* count, int32_t max_sel, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  return select_impl(scores, B, Tq, Hkv, N, q_pos0, q_pos0_b, k, window, block_size, flags, idx, count, max_sel,
                     workspace, workspace_bytes, stream, false);
}

}  // extern "C"

namespace {
int full_attn_topk_impl(const char* name, const hs2_kv_desc* kv, const hs2_page_table* pages, const void* q,
                        hs2_dtype q_dtype, int32_t Tq, int32_t Hq, int32_t q_pos0, const int32_t* q_pos0_b,
                        float softmax_scale, void* out, float* lse, float* scores, int32_t k, int32_t window,
                        int32_t flags, int32_t* idx, int32_t* count, int32_t max_sel, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  int st = check_kv(kv, "hs2_full_attn_topk");
  if (st) return st;
  if (!idx || !count) return fail(HS2_ERR_INVALID_ARG, std::string(name) + ": NULL idx/count");
  if (k < 0 || window < 0) return fail(HS2_ERR_INVALID_ARG, std::string(name) + ": need k >= 0 and window >= 0");
  if (flags & ~HS2_SEL_WINDOW_COMPETES) return fail(HS2_ERR_INVALID_ARG, std::string(name) + ": unknown flags");
  const int64_t need_sel = std::min<int64_t>((int64_t)k + window, kv->N);
  if (max_sel < need_sel)
    return fail(HS2_ERR_INVALID_ARG, std::string(name) + ": max_sel must be >= min(k + window, N) = " +
                                         std::to_string(need_sel));
  if (((uintptr_t)idx & 3) || ((uintptr_t)count & 3))
    return fail(HS2_ERR_INVALID_ARG, std::string(name) + ": idx/count must be 4-byte aligned");
  if (Tq <= 0 || Hq <= 0 || Hq % kv->Hkv) return check_q(kv, q, q_dtype, Tq, Hq, "hs2_full_attn_topk");
  const size_t need_ws = hs2_full_attn_topk_workspace(kv, Tq, Hq);
  if (!workspace || workspace_bytes < need_ws)
    return fail(HS2_ERR_WORKSPACE, std::string(name) + ": workspace needs " + std::to_string(need_ws) + " bytes");
  const size_t full_bytes = plan_full(kv, Tq, Hq).total;
  void* rest = static_cast<char*>(workspace) + full_bytes;
  const int32_t cand_window = (flags & HS2_SEL_WINDOW_COMPETES) ? 0 : window;
  SelPrep sel{k, window, cand_window, rest};
  st = full_layer(kv, q, q_dtype, Tq, Hq, q_pos0, q_pos0_b, softmax_scale, out, lse, scores, workspace, full_bytes,
                  stream, &sel, pages);
  if (st) return st;
  return select_impl(scores, kv->B, Tq, kv->Hkv, kv->N, q_pos0, q_pos0_b, k, window, 1, flags, idx, count, max_sel,
                     rest, workspace_bytes - full_bytes, stream, sel.hist0_done);
}

int select_impl(const float* scores, int32_t B, int32_t Tq, int32_t Hkv, int32_t N, int32_t q_pos0,
                const int32_t* q_pos0_b, int32_t k, int32_t window, int32_t block_size, int32_t flags, int32_t* idx,
                int32_t* count, int32_t max_sel, void* workspace, size_t workspace_bytes, hipStream_t stream,
                bool pre_hist0) {
  if (!scores || !idx || !count) return fail(HS2_ERR_INVALID_ARG, "hs2_select_topk_window: NULL scores/idx/count");
  if (B <= 0 || Tq <= 0 || Hkv <= 0 || N <= 0)
    return fail(HS2_ERR_INVALID_ARG, "hs2_select_topk_window: B, Tq, Hkv, N must be positive");
  if (q_pos0 < 0 || (int64_t)q_pos0 + Tq > N)
    return fail(HS2_ERR_INVALID_ARG, "hs2_select_topk_window: need 0 <= q_pos0 and q_pos0 + Tq <= N");
  if (k < 0 || window < 0 || block_size < 1)
    return fail(HS2_ERR_INVALID_ARG, "hs2_select_topk_window: need k >= 0, window >= 0, block_size >= 1");
  if (flags & ~HS2_SEL_WINDOW_COMPETES) return fail(HS2_ERR_INVALID_ARG, "hs2_select_topk_window: unknown flags");
  const bool competes = (flags & HS2_SEL_WINDOW_COMPETES) != 0;
  if (competes && block_size != 1)
    return fail(HS2_ERR_UNSUPPORTED, "hs2_select_topk_window: the competing window is token mode only");
  const int64_t need_sel = std::min<int64_t>((int64_t)k * block_size + window, N);
  if (max_sel < need_sel)
    return fail(HS2_ERR_INVALID_ARG, "hs2_select_topk_window: max_sel must be >= min(k*block_size + window, N) = " +
                                         std::to_string(need_sel));
  if (!al16(scores) || ((uintptr_t)idx & 3) || ((uintptr_t)count & 3) || ((uintptr_t)q_pos0_b & 3))
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
  p.qpos_b = q_pos0_b;
  p.k = k;
  p.window = window;
  p.cand_window = competes ? 0 : window;
  p.competes = competes ? 1 : 0;
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
  return gather_single(kv, nullptr, q, Tq, Hq, softmax_scale, idx, count, max_sel, out, lse, stream);
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

}  // extern "C"

namespace {
// The one-workgroup gather on checked arguments (pages nullptr: contiguous cache).
int gather_single(const hs2_kv_desc* kv, const hs2_page_table* pages, const void* q, int32_t Tq, int32_t Hq,
                  float softmax_scale, const int32_t* idx, const int32_t* count, int32_t max_sel, void* out,
                  float* lse, hipStream_t stream) {
  hs2::ScanParams p{};
  p.pages = page_map(pages);
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

// Checks shared by the split gather's entry points.
int check_gather_args(const char* name, const hs2_kv_desc* kv, const void* q, hs2_dtype q_dtype, int32_t Tq,
                      int32_t Hq, float softmax_scale, const int32_t* idx, const int32_t* count, int32_t max_sel,
                      void* out, float* lse) {
  const std::string w(name);
  int st = check_kv(kv, name);
  if (st) return st;
  if ((st = check_q(kv, q, q_dtype, Tq, Hq, name))) return st;
  if (!idx || !count || !out) return fail(HS2_ERR_INVALID_ARG, w + ": NULL idx/count/out");
  if (max_sel <= 0) return fail(HS2_ERR_INVALID_ARG, w + ": max_sel must be positive");
  if (!al16(out) || ((uintptr_t)idx & 3) || ((uintptr_t)count & 3) || (lse && ((uintptr_t)lse & 3)))
    return fail(HS2_ERR_INVALID_ARG, w + ": out must be 16-byte aligned, idx/count/lse 4-byte");
  if (!std::isfinite(softmax_scale)) return fail(HS2_ERR_INVALID_ARG, w + ": softmax_scale not finite");
  return HS2_OK;
}

// The split form pays off only while one workgroup per (b, t, g) leaves the
// GPU mostly idle; from kSplitGatherMaxUnits units on, the one-workgroup
// kernel is used (it needs no workspace).  The merging workgroup also keeps
// a maximum (then weight) and a sum per (slice, row) in its 4-wave merge
// buffer (4 * 16 * (D + 1) floats), so longer lists take the one-workgroup
// kernel too, as does an fp32 cache (no split form).
bool use_split_gather(const hs2_kv_desc* kv, int units, const GatherPlan& gp) {
  return kv->dtype != HS2_F32 && units < kSplitGatherMaxUnits && (int64_t)2 * gp.nsplit * 16 <= 4 * 16 * (kv->D + 1);
}

// Launch of the split gather on a workspace already checked for size and
// alignment (arrival counters zero on entry; zero again on exit).
int launch_split_gather(const char* name, const hs2_kv_desc* kv, const void* q, int32_t Tq, int32_t Hq,
                        float softmax_scale, const int32_t* idx, const int32_t* count, int32_t max_sel, void* out,
                        float* lse, const GatherPlan& gp, void* workspace, hipStream_t stream,
                        const hs2_page_table* pages = nullptr) {
  hs2::ScanParams p{};
  p.pages = page_map(pages);
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
  if (e != hipSuccess) return hip_fail(e, (std::string(name) + ": sparse_gather launch").c_str());
  return HS2_OK;
}

// hs2_sparse_attn_gather_ws on a contiguous (pages nullptr) or paged cache.
int gather_ws_impl(const char* name, const hs2_kv_desc* kv, const hs2_page_table* pages, const void* q,
                   hs2_dtype q_dtype, int32_t Tq, int32_t Hq, float softmax_scale, const int32_t* idx,
                   const int32_t* count, int32_t max_sel, void* out, float* lse, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  int st = check_gather_args(name, kv, q, q_dtype, Tq, Hq, softmax_scale, idx, count, max_sel, out, lse);
  if (st) return st;
  if (kv->dtype == HS2_F32)  // the fp32 path has no split form; it needs no workspace
    return gather_single(kv, nullptr, q, Tq, Hq, softmax_scale, idx, count, max_sel, out, lse, stream);
  const int units = kv->B * Tq * kv->Hkv;
  const GatherPlan gp = plan_gather(units, max_sel, kv->D);
  if (!workspace || workspace_bytes < gp.total)
    return fail(HS2_ERR_WORKSPACE, std::string(name) + ": workspace needs " + std::to_string(gp.total) + " bytes");
  if (!use_split_gather(kv, units, gp))
    return gather_single(kv, pages, q, Tq, Hq, softmax_scale, idx, count, max_sel, out, lse, stream);
  if ((uintptr_t)workspace & 255) return fail(HS2_ERR_INVALID_ARG, std::string(name) + ": workspace must be 256-byte aligned");
  return launch_split_gather(name, kv, q, Tq, Hq, softmax_scale, idx, count, max_sel, out, lse, gp, workspace, stream,
                             pages);
}

// ---- the no-allocation variant's scratch --------------------------------
// The split gather's partials and arrival counters for
// hs2_sparse_attn_gather_static live in this file-scope device array (one
// copy per GPU, held until the process ends).  Host code never passes the
// array's name to a kernel: the device address of each GPU's copy comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kStaticScratchBytes = size_t(4) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Clears the arrival-counter region (the first 4 KiB) of a device's copy.
__global__ void clear_scratch_words(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Device address of the current device's scratch; the first call on a device
// resolves it and clears the counter region on `stream`.
int static_scratch(hipStream_t stream, void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hs2_sparse_attn_gather_static: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(HS2_ERR_UNSUPPORTED, "hs2_sparse_attn_gather_static: device index above 63");
  std::call_once(g_scratch_once[dev], [&] {
    void* p = nullptr;
    hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (r == hipSuccess && p == nullptr) r = hipErrorInvalidSymbol;
    if (r == hipSuccess) {
      hipLaunchKernelGGL(clear_scratch_words, dim3(4), dim3(256), 0, stream, static_cast<uint32_t*>(p), 1024);
      r = hipGetLastError();
    }
    g_scratch_err[dev] = r;
    g_scratch_ptr[dev] = r == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess)
    return hip_fail(g_scratch_err[dev], "hs2_sparse_attn_gather_static: scratch set-up");
  *ptr = g_scratch_ptr[dev];
  return HS2_OK;
}
}  // namespace

extern "C" {

int hs2_sparse_attn_gather_ws(const hs2_kv_desc* kv, const void* q, hs2_dtype q_dtype, int32_t Tq, int32_t Hq,
                              float softmax_scale, const int32_t* idx, const int32_t* count, int32_t max_sel,
                              void* out, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return gather_ws_impl("hs2_sparse_attn_gather_ws", kv, nullptr, q, q_dtype, Tq, Hq, softmax_scale, idx, count,
                        max_sel, out, lse, workspace, workspace_bytes, stream);
}

int hs2_sparse_attn_gather_paged(const hs2_kv_desc* kv, const hs2_page_table* pages, const void* q,
                                 hs2_dtype q_dtype, int32_t Tq, int32_t Hq, float softmax_scale, const int32_t* idx,
                                 const int32_t* count, int32_t max_sel, void* out, float* lse, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  const char* name = "hs2_sparse_attn_gather_paged";
  int st = check_kv(kv, name);
  if (st) return st;
  if ((st = check_pages(kv, pages, name))) return st;
  return gather_ws_impl(name, kv, pages, q, q_dtype, Tq, Hq, softmax_scale, idx, count, max_sel, out, lse, workspace,
                        workspace_bytes, stream);
}

size_t hs2_sparse_attn_static_limit(void) { return kStaticScratchBytes; }

int hs2_sparse_attn_gather_static(const hs2_kv_desc* kv, const void* q, hs2_dtype q_dtype, int32_t Tq, int32_t Hq,
                                  float softmax_scale, const int32_t* idx, const int32_t* count, int32_t max_sel,
                                  void* out, float* lse, hipStream_t stream) {
  const char* name = "hs2_sparse_attn_gather_static";
  int st = check_gather_args(name, kv, q, q_dtype, Tq, Hq, softmax_scale, idx, count, max_sel, out, lse);
  if (st) return st;
  const int units = kv->B * Tq * kv->Hkv;
  const GatherPlan gp = plan_gather(units, max_sel, kv->D);
  if (!use_split_gather(kv, units, gp))  // the one-workgroup kernel: no scratch
    return hs2_sparse_attn_gather(kv, q, q_dtype, Tq, Hq, softmax_scale, idx, count, max_sel, out, lse, stream);
  if (gp.total > kStaticScratchBytes)
    return fail(HS2_ERR_WORKSPACE, std::string(name) + ": needs " + std::to_string(gp.total) +
                                       " bytes of scratch; the library's static scratch holds " +
                                       std::to_string(kStaticScratchBytes));
  void* ws = nullptr;
  if ((st = static_scratch(stream, &ws))) return st;
  return launch_split_gather(name, kv, q, Tq, Hq, softmax_scale, idx, count, max_sel, out, lse, gp, ws, stream);
}

int hs2_swa_attn(const hs2_kv_desc* kv, const void* q, hs2_dtype q_dtype, int32_t Tq, int32_t Hq, int32_t q_pos0,
                 const int32_t* q_pos0_b, int32_t window, float softmax_scale, void* out, float* lse,
                 hipStream_t stream) {
  const char* name = "hs2_swa_attn";
  int st = check_kv(kv, name);
  if (st) return st;
  if ((st = check_q(kv, q, q_dtype, Tq, Hq, name))) return st;
  if (q_pos0 < 0 || (int64_t)q_pos0 + Tq > kv->N)
    return fail(HS2_ERR_INVALID_ARG, "hs2_swa_attn: need 0 <= q_pos0 and q_pos0 + Tq <= N");
  if (window < 1) return fail(HS2_ERR_INVALID_ARG, "hs2_swa_attn: window must be at least 1");
  if (!out) return fail(HS2_ERR_INVALID_ARG, "hs2_swa_attn: out must not be NULL");
  if ((uintptr_t)q_pos0_b & 3) return fail(HS2_ERR_INVALID_ARG, "hs2_swa_attn: q_pos0_b must be 4-byte aligned");
  if (!al16(out) || (lse && ((uintptr_t)lse & 3)))
    return fail(HS2_ERR_INVALID_ARG, "hs2_swa_attn: out must be 16-byte aligned, lse 4-byte");
  if (!std::isfinite(softmax_scale)) return fail(HS2_ERR_INVALID_ARG, "hs2_swa_attn: softmax_scale not finite");
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
  p.qpos_b = q_pos0_b;
  p.scale_log2 = softmax_scale * 1.44269504088896340736f;
  p.band = window;
  p.out = out;
  p.lse = lse;
  p.nsplit = 1;
  const FullPlan pl = plan_full(kv, Tq, Hq);
  hipError_t e;
  if (pl.chunk) {  // many query tokens: the banded matrix-core pass, one split, final outputs
    p.tpack = pl.tpack;
    p.n_tpacks = pl.n_tpacks;
    p.rows = pl.rows;
    p.split_len = kv->N;
    e = hs2::launch_chunk_full(p, kv->dtype, stream);
  } else {  // few query tokens: one workgroup per (b, t, g) over its contiguous window
    p.tpack = 1;
    p.n_tpacks = Tq;
    p.rows = p.G;
    e = hs2::launch_scan(p, kv->dtype, true, false, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "hs2_swa_attn launch");
  return HS2_OK;
}

}  // extern "C"

namespace {
struct BridgePlan {
  size_t off_y, off_amax, off_scale, total;
};
BridgePlan plan_bridge(int L, int T, int Hkv, int D) {
  BridgePlan b{};
  size_t off = 0;
  b.off_y = off;
  off = a256(off + (size_t)L * T * 2 * Hkv * D * sizeof(float));
  b.off_amax = off;
  off = a256(off + (size_t)L * 2 * Hkv * sizeof(uint32_t));
  b.off_scale = off;
  off = a256(off + (size_t)L * 2 * Hkv * sizeof(float));
  b.total = off;
  return b;
}

int bridge_impl(const char* name, const void* hidden, int32_t T, int32_t d_model, const void* w_kv, int32_t L,
                const hs2_kv_out_desc* caches, int32_t batch_index, int32_t pos0, int32_t scale_mode, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  const std::string w(name);
  if (!caches) return fail(HS2_ERR_INVALID_ARG, w + ": cache descriptor is NULL");
  if (L < 1 || L > hs2::kMaxBridgeLayers)
    return fail(HS2_ERR_INVALID_ARG, w + ": layers must be 1.." + std::to_string(hs2::kMaxBridgeLayers));
  if (scale_mode != HS2_SCALE_KEEP && scale_mode != HS2_SCALE_GROW)
    return fail(HS2_ERR_INVALID_ARG, w + ": unknown scale mode");
  if (!hidden || !w_kv) return fail(HS2_ERR_INVALID_ARG, w + ": NULL hidden or w_kv");
  if (T <= 0 || d_model <= 0) return fail(HS2_ERR_INVALID_ARG, w + ": T and d_model must be positive");
  if (d_model % 64) return fail(HS2_ERR_UNSUPPORTED, w + ": d_model must be a multiple of 64");
  if (!al16(hidden) || !al16(w_kv)) return fail(HS2_ERR_INVALID_ARG, w + ": hidden/w_kv must be 16-byte aligned");
  const hs2_kv_out_desc& c0 = caches[0];
  hs2::BridgeLayers P{};
  P.L = L;
  P.pos0 = pos0;
  for (int l = 0; l < L; ++l) {
    const hs2_kv_out_desc& c = caches[l];
    const hs2_kv_desc view = as_read_desc(c);
    int st = check_kv(&view, name);
    if (st) return st;
    if (c.dtype != HS2_BF16 && c.dtype != HS2_FP8_E4M3FN)
      return fail(HS2_ERR_UNSUPPORTED, w + ": output cache must be BF16 or FP8_E4M3FN");
    if (c.dtype != c0.dtype || c.Hkv != c0.Hkv || c.D != c0.D)
      return fail(HS2_ERR_INVALID_ARG, w + ": the layers' caches must share dtype, Hkv and D");
    if (batch_index < 0 || batch_index >= c.B) return fail(HS2_ERR_INVALID_ARG, w + ": batch_index out of range");
    if (pos0 < 0 || (int64_t)pos0 + T > c.N)
      return fail(HS2_ERR_INVALID_ARG, w + ": need 0 <= pos0 and pos0 + T <= N");
    const bool fp8 = c.dtype == HS2_FP8_E4M3FN;
    const size_t esz = fp8 ? 1 : 2;
    hs2::BridgeOut& o = P.out[l];
    o.k = static_cast<char*>(c.k) + (int64_t)batch_index * c.stride_b * esz;
    o.v = static_cast<char*>(c.v) + (int64_t)batch_index * c.stride_b * esz;
    o.sn = c.stride_n;
    o.sh = c.stride_h;
    o.k_scale = fp8 ? c.k_scale + (int64_t)batch_index * c.Hkv : nullptr;
    o.v_scale = fp8 ? c.v_scale + (int64_t)batch_index * c.Hkv : nullptr;
  }
  if (scale_mode == HS2_SCALE_GROW && c0.dtype == HS2_FP8_E4M3FN) {
    if (L * 2 * c0.Hkv > 1024)
      return fail(HS2_ERR_UNSUPPORTED, w + ": scale maintenance handles at most 1024 (layer, K/V, head) scales");
    const BridgePlan bp = plan_bridge(L, T, c0.Hkv, c0.D);
    if (!workspace || workspace_bytes < bp.total)
      return fail(HS2_ERR_WORKSPACE, w + ": workspace needs " + std::to_string(bp.total) + " bytes");
    if ((uintptr_t)workspace & 255) return fail(HS2_ERR_INVALID_ARG, w + ": workspace must be 256-byte aligned");
    P.y = at<float>(workspace, bp.off_y);
    P.amax = at<uint32_t>(workspace, bp.off_amax);
    P.old_scale = at<float>(workspace, bp.off_scale);
  }
  const hipError_t e = hs2::launch_bridge(static_cast<const uint16_t*>(hidden), T, d_model,
                                          static_cast<const uint16_t*>(w_kv), c0.Hkv, c0.D, P, stream);
  if (e != hipSuccess) return hip_fail(e, (w + " launch").c_str());
  return HS2_OK;
}
}  // namespace

extern "C" {

int hs2_kv_bridge(const void* hidden, int32_t T, int32_t d_model, const void* w_kv, const hs2_kv_out_desc* kv_out,
                  int32_t batch_index, int32_t pos0, hipStream_t stream) {
  return bridge_impl("hs2_kv_bridge", hidden, T, d_model, w_kv, 1, kv_out, batch_index, pos0, HS2_SCALE_KEEP, nullptr,
                     0, stream);
}

size_t hs2_kv_bridge_layers_workspace(int32_t L, int32_t T, int32_t Hkv, int32_t D) {
  if (L <= 0 || T <= 0 || Hkv <= 0 || D <= 0) return 0;
  return plan_bridge(L, T, Hkv, D).total;
}

int hs2_kv_bridge_layers(const void* hidden, int32_t T, int32_t d_model, const void* w_kv, int32_t L,
                         const hs2_kv_out_desc* caches, int32_t batch_index, int32_t pos0, int32_t scale_mode,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return bridge_impl("hs2_kv_bridge_layers", hidden, T, d_model, w_kv, L, caches, batch_index, pos0, scale_mode,
                     workspace, workspace_bytes, stream);
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

int hs2_debug_scan_read_probe(const hs2_kv_desc* kv, int32_t Hq, int32_t with_codes, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  const char* name = "hs2_debug_scan_read_probe";
  int st = check_kv(kv, name);
  if (st) return st;
  if (kv->dtype == HS2_F32) return fail(HS2_ERR_UNSUPPORTED, std::string(name) + ": bf16 or FP8_E4M3FN cache only");
  if (Hq <= 0 || Hq % kv->Hkv || Hq / kv->Hkv > 16)
    return fail(HS2_ERR_INVALID_ARG, std::string(name) + ": Hq must be a multiple of Hkv with at most 16 heads per group");
  const FullPlan pl = plan_full(kv, 1, Hq);
  if (!workspace || workspace_bytes < pl.total)
    return fail(HS2_ERR_WORKSPACE, std::string(name) + ": workspace needs " + std::to_string(pl.total) + " bytes");
  if ((uintptr_t)workspace & 255) return fail(HS2_ERR_INVALID_ARG, std::string(name) + ": workspace must be 256-byte aligned");
  hs2::ScanParams p{};
  p.k = kv->k;
  p.v = kv->v;
  p.sb = kv->stride_b;
  p.sh = kv->stride_h;
  p.sn = kv->stride_n;
  p.B = kv->B;
  p.Hkv = kv->Hkv;
  p.N = kv->N;
  p.D = kv->D;
  p.G = Hq / kv->Hkv;
  p.Tq = 1;
  p.Hq = Hq;
  p.q_pos0 = kv->N - 1;  // one query token at the last position: the whole cache
  p.tpack = pl.tpack;
  p.n_tpacks = pl.n_tpacks;
  p.rows = pl.rows;
  p.nsplit = pl.nsplit;
  p.split_len = pl.split_len;
  p.part_o = at<float>(workspace, pl.off_o);
  p.lg16 = at<uint16_t>(workspace, pl.off_lg16);
  p.lgmax = at<float>(workspace, pl.off_lgmax);
  p.npad = pl.npad;
  const hipError_t e = hs2::launch_scan_read_probe(p, kv->dtype, with_codes != 0, stream);
  if (e != hipSuccess) return hip_fail(e, "scan_read_probe launch");
  return HS2_OK;
}

int hs2_timing_enable(int on) {
  g_timing.store(on != 0, std::memory_order_release);
  return HS2_OK;
}

int hs2_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_tmu);
  for (auto& r : g_recs) {
    (void)hipEventSynchronize(r.b);
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
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
