/*
 * hs2.h -- C ABI of the MI355X (gfx950) HySparse2 cross-decoder attention hot path.
 *
 * The method ("HySparse2: Hybrid Sparse Attention with Two-Level KV Sharing",
 * as described on javabetter.cn "mimo-v3-hysparse2", zgeo.com.cn
 * "xiaomi-mimo-v3-hysparse2-long-context-geo", aitop.news item 35442 and
 * siami.tw "xiaomi-mimo-v3-hysparse-2"): each cross-decoder hybrid block is one
 * full-attention layer followed by several sparse-attention layers
 * (javabetter.cn, the Cross-Decoder paragraph).  The full layer scans the whole
 * KV cache and its attention scores pick the tokens (javabetter.cn, first of
 * the two changes); a token-level top-k is merged with a forced window of the
 * most recent tokens (zgeo.com.cn, "core principle": 1024 global + 128 recent);
 * the sparse layers reuse the full layer's KV cache and selection indices
 * (aitop.news item 35442; javabetter.cn, KV Reuse paragraph); the full layer's
 * K/V come from a self-decoder hidden state through that layer's own
 * projection (javabetter.cn, KV Bridging paragraph).
 *
 * Conventions shared by every call:
 *   - All tensor pointers are DEVICE pointers unless stated otherwise; the
 *     caller allocates and owns every buffer (inputs, outputs, workspace).  The
 *     library never allocates, frees or retains a pointer beyond the call.
 *   - Calls are asynchronous on `stream`; results are valid once the stream
 *     reaches the call.  Calls never synchronise, print or abort.
 *   - The library keeps no state of its own beyond the per-kernel timing
 *     records (hs2_timing_*); every call is thread-safe.  Calls that share a
 *     workspace must be ordered on one stream.
 *   - Every call validates its arguments before any launch and returns an
 *     hs2 status; on failure hs2_last_error() holds a thread-local message.
 *   - Layouts are dense row-major unless strides are given:
 *       q, out : [B, Tq, Hq, D]     lse : [B, Tq, Hq] fp32
 *       scores : [B, Tq, Hkv, N] fp32
 *       idx    : [B, Tq, Hkv, max_sel] int32, count : [B, Tq, Hkv] int32
 *     Query head h belongs to KV group g = h / (Hq / Hkv).  Query token t sits
 *     at cache position p = q_pos0 + t and attends to positions [0, p].
 *   - Variable-length batches: the calls that take q_pos0 also take
 *     q_pos0_b, a DEVICE array of B int32 (or NULL).  When given, query token
 *     t of batch entry b sits at q_pos0_b[b] + t instead (each entry's own
 *     context length, up to N); values outside [0, N - Tq] are clamped into
 *     it on the device (the host cannot read them without a sync), so every
 *     access stays inside the cache.  q_pos0 itself must still be valid.
 *   - Base pointers must be 16-byte aligned; the K/V row stride (stride_n
 *     times the element size) and the other K/V strides must be multiples of
 *     16 bytes.
 *   - Supported: head_dim D in {64, 128}; group size Hq/Hkv <= 16; (q, kv)
 *     element types (F32, F32), (BF16, BF16), (BF16, FP8_E4M3FN).
 */
#ifndef HS2_H
#define HS2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t* hipStream_t;

#define HS2_ABI_VERSION 3

typedef enum { HS2_F32 = 0, HS2_BF16 = 1, HS2_FP8_E4M3FN = 2 } hs2_dtype;

/* Selection flags (hs2_select_topk_window, hs2_full_attn_topk). */
enum { HS2_SEL_WINDOW_COMPETES = 1 };

enum {
  HS2_OK = 0,
  HS2_ERR_INVALID_ARG = -1, /* bad shape, pointer, alignment or range          */
  HS2_ERR_UNSUPPORTED = -2, /* valid but not implemented (D, G, dtype pair)    */
  HS2_ERR_WORKSPACE = -3,   /* workspace smaller than the *_workspace() figure */
  HS2_ERR_HIP = -4          /* a HIP launch failed; see hs2_last_error()       */
};

/* One layer's shared K/V cache.  Element (b, h, n, d) of K is at
 * k[b*stride_b + h*stride_h + n*stride_n + d] (strides in elements, d
 * contiguous).  For FP8_E4M3FN caches (OCP E4M3FN codes, as the pages' FP8 KV
 * cache accounting -- zgeo.com.cn comparison table), k_scale and v_scale hold
 * one fp32 scale per (b, kv head), index b*Hkv + h, and the cache value is
 * decode(code) * scale; they are ignored (may be NULL) otherwise.  The
 * attention calls only read through this descriptor. */
typedef struct {
  const void* k;
  const void* v;
  int32_t dtype; /* hs2_dtype */
  int64_t stride_b, stride_h, stride_n;
  const float* k_scale;
  const float* v_scale;
  int32_t B, Hkv, N, D;
} hs2_kv_desc;

/* The same cache seen by a call that writes it (hs2_kv_bridge): same fields,
 * layout and rules as hs2_kv_desc, with writable pointers. */
typedef struct {
  void* k;
  void* v;
  int32_t dtype; /* hs2_dtype */
  int64_t stride_b, stride_h, stride_n;
  float* k_scale;
  float* v_scale;
  int32_t B, Hkv, N, D;
} hs2_kv_out_desc;

int hs2_abi_version(void);
const char* hs2_status_string(int status);
/* Message of the calling thread's last failure ("" if none). */
const char* hs2_last_error(void);

/* Full-attention layer of a hybrid block (javabetter.cn: the full layer looks
 * at everything from start to end, and its attention scores -- how related the
 * current token is to each earlier token -- are what the selection uses).
 * For every (b, t, h), logits s_j = softmax_scale * <q[b,t,h], k[b,g,j]> for
 * j in [0, p]:
 *   out[b,t,h]  = sum_j softmax(s)_j * v[b,g,j]    (q's element type, RNE)
 *   lse[b,t,h]  = log sum_j exp(s_j)               (natural log; may be NULL)
 *   scores[b,t,g,j] = sum over the query heads h of group g of softmax(s)_j
 *                     for j <= p, and 0 for p < j < N.
 * Requires 0 <= q_pos0 and q_pos0 + Tq <= N.  Workspace: at least
 * hs2_full_attn_scores_workspace(kv, Tq, Hq) bytes, 256-byte aligned, device
 * memory; its contents on entry are ignored.  Two calls that share one
 * workspace must not run concurrently (different streams).
 * Execution: a scan, a merge and a score kernel.  With many query tokens
 * (bf16 or FP8 cache, 4, 8 or 16 query heads per kv head, at least 4 packs of
 * 16/G tokens per (b, kv head), as in a 512-token chunk) the scan is a
 * matrix-core pass over K/V tiles staged in LDS, and the score kernel
 * recomputes the logits against the merged log-sum-exp instead of reading
 * stored codes.  Both compute the same quantities to the same bounds.  Rows
 * of the cache must be 16-byte aligned; the chunk kernels also need 32 rows
 * to span less than 2 GiB
 * (HS2_ERR_HIP otherwise). */
size_t hs2_full_attn_scores_workspace(const hs2_kv_desc* kv, int32_t Tq, int32_t Hq);
int hs2_full_attn_scores(const hs2_kv_desc* kv, const void* q, hs2_dtype q_dtype, int32_t Tq,
                         int32_t Hq, int32_t q_pos0, const int32_t* q_pos0_b, float softmax_scale,
                         void* out, float* lse, float* scores, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* Token-level top-k with a forced recent window (zgeo.com.cn "core
 * principle": 1024 global tokens picked and the most recent 128 always kept;
 * javabetter.cn, the two changes versus HySparse).  For each (b, t, g) with
 * p = q_pos0 + t: window Wn = [max(0, p-window+1), p]; candidates
 * C = [0, p-window] (empty when p < window).
 *   block_size == 1: T = the min(k, |C|) candidates with the largest scores,
 *     ties to the lower position.
 *   block_size  > 1: the previous generation's block baseline (zgeo.com.cn
 *     comparison table: 64-token blocks): aligned blocks of block_size
 *     positions clipped to C, block mass = sum of its scores (fp64 sum in
 *     ascending position), the min(k, #blocks) heaviest blocks (ties to the
 *     lower block), T = their positions; k counts blocks.
 *   idx[b,t,g,:count] = ascending(T union Wn); idx[b,t,g,count:] = -1.
 * flags: 0, or HS2_SEL_WINDOW_COMPETES (token mode only; HS2_ERR_UNSUPPORTED
 * with block_size > 1): the other reading of the two budgets, where the
 * window does not reserve its own: C = [0, p], T = its min(k, p+1) best, and
 * the list is the ascending union of T and Wn (count between
 * min(k, p+1) and min(k, p+1) + |Wn|; the pages name 1024 global tokens and
 * 128 forced recent ones without saying whether the two sets may overlap).
 * Scores must be finite and >= 0 (the full layer's scores are).
 * max_sel >= min(k*block_size + window, N) is required.  Workspace: at least
 * hs2_select_workspace(B, Tq, Hkv, N) bytes (covers both modes). */
size_t hs2_select_workspace(int32_t B, int32_t Tq, int32_t Hkv, int32_t N);
/* Tighter figure for one block_size (what the call actually checks). */
size_t hs2_select_workspace_for(int32_t B, int32_t Tq, int32_t Hkv, int32_t N, int32_t block_size);
int hs2_select_topk_window(const float* scores, int32_t B, int32_t Tq, int32_t Hkv, int32_t N,
                           int32_t q_pos0, const int32_t* q_pos0_b, int32_t k, int32_t window,
                           int32_t block_size, int32_t flags, int32_t* idx, int32_t* count,
                           int32_t max_sel, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Sparse-attention layer with KV reuse (aitop.news item 35442: sparse layers
 * reuse the previous full-attention layer's KV cache and selection indices;
 * javabetter.cn: they neither compute nor store K/V).  For every (b, t, h),
 * g = h / (Hq/Hkv), rows j in idx[b,t,g,0:count[b,t,g]]:
 *   out[b,t,h] = sum_j softmax_j(softmax_scale * <q[b,t,h], k[b,g,j]>) v[b,g,j]
 *   lse[b,t,h] = log sum_j exp(...)       (may be NULL)
 * Every listed index must lie in [0, N) (not checked on the device: the list
 * is read on the GPU); 0 <= count <= max_sel.  An empty list gives out = 0
 * and lse = -inf.  No workspace. */
int hs2_sparse_attn_gather(const hs2_kv_desc* kv, const void* q, hs2_dtype q_dtype, int32_t Tq,
                           int32_t Hq, float softmax_scale, const int32_t* idx,
                           const int32_t* count, int32_t max_sel, void* out, float* lse,
                           hipStream_t stream);

/* The same sparse layer with a caller workspace: each (b, t, g) list is cut
 * into slices of 128 entries, one workgroup per slice, and the last slice to
 * finish merges the partials -- many more workgroups at small batch.  The
 * workspace (device, 256-byte aligned, at least hs2_sparse_attn_workspace()
 * bytes) holds per-(b, t, g) arrival counters that MUST be zero before the
 * first call on it (e.g. zero-filled at allocation); every call leaves them
 * zero again.  Calls that share a workspace must be ordered on one stream.
 * fp32 caches, and calls with 64 or more (b, t, g) lists (where one
 * workgroup per list already fills the GPU), take the workspace-free path. */
size_t hs2_sparse_attn_workspace(int32_t B, int32_t Tq, int32_t Hkv, int32_t D, int32_t max_sel);
int hs2_sparse_attn_gather_ws(const hs2_kv_desc* kv, const void* q, hs2_dtype q_dtype, int32_t Tq,
                              int32_t Hq, float softmax_scale, const int32_t* idx,
                              const int32_t* count, int32_t max_sel, void* out, float* lse,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The same split sparse layer for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): same arguments, rules and results as hs2_sparse_attn_gather_ws
 * without the workspace.  The split's partials and arrival counters live in a
 * static device array of the library, hs2_sparse_attn_static_limit() bytes
 * (4 MiB) on every GPU the library runs on, held until the process ends; a
 * call whose split would need more returns HS2_ERR_WORKSPACE (the split
 * needs about units * ceil(max_sel / 128) * 16 * (D + 2) * 4 bytes, units =
 * B * Tq * Hkv; a call that takes the one-workgroup path -- fp32 caches, 64
 * or more lists, lists too long for the split's merge -- needs none).  The first call on a
 * device also clears the counters on `stream`.  The call itself allocates
 * nothing.  Every call on one GPU shares that GPU's array: calls that overlap
 * on one GPU (any streams, any threads) race and must be ordered by the
 * caller. */
size_t hs2_sparse_attn_static_limit(void);
int hs2_sparse_attn_gather_static(const hs2_kv_desc* kv, const void* q, hs2_dtype q_dtype, int32_t Tq,
                                  int32_t Hq, float softmax_scale, const int32_t* idx,
                                  const int32_t* count, int32_t max_sel, void* out, float* lse,
                                  hipStream_t stream);

/* Sliding-window attention of the self-decoder's hybrid layers
 * (javabetter.cn: MiMo-V2.6-Flash's 39 sliding-window layers, each token
 * attending to its nearest 128 tokens; the self-decoder mixes such layers
 * with full attention -- javabetter.cn, Self-Decoder paragraph; siami.tw
 * section one).  For every (b, t, h), p = q_pos0 + t, rows
 * j in [max(0, p - window + 1), p] (the current token included):
 *   out[b,t,h] = sum_j softmax_j(softmax_scale * <q[b,t,h], k[b,g,j]>) v[b,g,j]
 *   lse[b,t,h] = log sum_j exp(...)       (may be NULL)
 * This is the sparse layer with k = 0 and the window alone; it reads the
 * window's rows directly (no index list).  Prefill-sized calls (bf16 or FP8
 * cache, 4, 8 or 16 query heads per kv head, at least 4 packs of 16/G tokens
 * per (b, kv head)) run a banded matrix-core pass over the LDS-staged K/V
 * tiles of each 16-token block's window; others one workgroup per
 * (b, t, g).  Requires 0 <= q_pos0, q_pos0 + Tq <= N, window >= 1.  No
 * workspace. */
int hs2_swa_attn(const hs2_kv_desc* kv, const void* q, hs2_dtype q_dtype, int32_t Tq, int32_t Hq,
                 int32_t q_pos0, const int32_t* q_pos0_b, int32_t window, float softmax_scale,
                 void* out, float* lse, hipStream_t stream);

/* KV bridge (javabetter.cn, KV Bridging paragraph: a cross-decoder full layer
 * computes its K and V from a self-decoder layer's hidden state, with its own
 * parameters).  y = hidden [T, d_model] (bf16) x w_kv [d_model, 2*Hkv*D]
 * (bf16), fp32 accumulation; columns [0, Hkv*D) are K heads 0..Hkv-1 and
 * [Hkv*D, 2*Hkv*D) are V heads, head-major.  The rows are written into
 * kv_out at batch batch_index, positions [pos0, pos0 + T): a BF16 cache
 * receives y rounded to bf16 (RNE); an FP8_E4M3FN cache (the pages' FP8 KV
 * cache -- zgeo.com.cn comparison table) receives the E4M3FN code of
 * y / scale, scale = kv_out's k_scale or v_scale entry of (batch_index, head)
 * (read, not changed: the caller keeps each head's scale, which must be
 * positive), rounded to nearest even with magnitudes above 448 saturating to
 * 448.  Requires d_model % 64 == 0. */
int hs2_kv_bridge(const void* hidden, int32_t T, int32_t d_model, const void* w_kv,
                  const hs2_kv_out_desc* kv_out, int32_t batch_index, int32_t pos0, hipStream_t stream);

/* The bridge of L cross-decoder full layers from one hidden state (javabetter.cn,
 * KV Bridging paragraph: every cross-decoder full layer derives its own K/V
 * from the same self-decoder hidden state with its own parameters), in one
 * launch: layer l projects `hidden` with w_kv + l * d_model * 2*Hkv*D
 * ([L, d_model, 2*Hkv*D] bf16, contiguous) into caches[l] (a HOST array of L
 * descriptors, 1 <= L <= 16, sharing dtype, Hkv and D), batch batch_index,
 * rows [pos0, pos0 + T).  T = 1 is the per-token append of decoding.
 * bf16 caches: as hs2_kv_bridge.  FP8_E4M3FN caches, by scale_mode:
 *   HS2_SCALE_KEEP: as hs2_kv_bridge (the scales are read and must be > 0);
 *   HS2_SCALE_GROW: per-head scale maintenance (the pages give no rule; this
 *     is this library's reading): for each (layer, K/V, head), s' = max(s,
 *     max|y| / 448) over the new rows y (fp32); the scale is set to s'; if s'
 *     > s, the head's rows [0, pos0) are re-encoded in place as
 *     encode(fp32(decode(code) * s) / s') -- a pass over those rows, paid only
 *     when a scale grows; the new rows get encode(y / s') (zero codes while s'
 *     is 0).  Needs a workspace of hs2_kv_bridge_layers_workspace(L, T, Hkv, D)
 *     bytes (256-byte aligned).  A head's scale may start at 0 (empty cache).
 * encode() rounds to nearest even and saturates at +-448.  Requires d_model %
 * 64 == 0. */
enum { HS2_SCALE_KEEP = 0, HS2_SCALE_GROW = 1 };
size_t hs2_kv_bridge_layers_workspace(int32_t L, int32_t T, int32_t Hkv, int32_t D);
int hs2_kv_bridge_layers(const void* hidden, int32_t T, int32_t d_model, const void* w_kv, int32_t L,
                         const hs2_kv_out_desc* caches, int32_t batch_index, int32_t pos0,
                         int32_t scale_mode, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Diagnostic: decode n OCP E4M3FN codes (device array) to fp32 through the
 * same in-register conversion the attention kernels use.  Lets a test compare
 * the hardware conversion with the format's definition code by code. */
int hs2_debug_e4m3fn_to_f32(const uint8_t* codes, float* out, int32_t n, hipStream_t stream);

/* Diagnostic: streaming-read probe.  Reads `bytes` (a multiple of 16) of the
 * 16-byte aligned device buffer `buf` once with 16-byte non-temporal loads
 * from `blocks` workgroups of 256 threads, and writes one word per thread to
 * `out` (blocks*256 uint32).  Its duration (kernel "stream_read") gives the
 * HBM read bandwidth this GPU actually sustains, the ceiling the scan is
 * compared with. */
int hs2_debug_stream_read(const void* buf, size_t bytes, uint32_t* out, int32_t blocks, hipStream_t stream);

/* Diagnostic: read-pattern probe of the decode scan.  Runs the full layer's
 * decode plan (one query token at position N-1 of every batch row, Hq query
 * heads) with the scan's grid, position splits, per-lane loads and tile loop
 * over the cache `kv` (bf16 or FP8_E4M3FN, D = 64 or 128), with the attention
 * arithmetic replaced by an xor of the loaded words; with_codes != 0 adds the
 * scan's stores of 16-bit logit codes and tile maxima.  The results are
 * scratch: the workspace (hs2_full_attn_scores_workspace(kv, 1, Hq) bytes,
 * 256-byte aligned) receives the codes and one word per thread.  Its duration
 * (kernels "scan_read_probe" and "scan_read_probe_codes") beside the scan's
 * ("full_scan") separates the cache read, the code writes and the arithmetic
 * in the scan's cost.  Errors: HS2_ERR_INVALID_ARG for a bad descriptor, Hq
 * or alignment, HS2_ERR_UNSUPPORTED for an fp32 cache, HS2_ERR_WORKSPACE when
 * the workspace is short. */
int hs2_debug_scan_read_probe(const hs2_kv_desc* kv, int32_t Hq, int32_t with_codes, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* Full layer and token selection in one call: the results of
 * hs2_full_attn_scores followed by hs2_select_topk_window with block_size 1
 * (same layouts, rules, flags and requirements; both passages above).  With one
 * query token per (b, kv head) unit, the full layer sets the selection's rows
 * up (a bf16/FP8 scan itself, an fp32 cache in its merge kernel) and its score
 * kernel counts the selection's first radix digit while writing the scores,
 * which saves the selection two passes over them; with a bf16/FP8 cache the
 * split merge runs in the same launch as the scores.  Workspace: at least hs2_full_attn_topk_workspace() bytes, 256-byte
 * aligned. */
size_t hs2_full_attn_topk_workspace(const hs2_kv_desc* kv, int32_t Tq, int32_t Hq);
int hs2_full_attn_topk(const hs2_kv_desc* kv, const void* q, hs2_dtype q_dtype, int32_t Tq, int32_t Hq,
                       int32_t q_pos0, const int32_t* q_pos0_b, float softmax_scale, void* out, float* lse,
                       float* scores, int32_t k, int32_t window, int32_t flags, int32_t* idx,
                       int32_t* count, int32_t max_sel, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* Paged cache (decode path): the rows of all sequences live in a shared pool
 * of fixed-size pages, and a table maps each sequence's logical pages to pool
 * pages, as a serving layer that owns the cache memory hands them out (the
 * pages treat the cache as one array per layer; paging is a layout of that
 * array, not part of the method).  The descriptor's k/v point at the pool:
 * row r of kv head h at k + h*stride_h + r*stride_n, stride_b = 0, N the
 * logical length of every sequence; logical row j of sequence b is pool row
 * table[b*pages_per_seq + j/page_rows]*page_rows + j%page_rows.  Results are
 * those of the contiguous cache holding the same rows, bit for bit. */
typedef struct {
  const int32_t* table;  /* device [B][pages_per_seq]; entries are clamped to [0, pool_pages) */
  int32_t page_rows;     /* rows per page: a power of two, at least 32 */
  int32_t pages_per_seq; /* table entries per sequence; pages_per_seq * page_rows >= N */
  int32_t pool_pages;    /* pages in the pool; pool_pages * page_rows < 2^31 */
} hs2_page_table;

/* hs2_full_attn_topk over a paged cache: same arguments, rules, results and
 * workspace (hs2_full_attn_topk_workspace with the logical N) plus `pages`.
 * bf16/FP8 caches; calls that take the multi-query chunk path (many query
 * tokens per kv head) return HS2_ERR_UNSUPPORTED, as does an fp32 cache;
 * HS2_ERR_INVALID_ARG for a page table outside the rules above. */
int hs2_full_attn_topk_paged(const hs2_kv_desc* kv, const hs2_page_table* pages, const void* q, hs2_dtype q_dtype,
                             int32_t Tq, int32_t Hq, int32_t q_pos0, const int32_t* q_pos0_b, float softmax_scale,
                             void* out, float* lse, float* scores, int32_t k, int32_t window, int32_t flags,
                             int32_t* idx, int32_t* count, int32_t max_sel, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);
/* hs2_sparse_attn_gather_ws over a paged cache (the index lists hold logical
 * positions): same arguments, rules, results and workspace plus `pages`;
 * bf16/FP8 caches. */
int hs2_sparse_attn_gather_paged(const hs2_kv_desc* kv, const hs2_page_table* pages, const void* q,
                                 hs2_dtype q_dtype, int32_t Tq, int32_t Hq, float softmax_scale, const int32_t* idx,
                                 const int32_t* count, int32_t max_sel, void* out, float* lse, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/* Per-kernel timing with HIP events on the launch stream (off by default; a
 * measurement aid, process-wide).  While enabled, every kernel launch of the
 * library is bracketed by an event pair on its stream.  hs2_timing_collect
 * synchronises those events and returns, for launches of the named kernel
 * since the last reset, the summed milliseconds and the launch count;
 * hs2_timing_reset waits for and destroys the recorded events.  Names: see
 * hs2_timing_kernel_name. */
int hs2_timing_enable(int on);
int hs2_timing_reset(void);
int hs2_timing_collect(const char* kernel_name, double* total_ms, int32_t* launches);
/* i-th kernel name (NULL past the end). */
const char* hs2_timing_kernel_name(int32_t i);

#ifdef __cplusplus
}
#endif
#endif /* HS2_H */
