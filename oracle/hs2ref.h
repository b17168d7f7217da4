/*
 * hs2ref.h -- plain fp64 CPU oracle for the HySparse2 cross-decoder attention
 * hot path.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg use it to check and time the HIP library; the
 * library itself never includes, links or calls anything here.
 *
 * What it computes, following the pages ("HySparse2: Hybrid Sparse Attention
 * with Two-Level KV Sharing", as retold on javabetter.cn "mimo-v3-hysparse2",
 * zgeo.com.cn "xiaomi-mimo-v3-hysparse2-long-context-geo", aitop.news item 35442
 * and siami.tw "xiaomi-mimo-v3-hysparse-2"):
 *
 *   full layer     : causal softmax attention of every query head over the
 *                    whole shared K/V cache, plus per-token importance scores
 *                    taken from that layer's attention (javabetter.cn, the
 *                    paragraph on what the selection is based on).
 *   selection      : token-level top-k (1024 in the pages) plus a forced window
 *                    of the most recent tokens (128) (zgeo.com.cn, "core
 *                    principle" section and comparison table; javabetter.cn,
 *                    the "second change" paragraph).
 *   sparse layers  : attention over only the selected rows of the same cache,
 *                    reusing the full layer's K/V and index list
 *                    (aitop.news item 35442; javabetter.cn, KV Reuse paragraph).
 *   KV bridge      : K/V of a cross-decoder full layer computed from a
 *                    self-decoder hidden state with that layer's own projection
 *                    (javabetter.cn, KV Bridging paragraph).
 *
 * Where the pages are silent (score aggregation over GQA heads, tie rule,
 * whether the window competes, whether the window includes the current token,
 * output rounding, ...), each function below states the reading it uses.
 *
 * All arithmetic is IEEE fp64, two-pass softmax, sequential sums; no blocking,
 * no fusion, no reordering beyond what the definitions state.
 */
#ifndef HS2REF_H
#define HS2REF_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { HS2REF_F32 = 0, HS2REF_BF16 = 1, HS2REF_E4M3FN = 2 };

enum {
  HS2REF_OK = 0,
  HS2REF_ERR_ARG = -1,
  HS2REF_ERR_MEM = -2,
  HS2REF_ERR_CAPACITY = -3
};

/* One layer's K/V cache: element (b, h, n, d) of K is at
 * k[b*stride_b + h*stride_h + n*stride_n + d] (element units).  For E4M3FN
 * caches k_scale/v_scale hold one fp32 scale per (b, kv-head), index b*Hkv+h;
 * the dequantised value is fp32(decode(code) * scale), as a float32 multiply. */
typedef struct {
  const void* k;
  const void* v;
  int32_t dtype;
  int64_t stride_b, stride_h, stride_n;
  const float* k_scale;
  const float* v_scale;
  int32_t B, Hkv, N, D;
} hs2ref_kv;

/* OCP E4M3FN closed form: sign, 4 exponent bits (bias 7), 3 mantissa bits;
 * exponent 0 is subnormal 2^-6 * m/8; code S.1111.111 is NaN; no infinities. */
double hs2ref_e4m3fn_decode(uint32_t code);
/* bfloat16 bits -> value (upper half of an IEEE binary32). */
double hs2ref_bf16_decode(uint32_t bits);

int hs2ref_num_threads(void);

/* Full causal attention + importance scores.
 * q [B,Tq,Hq,D] (q_dtype F32 or BF16), query t sits at position p = q_pos0+t.
 * For every (b,t,h) with g = h / (Hq/Hkv):
 *   s_j = scale * <q, k_j>,  j in [0, p];  m = max s;  w = exp(s - m);
 *   L = sum w;  P = w / L;  out = sum_j P_j v_j;  lse = m + log L.
 * scores[b,t,g,j] = sum over the Hq/Hkv heads of group g of P_j for j <= p,
 * and 0 for p < j < N.  Any output pointer may be NULL. */
int hs2ref_full_attn_scores(const hs2ref_kv* kv, const void* q, int32_t q_dtype,
                            int32_t Tq, int32_t Hq, int32_t q_pos0, double scale,
                            double* out, double* lse, double* scores);

/* Token-level top-k with a forced recent window, or the 64-token-block
 * baseline when block_size > 1 (then k counts blocks).
 * For each (b,t,g) with p = q_pos0 + t:
 *   window Wn = [max(0, p-window+1), p];  candidates C = [0, p-window]
 *   (C = [0, p] when window_competes != 0).
 *   token mode: T = first min(k,|C|) of C ordered by (score desc, position asc).
 *   block mode: blocks beta with C meeting [bs*beta, bs*beta+bs-1]; block mass =
 *   sum of scores over that intersection; take the first min(k, #blocks) by
 *   (mass desc, beta asc); T = their C positions.
 *   Sel = ascending(T union Wn); idx[b,t,g, 0..count) = Sel, rest = -1.
 * scores [B,Tq,Hkv,N]; idx [B,Tq,Hkv,max_sel]; count [B,Tq,Hkv].
 * Returns HS2REF_ERR_CAPACITY when a selection exceeds max_sel. */
int hs2ref_select_topk_window(const double* scores, int32_t B, int32_t Tq, int32_t Hkv,
                              int32_t N, int32_t q_pos0, int32_t k, int32_t window,
                              int32_t block_size, int32_t window_competes,
                              int32_t* idx, int32_t* count, int32_t max_sel);

/* Sparse attention over an index list (KV reuse): for every (b,t,h), g = h/G,
 * rows j in idx[b,t,g,0..count): s = scale*<q,k_j>, two-pass softmax, out,
 * lse.  Indices must lie in [0, N). */
int hs2ref_sparse_attn(const hs2ref_kv* kv, const void* q, int32_t q_dtype,
                       int32_t Tq, int32_t Hq, double scale,
                       const int32_t* idx, const int32_t* count, int32_t max_sel,
                       double* out, double* lse);

/* KV bridge: y[t, c] = sum_r hidden[t, r] * w[r, c] for c in [0, 2*Hkv*D),
 * bf16 inputs, fp64 sums.  Columns [0, Hkv*D) are K heads 0..Hkv-1 (head-major),
 * columns [Hkv*D, 2*Hkv*D) are V heads.  y is [T, 2*Hkv*D]. */
int hs2ref_kv_bridge(const uint16_t* hidden, int32_t T, int32_t d_model,
                     const uint16_t* w_kv, int32_t Hkv, int32_t D, double* y);

#ifdef __cplusplus
}
#endif
#endif
