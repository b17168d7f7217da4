/*
 * hs2ref.c -- plain fp64 CPU oracle for the HySparse2 cross-decoder attention
 * hot path.  TEST INFRASTRUCTURE ONLY (see hs2ref.h for what each function
 * computes and which page passage it follows).  Nothing in the HIP library
 * includes, links or calls this file.
 *
 * HS2REF_MUTANT: the default build (0) is the oracle.  Non-zero values plant
 * one deliberate mistake each; the CPU test suite builds those variants to
 * show that its pins catch every one of them.  They are never used otherwise.
 */
#include "hs2ref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef HS2REF_MUTANT
#define HS2REF_MUTANT 0
#endif

/* ------------------------------------------------------------------ */
/* element decoding                                                     */
/* ------------------------------------------------------------------ */

double hs2ref_e4m3fn_decode(uint32_t code) {
  const uint32_t s = (code >> 7) & 1u, e = (code >> 3) & 15u, m = code & 7u;
#if HS2REF_MUTANT == 11
  const int bias = 8;
#else
  const int bias = 7;
#endif
  double mag;
  if (e == 15u && m == 7u) return NAN;
  if (e == 0u)
    mag = ldexp((double)m / 8.0, 1 - bias);
  else
    mag = ldexp(1.0 + (double)m / 8.0, (int)e - bias);
  return s ? -mag : mag;
}

double hs2ref_bf16_decode(uint32_t bits) {
  uint32_t u = (bits & 0xFFFFu) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

int hs2ref_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

static float g_e4m3[256];
static int g_e4m3_ready = 0;

static void ensure_tables(void) {
  if (g_e4m3_ready) return;
#ifdef _OPENMP
#pragma omp critical(hs2ref_tables)
#endif
  {
    if (!g_e4m3_ready) {
      for (int c = 0; c < 256; ++c) g_e4m3[c] = (float)hs2ref_e4m3fn_decode((uint32_t)c);
      g_e4m3_ready = 1;
    }
  }
}

/* One element of a K or V cache, dequantised as the pages' FP8 cache would be
 * read: fp32(decode(code) * scale) for E4M3FN, the stored value otherwise. */
static double kv_elem(const hs2ref_kv* kv, int which_v, int64_t b, int64_t h, int64_t n, int64_t d) {
  const int64_t off = b * kv->stride_b + h * kv->stride_h + n * kv->stride_n + d;
  const void* base = which_v ? kv->v : kv->k;
  switch (kv->dtype) {
    case HS2REF_F32:
      return (double)((const float*)base)[off];
    case HS2REF_BF16:
      return hs2ref_bf16_decode(((const uint16_t*)base)[off]);
    default: {
      const float sc = (which_v ? kv->v_scale : kv->k_scale)[b * kv->Hkv + h];
      const float prod = g_e4m3[((const uint8_t*)base)[off]] * sc;
      return (double)prod;
    }
  }
}

static double q_elem(const void* q, int32_t q_dtype, int64_t off) {
  if (q_dtype == HS2REF_F32) return (double)((const float*)q)[off];
  return hs2ref_bf16_decode(((const uint16_t*)q)[off]);
}

static int check_kv(const hs2ref_kv* kv) {
  if (!kv || !kv->k || !kv->v) return 0;
  if (kv->B <= 0 || kv->Hkv <= 0 || kv->N <= 0 || kv->D <= 0) return 0;
  if (kv->dtype != HS2REF_F32 && kv->dtype != HS2REF_BF16 && kv->dtype != HS2REF_E4M3FN) return 0;
  if (kv->dtype == HS2REF_E4M3FN && (!kv->k_scale || !kv->v_scale)) return 0;
  return 1;
}

/* ------------------------------------------------------------------ */
/* full layer: attention output, LSE and importance scores              */
/* ------------------------------------------------------------------ */

/* One (b, t, g): the G query heads of group g of token t (javabetter.cn: the
 * full layer looks at every earlier token; its attention scores, i.e. how
 * related the current token is to each earlier one, pick the tokens). */
static int full_unit(const hs2ref_kv* kv, const void* q, int32_t q_dtype, int32_t Tq, int32_t Hq,
                     int32_t q_pos0, double scale, int b, int t, int g,
                     double* out, double* lse, double* scores, int par) {
  const int D = kv->D, N = kv->N, G = Hq / kv->Hkv;
#if HS2REF_MUTANT == 3
  const int64_t p = (int64_t)q_pos0 + t - 1; /* drops the current token */
#else
  const int64_t p = (int64_t)q_pos0 + t;
#endif
  const int64_t npos = p + 1;
  double* prob = (double*)malloc(sizeof(double) * (size_t)G * (size_t)(npos > 0 ? npos : 1));
  double* qv = (double*)malloc(sizeof(double) * (size_t)D);
  double* row = (double*)malloc(sizeof(double) * (size_t)D);
  if (!prob || !qv || !row) {
    free(prob); free(qv); free(row);
    return HS2REF_ERR_MEM;
  }
  for (int i = 0; i < G; ++i) {
#if HS2REF_MUTANT == 2
    const int h = i * kv->Hkv + g; /* wrong GQA mapping */
#else
    const int h = g * G + i;
#endif
    const int64_t qoff = (((int64_t)b * Tq + t) * Hq + h) * D;
    for (int d = 0; d < D; ++d) qv[d] = q_elem(q, q_dtype, qoff + d);
    double* s = prob + (size_t)i * (size_t)npos;
    /* logits */
#ifdef _OPENMP
#pragma omp parallel for schedule(static) if (par)
#endif
    for (int64_t j = 0; j < npos; ++j) {
      double acc = 0.0;
      for (int d = 0; d < D; ++d) acc += qv[d] * kv_elem(kv, 0, b, g, j, d);
#if HS2REF_MUTANT == 1
      s[j] = acc; /* scale dropped */
#else
      s[j] = scale * acc;
#endif
    }
    /* two-pass softmax */
    double m = -INFINITY;
    for (int64_t j = 0; j < npos; ++j) m = s[j] > m ? s[j] : m;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) if (par)
#endif
    for (int64_t j = 0; j < npos; ++j) s[j] = exp(s[j] - m);
    double L = 0.0;
    for (int64_t j = 0; j < npos; ++j) L += s[j];
#if HS2REF_MUTANT != 4
#ifdef _OPENMP
#pragma omp parallel for schedule(static) if (par)
#endif
    for (int64_t j = 0; j < npos; ++j) s[j] = s[j] / L;
#endif
    /* output */
    if (out) {
      /* each element: its terms added in ascending position */
#ifdef _OPENMP
#pragma omp parallel for schedule(static) if (par)
#endif
      for (int d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int64_t j = 0; j < npos; ++j) {
#if HS2REF_MUTANT == 4
          const double pj = s[j] / L;
#else
          const double pj = s[j];
#endif
#if HS2REF_MUTANT == 15
          acc += pj * kv_elem(kv, 0, b, g, j, d); /* K for V */
#else
          acc += pj * kv_elem(kv, 1, b, g, j, d);
#endif
        }
        row[d] = acc;
      }
      const int64_t ooff = (((int64_t)b * Tq + t) * Hq + (g * G + i)) * D;
      for (int d = 0; d < D; ++d) out[ooff + d] = row[d];
    }
    if (lse) {
#if HS2REF_MUTANT == 12
      lse[((int64_t)b * Tq + t) * Hq + (g * G + i)] = m + L;
#else
      lse[((int64_t)b * Tq + t) * Hq + (g * G + i)] = m + log(L);
#endif
    }
  }
  if (scores) {
    double* srow = scores + (((int64_t)b * Tq + t) * kv->Hkv + g) * (int64_t)N;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) if (par)
#endif
    for (int64_t j = 0; j < N; ++j) {
      double acc = 0.0;
      if (j < npos)
        for (int i = 0; i < G; ++i) acc += prob[(size_t)i * (size_t)npos + (size_t)j];
      srow[j] = acc;
    }
  }
  free(prob); free(qv); free(row);
  return HS2REF_OK;
}

int hs2ref_full_attn_scores(const hs2ref_kv* kv, const void* q, int32_t q_dtype,
                            int32_t Tq, int32_t Hq, int32_t q_pos0, double scale,
                            double* out, double* lse, double* scores) {
  if (!check_kv(kv) || !q || Tq <= 0 || Hq <= 0 || Hq % kv->Hkv != 0) return HS2REF_ERR_ARG;
  if (q_dtype != HS2REF_F32 && q_dtype != HS2REF_BF16) return HS2REF_ERR_ARG;
  if (q_pos0 < 0 || (int64_t)q_pos0 + Tq > kv->N) return HS2REF_ERR_ARG;
  ensure_tables();
  const int64_t units = (int64_t)kv->B * Tq * kv->Hkv;
  int rc = HS2REF_OK;
  /* Threads go to the units; when there are fewer units than threads, to the
     positions (logits, exponentials, scores) and head dimensions (outputs) of
     one unit at a time.  Every value is formed by the same operations in the
     same order either way (the one sequential sum, L, stays sequential), so
     the results do not depend on the split. */
  const int inner = units < hs2ref_num_threads();
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) if (!inner)
#endif
  for (int64_t u = 0; u < units; ++u) {
    const int g = (int)(u % kv->Hkv);
    const int t = (int)((u / kv->Hkv) % Tq);
    const int b = (int)(u / ((int64_t)kv->Hkv * Tq));
    int r = full_unit(kv, q, q_dtype, Tq, Hq, q_pos0, scale, b, t, g, out, lse, scores, inner);
    if (r != HS2REF_OK) {
#ifdef _OPENMP
#pragma omp critical(hs2ref_rc)
#endif
      rc = r;
    }
  }
  return rc;
}

/* ------------------------------------------------------------------ */
/* selection: token top-k (or 64-token blocks) + forced recent window    */
/* ------------------------------------------------------------------ */

typedef struct {
  double s;
  int64_t j;
} keyed;

/* (score desc, position asc): the lower position wins a tie. */
static int cmp_keyed(const void* a, const void* b) {
  const keyed* x = (const keyed*)a;
  const keyed* y = (const keyed*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
#if HS2REF_MUTANT == 5
  return (x->j > y->j) ? -1 : (x->j < y->j); /* tie to the higher position */
#else
  return (x->j < y->j) ? -1 : (x->j > y->j);
#endif
}

int hs2ref_select_topk_window(const double* scores, int32_t B, int32_t Tq, int32_t Hkv,
                              int32_t N, int32_t q_pos0, int32_t k, int32_t window,
                              int32_t block_size, int32_t window_competes,
                              int32_t* idx, int32_t* count, int32_t max_sel) {
  if (!scores || !idx || !count || B <= 0 || Tq <= 0 || Hkv <= 0 || N <= 0) return HS2REF_ERR_ARG;
  if (k < 0 || window < 0 || block_size < 1 || max_sel < 0) return HS2REF_ERR_ARG;
  if (q_pos0 < 0 || (int64_t)q_pos0 + Tq > N) return HS2REF_ERR_ARG;
  const int64_t units = (int64_t)B * Tq * Hkv;
  int rc = HS2REF_OK;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t u = 0; u < units; ++u) {
    const int t = (int)((u / Hkv) % Tq);
    const int64_t p = (int64_t)q_pos0 + t;
    const double* srow = scores + u * (int64_t)N;
    int32_t* irow = idx + u * (int64_t)max_sel;
    unsigned char* mark = (unsigned char*)calloc((size_t)(p + 1), 1);
    keyed* items = (keyed*)malloc(sizeof(keyed) * (size_t)(p + 1));
    if (!mark || !items) {
      free(mark); free(items);
#ifdef _OPENMP
#pragma omp critical(hs2ref_rc)
#endif
      rc = HS2REF_ERR_MEM;
      continue;
    }
    /* forced window: the most recent `window` positions, current one included */
#if HS2REF_MUTANT == 6
    const int64_t wlo = p - window, whi = p - 1; /* excludes the current token */
#else
    const int64_t wlo = p - window + 1, whi = p;
#endif
    /* candidate range C = [0, clast] */
    const int64_t clast = window_competes ? p : (p - window);
    if (block_size == 1) {
      int64_t nc = 0;
      for (int64_t j = 0; j <= clast; ++j) {
        items[nc].s = srow[j];
        items[nc].j = j;
        ++nc;
      }
      qsort(items, (size_t)nc, sizeof(keyed), cmp_keyed);
#if HS2REF_MUTANT == 14
      const int64_t take = (k + 1 < nc) ? k + 1 : nc;
#else
      const int64_t take = (k < nc) ? k : nc;
#endif
      for (int64_t r = 0; r < take; ++r) mark[items[r].j] = 1;
    } else {
      const int64_t nb = clast >= 0 ? clast / block_size + 1 : 0;
      for (int64_t beta = 0; beta < nb; ++beta) {
        const int64_t lo = beta * block_size;
        const int64_t hi = (lo + block_size - 1 < clast) ? lo + block_size - 1 : clast;
        double mass = 0.0;
        for (int64_t j = lo; j <= hi; ++j) {
#if HS2REF_MUTANT == 13
          mass = srow[j] > mass ? srow[j] : mass; /* max instead of sum */
#else
          mass += srow[j];
#endif
        }
        items[beta].s = mass;
        items[beta].j = beta;
      }
      qsort(items, (size_t)nb, sizeof(keyed), cmp_keyed);
      const int64_t take = (k < nb) ? k : nb;
      for (int64_t r = 0; r < take; ++r) {
        const int64_t lo = items[r].j * block_size;
        const int64_t hi = (lo + block_size - 1 < clast) ? lo + block_size - 1 : clast;
        for (int64_t j = lo; j <= hi; ++j) mark[j] = 1;
      }
    }
    for (int64_t j = (wlo > 0 ? wlo : 0); j <= whi; ++j) mark[j] = 1;
    int64_t c = 0;
    int overflow = 0;
    for (int64_t j = 0; j <= p; ++j) {
      if (!mark[j]) continue;
      if (c < max_sel)
        irow[c] = (int32_t)j;
      else
        overflow = 1;
      ++c;
    }
    for (int64_t r = c; r < max_sel; ++r) irow[r] = -1;
    count[u] = (int32_t)c;
    if (overflow) {
#ifdef _OPENMP
#pragma omp critical(hs2ref_rc)
#endif
      rc = HS2REF_ERR_CAPACITY;
    }
    free(mark); free(items);
  }
  return rc;
}

/* ------------------------------------------------------------------ */
/* sparse layers: attention over the shared index list (KV reuse)        */
/* ------------------------------------------------------------------ */

int hs2ref_sparse_attn(const hs2ref_kv* kv, const void* q, int32_t q_dtype,
                       int32_t Tq, int32_t Hq, double scale,
                       const int32_t* idx, const int32_t* count, int32_t max_sel,
                       double* out, double* lse) {
  if (!check_kv(kv) || !q || !idx || !count || Tq <= 0 || Hq <= 0 || Hq % kv->Hkv != 0) return HS2REF_ERR_ARG;
  if (q_dtype != HS2REF_F32 && q_dtype != HS2REF_BF16) return HS2REF_ERR_ARG;
  ensure_tables();
  const int D = kv->D, G = Hq / kv->Hkv;
  const int64_t rows = (int64_t)kv->B * Tq * Hq;
  for (int64_t u = 0; u < (int64_t)kv->B * Tq * kv->Hkv; ++u) {
    if (count[u] < 0 || count[u] > max_sel) return HS2REF_ERR_ARG;
    for (int32_t r = 0; r < count[u]; ++r) {
      const int32_t j = idx[u * (int64_t)max_sel + r];
      if (j < 0 || j >= kv->N) return HS2REF_ERR_ARG;
    }
  }
  int rc = HS2REF_OK;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t rrow = 0; rrow < rows; ++rrow) {
    const int h = (int)(rrow % Hq);
    const int t = (int)((rrow / Hq) % Tq);
    const int b = (int)(rrow / ((int64_t)Hq * Tq));
    const int g = h / G;
    const int64_t u = ((int64_t)b * Tq + t) * kv->Hkv + g;
    const int32_t n = count[u];
    const int32_t* list = idx + u * (int64_t)max_sel;
    double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double* qv = (double*)malloc(sizeof(double) * (size_t)D);
    double* acc = (double*)malloc(sizeof(double) * (size_t)D);
    if (!s || !qv || !acc) {
      free(s); free(qv); free(acc);
#ifdef _OPENMP
#pragma omp critical(hs2ref_rc)
#endif
      rc = HS2REF_ERR_MEM;
      continue;
    }
#if HS2REF_MUTANT == 9
    const int64_t qoff = (((int64_t)b * Tq + t) * Hq + (h ^ 1)) * D; /* neighbour head's query */
#else
    const int64_t qoff = (((int64_t)b * Tq + t) * Hq + h) * D;
#endif
    for (int d = 0; d < D; ++d) qv[d] = q_elem(q, q_dtype, qoff + d);
    double m = -INFINITY;
    for (int32_t r = 0; r < n; ++r) {
      double a = 0.0;
      for (int d = 0; d < D; ++d) a += qv[d] * kv_elem(kv, 0, b, g, list[r], d);
      s[r] = scale * a;
      m = s[r] > m ? s[r] : m;
    }
    double L = 0.0;
    for (int32_t r = 0; r < n; ++r) {
      s[r] = exp(s[r] - m);
      L += s[r];
    }
    for (int d = 0; d < D; ++d) acc[d] = 0.0;
    for (int32_t r = 0; r < n; ++r) {
      const double pr = s[r] / L;
      for (int d = 0; d < D; ++d) acc[d] += pr * kv_elem(kv, 1, b, g, list[r], d);
    }
    if (out)
      for (int d = 0; d < D; ++d) out[rrow * D + d] = (n > 0) ? acc[d] : 0.0;
    if (lse) lse[rrow] = (n > 0) ? m + log(L) : -INFINITY;
    free(s); free(qv); free(acc);
  }
  return rc;
}

/* ------------------------------------------------------------------ */
/* KV bridge: per-layer projection of a self-decoder hidden state        */
/* ------------------------------------------------------------------ */

int hs2ref_kv_bridge(const uint16_t* hidden, int32_t T, int32_t d_model,
                     const uint16_t* w_kv, int32_t Hkv, int32_t D, double* y) {
  if (!hidden || !w_kv || !y || T <= 0 || d_model <= 0 || Hkv <= 0 || D <= 0) return HS2REF_ERR_ARG;
  const int64_t C = 2LL * Hkv * D;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t c = 0; c < C; ++c) {
      double acc = 0.0;
      for (int64_t r = 0; r < d_model; ++r) {
#if HS2REF_MUTANT == 10
        const double w = hs2ref_bf16_decode(w_kv[(c * d_model + r) % (C * d_model)]); /* transposed W */
#else
        const double w = hs2ref_bf16_decode(w_kv[r * C + c]);
#endif
        acc += hs2ref_bf16_decode(hidden[t * d_model + r]) * w;
      }
      y[t * C + c] = acc;
    }
  }
  return HS2REF_OK;
}
