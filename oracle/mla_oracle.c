/*
 * mla_oracle.c - plain CPU fp64 reference for MLA decode (DeepSeek-R1
 * forward_absorb).  TEST INFRASTRUCTURE ONLY: the GPU library never includes,
 * links or calls this file; only the tests, the smoke check and the bench's
 * CPU baseline use it.
 *
 * What it computes (kernelbot-amd-mixed-mla template page: the docstring's
 * "DeepSeek R1 forward_absorb MLA config" and "KV buffer format", and the naive
 * bf16 reference custom_kernel_bf16 / fp8 reference custom_kernel_fp8): for
 * every sequence b, every query row t in [qo_indptr[b], qo_indptr[b+1]) and
 * every head h,
 *
 *     s_j       = sm_scale * sum_{d < qk_dim} Q[t,h,d] * KV[j,d]
 *     O[t,h,v]  = sum_j softmax_j(s) * KV[j,v]            (v < v_dim)
 *
 * with, when logit_cap > 0, every scaled score first soft-capped as
 * s_j <- logit_cap * tanh(s_j / logit_cap).  The pages name logit_cap only as an
 * argument of a library decode call (submission 753817's fallback, set to 0.0);
 * the formula is the usual soft-cap reading of that argument.
 *
 * over the KV rows j in [kv_indptr[b], kv_indptr[b+1]).  Keys are the full
 * qk_dim-wide row, values its first v_dim columns; all heads share the one KV
 * row.  No mask: every query row sees every KV row of its sequence.
 *
 * Precision: every input is decoded exactly to double and all arithmetic is
 * done in double, in the order written below (no blocking, no reordering).
 * Quantised inputs are used through their decoded values for both K and V:
 *   fp8 E4M3FN   value(code) * scale            (one fp32 scale per tensor)
 *   MXFP4        value_E2M1(nibble) * 2^(E8M0 - 127)   (one scale per 32 columns)
 * Paged KV (the kv_indices / page_size arguments of the library decode call on
 * submission 753817's page, which passes page_size 1): with page size 1 the
 * rows of sequence b are KV[kv_indices[j]] for j in [kv_indptr[b],
 * kv_indptr[b+1]).  With page size P > 1, kv_indices lists pages: row i of
 * sequence b (i counted from 0) is row i mod P of page
 * kv_indices[kv_page_indptr[b] + i div P], that is KV[page * P + i mod P].
 * Without kv_indices the rows are KV[j].
 *
 * The fp8 a8w8 reference on the template page multiplies the two per-tensor
 * scales into the fp8 product (torch._scaled_mm with scale_a, scale_b), which
 * is the same number as decoding each operand first.
 *
 * Every function is pinned by tests other than re-typing it: exhaustive decode
 * tables against torch's float8 casts and the OCP format definitions, closed
 * forms (one row, two rows, identical scores), brute force in exact/decimal
 * arithmetic on tiny inputs, split recombination, symmetries, and an
 * independent torch fp64 formulation.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_BF16 = 0, ORACLE_FP8_E4M3FN = 1, ORACLE_MXFP4 = 2 };

/* ------------------------------------------------------------- decoders */

/* bf16: the upper 16 bits of an IEEE binary32. */
double oracle_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OCP 8-bit floating point, E4M3 ("fn": finite, no infinities).
 * Fields: sign(1) exponent(4, bias 7) mantissa(3).
 *   exponent 0:               (-1)^s * (m / 8) * 2^(1 - 7)       subnormal
 *   exponent 1..15:           (-1)^s * (1 + m / 8) * 2^(e - 7)
 *   except S.1111.111:        NaN (the only NaN; there is no inf) */
double oracle_e4m3fn_value(uint8_t code) {
  const int s = code >> 7, e = (code >> 3) & 0xF, m = code & 0x7;
  double mag;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, 1 - 7);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* OCP MX E2M1 element: sign(1) exponent(2, bias 1) mantissa(1).
 *   exponent 0: (-1)^s * (m / 2) * 2^0 ; otherwise (-1)^s * (1 + m/2) * 2^(e-1). */
double oracle_e2m1_value(uint8_t nibble) {
  const int s = (nibble >> 3) & 1, e = (nibble >> 1) & 0x3, m = nibble & 1;
  double mag = (e == 0) ? (double)m / 2.0 : ldexp(1.0 + (double)m / 2.0, e - 1);
  return s ? -mag : mag;
}

/* OCP MX E8M0 scale: 2^(code - 127); code 255 is NaN. */
double oracle_e8m0_value(uint8_t code) {
  if (code == 0xFF) return NAN;
  return ldexp(1.0, (int)code - 127);
}

/* Decode n fp8 codes times a scale into doubles (exact product). */
void oracle_decode_fp8(const uint8_t* codes, int64_t n, float scale, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3fn_value(codes[i]) * (double)scale;
}

/* Decode MXFP4 rows: packed [rows][dim/2] (element 2i in the low nibble of
 * byte i, 2i+1 in the high nibble), scales [rows][dim/32]. */
void oracle_decode_mxfp4(const uint8_t* packed, const uint8_t* scales, int64_t rows, int dim, double* out) {
  for (int64_t r = 0; r < rows; ++r)
    for (int c = 0; c < dim; ++c) {
      const uint8_t byte = packed[r * (dim / 2) + c / 2];
      const uint8_t nib = (c & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0xF);
      out[r * dim + c] = oracle_e2m1_value(nib) * oracle_e8m0_value(scales[r * (dim / 32) + c / 32]);
    }
}

/* ------------------------------------------------------------- attention */

typedef struct {
  int32_t batch_size;
  int32_t num_heads;
  int32_t qk_dim;
  int32_t v_dim;
  int32_t q_dtype;  /* ORACLE_BF16 or ORACLE_FP8_E4M3FN */
  int32_t kv_dtype; /* ORACLE_BF16, ORACLE_FP8_E4M3FN or ORACLE_MXFP4 */
  double sm_scale;
  double logit_cap; /* > 0: soft-cap of the scaled scores; 0: none */
} oracle_problem;

/* Decode KV row j (all qk_dim columns) into dst. */
static void decode_kv_row(const oracle_problem* p, const void* kv, const void* kv_scale, int64_t j, double* dst) {
  const int D = p->qk_dim;
  if (p->kv_dtype == ORACLE_BF16) {
    const uint16_t* row = (const uint16_t*)kv + j * D;
    for (int d = 0; d < D; ++d) dst[d] = oracle_bf16_value(row[d]);
  } else if (p->kv_dtype == ORACLE_FP8_E4M3FN) {
    const uint8_t* row = (const uint8_t*)kv + j * D;
    const double s = (double)*(const float*)kv_scale;
    for (int d = 0; d < D; ++d) dst[d] = oracle_e4m3fn_value(row[d]) * s;
  } else {
    oracle_decode_mxfp4((const uint8_t*)kv + j * (D / 2), (const uint8_t*)kv_scale + j * (D / 32), 1, D, dst);
  }
}

/* Decode query row t, head h into dst. */
static void decode_q_row(const oracle_problem* p, const void* q, const float* q_scale, int64_t t, int h, double* dst) {
  const int D = p->qk_dim;
  const int64_t base = (t * p->num_heads + h) * (int64_t)D;
  if (p->q_dtype == ORACLE_BF16) {
    for (int d = 0; d < D; ++d) dst[d] = oracle_bf16_value(((const uint16_t*)q)[base + d]);
  } else {
    const double s = (double)*q_scale;
    for (int d = 0; d < D; ++d) dst[d] = oracle_e4m3fn_value(((const uint8_t*)q)[base + d]) * s;
  }
}

/* Softmax attention of one query row over n decoded KV rows, as defined above.
 * out[v_dim] and *lse (natural log of sum_j exp(s_j)).  n == 0 gives O = 0 and
 * lse = -inf. */
static void attend_one(const oracle_problem* p, const double* qrow, const double* kvrows, int64_t n, double* scores,
                       double* out, double* lse) {
  const int D = p->qk_dim, V = p->v_dim;
  for (int v = 0; v < V; ++v) out[v] = 0.0;
  if (n == 0) {
    *lse = -INFINITY;
    return;
  }
  double m = -INFINITY;
  for (int64_t j = 0; j < n; ++j) {
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += qrow[d] * kvrows[j * D + d];
    scores[j] = p->sm_scale * dot;
    if (p->logit_cap > 0.0) scores[j] = p->logit_cap * tanh(scores[j] / p->logit_cap);
    if (scores[j] > m) m = scores[j];
  }
  double l = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    const double w = exp(scores[j] - m);
    scores[j] = w;
    l += w;
  }
  for (int64_t j = 0; j < n; ++j)
    for (int v = 0; v < V; ++v) out[v] += scores[j] * kvrows[j * D + v];
  for (int v = 0; v < V; ++v) out[v] /= l;
  *lse = m + log(l);
}

typedef struct {
  const oracle_problem* p;
  const void *q, *kv, *kv_scale;
  const float* q_scale;
  const int32_t *qo_indptr, *kv_indptr, *kv_indices, *kv_page_indptr, *seq_ids;
  int n_seq, page_size;
  double *out, *lse;
  int next; /* shared work counter, guarded by mu */
  pthread_mutex_t mu;
  int status;
} shared_t;

static void* worker(void* arg) {
  shared_t* sh = (shared_t*)arg;
  const oracle_problem* p = sh->p;
  const int D = p->qk_dim, V = p->v_dim, H = p->num_heads;
  double* kvrows = NULL;
  double* scores = NULL;
  int64_t cap = 0;
  double* qrow = (double*)malloc(sizeof(double) * (size_t)D);
  for (;;) {
    pthread_mutex_lock(&sh->mu);
    const int k = sh->next++;
    pthread_mutex_unlock(&sh->mu);
    if (k >= sh->n_seq) break;
    const int b = sh->seq_ids ? sh->seq_ids[k] : k;
    const int64_t j0 = sh->kv_indptr[b], j1 = sh->kv_indptr[b + 1];
    const int64_t n = j1 - j0;
    if (n > cap) {
      free(kvrows);
      free(scores);
      cap = n;
      kvrows = (double*)malloc(sizeof(double) * (size_t)(cap * D));
      scores = (double*)malloc(sizeof(double) * (size_t)cap);
      if (!kvrows || !scores) {
        sh->status = -2;
        break;
      }
    }
    for (int64_t j = 0; j < n; ++j) {
      int64_t row = j0 + j;
      if (sh->kv_page_indptr)
        row = (int64_t)sh->kv_indices[sh->kv_page_indptr[b] + j / sh->page_size] * sh->page_size + j % sh->page_size;
      else if (sh->kv_indices)
        row = sh->kv_indices[j0 + j];
      decode_kv_row(p, sh->kv, sh->kv_scale, row, kvrows + j * D);
    }
    for (int64_t t = sh->qo_indptr[b]; t < sh->qo_indptr[b + 1]; ++t)
      for (int h = 0; h < H; ++h) {
        decode_q_row(p, sh->q, sh->q_scale, t, h, qrow);
        attend_one(p, qrow, kvrows, n, scores, sh->out + (t * H + h) * (int64_t)V, sh->lse + t * H + h);
      }
  }
  free(kvrows);
  free(scores);
  free(qrow);
  return NULL;
}

/* Reference decode for the sequences listed in seq_ids (all sequences when
 * seq_ids is NULL; n_seq is then the batch size).  out is indexed by global
 * query row: out[(t*num_heads + h)*v_dim + v], lse[t*num_heads + h]; entries of
 * sequences not listed are left untouched.  Returns 0, or a negative value on
 * bad arguments / allocation failure. */
int oracle_mla_decode_paged(const oracle_problem* p, const void* q, const float* q_scale, const void* kv,
                            const void* kv_scale, const int32_t* qo_indptr, const int32_t* kv_indptr,
                            const int32_t* kv_indices, const int32_t* seq_ids, int n_seq, double* out, double* lse,
                            int nthreads);

int oracle_mla_decode(const oracle_problem* p, const void* q, const float* q_scale, const void* kv,
                      const void* kv_scale, const int32_t* qo_indptr, const int32_t* kv_indptr,
                      const int32_t* seq_ids, int n_seq, double* out, double* lse, int nthreads) {
  return oracle_mla_decode_paged(p, q, q_scale, kv, kv_scale, qo_indptr, kv_indptr, NULL, seq_ids, n_seq, out, lse,
                                 nthreads);
}

int oracle_mla_decode_pages(const oracle_problem* p, const void* q, const float* q_scale, const void* kv,
                            const void* kv_scale, const int32_t* qo_indptr, const int32_t* kv_indptr,
                            const int32_t* kv_indices, const int32_t* kv_page_indptr, int page_size,
                            const int32_t* seq_ids, int n_seq, double* out, double* lse, int nthreads);

/* The same with KV row j of the CSR space read from KV[kv_indices[j]] (NULL:
 * KV[j]); the caller guarantees every index is a row of kv. */
int oracle_mla_decode_paged(const oracle_problem* p, const void* q, const float* q_scale, const void* kv,
                            const void* kv_scale, const int32_t* qo_indptr, const int32_t* kv_indptr,
                            const int32_t* kv_indices, const int32_t* seq_ids, int n_seq, double* out, double* lse,
                            int nthreads) {
  return oracle_mla_decode_pages(p, q, q_scale, kv, kv_scale, qo_indptr, kv_indptr, kv_indices, NULL, 1, seq_ids,
                                 n_seq, out, lse, nthreads);
}

/* The same with pages of page_size rows: kv_page_indptr[b] is the first entry
 * of sequence b's page list in kv_indices (NULL: one index per CSR row, as
 * above); the caller guarantees every page it names lies inside kv. */
int oracle_mla_decode_pages(const oracle_problem* p, const void* q, const float* q_scale, const void* kv,
                            const void* kv_scale, const int32_t* qo_indptr, const int32_t* kv_indptr,
                            const int32_t* kv_indices, const int32_t* kv_page_indptr, int page_size,
                            const int32_t* seq_ids, int n_seq, double* out, double* lse, int nthreads) {
  if (!p || !q || !kv || !qo_indptr || !kv_indptr || !out || !lse) return -1;
  if (kv_page_indptr && (!kv_indices || page_size < 1)) return -1;
  if (p->num_heads <= 0 || p->qk_dim <= 0 || p->v_dim <= 0 || p->v_dim > p->qk_dim) return -1;
  if (!(p->logit_cap >= 0.0)) return -1;
  if (p->kv_dtype == ORACLE_MXFP4 && p->qk_dim % 32) return -1;
  if (p->kv_dtype != ORACLE_BF16 && !kv_scale) return -1;
  if (p->q_dtype != ORACLE_BF16 && !q_scale) return -1;
  if (!seq_ids) n_seq = p->batch_size;
  shared_t sh;
  memset(&sh, 0, sizeof sh);
  sh.p = p;
  sh.q = q;
  sh.q_scale = q_scale;
  sh.kv = kv;
  sh.kv_scale = kv_scale;
  sh.qo_indptr = qo_indptr;
  sh.kv_indptr = kv_indptr;
  sh.kv_indices = kv_indices;
  sh.kv_page_indptr = kv_page_indptr;
  sh.page_size = page_size;
  sh.seq_ids = seq_ids;
  sh.n_seq = n_seq;
  sh.out = out;
  sh.lse = lse;
  pthread_mutex_init(&sh.mu, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &sh);
  worker(&sh);
  for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
  pthread_mutex_destroy(&sh.mu);
  return sh.status;
}
