/*
 * dsa_ref.c -- plain, slow CPU reference of the DeepSeek Sparse Attention (DSA) hot path in C.
 *
 * TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU baseline load
 * it (through oracle/cref.py); the GPU library never does, and the two share no code, tables
 * or constants. It computes what oracle/dsa.py computes, from the same definitions, in double
 * precision with plain loops, one query token at a time ("LLM architecture survey", section
 * 2.2 DeepSeek-V3.2: score every preceding token with the lightning indexer, keep the k best,
 * attend over them in MLA's MQA mode; section 2.1 DeepSeek-V3: latent row = 512 + 64 dims).
 *
 *   dsa_ref_index_scores  s_t = sum_h w_h * max(q_h . k_t, 0) for t <= p, -inf after
 *                         (E4M3 products and their sums are exact in double)
 *   dsa_ref_select_topk   the min(k, p+1) best of scores[0..p] by (score desc, position asc),
 *                         ascending, -1 padded (qsort as the sort)
 *   dsa_ref_sparse_mla    z_i = scale * q_h . c_i over 576 dims, softmax over the rows given,
 *                         o_h = sum_i P_i c_i[0:512], lse_h = log sum_i exp z_i
 *
 * Inputs are one sequence in logical token order (the caller resolves paging). OpenMP, when
 * the compiler is given -fopenmp, splits the loops over keys and over heads across cores.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* OCP FP8 E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is subnormal
 * (m * 2^-9); S.1111.111 is NaN; no infinities. */
static double e4m3_value(uint8_t code) {
  const int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m, -9);
  else v = ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -v : v;
}

/* bfloat16: the upper half of an IEEE binary32 */
static double bf16_value(uint16_t bits) {
  const uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* q [Hi][128] E4M3 codes, w [Hi], keys [>= p+1][128] E4M3 codes in token order -> out [L_max] */
void dsa_ref_index_scores(const uint8_t* q, const float* w, int Hi, const uint8_t* keys, int p, int L_max,
                          double* out) {
  double* qd = (double*)malloc(sizeof(double) * (size_t)Hi * 128);
  for (int i = 0; i < Hi * 128; ++i) qd[i] = e4m3_value(q[i]);
#pragma omp parallel for schedule(static)
  for (int t = 0; t <= p; ++t) {
    double kd[128];
    for (int i = 0; i < 128; ++i) kd[i] = e4m3_value(keys[(size_t)t * 128 + i]);
    double s = 0.0;
    for (int h = 0; h < Hi; ++h) {
      double d = 0.0;
      for (int i = 0; i < 128; ++i) d += qd[h * 128 + i] * kd[i];
      if (d > 0.0) s += (double)w[h] * d;
    }
    out[t] = s;
  }
  for (int t = p + 1; t < L_max; ++t) out[t] = -INFINITY;
  free(qd);
}

typedef struct {
  float s;
  int32_t pos;
} scored_t;

/* descending score, then ascending position; -0 and +0 compare equal */
static int by_score_then_position(const void* a, const void* b) {
  const scored_t* x = (const scored_t*)a;
  const scored_t* y = (const scored_t*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->pos > y->pos) - (x->pos < y->pos);
}

static int ascending_int(const void* a, const void* b) {
  const int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* scores [>= p+1] float (the precision the GPU stores them in) -> out [k] */
void dsa_ref_select_topk(const float* scores, int p, int k, int32_t* out) {
  const int n = p + 1, m = k < n ? k : n;
  scored_t* all = (scored_t*)malloc(sizeof(scored_t) * (size_t)n);
  for (int t = 0; t < n; ++t) {
    all[t].s = scores[t];
    all[t].pos = t;
  }
  qsort(all, (size_t)n, sizeof(scored_t), by_score_then_position);
  for (int i = 0; i < m; ++i) out[i] = all[i].pos;
  qsort(out, (size_t)m, sizeof(int32_t), ascending_int);
  for (int i = m; i < k; ++i) out[i] = -1;
  free(all);
}

/* Rows of the selected tokens: bf16 bits (row_scale == 0) or E4M3 codes times row_scale. */
static double row_value(const void* rows, int row_scale_is_e4m3, double row_scale, size_t i) {
  if (row_scale_is_e4m3) return row_scale * e4m3_value(((const uint8_t*)rows)[i]);
  return bf16_value(((const uint16_t*)rows)[i]);
}

/* q [H][576] bf16 bits; rows [m][576] (bf16 bits, or E4M3 codes when e4m3_scale > 0) ->
 * o [H][512], lse [H]; m == 0 gives o = 0 and lse = -inf. */
void dsa_ref_sparse_mla(const uint16_t* q, int H, const void* rows, int m, double scale, double e4m3_scale,
                        double* o, double* lse) {
  const int is8 = e4m3_scale > 0.0;
  double* c = (double*)malloc(sizeof(double) * ((size_t)m * 576 + 1));
  for (size_t i = 0; i < (size_t)m * 576; ++i) c[i] = row_value(rows, is8, e4m3_scale, i);
#pragma omp parallel for schedule(static)
  for (int h = 0; h < H; ++h) {
    double* oh = o + (size_t)h * 512;
    for (int v = 0; v < 512; ++v) oh[v] = 0.0;
    if (m == 0) {
      lse[h] = -INFINITY;
      continue;
    }
    double qd[576];
    for (int d = 0; d < 576; ++d) qd[d] = bf16_value(q[(size_t)h * 576 + d]);
    double* z = (double*)malloc(sizeof(double) * (size_t)m);
    double zmax = -INFINITY;
    for (int i = 0; i < m; ++i) {
      double acc = 0.0;
      for (int d = 0; d < 576; ++d) acc += qd[d] * c[(size_t)i * 576 + d];
      z[i] = scale * acc;
      if (z[i] > zmax) zmax = z[i];
    }
    double denom = 0.0;
    for (int i = 0; i < m; ++i) {
      const double e = exp(z[i] - zmax);
      denom += e;
      for (int v = 0; v < 512; ++v) oh[v] += e * c[(size_t)i * 576 + v];
    }
    for (int v = 0; v < 512; ++v) oh[v] /= denom;
    lse[h] = zmax + log(denom);
    free(z);
  }
  free(c);
}
