/*
 * moe_oracle.c -- plain, slow, fp64 CPU oracle of the W4A16 routed-expert MoE
 * layer. TEST INFRASTRUCTURE ONLY: it exists to check the GPU library. Only
 * the tests, the package smoke check and the bench's CPU-baseline leg may load
 * it. It shares no code, header or table with the GPU library.
 *
 * What it computes (the plain definition, evaluated in fp64 with no
 * intermediate rounding):
 *
 *   ref[t] = S(x_t) + sum_{j<k, id_tj local} w_tj * F_{id_tj - base}(x_t)
 *   F_e(v) = W2_e ( silu(W1_e v) * (W3_e v) ),  W1 = W13[0:I], W3 = W13[I:2I]
 *   W[n][c] = q[n][c] * s[n][c/32],  q = (4-bit field c%8 of word c/8) - 8
 *   silu(z) = z / (1 + exp(-z))
 *   S = the same MLP with the bf16 shared-expert weights, weight 1 (absent if
 *       no shared weights are given)
 *
 * Sources: Kimi-K2.6 inference-research catalog entry -- MoE paragraph
 * (384 routed experts, 8 per token, one shared expert, moe_intermediate 2048),
 * QUANT paragraph (routed experts are compressed-tensors INT4, group size 32,
 * symmetric, pack-quantized; the shared expert stays in higher precision) and
 * PARAMS paragraph (int4 values held in int32 containers). The pages do not
 * fix the nibble order, the sign encoding, the gate/up row order, the
 * activation or the combine rule; the readings used here are: low nibble
 * first along the input dimension, excess-8 codes, gate rows before up rows,
 * SwiGLU, routing weights applied as given and ids outside [base, base+E)
 * skipped.
 *
 * Parity against the pages' own numbers: unpinned (the pages print no layer
 * output); the tests pin this file to closed forms, a library SwiGLU MLP, an
 * independent dense formulation and invariants instead.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GROUP 32

static double bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* signed 4-bit value of input element c of a row of packed words */
static int int4_code(const int32_t *row_words, int64_t c) {
  uint32_t word = (uint32_t)row_words[c / 8];
  int field = (int)((word >> (4 * (c % 8))) & 0xFu);
  return field - 8;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* dequantised int4 weight W[n][c] of an [N, C] matrix */
static double w_int4(const int32_t *packed, const uint16_t *scales, int64_t C,
                     int64_t n, int64_t c) {
  const int32_t *row = packed + n * (C / 8);
  double s = bf16_value(scales[n * (C / GROUP) + c / GROUP]);
  return (double)int4_code(row, c) * s;
}

/* y = W2 (silu(W1 v) * W3 v) for one int4 expert; a: [2I], h: [I] scratch */
static void mlp_int4(const double *v, const int32_t *pw13, const uint16_t *s13,
                     const int32_t *pw2, const uint16_t *s2, int64_t H, int64_t I,
                     double *a, double *h, double *y) {
  for (int64_t n = 0; n < 2 * I; ++n) {
    double acc = 0.0;
    for (int64_t c = 0; c < H; ++c) acc += w_int4(pw13, s13, H, n, c) * v[c];
    a[n] = acc;
  }
  for (int64_t i = 0; i < I; ++i) h[i] = silu(a[i]) * a[I + i];
  for (int64_t n = 0; n < H; ++n) {
    double acc = 0.0;
    for (int64_t i = 0; i < I; ++i) acc += w_int4(pw2, s2, I, n, i) * h[i];
    y[n] = acc;
  }
}

/* the same MLP with dense bf16 weights: w13 [2I, H], w2 [H, I] */
static void mlp_bf16(const double *v, const uint16_t *w13, const uint16_t *w2,
                     int64_t H, int64_t I, double *a, double *h, double *y) {
  for (int64_t n = 0; n < 2 * I; ++n) {
    double acc = 0.0;
    for (int64_t c = 0; c < H; ++c) acc += bf16_value(w13[n * H + c]) * v[c];
    a[n] = acc;
  }
  for (int64_t i = 0; i < I; ++i) h[i] = silu(a[i]) * a[I + i];
  for (int64_t n = 0; n < H; ++n) {
    double acc = 0.0;
    for (int64_t i = 0; i < I; ++i) acc += bf16_value(w2[n * I + i]) * h[i];
    y[n] = acc;
  }
}

typedef struct {
  const uint16_t *x;
  const int32_t *ids;
  const float *wts;
  const int32_t *pw13;
  const uint16_t *s13;
  const int32_t *pw2;
  const uint16_t *s2;
  const uint16_t *shared;
  double *out;
  const int64_t *rows;
  int64_t n_rows, H, I, E, base, k;
  int64_t r_begin, r_end;
} job_t;

static void *worker(void *arg) {
  job_t *jb = (job_t *)arg;
  int64_t H = jb->H, I = jb->I;
  double *v = malloc(sizeof(double) * H);
  double *a = malloc(sizeof(double) * 2 * I);
  double *h = malloc(sizeof(double) * I);
  double *y = malloc(sizeof(double) * H);
  for (int64_t r = jb->r_begin; r < jb->r_end; ++r) {
    int64_t t = jb->rows ? jb->rows[r] : r;
    double *o = jb->out + r * H;
    for (int64_t c = 0; c < H; ++c) v[c] = bf16_value(jb->x[t * H + c]);
    for (int64_t n = 0; n < H; ++n) o[n] = 0.0;
    if (jb->shared) {
      mlp_bf16(v, jb->shared, jb->shared + 2 * I * H, H, I, a, h, y);
      for (int64_t n = 0; n < H; ++n) o[n] += y[n];
    }
    for (int64_t j = 0; j < jb->k; ++j) {
      int64_t id = jb->ids[t * jb->k + j];
      if (id < jb->base || id >= jb->base + jb->E) continue;
      int64_t e = id - jb->base;
      double w = (double)jb->wts[t * jb->k + j];
      mlp_int4(v, jb->pw13 + e * 2 * I * (H / 8), jb->s13 + e * 2 * I * (H / GROUP),
               jb->pw2 + e * H * (I / 8), jb->s2 + e * H * (I / GROUP), H, I, a, h, y);
      for (int64_t n = 0; n < H; ++n) o[n] += w * y[n];
    }
  }
  free(v);
  free(a);
  free(h);
  free(y);
  return NULL;
}

/*
 * ref[r, :] for r < n_rows, token t = rows[r] (or r when rows is NULL).
 * Returns 0, or -1 on bad arguments.
 */
int oracle_forward(const uint16_t *x, const int32_t *topk_ids, const float *topk_weights,
                   const int32_t *packed_w13, const uint16_t *scales_w13,
                   const int32_t *packed_w2, const uint16_t *scales_w2,
                   const uint16_t *shared_w, double *ref, int64_t num_tokens,
                   int64_t hidden, int64_t inter, int64_t num_experts, int64_t expert_base,
                   int64_t top_k, const int64_t *rows, int64_t n_rows, int64_t n_threads) {
  if (hidden % GROUP || inter % GROUP || top_k < 1 || num_tokens < 0) return -1;
  if (!rows) n_rows = num_tokens;
  if (n_rows == 0) return 0;
  if (n_threads < 1) n_threads = 1;
  if (n_threads > n_rows) n_threads = n_rows;
  for (int64_t r = 0; rows && r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= num_tokens) return -1;
  pthread_t *th = malloc(sizeof(pthread_t) * n_threads);
  job_t *jobs = malloc(sizeof(job_t) * n_threads);
  for (int64_t i = 0; i < n_threads; ++i) {
    job_t jb = {x, topk_ids, topk_weights, packed_w13, scales_w13, packed_w2, scales_w2,
                shared_w, ref, rows, n_rows, hidden, inter, num_experts, expert_base, top_k,
                n_rows * i / n_threads, n_rows * (i + 1) / n_threads};
    jobs[i] = jb;
    pthread_create(&th[i], NULL, worker, &jobs[i]);
  }
  for (int64_t i = 0; i < n_threads; ++i) pthread_join(th[i], NULL);
  free(th);
  free(jobs);
  return 0;
}

/* fp64 silu as used above, exported for the identity check in the tests */
double oracle_silu(double z) { return silu(z); }

/* signed code of element c of a packed row, exported for the unpack pins */
int oracle_int4_code(const int32_t *row_words, int64_t c) { return int4_code(row_words, c); }
