/* Drives the fp64 oracle (oracle/moe_oracle.c) on small problems, built with
 * AddressSanitizer and UndefinedBehaviorSanitizer: several thread counts,
 * token subsets, invalid and non-local routing ids, with and without the
 * shared expert, and the argument errors. A token's row must not depend on
 * the thread count or on the subset it is computed in (the same arithmetic
 * in the same order). Exits non-zero on a failed expectation. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_forward(const uint16_t *x, const int32_t *topk_ids, const float *topk_weights,
                   const int32_t *packed_w13, const uint16_t *scales_w13,
                   const int32_t *packed_w2, const uint16_t *scales_w2,
                   const uint16_t *shared_w, double *ref, int64_t num_tokens,
                   int64_t hidden, int64_t inter, int64_t num_experts, int64_t expert_base,
                   int64_t top_k, const int64_t *rows, int64_t n_rows, int64_t n_threads);
int oracle_int4_code(const int32_t *row_words, int64_t c);
double oracle_silu(double z);

static int checks = 0, fails = 0;
#define EXPECT(c)                                                   \
  do {                                                              \
    ++checks;                                                       \
    if (!(c)) {                                                     \
      fprintf(stderr, "line %d: expected %s\n", __LINE__, #c);      \
      ++fails;                                                      \
    }                                                               \
  } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next32(void) {  /* xorshift64* */
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return (uint32_t)((rng * 0x2545F4914F6CDD1Dull) >> 32);
}
/* a bf16 of magnitude about `scale` (top half of an fp32) */
static uint16_t bf16_about(double scale) {
  float f = (float)(scale * ((double)next32() / 4294967296.0 * 2.0 - 1.0));
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static void *alloc(size_t n) {
  void *p = malloc(n ? n : 1);
  if (!p) abort();
  return p;
}

static void run(int64_t T, int64_t H, int64_t I, int64_t E, int64_t base, int64_t k,
                int shared) {
  uint16_t *x = alloc(2 * T * H);
  int32_t *ids = alloc(4 * T * k);
  float *w = alloc(4 * T * k);
  int32_t *p13 = alloc(4 * E * 2 * I * (H / 8));
  uint16_t *s13 = alloc(2 * E * 2 * I * (H / 32));
  int32_t *p2 = alloc(4 * E * H * (I / 8));
  uint16_t *s2 = alloc(2 * E * H * (I / 32));
  uint16_t *sw = shared ? alloc(2 * (2 * I * H + H * I)) : NULL;
  for (int64_t i = 0; i < T * H; ++i) x[i] = bf16_about(2.0);
  for (int64_t i = 0; i < T * k; ++i) {
    const uint32_t r = next32() % (uint32_t)(E + 3);
    ids[i] = (r == 0) ? -1 : (int32_t)(base + r - 1); /* -1, local, and two past the range */
    w[i] = (float)((double)next32() / 4294967296.0);
  }
  for (int64_t i = 0; i < E * 2 * I * (H / 8); ++i) p13[i] = (int32_t)next32();
  for (int64_t i = 0; i < E * H * (I / 8); ++i) p2[i] = (int32_t)next32();
  for (int64_t i = 0; i < E * 2 * I * (H / 32); ++i) s13[i] = bf16_about(0.02);
  for (int64_t i = 0; i < E * H * (I / 32); ++i) s2[i] = bf16_about(0.02);
  if (sw)
    for (int64_t i = 0; i < 2 * I * H + H * I; ++i) sw[i] = bf16_about(0.05);

  double *full = alloc(8 * T * H), *again = alloc(8 * T * H), *sub = alloc(8 * T * H);
  EXPECT(oracle_forward(x, ids, w, p13, s13, p2, s2, sw, full, T, H, I, E, base, k, NULL, 0, 1) ==
         0);
  EXPECT(oracle_forward(x, ids, w, p13, s13, p2, s2, sw, again, T, H, I, E, base, k, NULL, 0,
                        3) == 0);
  EXPECT(memcmp(full, again, 8 * T * H) == 0);
  for (int64_t i = 0; i < T * H; ++i) EXPECT(isfinite(full[i]));
  /* a subset in reverse order, computed with two threads */
  int64_t *rows = alloc(8 * T);
  for (int64_t r = 0; r < T; ++r) rows[r] = T - 1 - r;
  EXPECT(oracle_forward(x, ids, w, p13, s13, p2, s2, sw, sub, T, H, I, E, base, k, rows, T, 2) ==
         0);
  for (int64_t r = 0; r < T; ++r) EXPECT(memcmp(sub + r * H, full + rows[r] * H, 8 * H) == 0);
  /* argument errors */
  EXPECT(oracle_forward(x, ids, w, p13, s13, p2, s2, sw, sub, T, H + 1, I, E, base, k, NULL, 0,
                        1) == -1);
  EXPECT(oracle_forward(x, ids, w, p13, s13, p2, s2, sw, sub, T, H, I, E, base, 0, NULL, 0, 1) ==
         -1);
  rows[0] = T; /* past the last token */
  EXPECT(oracle_forward(x, ids, w, p13, s13, p2, s2, sw, sub, T, H, I, E, base, k, rows, 1, 1) ==
         -1);
  EXPECT(oracle_forward(x, ids, w, p13, s13, p2, s2, sw, sub, 0, H, I, E, base, k, NULL, 0, 4) ==
         0);
  free(x), free(ids), free(w), free(p13), free(s13), free(p2), free(s2), free(sw);
  free(full), free(again), free(sub), free(rows);
}

int main(void) {
  /* the unpack convention on a hand-worked word: fields 0..7 = codes 0..7 */
  const int32_t word[2] = {0x76543210, (int32_t)0xFEDCBA98u};
  for (int c = 0; c < 16; ++c) EXPECT(oracle_int4_code(word, c) == c - 8);
  EXPECT(oracle_silu(0.0) == 0.0);
  run(5, 64, 64, 4, 1, 3, 1);
  run(7, 96, 32, 3, 0, 2, 0);
  run(1, 128, 64, 6, 2, 4, 1);
  printf("oracle checks: %d, failed: %d\n", checks, fails);
  return fails ? 1 : 0;
}
