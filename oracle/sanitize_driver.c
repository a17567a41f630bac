/*
 * sanitize_driver.c -- TEST INFRASTRUCTURE ONLY.  A plain C program that calls every entry
 * point of the CPU oracle (pkv_oracle.c) on small inputs, error paths included, so that the
 * oracle can be built and run under AddressSanitizer and UndefinedBehaviorSanitizer (gcc,
 * host code only).  tests/test_oracle_sanitizers.py compiles it together with pkv_oracle.c
 * and runs it; any invalid access, leak or undefined operation aborts the run.  It checks a
 * few results as well (a single token returns V, split equals unsplit, the write lands at its
 * slot), so that a run that exercises nothing cannot pass.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* the oracle's entry points (pkv_oracle.c) */
int64_t oracle_physical_index(const int32_t *table, int64_t block_size, int64_t pos);
int oracle_slot_mapping(int64_t *slots, const int32_t *tables, int64_t max_blocks, const int64_t *positions,
                        int64_t n, int64_t block_size);
int oracle_kv_write(const void *k_new, const void *v_new, void *k_cache, void *v_cache, const int64_t *slots,
                    int64_t num_tokens, int64_t num_blocks, int64_t block_size, int64_t num_kv_heads,
                    int64_t head_dim, int dtype);
int oracle_copy_blocks(void *k_cache, void *v_cache, const int64_t *pairs, int64_t num_pairs, int64_t num_blocks,
                       int64_t block_size, int64_t num_kv_heads, int64_t head_dim, int dtype);
int oracle_paged_attention(double *out, const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *block_tables, int64_t max_blocks, const int32_t *context_lens,
                           int64_t num_seqs, int64_t num_heads, int64_t num_kv_heads, int64_t head_dim,
                           int64_t block_size, int64_t num_blocks, double scale, int64_t partition_size,
                           const int64_t *items, int64_t num_items, int dtype, int num_threads);
int oracle_max_threads(void);

static int failures = 0;
#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                    \
    }                                                                \
  } while (0)

static uint32_t lcg = 12345u;
static float rnd(void) {
  lcg = lcg * 1664525u + 1013904223u;
  return (float)((lcg >> 8) & 0xffff) / 32768.0f - 1.0f;
}

/* fp32 or bf16 (high halves of fp32) buffers of n elements */
static void *make_buf(int64_t n, int dtype) {
  if (dtype == 0) {
    float *p = (float *)malloc((size_t)n * 4);
    for (int64_t i = 0; i < n; ++i) p[i] = rnd();
    return p;
  }
  uint16_t *p = (uint16_t *)malloc((size_t)n * 2);
  for (int64_t i = 0; i < n; ++i) {
    float f = rnd();
    uint32_t w;
    memcpy(&w, &f, 4);
    p[i] = (uint16_t)(w >> 16);
  }
  return p;
}

static void attention_case(int dtype, int64_t S, int64_t Hq, int64_t Hkv, int64_t D, int64_t B) {
  const int64_t e = dtype == 0 ? 4 : 2;
  const int64_t maxblk = 9, N = S * maxblk + 3;
  int32_t *tables = (int32_t *)malloc((size_t)(S * maxblk) * 4);
  int32_t *ctx = (int32_t *)malloc((size_t)S * 4);
  for (int64_t s = 0; s < S; ++s) {
    ctx[s] = (int32_t)(1 + (s * 7 + 3) % (maxblk * B));
    for (int64_t j = 0; j < maxblk; ++j) tables[s * maxblk + j] = (int32_t)((s * maxblk + j) * 5 % N);
  }
  ctx[0] = 1;   /* a single token */
  void *q = make_buf(S * Hq * D, dtype);
  void *k = make_buf(N * B * Hkv * D, dtype);
  void *v = make_buf(N * B * Hkv * D, dtype);
  double *o0 = (double *)malloc((size_t)(S * Hq * D) * sizeof(double));
  double *o1 = (double *)malloc((size_t)(S * Hq * D) * sizeof(double));
  const double scale = 1.0 / sqrt((double)D);
  CHECK(oracle_paged_attention(o0, q, k, v, tables, maxblk, ctx, S, Hq, Hkv, D, B, N, scale, 0, NULL, 0, dtype, 0) == 0);
  CHECK(oracle_paged_attention(o1, q, k, v, tables, maxblk, ctx, S, Hq, Hkv, D, B, N, scale, 2 * B, NULL, 0, dtype, 1) ==
        0);
  for (int64_t i = 0; i < S * Hq * D; ++i) CHECK(fabs(o0[i] - o1[i]) < 1e-12);
  /* sequence 0 has one token: its output is V of slot table[0][0] * B, exactly */
  for (int64_t h = 0; h < Hq; ++h)
    for (int64_t d = 0; d < D; ++d) {
      const int64_t idx = ((int64_t)tables[0] * B * Hkv + h / (Hq / Hkv)) * D + d;
      double want;
      if (dtype == 0) {
        want = ((const float *)v)[idx];
      } else {
        uint32_t w = (uint32_t)((const uint16_t *)v)[idx] << 16;
        float f;
        memcpy(&f, &w, 4);
        want = f;
      }
      CHECK(o0[h * D + d] == want);
    }
  /* a subset of items, in any order */
  int64_t items[3] = {S * Hq - 1, 0, (S * Hq) / 2};
  CHECK(oracle_paged_attention(o1, q, k, v, tables, maxblk, ctx, S, Hq, Hkv, D, B, N, scale, B, items, 3, dtype, 2) ==
        0);
  for (int i = 0; i < 3; ++i)
    for (int64_t d = 0; d < D; ++d) CHECK(fabs(o1[i * D + d] - o0[items[i] * D + d]) < 1e-12);
  /* errors: context 0, an item out of range, a table entry outside the pool, a bad partition */
  ctx[1] = 0;
  CHECK(oracle_paged_attention(o1, q, k, v, tables, maxblk, ctx, S, Hq, Hkv, D, B, N, scale, 0, NULL, 0, dtype, 0) != 0);
  ctx[1] = 5;
  items[0] = S * Hq;
  CHECK(oracle_paged_attention(o1, q, k, v, tables, maxblk, ctx, S, Hq, Hkv, D, B, N, scale, 0, items, 3, dtype, 0) != 0);
  tables[1 * maxblk] = (int32_t)N;
  CHECK(oracle_paged_attention(o1, q, k, v, tables, maxblk, ctx, S, Hq, Hkv, D, B, N, scale, 0, NULL, 0, dtype, 0) != 0);
  CHECK(oracle_paged_attention(o1, q, k, v, tables, maxblk, ctx, S, Hq, Hkv, D, B, N, scale, B + 1, NULL, 0, dtype, 0) !=
        0);
  free(tables);
  free(ctx);
  free(q);
  free(k);
  free(v);
  free(o0);
  free(o1);
  (void)e;
}

static void movers_case(int dtype) {
  const int64_t N = 6, B = 4, Hkv = 2, D = 8, e = dtype == 0 ? 4 : 2;
  const int64_t row = Hkv * D * e, blk = B * row;
  void *k = make_buf(N * B * Hkv * D, dtype), *v = make_buf(N * B * Hkv * D, dtype);
  void *kn = make_buf(3 * Hkv * D, dtype), *vn = make_buf(3 * Hkv * D, dtype);
  int64_t slots[3] = {5, 0, 23};
  CHECK(oracle_kv_write(kn, vn, k, v, slots, 3, N, B, Hkv, D, dtype) == 0);
  CHECK(memcmp((char *)k + 5 * row, kn, (size_t)row) == 0 && memcmp((char *)v + 23 * row, (char *)vn + 2 * row,
                                                                    (size_t)row) == 0);
  CHECK(oracle_kv_write(kn, vn, k, v, slots, 0, N, B, Hkv, D, dtype) == 0);   /* empty */
  slots[2] = 5;
  CHECK(oracle_kv_write(kn, vn, k, v, slots, 3, N, B, Hkv, D, dtype) != 0);   /* duplicate */
  slots[2] = N * B;
  CHECK(oracle_kv_write(kn, vn, k, v, slots, 3, N, B, Hkv, D, dtype) != 0);   /* past the pool */
  slots[2] = -1;
  CHECK(oracle_kv_write(kn, vn, k, v, slots, 3, N, B, Hkv, D, dtype) != 0);
  int64_t pairs[4] = {1, 4, 2, 5};
  CHECK(oracle_copy_blocks(k, v, pairs, 2, N, B, Hkv, D, dtype) == 0);
  CHECK(memcmp((char *)k + 4 * blk, (char *)k + 1 * blk, (size_t)blk) == 0);
  CHECK(oracle_copy_blocks(k, v, pairs, 0, N, B, Hkv, D, dtype) == 0);        /* empty */
  pairs[2] = 4;                                                               /* a destination as a source */
  CHECK(oracle_copy_blocks(k, v, pairs, 2, N, B, Hkv, D, dtype) != 0);
  pairs[2] = 2;
  pairs[3] = 4;                                                               /* a repeated destination */
  CHECK(oracle_copy_blocks(k, v, pairs, 2, N, B, Hkv, D, dtype) != 0);
  pairs[3] = N;
  CHECK(oracle_copy_blocks(k, v, pairs, 2, N, B, Hkv, D, dtype) != 0);
  free(k);
  free(v);
  free(kn);
  free(vn);
}

int main(void) {
  const int32_t table[3] = {47, 12, 83};
  int64_t slots[2], pos[2] = {257, 300};
  CHECK(oracle_physical_index(table, 256, 257) == 3073);
  CHECK(oracle_slot_mapping(slots, table, 3, pos, 1, 256) == 0 && slots[0] == 3073);
  pos[0] = 3 * 256;
  CHECK(oracle_slot_mapping(slots, table, 3, pos, 1, 256) != 0);
  CHECK(oracle_max_threads() >= 1);
  for (int dtype = 0; dtype < 2; ++dtype) {
    movers_case(dtype);
    attention_case(dtype, 3, 4, 4, 64, 4);
    attention_case(dtype, 4, 8, 2, 128, 16);
    attention_case(dtype, 2, 6, 2, 16, 8);
  }
  printf("sanitize_driver: %d failure(s)\n", failures);
  return failures != 0;
}
