/*
 * pkv_oracle.c -- plain, slow, obviously-correct CPU oracle for the paged KV
 * cache decode path.  TEST INFRASTRUCTURE ONLY: tests, the smoke check and the
 * bench's CPU-baseline leg use it; the GPU library never links or calls it, and
 * it shares no code, header or constant with the GPU library.
 *
 * Sources (web pages on PagedAttention; cited by title and section):
 *   [P1] "nano-vLLM . Ch04 . PagedAttention", section 4 "The Three Mechanisms"
 *        (block table, slot mapping), section 6 "Copy-on-write block sharing",
 *        section 9 "Common Mistakes" (Myth 1: same math, only the memory layout
 *        differs).
 *   [P2] "PagedAttention" (PidokuInfra, topic 10), section 4 "Tiny example"
 *        (PhysicalIndex), section 5 "Technical explanation" / "The kernel side"
 *        (kernel arguments, cache layout [num_blocks, block_size, kv_heads,
 *        head_dim], block-table walk with online softmax).
 *   [P3] "PagedAttention" (tokentrails), step 3 "Attention across blocks" and
 *        the "Code" box (write kv[b, t % BLOCK]; gather blocks, then attend).
 *
 * Arithmetic is fp64.  Inputs are fp32 or bf16; bf16 widens to fp32 exactly
 * (it is the high half of an fp32 word) and then to fp64.
 *
 * Readings where the pages are silent (each restated where it is used):
 *   - GQA: query head h reads KV head h / (Hq / Hkv) (contiguous groups).
 *   - Only positions t < ctx are attended; slots past ctx in the last block and
 *     table entries past ceil(ctx / B) are never read.
 *   - ctx >= 1 (a decode step always contains its own token); ctx < 1 is an
 *     error here.
 *   - Split-K: partition p covers [p*P, min((p+1)*P, ctx)); the partials are
 *     merged by log-sum-exp.  Equal to the unsplit result in exact arithmetic.
 *   - Duplicate slots in one write, a repeated copy destination, or a copy
 *     destination that is also a source in the same call are caller errors.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

enum {
  ORACLE_OK = 0,
  ORACLE_EINVAL = -1,    /* bad sizes / unsupported dtype                       */
  ORACLE_ERANGE = -2,    /* slot, block id or context length out of range       */
  ORACLE_EDUP = -3,      /* duplicate slot / copy destination, or dst == a src  */
  ORACLE_ENOMEM = -4
};

static int64_t elem_size(int dtype) { return dtype == ORACLE_F32 ? 4 : (dtype == ORACLE_BF16 ? 2 : 0); }

/* Element `idx` of a flat fp32 or bf16 array, widened exactly to double. */
static double load_elem(const void *base, int64_t idx, int dtype) {
  float f;
  if (dtype == ORACLE_F32) {
    memcpy(&f, (const char *)base + idx * 4, 4);
  } else {
    uint16_t h;
    uint32_t w;
    memcpy(&h, (const char *)base + idx * 2, 2);
    w = (uint32_t)h << 16;
    memcpy(&f, &w, 4);
  }
  return (double)f;
}

/* [P2] section 4, PhysicalIndex; [P1] section 4, "Mechanism 3 -- The slot mapping":
 * the slot of logical position `pos` is table[pos / B] * B + pos % B. */
int64_t oracle_physical_index(const int32_t *table, int64_t block_size, int64_t pos) {
  return (int64_t)table[pos / block_size] * block_size + pos % block_size;
}

/* Slots for a batch: slots[i] = PhysicalIndex(table of seq i, pos[i]).  Tables are rows of
 * a [num_seqs, max_blocks] array. */
int oracle_slot_mapping(int64_t *slots, const int32_t *tables, int64_t max_blocks,
                        const int64_t *positions, int64_t n, int64_t block_size) {
  int64_t i;
  if (block_size <= 0 || n < 0) return ORACLE_EINVAL;
  for (i = 0; i < n; ++i) {
    if (positions[i] < 0 || positions[i] / block_size >= max_blocks) return ORACLE_ERANGE;
    slots[i] = oracle_physical_index(tables + i * max_blocks, block_size, positions[i]);
  }
  return ORACLE_OK;
}

/* KV write ([P1] section 4; [P3] Code: kv[b, t % BLOCK] = (k, v)).
 * For token i with slot s: block b = s / B, offset o = s % B; the bytes of
 * k_new[i, :, :] go to k_cache[b, o, :, :] and those of v_new[i] to v_cache[b, o].
 * Pure byte movement: NaN payloads, -0 and subnormals survive.  Every other byte of
 * both pools is left as it was. */
int oracle_kv_write(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                    const int64_t *slots, int64_t num_tokens, int64_t num_blocks,
                    int64_t block_size, int64_t num_kv_heads, int64_t head_dim, int dtype) {
  const int64_t e = elem_size(dtype);
  const int64_t row = num_kv_heads * head_dim * e;     /* bytes of one [Hkv, D] row */
  int64_t i, j;
  if (e == 0 || num_tokens < 0 || num_blocks <= 0 || block_size <= 0 || row <= 0) return ORACLE_EINVAL;
  for (i = 0; i < num_tokens; ++i) {
    if (slots[i] < 0 || slots[i] >= num_blocks * block_size) return ORACLE_ERANGE;
    for (j = 0; j < i; ++j)
      if (slots[j] == slots[i]) return ORACLE_EDUP;
  }
  for (i = 0; i < num_tokens; ++i) {
    const int64_t b = slots[i] / block_size, o = slots[i] % block_size;
    const int64_t dst = (b * block_size + o) * row;
    memcpy((char *)k_cache + dst, (const char *)k_new + i * row, (size_t)row);
    memcpy((char *)v_cache + dst, (const char *)v_new + i * row, (size_t)row);
  }
  return ORACLE_OK;
}

/* Copy-on-write block copy ([P1] section 6: copy the block first, then write;
 * [P3] Code: copy_block).  pairs is [num_pairs, 2] (src, dst).  Whole blocks are
 * copied, all B slots including unfilled ones, for K and for V. */
int oracle_copy_blocks(void *k_cache, void *v_cache, const int64_t *pairs, int64_t num_pairs,
                       int64_t num_blocks, int64_t block_size, int64_t num_kv_heads,
                       int64_t head_dim, int dtype) {
  const int64_t e = elem_size(dtype);
  const int64_t blk = block_size * num_kv_heads * head_dim * e;
  int64_t i, j;
  if (e == 0 || num_pairs < 0 || num_blocks <= 0 || blk <= 0) return ORACLE_EINVAL;
  for (i = 0; i < num_pairs; ++i) {
    const int64_t s = pairs[2 * i], d = pairs[2 * i + 1];
    if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks) return ORACLE_ERANGE;
    for (j = 0; j < num_pairs; ++j) {
      if (j != i && pairs[2 * j + 1] == d) return ORACLE_EDUP;
      if (pairs[2 * j] == d) return ORACLE_EDUP;
    }
  }
  for (i = 0; i < num_pairs; ++i) {
    const int64_t s = pairs[2 * i], d = pairs[2 * i + 1];
    memcpy((char *)k_cache + d * blk, (const char *)k_cache + s * blk, (size_t)blk);
    memcpy((char *)v_cache + d * blk, (const char *)v_cache + s * blk, (size_t)blk);
  }
  return ORACLE_OK;
}

typedef struct {
  const void *q, *k, *v;
  const int32_t *tables;
  const int32_t *ctx;
  int64_t max_blocks, S, Hq, Hkv, D, B, N;
  double scale;
  int dtype;
} attn_args;

/* Attention of query (s, h) restricted to positions [t0, t1), unnormalised:
 * x_t = scale * sum_d q[d] k_t[d];  m = max_t x_t;  w_t = exp(x_t - m);
 * L = sum_t w_t;  o[d] = sum_t w_t v_t[d].
 * Position t lives in block table[t / B] at offset t % B ([P2] section 5 "The kernel
 * side": the walk over ceil(ctx / B) blocks through the block table). */
static int attend_range(const attn_args *a, int64_t s, int64_t h, int64_t t0, int64_t t1,
                        double *x, double *o, double *m_out, double *l_out) {
  const int64_t g = a->Hq / a->Hkv;
  const int64_t kvh = h / g;                          /* GQA reading: contiguous groups */
  const int32_t *table = a->tables + s * a->max_blocks;
  const int64_t qoff = (s * a->Hq + h) * a->D;
  double m = -INFINITY, L = 0.0;
  int64_t t, d;
  for (t = t0; t < t1; ++t) {
    const int64_t b = table[t / a->B], off = t % a->B;
    int64_t krow;
    double acc = 0.0;
    if (b < 0 || b >= a->N) return ORACLE_ERANGE;
    krow = ((b * a->B + off) * a->Hkv + kvh) * a->D;
    for (d = 0; d < a->D; ++d) acc += load_elem(a->q, qoff + d, a->dtype) * load_elem(a->k, krow + d, a->dtype);
    x[t - t0] = a->scale * acc;
    if (x[t - t0] > m) m = x[t - t0];
  }
  for (d = 0; d < a->D; ++d) o[d] = 0.0;
  for (t = t0; t < t1; ++t) {
    const int64_t b = table[t / a->B], off = t % a->B;
    const int64_t vrow = ((b * a->B + off) * a->Hkv + kvh) * a->D;
    const double w = exp(x[t - t0] - m);
    L += w;
    for (d = 0; d < a->D; ++d) o[d] += w * load_elem(a->v, vrow + d, a->dtype);
  }
  *m_out = m;
  *l_out = L;
  return ORACLE_OK;
}

/* out[i, :] = softmax(scale * q K^T) V for query item items[i] = s * Hq + h, over the
 * sequence's first ctx[s] positions gathered through its block table.
 * partition_size == 0: one pass over [0, ctx).  partition_size = P > 0: partials
 * (m_p, L_p, o_p) over [p*P, min((p+1)*P, ctx)), merged as
 *   M = max_p m_p,  L = sum_p L_p e^(m_p - M),  out = sum_p e^(m_p - M) o_p / L.
 * items == NULL means every (s, h) in order.  Returns the first error found. */
int oracle_paged_attention(double *out, const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *block_tables, int64_t max_blocks, const int32_t *context_lens,
                           int64_t num_seqs, int64_t num_heads, int64_t num_kv_heads, int64_t head_dim,
                           int64_t block_size, int64_t num_blocks, double scale, int64_t partition_size,
                           const int64_t *items, int64_t num_items, int dtype, int num_threads) {
  attn_args a;
  int64_t i, n = items ? num_items : num_seqs * num_heads, max_ctx = 0;
  int err = ORACLE_OK;
  if (elem_size(dtype) == 0 || num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 ||
      num_heads % num_kv_heads != 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0 ||
      max_blocks <= 0 || partition_size < 0 || (partition_size > 0 && partition_size % block_size != 0))
    return ORACLE_EINVAL;
  for (i = 0; i < num_seqs; ++i) {
    if (context_lens[i] < 1 || context_lens[i] > max_blocks * block_size) return ORACLE_ERANGE;
    if (context_lens[i] > max_ctx) max_ctx = context_lens[i];
  }
  for (i = 0; items && i < num_items; ++i)
    if (items[i] < 0 || items[i] >= num_seqs * num_heads) return ORACLE_EINVAL;
  a.q = q; a.k = k_cache; a.v = v_cache; a.tables = block_tables; a.ctx = context_lens;
  a.max_blocks = max_blocks; a.S = num_seqs; a.Hq = num_heads; a.Hkv = num_kv_heads;
  a.D = head_dim; a.B = block_size; a.N = num_blocks; a.scale = scale; a.dtype = dtype;
#ifdef _OPENMP
  /* a clause, not omp_set_num_threads: the count holds for this call only */
  if (num_threads <= 0) num_threads = omp_get_max_threads();
#else
  (void)num_threads;
#endif
#pragma omp parallel num_threads(num_threads)
  {
    double *x = (double *)malloc(sizeof(double) * (size_t)max_ctx);
    double *o = (double *)malloc(sizeof(double) * (size_t)head_dim);
    double *acc = (double *)malloc(sizeof(double) * (size_t)head_dim);
    int64_t it, d;
    if (!x || !o || !acc) {
#pragma omp critical
      err = ORACLE_ENOMEM;
    }
#pragma omp for schedule(dynamic, 1)
    for (it = 0; it < n; ++it) {
      const int64_t item = items ? items[it] : it;
      const int64_t s = item / num_heads, h = item % num_heads;
      const int64_t ctx = context_lens[s];
      double *dst = out + it * head_dim;
      int rc = ORACLE_OK;
      if (!x || !o || !acc) continue;
      if (partition_size == 0) {
        double m, L;
        rc = attend_range(&a, s, h, 0, ctx, x, o, &m, &L);
        for (d = 0; d < head_dim && rc == ORACLE_OK; ++d) dst[d] = o[d] / L;
      } else {
        /* two sweeps over the partitions: the max of the partial maxima, then the merge */
        const int64_t np = (ctx + partition_size - 1) / partition_size;
        double M = -INFINITY, L = 0.0, m, Lp;
        int64_t p;
        for (p = 0; p < np && rc == ORACLE_OK; ++p) {
          const int64_t t1 = (p + 1) * partition_size < ctx ? (p + 1) * partition_size : ctx;
          rc = attend_range(&a, s, h, p * partition_size, t1, x, o, &m, &Lp);
          if (m > M) M = m;
        }
        for (d = 0; d < head_dim; ++d) acc[d] = 0.0;
        for (p = 0; p < np && rc == ORACLE_OK; ++p) {
          const int64_t t1 = (p + 1) * partition_size < ctx ? (p + 1) * partition_size : ctx;
          double w;
          rc = attend_range(&a, s, h, p * partition_size, t1, x, o, &m, &Lp);
          w = exp(m - M);
          L += Lp * w;
          for (d = 0; d < head_dim; ++d) acc[d] += w * o[d];
        }
        for (d = 0; d < head_dim && rc == ORACLE_OK; ++d) dst[d] = acc[d] / L;
      }
      if (rc != ORACLE_OK) {
#pragma omp critical
        if (err == ORACLE_OK) err = rc;
      }
    }
    free(x);
    free(o);
    free(acc);
  }
  return err;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
