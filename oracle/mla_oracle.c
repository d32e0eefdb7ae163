/*
 * TEST INFRASTRUCTURE ONLY.  A plain, slow fp64 CPU reference for MLA decode
 * attention over a paged latent KV cache.  Only tests/, the smoke check and the
 * benchmark's CPU-baseline leg may build, load or call it; the product library
 * never does.  It shares no code, header or table with the HIP path.
 *
 * What it computes, following the pages:
 *  - "RFC: MsModeling 支持 Decode Context Parallel 仿真", §2.1.4 symbol table:
 *    B sequences, Q query tokens per sequence (Q = 1 + speculative tokens),
 *    h_q query heads, one latent KV head (h_kv = 1 for MLA), row width
 *    D = kv_lora_rank + qk_rope_head_dim.
 *  - same page, §2.1.4.1 (table A): the MLA cache is [N_blk, block_size, D],
 *    addressed through block_table [B, max_blocks].
 *  - same page, §2.1.4.2 (table B): the attention op returns an output plus an
 *    fp32 log-sum-exp (lse) per (token, head); under DCP each rank attends only
 *    its share of the sequence and the partial (output, lse) pairs are
 *    recombined by an online-softmax merge (§1.1, §2.1.1, §2.1.4.3).
 *  - same page, §2.1.4.1: tokens are dealt to DCP ranks in runs of
 *    cp_kv_cache_interleave_size; shard(p) = floor(p / I) mod N.
 *  - same page §1.3 and "RFC: Context Parallel Modeling for DeepSeek-Style
 *    Attention" §3.6: the SFA sparse path replaces the S context positions by
 *    the top_k indexer-selected positions, with bf16 inputs.
 *
 * Readings where the pages are silent (each one is listed in the design notes):
 *  - absorbed MLA: every head dots its D = 576 query with the shared latent row;
 *    V is the row's first d_v = 512 columns; the output stays in latent space.
 *  - s_p = scale * <q, k_p>; lse = ln sum_{p in A} exp(s_p); O = sum exp(s_p - lse) v_p.
 *  - query token q of sequence b sits at position pos = S_b - Q + q and attends
 *    positions <= pos (causal within the speculative tokens).
 *  - sparse indices are logical token positions; -1 is padding; any value
 *    outside [0, pos] is dropped; duplicates count with multiplicity.
 *  - an empty attended set gives O = 0 and lse = -inf.
 *
 * The attended set A is built explicitly as a list, and softmax is evaluated in
 * the two-pass form m = max s, l = sum exp(s - m) (the same number as the
 * definition, written so that exp cannot overflow).  No tiling, no online
 * rescaling, no fusion.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum {
  ORACLE_OK = 0,
  ORACLE_ERR_ARG = 1,        /* null pointer or non-positive size */
  ORACLE_ERR_BLOCK = 2,      /* a block-table entry that a used position needs is out of range */
  ORACLE_ERR_NOMEM = 3
};

typedef struct {
  int32_t B, Q, h_q, d_qk, d_v;
  double scale;
  const uint16_t *q;          /* bf16 bits [B, Q, h_q, d_qk] */
  const uint16_t *kv;         /* bf16 bits [num_blocks, block_size, d_qk] */
  int32_t num_blocks, block_size;
  const int32_t *block_table; /* [B, max_blocks] */
  int32_t max_blocks;
  const int32_t *seq_lens;    /* [B] */
  /* int8 cache, used instead of kv when kv8 is non-null: codes [num_blocks,
   * block_size, d_qk] and one factor per row [num_blocks, block_size]. */
  const int8_t *kv8;
  const float *kv_scale;
} oracle_problem;

/* bf16 is the upper half of an IEEE binary32; the widening to double is exact. */
static double bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Column c of latent cache row `row`.  bf16 cache: the stored value.  int8
 * cache (the one-byte kv-int8 element type of the DCP page, notation table of
 * §2.1.4 and the open items of §3.3; the pages leave its dequantisation open): the row's factor times the code, both
 * exact in double. */
static double latent_value(const oracle_problem *P, int64_t row, int c) {
  if (P->kv8) return (double)P->kv_scale[row] * (double)P->kv8[row * P->d_qk + c];
  return bf16_value(P->kv[row * P->d_qk + c]);
}

/* Physical cache row of logical position p of sequence b (table A of the DCP page). */
static int64_t physical_row(const oracle_problem *P, int b, int64_t p) {
  int64_t blk_slot = p / P->block_size;
  if (blk_slot < 0 || blk_slot >= P->max_blocks) return -1;
  int32_t blk = P->block_table[(int64_t)b * P->max_blocks + blk_slot];
  if (blk < 0 || blk >= P->num_blocks) return -1;
  return (int64_t)blk * P->block_size + p % P->block_size;
}

/* Softmax-weighted sum over an explicit list of attended positions for one
 * (b, q, h).  Returns ORACLE_OK or ORACLE_ERR_BLOCK. */
static int attend(const oracle_problem *P, int b, int qi, int h, const int64_t *pos,
                  int64_t n, double *s, double *out, double *lse) {
  const int D = P->d_qk, DV = P->d_v;
  for (int c = 0; c < DV; ++c) out[c] = 0.0;
  if (n == 0) {
    *lse = -INFINITY;
    return ORACLE_OK;
  }
  const uint16_t *qrow = P->q + (((int64_t)b * P->Q + qi) * P->h_q + h) * D;
  /* scores s_p = scale * <q, k_p> over all D columns */
  for (int64_t j = 0; j < n; ++j) {
    int64_t row = physical_row(P, b, pos[j]);
    if (row < 0) return ORACLE_ERR_BLOCK;
    double dot = 0.0;
    for (int k = 0; k < D; ++k) dot += bf16_value(qrow[k]) * latent_value(P, row, k);
    s[j] = P->scale * dot;
  }
  double m = s[0];
  for (int64_t j = 1; j < n; ++j)
    if (s[j] > m) m = s[j];
  double l = 0.0;
  for (int64_t j = 0; j < n; ++j) l += exp(s[j] - m);
  /* O = sum_p softmax_p * v_p with v_p = the first d_v columns of the latent row */
  for (int64_t j = 0; j < n; ++j) {
    double w = exp(s[j] - m) / l;
    const int64_t vrow = physical_row(P, b, pos[j]);
    for (int c = 0; c < DV; ++c) out[c] += w * latent_value(P, vrow, c);
  }
  *lse = m + log(l);
  return ORACLE_OK;
}

static int check_problem(const oracle_problem *P) {
  if (!P || !P->q || (!P->kv && !P->kv8) || (P->kv8 && !P->kv_scale) || !P->block_table ||
      !P->seq_lens)
    return ORACLE_ERR_ARG;
  if (P->B <= 0 || P->Q <= 0 || P->h_q <= 0 || P->d_qk <= 0 || P->d_v <= 0 ||
      P->d_v > P->d_qk || P->block_size <= 0 || P->num_blocks <= 0 || P->max_blocks <= 0)
    return ORACLE_ERR_ARG;
  return ORACLE_OK;
}

/* Row id r of the flattened [B, Q, h_q] output.  sel == NULL means every row. */
static void split_row(const oracle_problem *P, int64_t r, int *b, int *qi, int *h) {
  *h = (int)(r % P->h_q);
  int64_t bq = r / P->h_q;
  *qi = (int)(bq % P->Q);
  *b = (int)(bq / P->Q);
}

/*
 * Dense decode.  Attended set for (b, q): every position p in [0, S_b - Q + q];
 * with num_shards > 1 only those with floor(p / interleave) mod num_shards ==
 * shard_id (the DCP interleaved placement).  Writes out[n_sel, d_v], lse[n_sel].
 */
int oracle_dense(const oracle_problem *P, int32_t num_shards, int32_t interleave,
                 int32_t shard_id, int64_t n_sel, const int64_t *sel, double *out,
                 double *lse) {
  int rc = check_problem(P);
  if (rc) return rc;
  if (num_shards < 1 || (num_shards > 1 && (interleave < 1 || shard_id < 0 ||
                                            shard_id >= num_shards)))
    return ORACLE_ERR_ARG;
  int64_t rows = (int64_t)P->B * P->Q * P->h_q;
  if (!sel) n_sel = rows;
  if (n_sel < 0 || !out || !lse) return ORACLE_ERR_ARG;
  int err = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < n_sel; ++t) {
    int64_t r = sel ? sel[t] : t;
    if (r < 0 || r >= rows) {
#pragma omp atomic write
      err = ORACLE_ERR_ARG;
      continue;
    }
    int b, qi, h;
    split_row(P, r, &b, &qi, &h);
    int64_t last = (int64_t)P->seq_lens[b] - P->Q + qi; /* causal limit */
    int64_t cap = last >= 0 ? last + 1 : 0;
    int64_t *pos = (int64_t *)malloc(sizeof(int64_t) * (cap > 0 ? cap : 1));
    double *s = (double *)malloc(sizeof(double) * (cap > 0 ? cap : 1));
    if (!pos || !s) {
      free(pos);
      free(s);
#pragma omp atomic write
      err = ORACLE_ERR_NOMEM;
      continue;
    }
    int64_t n = 0;
    for (int64_t p = 0; p <= last; ++p)
      if (num_shards == 1 || (p / interleave) % num_shards == shard_id) pos[n++] = p;
    int e = attend(P, b, qi, h, pos, n, s, out + t * P->d_v, lse + t);
    if (e) {
#pragma omp atomic write
      err = e;
    }
    free(pos);
    free(s);
  }
  return err;
}

/*
 * Sparse (SFA) decode.  indices[b * stride_b + q * stride_q + k], k < top_k,
 * are logical positions; the attended multiset for (b, q) holds each entry i
 * with 0 <= i <= S_b - Q + q (so -1 padding and out-of-range values drop out),
 * and with num_shards > 1 only the entries this DCP rank holds,
 * floor(i / interleave) mod num_shards == shard_id (the interleaved placement
 * of the DCP page, §2.1.4.1; sparse attention under DCP attends, on each rank,
 * the selected positions that rank stores).
 */
int oracle_sparse(const oracle_problem *P, const int32_t *indices, int32_t top_k,
                  int64_t stride_b, int64_t stride_q, int32_t num_shards, int32_t interleave,
                  int32_t shard_id, int64_t n_sel, const int64_t *sel, double *out, double *lse) {
  int rc = check_problem(P);
  if (rc) return rc;
  if (!indices || top_k < 0 || !out || !lse) return ORACLE_ERR_ARG;
  if (num_shards < 1 || (num_shards > 1 && (interleave < 1 || shard_id < 0 ||
                                            shard_id >= num_shards)))
    return ORACLE_ERR_ARG;
  int64_t rows = (int64_t)P->B * P->Q * P->h_q;
  if (!sel) n_sel = rows;
  int err = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < n_sel; ++t) {
    int64_t r = sel ? sel[t] : t;
    if (r < 0 || r >= rows) {
#pragma omp atomic write
      err = ORACLE_ERR_ARG;
      continue;
    }
    int b, qi, h;
    split_row(P, r, &b, &qi, &h);
    int64_t last = (int64_t)P->seq_lens[b] - P->Q + qi;
    int64_t *pos = (int64_t *)malloc(sizeof(int64_t) * (top_k > 0 ? top_k : 1));
    double *s = (double *)malloc(sizeof(double) * (top_k > 0 ? top_k : 1));
    if (!pos || !s) {
      free(pos);
      free(s);
#pragma omp atomic write
      err = ORACLE_ERR_NOMEM;
      continue;
    }
    const int32_t *list = indices + (int64_t)b * stride_b + (int64_t)qi * stride_q;
    int64_t n = 0;
    for (int32_t k = 0; k < top_k; ++k) {
      int64_t i = list[k];
      if (i >= 0 && i <= last && (num_shards == 1 || (i / interleave) % num_shards == shard_id))
        pos[n++] = i;
    }
    int e = attend(P, b, qi, h, pos, n, s, out + t * P->d_v, lse + t);
    if (e) {
#pragma omp atomic write
      err = e;
    }
    free(pos);
    free(s);
  }
  return err;
}

/*
 * Online-softmax merge of n partial results (DCP page, §1.1 and §2.1.4.3): for
 * each row, M = max_i lse_i, w_i = exp(lse_i - M), lse = M + ln sum w_i and
 * O = sum w_i O_i / sum w_i.  Parts with lse = -inf carry no weight; when every
 * part is -inf the row is O = 0, lse = -inf.
 * o_parts[n, rows, d_v], lse_parts[n, rows]; out[rows, d_v], lse_out[rows].
 */
int oracle_merge(const double *o_parts, const double *lse_parts, int32_t n, int64_t rows,
                 int32_t d_v, double *out, double *lse_out) {
  if (!o_parts || !lse_parts || !out || !lse_out || n < 1 || rows < 0 || d_v < 1)
    return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double M = -INFINITY;
    for (int32_t i = 0; i < n; ++i)
      if (lse_parts[(int64_t)i * rows + r] > M) M = lse_parts[(int64_t)i * rows + r];
    double *o = out + r * d_v;
    for (int32_t c = 0; c < d_v; ++c) o[c] = 0.0;
    if (M == -INFINITY) {
      lse_out[r] = -INFINITY;
      continue;
    }
    double W = 0.0;
    for (int32_t i = 0; i < n; ++i) {
      double li = lse_parts[(int64_t)i * rows + r];
      if (li == -INFINITY) continue;
      double w = exp(li - M);
      W += w;
      const double *oi = o_parts + ((int64_t)i * rows + r) * d_v;
      for (int32_t c = 0; c < d_v; ++c) o[c] += w * oi[c];
    }
    for (int32_t c = 0; c < d_v; ++c) o[c] /= W;
    lse_out[r] = M + log(W);
  }
  return ORACLE_OK;
}

/* Number of threads an OpenMP parallel region here would use. */
int oracle_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    {
#ifdef _OPENMP
      n = omp_get_num_threads();
#endif
    }
  }
  return n;
}
