/*
 * Paged-KV attention oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU definition of what the paged-KV path
 * computes.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline leg may load this library; the product path never does.  It shares
 * no code, header or constant with the GPU library.
 *
 * What it follows (pages as cited; no page prints a numeric worked example):
 *  - store: nano-vllm overview / devpress "nano-vllm解读", section on how
 *    PagedAttention is implemented (KV cache write): each new token's K and V
 *    row lands at cache row slot_mapping[i] of the cache viewed as
 *    [num_blocks * block_size, H_kv * d]; the AIInfraGuide 3.6 page, section 2,
 *    says a slot of -1 (padding) writes nothing.
 *  - attention: ascendai overview, section "FlashAttention 集成", the
 *    naive definition softmax(q k^T / sqrt(d)) v; paging only changes where
 *    key j of sequence b lives: physical block block_table[b][j / block_size],
 *    row j % block_size of that block (devpress page, "PagedAttention是如何实现的").
 *  - decode: one query per sequence over context_lens[b] keys, where
 *    context_lens counts the token stored this step (AIInfraGuide 3.6, section 2).
 *  - prefill: queries stacked along the token axis by cu_seqlens_q; the i-th new
 *    query of sequence b sits at absolute position c + i with
 *    c = (cu_seqlens_k[b+1]-cu_seqlens_k[b]) - (cu_seqlens_q[b+1]-cu_seqlens_q[b])
 *    cached tokens (AIInfraGuide 3.6, section 2, positions), and under the causal
 *    mask it sees keys 0 .. c + i.
 *  - grouped-query attention: query head h reads kv head h / (H_q / H_kv).  The
 *    pages give K/V H_kv heads but never state the grouping; this is the
 *    contiguous-group reading.  It is "parity unpinned" by the pages (only
 *    library convention backs it).
 *
 * Arithmetic: bf16 inputs are widened exactly; scores, softmax and the weighted
 * sum are carried in double precision with libm exp.  A sequence with no keys
 * gives an all-zero output row.
 *
 * Planted mistakes: building with -DPKV_ORACLE_PLANT=<n> (n > 0) compiles one
 * deliberate error so the test suite can show that its pins catch it.  The
 * default build (PKV_ORACLE_PLANT undefined or 0) has none.
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef PKV_ORACLE_PLANT
#define PKV_ORACLE_PLANT 0
#endif

enum {
  ORACLE_OK = 0,
  ORACLE_BAD_ARG = 1,      /* shape arguments inconsistent */
  ORACLE_BAD_SLOT = 2,     /* slot outside [-1, num_blocks * block_size) */
  ORACLE_DUP_SLOT = 3,     /* two tokens mapped to one slot */
  ORACLE_BAD_BLOCK = 4,    /* block table entry outside [0, num_blocks) for a read key */
  ORACLE_BAD_LEN = 5,      /* context / key length negative or beyond the table */
  ORACLE_NO_MEM = 6
};

static double widen_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

int pkv_oracle_plant(void) { return PKV_ORACLE_PLANT; }

/* Threads the parallel loops below use (OpenMP's current maximum). */
int pkv_oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------ store */
int pkv_oracle_store(uint16_t* k_cache, uint16_t* v_cache,
                     const uint16_t* key, int64_t key_stride,
                     const uint16_t* value, int64_t value_stride,
                     const int32_t* slot_mapping, int32_t n_tokens,
                     int32_t num_blocks, int32_t block_size, int32_t row_elems) {
  if (n_tokens < 0 || num_blocks <= 0 || block_size <= 0 || row_elems <= 0 ||
      key_stride < row_elems || value_stride < row_elems)
    return ORACLE_BAD_ARG;
  int64_t n_slots = (int64_t)num_blocks * block_size;
  /* check every slot before writing anything */
  unsigned char* seen = (unsigned char*)calloc((size_t)n_slots, 1);
  if (!seen) return ORACLE_NO_MEM;
  for (int32_t i = 0; i < n_tokens; ++i) {
    int32_t s = slot_mapping[i];
    if (s == -1) continue;
    if (s < -1 || (int64_t)s >= n_slots) { free(seen); return ORACLE_BAD_SLOT; }
    if (seen[s]) { free(seen); return ORACLE_DUP_SLOT; }
    seen[s] = 1;
  }
  free(seen);
  for (int32_t i = 0; i < n_tokens; ++i) {
    int32_t s = slot_mapping[i];
    if (s == -1) continue; /* padding token: nothing is written */
    memcpy(k_cache + (int64_t)s * row_elems, key + (int64_t)i * key_stride,
           sizeof(uint16_t) * (size_t)row_elems);
    memcpy(v_cache + (int64_t)s * row_elems, value + (int64_t)i * value_stride,
           sizeof(uint16_t) * (size_t)row_elems);
  }
  return ORACLE_OK;
}

/* -------------------------------------------------------------- attention */
struct cache_view {
  const uint16_t* k;       /* [num_blocks, block_size, H_kv, d] */
  const uint16_t* v;
  int32_t num_blocks, block_size, H_kv, d;
};

/* Pointer to the K (or V) vector of logical key j of a sequence, or NULL if the
 * table does not map it to a valid block. */
static const uint16_t* key_row(const struct cache_view* c, const uint16_t* base,
                               const int32_t* table_row, int32_t j, int32_t kv_head) {
  int32_t blk = table_row[j / c->block_size];
#if PKV_ORACLE_PLANT == 4
  blk = table_row[(j + 1) / c->block_size]; /* planted: page index off by one token */
#endif
  if (blk < 0 || blk >= c->num_blocks) return NULL;
  int64_t row = (int64_t)blk * c->block_size + j % c->block_size;
  return base + (row * c->H_kv + kv_head) * c->d;
}

/* out[0..d) = softmax over keys 0..n_keys-1 of (q . k_j) * scale, applied to v_j. */
static int attend(double* out, const uint16_t* q, const struct cache_view* c,
                  const int32_t* table_row, int32_t n_keys, int32_t kv_head,
                  double scale) {
  const int32_t d = c->d;
  for (int32_t e = 0; e < d; ++e) out[e] = 0.0;
  if (n_keys == 0) return ORACLE_OK;
#if PKV_ORACLE_PLANT == 1
  n_keys -= 1; /* planted: drops the newest key */
  if (n_keys == 0) return ORACLE_OK;
#endif
  double* s = (double*)malloc(sizeof(double) * (size_t)n_keys);
  if (!s) return ORACLE_NO_MEM;
  double m = -INFINITY;
  for (int32_t j = 0; j < n_keys; ++j) {
    const uint16_t* kj = key_row(c, c->k, table_row, j, kv_head);
    if (!kj) { free(s); return ORACLE_BAD_BLOCK; }
    double dot = 0.0;
    for (int32_t e = 0; e < d; ++e) dot += widen_bf16(q[e]) * widen_bf16(kj[e]);
#if PKV_ORACLE_PLANT == 3
    s[j] = dot; /* planted: scale dropped */
#else
    s[j] = dot * scale;
#endif
    if (s[j] > m) m = s[j];
  }
  double l = 0.0;
  for (int32_t j = 0; j < n_keys; ++j) {
    double w = exp(s[j] - m);
    l += w;
#if PKV_ORACLE_PLANT == 5
    const uint16_t* vj = key_row(c, c->k, table_row, j, kv_head); /* planted: K used as V */
#else
    const uint16_t* vj = key_row(c, c->v, table_row, j, kv_head);
#endif
    for (int32_t e = 0; e < d; ++e) out[e] += w * widen_bf16(vj[e]);
  }
  for (int32_t e = 0; e < d; ++e) out[e] /= l;
  free(s);
  return ORACLE_OK;
}

static int32_t kv_head_of(int32_t h, int32_t H_q, int32_t H_kv) {
#if PKV_ORACLE_PLANT == 2
  return h % H_kv; /* planted: interleaved instead of contiguous head groups */
#else
  return h / (H_q / H_kv);
#endif
}

static int check_geometry(int32_t H_q, int32_t H_kv, int32_t d, int32_t num_blocks,
                          int32_t block_size, int32_t max_blocks_per_seq) {
  if (H_q <= 0 || H_kv <= 0 || d <= 0 || H_q % H_kv != 0 || num_blocks <= 0 ||
      block_size <= 0 || max_blocks_per_seq < 0)
    return ORACLE_BAD_ARG;
  return ORACLE_OK;
}

/* out [B, H_q, d] (double); q [B, H_q, d] bf16 bits. */
int pkv_oracle_decode(double* out, const uint16_t* q, const uint16_t* k_cache,
                      const uint16_t* v_cache, const int32_t* block_tables,
                      const int32_t* context_lens, int32_t B, int32_t H_q, int32_t H_kv,
                      int32_t d, int32_t num_blocks, int32_t block_size,
                      int32_t max_blocks_per_seq, float softmax_scale) {
  int rc = check_geometry(H_q, H_kv, d, num_blocks, block_size, max_blocks_per_seq);
  if (rc) return rc;
  for (int32_t b = 0; b < B; ++b)
    if (context_lens[b] < 0 ||
        (int64_t)context_lens[b] > (int64_t)max_blocks_per_seq * block_size)
      return ORACLE_BAD_LEN;
  struct cache_view c = {k_cache, v_cache, num_blocks, block_size, H_kv, d};
  int err = ORACLE_OK;
  int64_t rows = (int64_t)B * H_q;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t r = 0; r < rows; ++r) {
    int32_t b = (int32_t)(r / H_q), h = (int32_t)(r % H_q);
    int e = attend(out + r * d, q + r * d, &c,
                   block_tables + (int64_t)b * max_blocks_per_seq, context_lens[b],
                   kv_head_of(h, H_q, H_kv), (double)softmax_scale);
    if (e) {
#pragma omp critical
      err = e;
    }
  }
  return err;
}

/* out [total_q, H_q, d] (double); q [total_q, H_q, d] bf16 bits. */
int pkv_oracle_prefill(double* out, const uint16_t* q, const uint16_t* k_cache,
                       const uint16_t* v_cache, const int32_t* block_tables,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                       int32_t B, int32_t H_q, int32_t H_kv, int32_t d,
                       int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                       float softmax_scale) {
  int rc = check_geometry(H_q, H_kv, d, num_blocks, block_size, max_blocks_per_seq);
  if (rc) return rc;
  if (cu_seqlens_q[0] != 0) return ORACLE_BAD_ARG;
  for (int32_t b = 0; b < B; ++b) {
    int32_t nq = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
    int32_t nk = cu_seqlens_k[b + 1] - cu_seqlens_k[b];
    if (nq < 0 || nk < nq || (int64_t)nk > (int64_t)max_blocks_per_seq * block_size)
      return ORACLE_BAD_LEN;
  }
  struct cache_view c = {k_cache, v_cache, num_blocks, block_size, H_kv, d};
  int err = ORACLE_OK;
  int64_t total_q = cu_seqlens_q[B];
  int64_t rows = total_q * H_q;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t r = 0; r < rows; ++r) {
    int64_t t = r / H_q;
    int32_t h = (int32_t)(r % H_q);
    int32_t b = 0; /* sequence owning query row t */
    while (cu_seqlens_q[b + 1] <= t) ++b;
    int32_t nq = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
    int32_t nk = cu_seqlens_k[b + 1] - cu_seqlens_k[b];
    int32_t cached = nk - nq;
    int32_t i = (int32_t)(t - cu_seqlens_q[b]);
    int e = attend(out + r * d, q + r * d, &c,
                   block_tables + (int64_t)b * max_blocks_per_seq, cached + i + 1,
                   kv_head_of(h, H_q, H_kv), (double)softmax_scale);
    if (e) {
#pragma omp critical
      err = e;
    }
  }
  return err;
}
