/*
 * Plain fp64 CPU oracle for one mixed chunked-prefill attention step.
 * TEST INFRASTRUCTURE ONLY: see oracle.h for who may call it and for the
 * passages each function follows.  Deliberately simple: no blocking, no online
 * softmax, no fusion.  Each output row is computed on its own, in two passes
 * over its visible keys in ascending position order.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Exact upcast of one stored element to double. */
static double load_elem(const void* base, size_t idx, int32_t dtype) {
  if (dtype == ORACLE_F32) {
    return (double)((const float*)base)[idx];
  }
  uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static size_t elem_size(int32_t dtype) { return dtype == ORACLE_F32 ? 4 : 2; }

/* Segment b spans packed rows [cu[b], cu[b+1]); its query length is
 * Lq = cu[b+1] - cu[b] and its KV length Lk = seqlens_k[b] counts the history
 * plus this step's new tokens (they were appended before attention runs). */
static int segment_shape(const int32_t* cu, const int32_t* seqlens_k, int32_t b,
                         int32_t* lq, int32_t* lk) {
  if (cu[b + 1] < cu[b]) return -1;
  *lq = cu[b + 1] - cu[b];
  *lk = seqlens_k[b];
  if (*lq > *lk) return -1;
  return 0;
}

int oracle_visible_counts(const int32_t* cu, const int32_t* seqlens_k,
                          int32_t num_seqs, int32_t* n_vis) {
  if (cu[0] != 0) return -1;
  for (int32_t b = 0; b < num_seqs; ++b) {
    int32_t lq, lk;
    if (segment_shape(cu, seqlens_k, b, &lq, &lk)) return -1;
    /* The query segment sits at the end of the KV segment: row i is the key
     * at position (Lk - Lq) + i and sees every key up to and including it. */
    for (int32_t i = 0; i < lq; ++i) n_vis[cu[b] + i] = (lk - lq) + i + 1;
  }
  return 0;
}

int oracle_check_slots(const int32_t* cu, const int32_t* seqlens_k,
                       const int32_t* block_table, const int32_t* slot_mapping,
                       int32_t num_seqs, int32_t max_blocks, int32_t page_size,
                       int32_t num_blocks) {
  if (cu[0] != 0) return -1;
  int32_t total = cu[num_seqs];
  int64_t pool_slots = (int64_t)num_blocks * page_size;
  /* every slot in range and used at most once */
  unsigned char* used = (unsigned char*)calloc((size_t)pool_slots, 1);
  if (!used) return -4;
  for (int32_t t = 0; t < total; ++t) {
    int32_t s = slot_mapping[t];
    if (s < 0 || (int64_t)s >= pool_slots || used[s]) {
      free(used);
      return -3;
    }
    used[s] = 1;
  }
  free(used);
  int mismatches = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    int32_t lq, lk;
    if (segment_shape(cu, seqlens_k, b, &lq, &lk)) return -1;
    const int32_t* row = block_table + (size_t)b * max_blocks;
    for (int32_t i = 0; i < lq; ++i) {
      int32_t pos = (lk - lq) + i;
      int32_t logical = pos / page_size;
      if (logical >= max_blocks) return -2;
      int32_t phys = row[logical];
      if (phys < 0 || phys >= num_blocks) return -2;
      int32_t slot = phys * page_size + pos % page_size;
      if (slot != slot_mapping[cu[b] + i]) ++mismatches;
    }
  }
  return mismatches;
}

int oracle_append(const void* key, const void* value, const int32_t* slot_mapping,
                  void* k_cache, void* v_cache, int32_t total_tokens,
                  int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                  int32_t num_blocks, int32_t dtype) {
  size_t es = elem_size(dtype);
  size_t row_elems = (size_t)num_kv_heads * head_dim;
  int64_t pool_slots = (int64_t)num_blocks * page_size;
  for (int32_t t = 0; t < total_tokens; ++t) {
    int32_t s = slot_mapping[t];
    if (s < 0) continue;
    if ((int64_t)s >= pool_slots) return -3;
    /* slot s is page s / P, offset s % P; a page holds P consecutive rows of
     * [Hkv, D], so the row's first element sits at s * Hkv * D. */
    for (size_t e = 0; e < row_elems; ++e) {
      size_t src = (size_t)t * row_elems + e;
      size_t dst = (size_t)s * row_elems + e;
      memcpy((char*)k_cache + dst * es, (const char*)key + src * es, es);
      memcpy((char*)v_cache + dst * es, (const char*)value + src * es, es);
    }
  }
  return 0;
}

/* Element index of (key position pos, kv head, channel d) of a segment whose
 * block-table row is `row`: page row[pos / P], offset pos % P. */
static size_t cache_index(const int32_t* row, int32_t pos, int32_t kvh, int32_t d,
                          int32_t page_size, int32_t num_kv_heads, int32_t head_dim) {
  size_t page = (size_t)row[pos / page_size];
  size_t off = (size_t)(pos % page_size);
  return ((page * page_size + off) * num_kv_heads + kvh) * head_dim + d;
}

int oracle_attention(const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* cu, const int32_t* seqlens_k,
                     const int32_t* block_table, int32_t num_seqs,
                     int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t page_size, int32_t num_blocks, int32_t max_blocks,
                     double scale, int32_t dtype, const uint8_t* row_select,
                     double* out) {
  if (cu[0] != 0 || num_heads % num_kv_heads != 0) return -1;
  int32_t max_lk = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    int32_t lq, lk;
    if (segment_shape(cu, seqlens_k, b, &lq, &lk)) return -1;
    if (lq == 0) continue;
    int32_t pages = (lk + page_size - 1) / page_size;
    if (pages > max_blocks) return -2;
    for (int32_t p = 0; p < pages; ++p) {
      int32_t id = block_table[(size_t)b * max_blocks + p];
      if (id < 0 || id >= num_blocks) return -2;
    }
    if (lk > max_lk) max_lk = lk;
  }
  const int32_t total = cu[num_seqs];
  const int32_t group = num_heads / num_kv_heads; /* query heads per KV head */
  const long long work = (long long)total * num_heads;

#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(max_lk > 0 ? max_lk : 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)head_dim);
    int32_t b = 0;
#pragma omp for schedule(dynamic, 4)
    for (long long w = 0; w < work; ++w) {
      int32_t r = (int32_t)(w / num_heads);
      int32_t h = (int32_t)(w % num_heads);
      if (row_select && !row_select[r]) continue;
      /* segment that owns packed row r */
      if (r < cu[b] || r >= cu[b + 1]) {
        b = 0;
        while (!(r >= cu[b] && r < cu[b + 1])) ++b;
      }
      const int32_t lq = cu[b + 1] - cu[b];
      const int32_t lk = seqlens_k[b];
      const int32_t i = r - cu[b];
      const int32_t n_vis = (lk - lq) + i + 1;
      const int32_t kvh = h / group;
      const int32_t* row = block_table + (size_t)b * max_blocks;
      const size_t q0 = ((size_t)r * num_heads + h) * head_dim;

      /* pass 1: scores of all visible keys and their maximum */
      double m = -INFINITY;
      for (int32_t j = 0; j < n_vis; ++j) {
        double dot = 0.0;
        for (int32_t d = 0; d < head_dim; ++d) {
          size_t kidx = cache_index(row, j, kvh, d, page_size, num_kv_heads, head_dim);
          dot += load_elem(q, q0 + d, dtype) * load_elem(k_cache, kidx, dtype);
        }
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
      }
      /* pass 2: softmax weights, their sum, and the weighted sum of values */
      double l = 0.0;
      for (int32_t d = 0; d < head_dim; ++d) acc[d] = 0.0;
      for (int32_t j = 0; j < n_vis; ++j) {
        double wgt = exp(s[j] - m);
        l += wgt;
        for (int32_t d = 0; d < head_dim; ++d) {
          size_t vidx = cache_index(row, j, kvh, d, page_size, num_kv_heads, head_dim);
          acc[d] += wgt * load_elem(v_cache, vidx, dtype);
        }
      }
      for (int32_t d = 0; d < head_dim; ++d) out[q0 + d] = acc[d] / l;
    }
    free(s);
    free(acc);
  }
  return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
