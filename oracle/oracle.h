/*
 * Plain CPU oracle for one mixed chunked-prefill attention step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path never
 * calls it, and it shares no code, header or table with the HIP library.
 *
 * Everything is fp64 on the host, computed straight from the definitions on
 * the source pages:
 *   - "大语言模型推理优化（二）：Chunked Prefill" (wangyu.me), sections
 *     "记录 KV Cache 的长度", "Flash Attention 的 varlen 接口" and
 *     "在 vLLM 中是如何实现的 / 输入组装": packed ragged query segments,
 *     segment isolation, causal masking with the query segment aligned to the
 *     END of its KV segment, new K/V written through slot_mapping before the
 *     paged attention reads pages through the block table.
 *   - kwkr.cn Triton hybrid-attention article, section "Triton 混合算子内核设计
 *     与实现": page = block_table[pos / PAGE_SIZE], offset = pos % PAGE_SIZE,
 *     scale = 1/sqrt(head_dim), natural exponential.
 *   - "技术融合剖析：Chunked Prefill如何借助FlashAttention/FlashInfer实现混合批次推理"
 *     (lpnh.cn), section 4.2: the append writes each new token's K/V into its
 *     physical page slot.
 *
 * Storage dtypes: ORACLE_F32 (IEEE binary32) and ORACLE_BF16 (upper 16 bits of
 * binary32, stored as uint16).  Upcasts to double are exact.
 *
 * Layouts (all dense, row-major):
 *   q           [T, Hq, D]
 *   key, value  [T, Hkv, D]                (this step's new tokens)
 *   k/v cache   [NB, P, Hkv, D]            (P = page size in tokens)
 *   cu_seqlens_q[B+1], seqlens_k[B], block_table[B, max_blocks], slot_mapping[T]
 *   out         [T, Hq, D] double
 *
 * Return codes: 0 = ok, negative = a precondition failed (see oracle.c).
 *
 * parity pins: every function here is pinned by tests/test_oracle_pins.py
 * (worked example, chunk invariance, closed forms, brute force, block-table
 * fingerprint, NaN hygiene, planted-mistake mutants).
 */
#ifndef CPMH_ORACLE_H
#define CPMH_ORACLE_H
#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

/* Number of keys row i of each segment may see, written for every packed row:
 * n_vis[cu[b]+i] = (Lk_b - Lq_b) + i + 1.  Returns 0, or -1 if a segment has
 * Lq > Lk or cu is not non-decreasing from 0. */
int oracle_visible_counts(const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                          int32_t num_seqs, int32_t* n_vis);

/* Re-derives, for every packed row, the slot its new K/V must land in
 * (slot = block_table[b][pos / P] * P + pos % P with pos = Lk - Lq + i) and
 * compares it with slot_mapping.  Returns the number of mismatching rows, or a
 * negative code if block ids are out of range (-2), slots collide or leave
 * the pool (-3), or the segment shape is invalid (-1). */
int oracle_check_slots(const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                       const int32_t* block_table, const int32_t* slot_mapping,
                       int32_t num_seqs, int32_t max_blocks, int32_t page_size,
                       int32_t num_blocks);

/* Copies key[t] / value[t] element by element into the cache slot
 * slot_mapping[t] (tokens with a negative slot are skipped).  Returns 0, or -3
 * for a slot outside the pool. */
int oracle_append(const void* key, const void* value, const int32_t* slot_mapping,
                  void* k_cache, void* v_cache, int32_t total_tokens,
                  int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                  int32_t num_blocks, int32_t dtype);

/* Paged varlen attention, right-aligned causal, fp64.
 * row_select (nullable, [T] bytes): when given, only rows with a nonzero entry
 * are computed; other rows of `out` are left untouched.
 * Returns 0, -1 (bad segment shape), -2 (a needed block id out of range). */
int oracle_attention(const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                     const int32_t* block_table, int32_t num_seqs,
                     int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t page_size, int32_t num_blocks, int32_t max_blocks,
                     double scale, int32_t dtype, const uint8_t* row_select,
                     double* out);

/* Number of OpenMP threads the oracle runs on. */
int oracle_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
