/*
 * hybrid_attn.h -- C ABI of libhybridattn.so: one mixed chunked-prefill step
 * of paged attention on an AMD Instinct MI355X (gfx950).
 *
 * A step packs ragged query segments -- decode segments of one token and
 * prefill chunks of many -- into one tensor, and every segment attends only to
 * its own KV history, which lives in fixed-size pages located through a
 * per-request block table.  Sources for what is computed:
 *   [VARLEN]  "大语言模型推理优化（二）：Chunked Prefill" (wangyu.me), sections
 *             "记录 KV Cache 的长度" and "Flash Attention 的 varlen 接口":
 *             cu_seqlens_q packing, segment isolation, causal mask with the
 *             query segment aligned to the END of its KV segment, decode =
 *             query length 1.
 *   [ORDER]   same page, section "在 vLLM 中是如何实现的 / 输入组装": the new
 *             K/V are written through slot_mapping into the paged cache first,
 *             then the varlen paged kernel gathers history via block_table.
 *   [PAGED]   kwkr.cn Triton hybrid-attention article, kernel section: page
 *             = block_table[pos / PAGE_SIZE], offset = pos % PAGE_SIZE,
 *             scale = 1/sqrt(head_dim), online softmax in fp32.
 *   [APPEND]  "技术融合剖析：Chunked Prefill如何借助FlashAttention/FlashInfer实现
 *             混合批次推理" (lpnh.cn), section 4.2: the append translates each
 *             new token through the block table and writes it into its page.
 *
 * Conventions shared by every entry point
 *   - All tensors are dense and row-major in the layouts given below; pointers
 *     marked "device" are HIP device pointers, the rest are host values.
 *   - The caller allocates and owns every buffer, the workspace included.  The
 *     library keeps no pointer after a call returns, allocates no device
 *     memory, and never synchronises: work is enqueued on `stream` (a
 *     hipStream_t; NULL = the default stream) and the call returns at once.
 *   - Calls from several host threads may run at once (each with its own
 *     workspace): the per-device attribute cache behind the launches is
 *     written through atomics, and the two-stream baseline creates its stream
 *     under a per-device lock.
 *   - No exception crosses the ABI.  Host-checkable argument problems are
 *     reported before anything is enqueued.  HA_ERR_HIP reports a failed
 *     launch (hipGetLastError after the launch).
 *   - Device-resident metadata is trusted for performance but never able to
 *     make a kernel read or write outside the buffers: segments that break a
 *     precondition (Lq > Lk, Lk > max_seqlen_k, Lq > max_seqlen_q, more pages
 *     than max_blocks_per_seq, cu_seqlens_q not non-decreasing or past
 *     total_q) are skipped and their output rows are left unwritten; block ids
 *     outside [0, num_blocks) read as zero rows; slots outside the pool are
 *     skipped by the append.
 *   - Supported: dtype F32 or BF16 (output = input dtype, fp32 -> bf16 by
 *     round-to-nearest-even), head_dim 64 or 128, page_size 16,
 *     num_heads % num_kv_heads == 0 (query head h reads KV head
 *     h / (num_heads / num_kv_heads)).
 */
#ifndef HYBRID_ATTN_H
#define HYBRID_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HA_OK = 0,
  HA_ERR_INVALID_ARGUMENT = 1, /* null pointer, non-positive size, bad head ratio, ... */
  HA_ERR_UNSUPPORTED = 2,      /* dtype, head_dim or page_size outside the supported set */
  HA_ERR_WORKSPACE_TOO_SMALL = 3,
  HA_ERR_HIP = 4 /* a HIP runtime call or kernel launch failed */
} ha_status;

typedef enum { HA_DTYPE_F32 = 0, HA_DTYPE_BF16 = 1 } ha_dtype;

/* Human-readable name of a status code (static storage, never NULL). */
const char* ha_status_string(ha_status status);

/*
 * paged_kv_append -- write this step's new keys/values into the paged pools
 * [ORDER][APPEND].  Call it BEFORE hybrid_attn_fwd for the same step, on the
 * same stream, so that seqlens_k can include the new tokens.
 *
 *   key, value    device [total_tokens, num_kv_heads, head_dim], dtype
 *   slot_mapping  device int32 [total_tokens]; token t goes to page
 *                 slot / page_size, offset slot % page_size.  A negative slot
 *                 skips the token (padding).  Slots must be distinct; two
 *                 tokens naming one slot leave either token's row there.
 *   k_cache, v_cache  device [num_blocks, page_size, num_kv_heads, head_dim]
 *
 * The copy is bit-exact; no other byte of either pool is written.
 * Returns HA_ERR_INVALID_ARGUMENT for null pointers or non-positive sizes
 * (total_tokens == 0 is a valid no-op), HA_ERR_UNSUPPORTED for other dtypes,
 * head_dim or page_size.
 */
ha_status paged_kv_append(const void* key, const void* value, const int32_t* slot_mapping,
                          void* k_cache, void* v_cache, int32_t total_tokens,
                          int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                          int32_t num_blocks, ha_dtype dtype, void* stream);

/*
 * hybrid_attn_workspace_size -- bytes of device workspace hybrid_attn_fwd
 * needs for a step with these bounds (plan arrays, work counters, split-KV
 * partial results of decode rows and of long chunk tiles).  Depends only on
 * host-known bounds; returns 0
 * for num_seqs < 1, total_q < 0, max_seqlen_k < 0, num_heads < 1 or head_dim < 1.
 */
size_t hybrid_attn_workspace_size(int32_t num_seqs, int32_t total_q, int32_t max_seqlen_k,
                                  int32_t num_heads, int32_t head_dim);

/*
 * hybrid_attn_fwd -- one fused varlen paged attention forward for a mixed
 * step, causal with right alignment [VARLEN][PAGED].
 *
 * For segment b with Lq = cu_seqlens_q[b+1] - cu_seqlens_q[b] and
 * Lk = seqlens_k[b] (history plus this step's new tokens), query row i
 * (packed row r = cu_seqlens_q[b] + i) of head h sees the keys at positions
 * 0 .. (Lk - Lq) + i of its own segment, and
 *   out[r, h, :] = sum_j softmax_j(sm_scale * <q[r, h, :], K_j>) * V_j
 * where K_j / V_j are read from page block_table[b][j / page_size], offset
 * j % page_size, KV head h / (num_heads / num_kv_heads).
 *
 *   q             device [total_q, num_heads, head_dim], dtype
 *   k_cache, v_cache  device [num_blocks, page_size, num_kv_heads, head_dim]
 *   cu_seqlens_q  device int32 [num_seqs + 1], cu_seqlens_q[0] = 0, non-decreasing,
 *                 cu_seqlens_q[num_seqs] = total_q
 *   seqlens_k     device int32 [num_seqs], 0 <= Lq_b <= Lk_b <= max_seqlen_k
 *   block_table   device int32 [num_seqs, max_blocks_per_seq]; the first
 *                 ceil(Lk_b / page_size) entries of row b are physical block
 *                 ids in [0, num_blocks); later entries are never read
 *   out           device [total_q, num_heads, head_dim], dtype; rows of
 *                 segments with Lq = 0 do not exist, every other row is written
 *   max_seqlen_q, max_seqlen_k  host upper bounds of Lq_b and Lk_b
 *   sm_scale      softmax scale (1/sqrt(head_dim) on the pages); values <= 0
 *                 select 1/sqrt(head_dim)
 *   workspace     device, at least hybrid_attn_workspace_size(...) bytes,
 *                 256-byte aligned; its content on entry does not matter.  It
 *                 is in use until the enqueued work finishes: calls that share
 *                 a workspace must be ordered (e.g. on one stream).
 *
 * Errors: HA_ERR_INVALID_ARGUMENT (null pointers, num_seqs < 1, total_q < 0,
 * num_heads % num_kv_heads != 0, max_seqlen_q > max_seqlen_k, non-positive
 * sizes), HA_ERR_UNSUPPORTED (dtype, head_dim, page_size),
 * HA_ERR_WORKSPACE_TOO_SMALL, HA_ERR_HIP.
 */
ha_status hybrid_attn_fwd(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                          const int32_t* block_table, void* out, int32_t num_seqs,
                          int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                          int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t page_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                          float sm_scale, ha_dtype dtype, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * hybrid_step_fwd -- one whole mixed step: paged_kv_append of this step's new
 * keys and values, then hybrid_attn_fwd, in the order the wangyu.me page
 * gives for vLLM (section "输入组装": the new K/V are written through
 * slot_mapping before the varlen paged attention reads the history).
 *
 * key, value    [total_q, num_kv_heads, head_dim], dtype -- the new tokens are
 *               this step's query rows, in the same packed order
 * slot_mapping  [total_q] int32, device: slot page * 16 + offset of each new
 *               token (negative: padding, skipped)
 * q, k_cache, v_cache, metadata, out, workspace: as for hybrid_attn_fwd; the
 * pools are written (the appended slots) and then read.
 *
 * Result: byte for byte what paged_kv_append followed by hybrid_attn_fwd on
 * the same stream produce (pools and out).  For steps of at most 64 segments
 * whose K/V rows are at least 128 16-byte chunks (num_kv_heads * head_dim *
 * element size >= 2 KB), the append and the planner share one launch, which
 * saves the planner's own launch; otherwise the kernels of the two calls run
 * in sequence.  Errors: those of both calls (HA_ERR_INVALID_ARGUMENT also for
 * null key, value or slot_mapping when total_q > 0); nothing is launched on
 * an error.
 */
ha_status hybrid_step_fwd(const void* key, const void* value, const int32_t* slot_mapping,
                          const void* q, void* k_cache, void* v_cache,
                          const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                          const int32_t* block_table, void* out, int32_t num_seqs,
                          int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                          int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t page_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                          float sm_scale, ha_dtype dtype, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * hybrid_step_fwd_noalloc -- hybrid_step_fwd without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine); its
 * workspace is a 64 MiB array in the library's device code, one copy per GPU,
 * held from the library's load until the process ends.  The first call on a
 * device looks up that array's address (hipGetSymbolAddress) with the device
 * current.
 *
 * Arguments, result and errors: those of hybrid_step_fwd, minus workspace and
 * workspace_bytes.  Steps whose workspace (hybrid_attn_workspace_size) fits in
 * 64 MiB get byte for byte the output of hybrid_step_fwd; for bigger steps the
 * split-KV partial-result capacities shrink to fit, the planner picks coarser
 * splits, and the output stays within the same tolerance of the exact result.
 * HA_ERR_WORKSPACE_TOO_SMALL: the per-segment plan arrays alone exceed the
 * array (more than about four million segments).
 *
 * The array keeps the last call's contents; every call rewrites what it reads
 * (plan, counters, partials), so contents on entry do not matter.  All calls
 * on one GPU share the array: calls that overlap in time on that GPU (two
 * streams, or two host threads whose streams are not ordered) race on it and
 * must be serialised by the caller, e.g. by issuing them on one stream.
 */
ha_status hybrid_step_fwd_noalloc(const void* key, const void* value, const int32_t* slot_mapping,
                                  const void* q, void* k_cache, void* v_cache,
                                  const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                                  const int32_t* block_table, void* out, int32_t num_seqs,
                                  int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                  int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t page_size, int32_t num_blocks,
                                  int32_t max_blocks_per_seq, float sm_scale, ha_dtype dtype,
                                  void* stream);

/*
 * hybrid_attn_fwd_two_launch -- the same computation as hybrid_attn_fwd, but
 * with the chunk (prefill) role and the decode role in two separate kernel
 * launches instead of one fused launch: the "separate prefill and decode
 * kernels" alternative the kwkr.cn hybrid-attention article argues against
 * (section on the hybrid batch).  It exists as a comparison baseline; results
 * are bitwise equal to hybrid_attn_fwd for the same inputs and workspace size,
 * except for bf16 steps of a single segment with at least one (256-row tile,
 * head) pair per compute unit: hybrid_attn_fwd runs those through a kernel
 * of their own (no decode work to share the GPU with), whose rounding differs
 * within the stated tolerance.
 *
 *   two_streams = 0  chunk launch, then decode launch, on `stream`
 *   two_streams != 0 the chunk launch runs on a second stream the library
 *                    creates on first use on each device (default priority),
 *                    concurrently with the decode launch on `stream`; each
 *                    launch gets half of the resident workgroups; `stream`
 *                    waits for both before the merge.  The library keeps
 *                    that stream and two events until the process ends.
 *
 * Other arguments, ownership and errors as for hybrid_attn_fwd.
 */
ha_status hybrid_attn_fwd_two_launch(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                                     const int32_t* block_table, void* out, int32_t num_seqs,
                                     int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                     int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t page_size, int32_t num_blocks,
                                     int32_t max_blocks_per_seq, float sm_scale, ha_dtype dtype,
                                     void* workspace, size_t workspace_bytes,
                                     int32_t two_streams, void* stream);

/*
 * varlen_attn_fwd -- the same right-aligned causal attention over K/V packed
 * contiguously per segment, the flash_attn_varlen_func contract the wangyu.me
 * page describes (section on the varlen interface): segment b's keys and
 * values are rows cu_seqlens_k[b] .. cu_seqlens_k[b+1] - 1 of k and v, so
 * Lk_b = cu_seqlens_k[b+1] - cu_seqlens_k[b]; query rows as for
 * hybrid_attn_fwd (right-aligned: row i sees keys 0 .. Lk_b - Lq_b + i).
 *
 *   k, v          device [total_k, num_kv_heads, head_dim], dtype
 *   cu_seqlens_k  device int32 [num_seqs + 1], non-decreasing, last <= total_k
 *   workspace     at least hybrid_attn_workspace_size(num_seqs, total_q,
 *                 max_seqlen_k, num_heads, head_dim) bytes, 256-byte aligned
 * Other arguments as for hybrid_attn_fwd (no block table, no page size).
 * Segments whose key rows fall outside [0, total_k) or that break the other
 * preconditions are skipped (rows untouched).  Same plan and arithmetic as
 * hybrid_attn_fwd: for the same keys the outputs are byte-identical.
 * Errors: as for hybrid_attn_fwd; HA_ERR_INVALID_ARGUMENT also for a null
 * cu_seqlens_k or total_k < 0.
 */
ha_status varlen_attn_fwd(const void* q, const void* k, const void* v,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* out,
                          int32_t num_seqs, int32_t total_q, int32_t total_k,
                          int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t num_heads,
                          int32_t num_kv_heads, int32_t head_dim, float sm_scale, ha_dtype dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HYBRID_ATTN_H */
