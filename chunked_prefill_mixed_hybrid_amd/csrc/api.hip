// C ABI of libhybridattn.so (declared in include/hybrid_attn.h): host-side
// argument checks, workspace sizing, then the launches on the caller's stream.
#include <mutex>

#include "hybrid_attn.h"
#include "ha_common.hpp"
#include "ha_internal.hpp"

namespace {

bool supported_shape(int head_dim, int page_size, ha_dtype dtype) {
  return (head_dim == 64 || head_dim == 128) && page_size == ha::kPage &&
         (dtype == HA_DTYPE_F32 || dtype == HA_DTYPE_BF16);
}

}  // namespace

extern "C" {

ha_status paged_kv_append(const void* key, const void* value, const int32_t* slot_mapping,
                          void* k_cache, void* v_cache, int32_t total_tokens,
                          int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                          int32_t num_blocks, ha_dtype dtype, void* stream) {
  if (total_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || page_size <= 0 ||
      num_blocks <= 0)
    return HA_ERR_INVALID_ARGUMENT;
  if (!supported_shape(head_dim, page_size, dtype)) return HA_ERR_UNSUPPORTED;
  if (!k_cache || !v_cache) return HA_ERR_INVALID_ARGUMENT;
  if (total_tokens == 0) return HA_OK;
  if (!key || !value || !slot_mapping) return HA_ERR_INVALID_ARGUMENT;
  if (static_cast<long long>(num_blocks) * page_size > 0x7fffffffLL) return HA_ERR_INVALID_ARGUMENT;
  hipError_t e = ha::launch_kv_append(key, value, slot_mapping, k_cache, v_cache, total_tokens,
                                      num_kv_heads, head_dim, num_blocks,
                                      dtype == HA_DTYPE_F32 ? 0 : 1,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? HA_OK : HA_ERR_HIP;
}

size_t hybrid_attn_workspace_size(int32_t num_seqs, int32_t total_q, int32_t max_seqlen_k,
                                  int32_t num_heads, int32_t head_dim) {
  if (num_seqs < 1 || total_q < 0 || max_seqlen_k < 0 || num_heads < 1 || head_dim < 1) return 0;
  return ha::ws_layout(num_seqs, total_q, max_seqlen_k, num_heads, head_dim).total;
}

}  // extern "C"

namespace {

// Host checks shared by the attention entry points (everything but the
// workspace pointer); on HA_OK, L holds the call's arguments and the layout
// `ws`.  Touches no GPU state.
ha_status prepare_launch(ha::AttnLaunch& L, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                         const int32_t* block_table, const int32_t* cu_seqlens_k,
                         int32_t total_k, void* out, int32_t num_seqs,
                         int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                         int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t page_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                         float sm_scale, ha_dtype dtype, void* stream, int launch_mode) {
  if (num_seqs < 1 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || num_heads < 1 ||
      num_kv_heads < 1 || head_dim < 1 || page_size < 1 || num_blocks < 1 ||
      max_blocks_per_seq < 1)
    return HA_ERR_INVALID_ARGUMENT;
  if (num_heads % num_kv_heads != 0 || max_seqlen_q > max_seqlen_k ||
      max_seqlen_k > ha::kMaxSeqlenK)
    return HA_ERR_INVALID_ARGUMENT;
  if (static_cast<long long>(num_blocks) * page_size > 0x7fffffffLL) return HA_ERR_INVALID_ARGUMENT;
  if (!supported_shape(head_dim, page_size, dtype)) return HA_ERR_UNSUPPORTED;
  if (!cu_seqlens_q || !k_cache || !v_cache) return HA_ERR_INVALID_ARGUMENT;
  if (cu_seqlens_k ? total_k < 0 : (!seqlens_k || !block_table)) return HA_ERR_INVALID_ARGUMENT;
  if (total_q > 0 && (!q || !out)) return HA_ERR_INVALID_ARGUMENT;

  L.q = q;
  L.k_cache = k_cache;
  L.v_cache = v_cache;
  L.cu_seqlens_q = cu_seqlens_q;
  L.seqlens_k = seqlens_k;
  L.block_table = block_table;
  L.cu_seqlens_k = cu_seqlens_k;
  L.total_k = total_k;
  L.out = out;
  L.num_seqs = num_seqs;
  L.total_q = total_q;
  L.max_seqlen_q = max_seqlen_q;
  L.max_seqlen_k = max_seqlen_k;
  L.num_heads = num_heads;
  L.num_kv_heads = num_kv_heads;
  L.head_dim = head_dim;
  L.num_blocks = num_blocks;
  L.max_blocks = max_blocks_per_seq;
  L.sm_scale = sm_scale > 0.f ? sm_scale : 1.0f / sqrtf(static_cast<float>(head_dim));
  L.dtype = dtype == HA_DTYPE_F32 ? 0 : 1;
  L.launch_mode = launch_mode;
  L.ws = ha::ws_layout(num_seqs, total_q, max_seqlen_k, num_heads, head_dim);
  L.stream = static_cast<hipStream_t>(stream);
  return HA_OK;
}

// The attention entry points with a caller-owned workspace: checks, then the
// launches (hybrid_step_fwd: the append first).
ha_status attention_launch(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                           const int32_t* block_table, const int32_t* cu_seqlens_k,
                           int32_t total_k, void* out, int32_t num_seqs,
                           int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                           int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t page_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                           float sm_scale, ha_dtype dtype, void* workspace,
                           size_t workspace_bytes, void* stream, int launch_mode,
                           const void* append_key = nullptr, const void* append_value = nullptr,
                           const int32_t* slot_mapping = nullptr) {
  ha::AttnLaunch L;
  const ha_status st = prepare_launch(L, q, k_cache, v_cache, cu_seqlens_q, seqlens_k, block_table,
                                      cu_seqlens_k, total_k, out, num_seqs, total_q, max_seqlen_q,
                                      max_seqlen_k, num_heads, num_kv_heads, head_dim, page_size,
                                      num_blocks, max_blocks_per_seq, sm_scale, dtype, stream,
                                      launch_mode);
  if (st != HA_OK) return st;
  if (!workspace || reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return HA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < L.ws.total) return HA_ERR_WORKSPACE_TOO_SMALL;
  if (total_q == 0) return HA_OK;
  L.workspace = static_cast<unsigned char*>(workspace);
  L.append_key = append_key;
  L.append_value = append_value;
  L.slot_mapping = slot_mapping;
  return ha::launch_attention(L) == hipSuccess ? HA_OK : HA_ERR_HIP;
}

// Scratch memory of hybrid_step_fwd_noalloc: one copy per GPU the library runs
// on, held until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device array: the device address comes from
// hipGetSymbolAddress, once per device with that device current, and only
// that address reaches kernels.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_lock;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(g_scratch_lock);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

ha_status hybrid_step_fwd_noalloc(const void* key, const void* value, const int32_t* slot_mapping,
                                  const void* q, void* k_cache, void* v_cache,
                                  const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                                  const int32_t* block_table, void* out, int32_t num_seqs,
                                  int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                  int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t page_size, int32_t num_blocks,
                                  int32_t max_blocks_per_seq, float sm_scale, ha_dtype dtype,
                                  void* stream) {
  if (total_q > 0 && (!key || !value || !slot_mapping)) return HA_ERR_INVALID_ARGUMENT;
  ha::AttnLaunch L;
  const ha_status st = prepare_launch(L, q, k_cache, v_cache, cu_seqlens_q, seqlens_k, block_table,
                                      nullptr, 0, out, num_seqs, total_q, max_seqlen_q,
                                      max_seqlen_k, num_heads, num_kv_heads, head_dim, page_size,
                                      num_blocks, max_blocks_per_seq, sm_scale, dtype, stream,
                                      ha::kLaunchFused);
  if (st != HA_OK) return st;
  // the workspace arrays within the scratch array: partial-slot capacities
  // shrink to fit; only a step whose per-segment arrays alone exceed it fails
  L.ws = ha::ws_layout_within(num_seqs, total_q, max_seqlen_k, num_heads, head_dim, kScratchBytes);
  if (L.ws.total > kScratchBytes) return HA_ERR_WORKSPACE_TOO_SMALL;
  if (total_q == 0) return HA_OK;
  void* buf = nullptr;
  if (scratch_address(&buf) != hipSuccess) return HA_ERR_HIP;
  L.workspace = static_cast<unsigned char*>(buf);
  L.append_key = key;
  L.append_value = value;
  L.slot_mapping = slot_mapping;
  return ha::launch_attention(L) == hipSuccess ? HA_OK : HA_ERR_HIP;
}

ha_status hybrid_attn_fwd(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                          const int32_t* block_table, void* out, int32_t num_seqs,
                          int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                          int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t page_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                          float sm_scale, ha_dtype dtype, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return attention_launch(q, k_cache, v_cache, cu_seqlens_q, seqlens_k, block_table, nullptr, 0,
                          out, num_seqs, total_q, max_seqlen_q, max_seqlen_k, num_heads,
                          num_kv_heads, head_dim, page_size, num_blocks, max_blocks_per_seq,
                          sm_scale, dtype, workspace, workspace_bytes, stream, ha::kLaunchFused);
}

ha_status hybrid_step_fwd(const void* key, const void* value, const int32_t* slot_mapping,
                          const void* q, void* k_cache, void* v_cache,
                          const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                          const int32_t* block_table, void* out, int32_t num_seqs,
                          int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                          int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t page_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                          float sm_scale, ha_dtype dtype, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (total_q > 0 && (!key || !value || !slot_mapping)) return HA_ERR_INVALID_ARGUMENT;
  return attention_launch(q, k_cache, v_cache, cu_seqlens_q, seqlens_k, block_table, nullptr, 0,
                          out, num_seqs, total_q, max_seqlen_q, max_seqlen_k, num_heads,
                          num_kv_heads, head_dim, page_size, num_blocks, max_blocks_per_seq,
                          sm_scale, dtype, workspace, workspace_bytes, stream, ha::kLaunchFused,
                          key, value, slot_mapping);
}

ha_status hybrid_attn_fwd_two_launch(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                                     const int32_t* block_table, void* out, int32_t num_seqs,
                                     int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                     int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t page_size, int32_t num_blocks,
                                     int32_t max_blocks_per_seq, float sm_scale, ha_dtype dtype,
                                     void* workspace, size_t workspace_bytes,
                                     int32_t two_streams, void* stream) {
  return attention_launch(q, k_cache, v_cache, cu_seqlens_q, seqlens_k, block_table, nullptr, 0,
                          out, num_seqs, total_q, max_seqlen_q, max_seqlen_k, num_heads,
                          num_kv_heads, head_dim, page_size, num_blocks, max_blocks_per_seq,
                          sm_scale, dtype, workspace, workspace_bytes, stream,
                          two_streams ? ha::kLaunchTwoStreams : ha::kLaunchSerial);
}

ha_status varlen_attn_fwd(const void* q, const void* k, const void* v,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* out,
                          int32_t num_seqs, int32_t total_q, int32_t total_k,
                          int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t num_heads,
                          int32_t num_kv_heads, int32_t head_dim, float sm_scale, ha_dtype dtype,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!cu_seqlens_k) return HA_ERR_INVALID_ARGUMENT;
  // the paged kernels read a packed buffer as pages of 16 rows starting at each
  // segment's first row (identity block table)
  const int32_t pages = max_seqlen_k > 0 ? (max_seqlen_k + ha::kPage - 1) / ha::kPage : 1;
  return attention_launch(q, k, v, cu_seqlens_q, nullptr, nullptr, cu_seqlens_k, total_k, out,
                          num_seqs, total_q, max_seqlen_q, max_seqlen_k, num_heads, num_kv_heads,
                          head_dim, ha::kPage, 1, pages, sm_scale, dtype, workspace,
                          workspace_bytes, stream, ha::kLaunchFused);
}

}  // extern "C"
