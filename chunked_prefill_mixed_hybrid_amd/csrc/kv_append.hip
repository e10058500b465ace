// paged_kv_append: copy each new token's K and V rows into the page slot its
// slot_mapping entry names.  A token row of one pool is [Hkv, D] contiguous
// both in key/value [T, Hkv, D] and in the cache [NB, P, Hkv, D] (slot s starts
// at element s * Hkv * D), so the append is a gather-free scatter of
// contiguous rows, done with 16-byte vector loads and stores.
// Sources: wangyu.me Chunked Prefill page, section "输入组装" (slot_mapping
// write before attention); lpnh.cn FlashInfer article, section 4.2 (append
// through the page table).  Slots are distinct by precondition, so no atomics.
#include "ha_common.hpp"
#include "ha_internal.hpp"

namespace ha {

// Short rows: one thread moves one 16-byte chunk of K and the same chunk of V.
// grid.x * blockDim.x >= total_tokens * chunks_per_row (checked by the launcher).
__global__ __launch_bounds__(kThreads) void kv_append_kernel(AppendRows a) {
  append_chunk(a, static_cast<long long>(blockIdx.x) * kThreads + threadIdx.x);
}

// Rows of at least half a workgroup of chunks (e.g. 32 heads x 128 bf16 = 512):
// one workgroup per token, whose slot is a single scalar load, and each thread
// moves chunks c, c + 256, ... of that row.
__global__ __launch_bounds__(kThreads) void kv_append_rows_kernel(AppendRows a) {
  append_row(a, blockIdx.x);
}

hipError_t launch_kv_append(const void* key, const void* value, const int32_t* slot_mapping,
                            void* k_cache, void* v_cache, int total_tokens, int num_kv_heads,
                            int head_dim, int num_blocks, int dtype, hipStream_t stream) {
  const int elem_bytes = dtype == 0 ? 4 : 2;
  const long long row_bytes = static_cast<long long>(num_kv_heads) * head_dim * elem_bytes;
  const int chunks_per_row = static_cast<int>(row_bytes / 16);  // head_dim * elem_bytes % 16 == 0
  const long long total = static_cast<long long>(total_tokens) * chunks_per_row;
  if (total == 0) return hipSuccess;
  const long long pool_slots = static_cast<long long>(num_blocks) * kPage;
  const AppendRows rows{static_cast<const uint4*>(key), static_cast<const uint4*>(value),
                        slot_mapping, static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache),
                        chunks_per_row, pool_slots, total_tokens};
  if (chunks_per_row >= kThreads / 2) {
    hipLaunchKernelGGL(kv_append_rows_kernel, dim3(static_cast<unsigned>(total_tokens)),
                       dim3(kThreads), 0, stream, rows);
    return hipGetLastError();
  }
  const long long blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_append_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     stream, rows);
  return hipGetLastError();
}

}  // namespace ha
