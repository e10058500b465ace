// Host/device contract between the C-ABI layer (api.hip) and the kernel files
// (kv_append.hip, attention.hip): workspace layout, tuning constants and the
// launcher entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ha_common.hpp"

namespace ha {

// ---- tuning constants (gfx950) ---------------------------------------------------
constexpr int kThreads = 256;       // 4 waves per workgroup for every kernel role
constexpr int kChunkRows = 128;     // query rows per chunk tile (32 per wave)
constexpr int kSplitMinLog2 = 8;
constexpr int kSplitMin = 1 << kSplitMinLog2;  // smallest decode KV split, in keys
constexpr int kSplitCandidates = 23;  // decode split sizes kSplitMin << k, k < 23 (up to 2^30)
constexpr int kPartsMax = 16384;    // cap on (segment, split) partial slots
constexpr int kItemsPerSlot = 16;   // decode splits aimed at per resident workgroup (tail pieces not counted)
constexpr int kHeadsPerDecodeItem = 4;  // bf16: one head per 16-lane row of every wave; fp32: one per wave
constexpr int kMaxSeqlenK = 1 << 30;
// Decode tail: when the decode split is at least 2^kTailMinLog2 keys, each
// segment's last split is cut into pieces of split / 2^kTailLog2 keys that are
// queued after every full split, so the queue ends with short items instead
// of full ones (fewer workgroups idle while the last items finish).
constexpr int kTailMinLog2 = 11;
constexpr int kTailLog2 = 2;
// Decode items of at least this many keys claim their successor only when they
// are done (in the instance with deferred claims), as chunk items do.
constexpr int kLateClaimKeys = 1 << kTailMinLog2;
// Full splits and tail pieces of a decode segment of lk keys at split 2^sh.
__host__ __device__ inline void decode_pieces(long long lk, int sh, long long& full, long long& tail) {
  const long long n = (lk + (1LL << sh) - 1) >> sh;
  if (sh >= kTailMinLog2 && n >= 1) {
    full = n - 1;
    const long long piece = 1LL << (sh - kTailLog2);
    tail = (lk - (full << sh) + piece - 1) >> (sh - kTailLog2);
  } else {
    full = n;
    tail = 0;
  }
}
// Chunk tiles are split along the keys only when a few long tiles would
// otherwise outlast the rest of the step: at most this many (tile, head, split)
// items in all (kChunkSplitItems; the one-wave planner counts only non-empty
// ranges against it), each range at least kChunkSplitMinKeys keys long, with
// partial slots for up to kChunkSlotItems (tile, head, range) triples.
constexpr int kChunkSplitItems = 512;
constexpr int kChunkSlotItems = 1024;
constexpr int kChunkSplitMinKeys = 512;
// Length of each of the nsplit key ranges of a split chunk segment of lk keys:
// equal ranges rounded up to 64 keys, so every range boundary other than a
// tile's end falls on a 64-key step (keys past a range end are never loaded and
// never need a mask).
__host__ __device__ inline int chunk_range_keys(int lk, int nsplit) {
  return ((lk + nsplit - 1) / nsplit + 63) & ~63;
}

// ---- workspace ---------------------------------------------------------------------
// [header 256 B][tile_prefix (B+1)][dec_prefix (B+1)][part_prefix (B+1)][seqlens (B+1)]
// [tail_prefix (B+1)]
// [partials parts_cap x H x (D + 4) fp32]
// [chunk_partials chunk_slots_cap x H x 128 x (D + 4) fp32]; every array starts
// on a 256-byte boundary.
// Chunk tiles are queued in kXcdGroups groups: the tiles of query head h go to
// group h % kXcdGroups, and workgroup b prefers group b % kXcdGroups.  Work-
// groups are dispatched to the 8 XCDs of an MI355X round robin, so the query
// tiles of one head run side by side on one XCD and re-read its KV history
// from that XCD's L2 instead of HBM.
constexpr int kXcdGroups = 8;
__host__ __device__ inline int chunk_group_heads(int num_heads, int x) {
  return num_heads / kXcdGroups + (x < num_heads % kXcdGroups ? 1 : 0);
}
// Chunk items in group x when each of the `pairs` (query tile, key range)
// pairs of a head is one item.  gsub == 1: the group holds every pair of heads
// x, x + 8, ...  gsub > 1 (fp32 steps with fewer heads than groups): head
// x % H deals its pairs over gsub groups, pair t going to group
// (t % gsub) * H + head, so that every group has work.
__host__ __device__ inline int chunk_group_items(int num_heads, int gsub, int pairs, int x) {
  if (gsub <= 1) return chunk_group_heads(num_heads, x) * pairs;
  if (x >= num_heads * gsub) return 0;
  const int sub = x / num_heads;
  return (pairs - sub + gsub - 1) / gsub;
}
// Workgroups b < n with b % kXcdGroups == x (the ones whose first items come
// from queue group x, the group of their own XCD).
__host__ __device__ constexpr int wgs_in_group(int n, int x) {
  return n > x ? (n - x + kXcdGroups - 1) / kXcdGroups : 0;
}
// Static first chunk items of a fused launch of `grid` workgroups: chunk-first
// workgroup b < half takes rank b / kXcdGroups of group b % kXcdGroups; with
// `spare`, a decode-first workgroup b >= half + n_dec (n_dec: decode items,
// at most grid - half) has no decode item and takes the next rank of its group.
__host__ __device__ inline int spare_chunk_rank(int b, int half, int n_dec) {
  const int x = b % kXcdGroups;
  return wgs_in_group(half, x) + b / kXcdGroups - wgs_in_group(half + n_dec, x);
}
// Ranks 0 .. this - 1 of group x are handed out statically (before the cap by
// the group's items): the group's counter starts there.
__host__ __device__ inline int static_chunk_ranks(int half, int n_dec, int grid, bool spare, int x) {
  const int n = wgs_in_group(half, x);
  return spare ? n + wgs_in_group(grid, x) - wgs_in_group(half + n_dec, x) : n;
}
// Sub-groups per head for a step of num_heads heads (see chunk_group_items).
__host__ __device__ inline int chunk_group_sub(bool fp32, int num_heads) {
  return (fp32 && num_heads < kXcdGroups) ? kXcdGroups / num_heads : 1;
}

struct PlanHeader {
  uint32_t chunk_counter[kXcdGroups];  // next chunk item of each group (set by the planner)
  uint32_t dec_counter;   // next decode item (set by the planner each call)
  int32_t n_chunk_tiles;  // query tiles (per head) over all chunk segments
  int32_t n_dec_items;    // decode (segment, split or tail piece, 4-head group) items
  int32_t n_dec_full;     // of which full splits (queued first; the tail pieces follow)
  int32_t split;          // decode split size in keys (multiple of 64)
  int32_t n_parts;        // partial slots in use
  int32_t bad_segments;   // segments skipped because they broke a precondition
  int32_t chunk_split;    // KV splits per chunk tile (1: tiles are not split)
  int32_t chunk_gsub;     // queue groups per head (chunk_group_items)
  int32_t pad[47];
};
static_assert(sizeof(PlanHeader) == 256, "header is 256 bytes");

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct WsLayout {
  size_t tile_prefix, dec_prefix, part_prefix, seqlens, tail_prefix, partials, chunk_partials, total;
  int parts_cap;
  int part_stride;      // floats per (part, head) or (chunk slot, head, row): m, l, 2 pad, acc[D]
  int tiles_cap;        // bound on query tiles over all chunk segments
  int chunk_slots_cap;  // (tile, split) partial slots available to split chunk tiles
};

inline int parts_cap_for(int num_seqs, int max_seqlen_k) {
  long long per_seq = (static_cast<long long>(max_seqlen_k) + kSplitMin - 1) / kSplitMin;
  long long cap = static_cast<long long>(num_seqs) * per_seq;
  return static_cast<int>(cap < kPartsMax ? cap : kPartsMax);
}

// Query tiles of all chunk segments: a chunk segment has Lq >= 2 rows, so there
// are at most total_q / 2 of them and sum(ceil(Lq / 128)) <= total_q / 128 + #chunks.
inline int tiles_cap_for(int num_seqs, int total_q) {
  const long long chunks = num_seqs < total_q / 2 ? num_seqs : total_q / 2;
  return static_cast<int>(total_q / kChunkRows + chunks);
}

inline int chunk_slots_cap_for(int num_seqs, int total_q, int max_seqlen_k, int num_heads) {
  const long long by_items = kChunkSlotItems / num_heads;
  const long long max_split = (static_cast<long long>(max_seqlen_k) + kChunkSplitMinKeys - 1) /
                              kChunkSplitMinKeys;
  const long long by_shape = static_cast<long long>(tiles_cap_for(num_seqs, total_q)) * max_split;
  const long long cap = by_items < by_shape ? by_items : by_shape;
  return static_cast<int>(cap < 2 ? 0 : cap);
}

inline WsLayout ws_layout(int num_seqs, int total_q, int max_seqlen_k, int num_heads, int head_dim) {
  WsLayout l;
  size_t off = sizeof(PlanHeader);
  size_t arr = align256(sizeof(int32_t) * (static_cast<size_t>(num_seqs) + 1));
  l.tile_prefix = off; off += arr;
  l.dec_prefix = off; off += arr;
  l.part_prefix = off; off += arr;
  l.seqlens = off; off += arr;  // Lk per segment, derived by the planner for contiguous K/V
  l.tail_prefix = off; off += arr;  // decode tail pieces (x head groups) per segment
  l.parts_cap = parts_cap_for(num_seqs, max_seqlen_k);
  l.part_stride = head_dim + 4;
  l.partials = off;
  off += align256(sizeof(float) * static_cast<size_t>(l.parts_cap) * num_heads * l.part_stride);
  l.tiles_cap = tiles_cap_for(num_seqs, total_q);
  l.chunk_slots_cap = chunk_slots_cap_for(num_seqs, total_q, max_seqlen_k, num_heads);
  l.chunk_partials = off;
  off += align256(sizeof(float) * static_cast<size_t>(l.chunk_slots_cap) * num_heads * kChunkRows *
                  l.part_stride);
  l.total = off;
  return l;
}

// The same layout within max_bytes: the partial-slot capacities shrink until
// the arrays fit -- decode partials first to at most half of the room left
// after the fixed arrays, then chunk-tile partials to what remains (none when
// fewer than 2 slots fit), then decode partials to the rest.  The planner
// adapts: it picks decode splits whose partial slots fit parts_cap (the
// largest split needs none) and splits chunk tiles only into slots that exist.
// total > max_bytes only when the fixed arrays alone do not fit.
inline WsLayout ws_layout_within(int num_seqs, int total_q, int max_seqlen_k, int num_heads,
                                 int head_dim, size_t max_bytes) {
  WsLayout l = ws_layout(num_seqs, total_q, max_seqlen_k, num_heads, head_dim);
  if (l.total <= max_bytes || l.partials > max_bytes) return l;
  const size_t part_bytes = sizeof(float) * static_cast<size_t>(num_heads) * l.part_stride;
  const size_t slot_bytes = part_bytes * kChunkRows;
  if (max_bytes - l.partials < 512) return l;
  const size_t room = max_bytes - l.partials - 512;  // the two arrays' alignment pads kept aside
  size_t parts = room / 2 / part_bytes;
  if (parts > static_cast<size_t>(l.parts_cap)) parts = l.parts_cap;
  size_t slots = (room - parts * part_bytes) / slot_bytes;
  if (slots > static_cast<size_t>(l.chunk_slots_cap)) slots = l.chunk_slots_cap;
  if (slots < 2) slots = 0;
  parts = (room - slots * slot_bytes) / part_bytes;
  if (parts > static_cast<size_t>(l.parts_cap)) parts = l.parts_cap;
  l.parts_cap = static_cast<int>(parts);
  l.chunk_slots_cap = static_cast<int>(slots);
  l.chunk_partials = l.partials + align256(parts * part_bytes);
  l.total = l.chunk_partials + align256(slots * slot_bytes);
  return l;
}

// ---- launchers ---------------------------------------------------------------------
// How the chunk role and the decode role are launched: one fused persistent
// kernel (the product path), or -- as a comparison baseline -- two launches,
// one per role, back to back on the caller's stream or concurrently on two
// streams with half of the resident workgroups each.
constexpr int kLaunchFused = 0, kLaunchSerial = 1, kLaunchTwoStreams = 2;
struct AttnLaunch {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* cu_seqlens_q;
  const int32_t* seqlens_k;    // paged K/V
  const int32_t* block_table;  // paged K/V
  const int32_t* cu_seqlens_k; // contiguous K/V (then seqlens_k and block_table are unused)
  int total_k;                 // contiguous K/V: rows of k and v
  void* out;
  int num_seqs, total_q, max_seqlen_q, max_seqlen_k;
  int num_heads, num_kv_heads, head_dim, num_blocks, max_blocks;
  float sm_scale;
  int dtype;  // 0 = f32, 1 = bf16
  int launch_mode;  // kLaunchFused, kLaunchSerial or kLaunchTwoStreams
  unsigned char* workspace;
  WsLayout ws;
  hipStream_t stream;
  // hybrid_step_fwd: this step's new keys and values go into the pools first
  // (key / value [total_q, Hkv, D], slot_mapping [total_q]); null for the
  // attention-only entry points
  const void* append_key = nullptr;
  const void* append_value = nullptr;
  const int32_t* slot_mapping = nullptr;
};

// One token row of the append: the row's K and V (chunks_per_row 16-byte
// chunks each) go to slot slot_mapping[t]; a padding token (slot < 0) or a
// slot outside the pool is skipped.  append_row: called by one workgroup per
// token; append_chunk: one thread per 16-byte chunk (short rows).
struct AppendRows {
  const uint4* key;
  const uint4* value;
  const int32_t* slot_mapping;
  uint4* k_cache;
  uint4* v_cache;
  int chunks_per_row;
  long long pool_slots;
  int total_tokens;
};
__device__ __forceinline__ void append_chunk(const AppendRows& a, long long idx) {
  if (idx >= static_cast<long long>(a.total_tokens) * a.chunks_per_row) return;
  const int t = static_cast<int>(idx / a.chunks_per_row);
  const int c = static_cast<int>(idx - static_cast<long long>(t) * a.chunks_per_row);
  const int slot = a.slot_mapping[t];
  if (slot < 0 || slot >= a.pool_slots) return;  // padding token or slot outside the pool
  const size_t dst = static_cast<size_t>(slot) * a.chunks_per_row + c;
  const uint4 kv = a.key[idx];
  const uint4 vv = a.value[idx];
  a.k_cache[dst] = kv;
  a.v_cache[dst] = vv;
}
// Each thread loads up to kAppendBatch chunks of K and of V before it stores
// any: the pools may alias the new rows as far as the compiler knows, so
// loads are never moved above earlier stores by themselves.
constexpr int kAppendBatch = 4;
__device__ __forceinline__ void append_row(const AppendRows& a, int t) {
  const int slot = __builtin_amdgcn_readfirstlane(a.slot_mapping[t]);
  if (slot < 0 || slot >= a.pool_slots) return;
  const size_t src = static_cast<size_t>(t) * a.chunks_per_row;
  const size_t dst = static_cast<size_t>(slot) * a.chunks_per_row;
  const u32x4_t* key = reinterpret_cast<const u32x4_t*>(a.key);
  const u32x4_t* value = reinterpret_cast<const u32x4_t*>(a.value);
  u32x4_t* kc = reinterpret_cast<u32x4_t*>(a.k_cache);
  u32x4_t* vc = reinterpret_cast<u32x4_t*>(a.v_cache);
  for (int c0 = 0; c0 < a.chunks_per_row; c0 += kAppendBatch * kThreads) {
    u32x4_t kv[kAppendBatch], vv[kAppendBatch];
#pragma unroll
    for (int u = 0; u < kAppendBatch; ++u) {  // past the row end: a chunk of the row, not stored
      const int c = min(c0 + u * kThreads + static_cast<int>(threadIdx.x), a.chunks_per_row - 1);
      kv[u] = key[src + c];
      vv[u] = value[src + c];
    }
#pragma unroll
    for (int u = 0; u < kAppendBatch; ++u) {
      const int c = c0 + u * kThreads + static_cast<int>(threadIdx.x);
      if (c < a.chunks_per_row) {
        kc[dst + c] = kv[u];
        vc[dst + c] = vv[u];
      }
    }
  }
}

hipError_t launch_kv_append(const void* key, const void* value, const int32_t* slot_mapping,
                            void* k_cache, void* v_cache, int total_tokens, int num_kv_heads,
                            int head_dim, int num_blocks, int dtype, hipStream_t stream);

hipError_t launch_attention(const AttnLaunch& a);

}  // namespace ha
