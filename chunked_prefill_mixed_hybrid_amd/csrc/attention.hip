// hybrid_attn_fwd kernels for gfx950: planner, one fused persistent attention
// kernel that serves both roles of a mixed chunked-prefill step, and the
// split-KV combine.
//
// What is computed (wangyu.me "大语言模型推理优化（二）：Chunked Prefill",
// section "Flash Attention 的 varlen 接口"): packed query segment b
// (rows cu[b] .. cu[b+1]) attends only to its own Lk = seqlens_k[b] keys; the
// query segment is right-aligned to the end of the key segment, so row i sees
// keys 0 .. (Lk - Lq) + i.  Keys and values of position j live in page
// block_table[b][j / 16], offset j % 16 (kwkr.cn Triton article, kernel
// section), and softmax uses scale 1/sqrt(D) with online (running max / running
// sum) accumulation in fp32 (same article).
//
// How it runs on CDNA4:
//   * plan_kernel (one workgroup) classifies segments -- Lq == 1 is decode,
//     Lq > 1 is a prefill chunk (the pages: decode and prefill are the same
//     computation with different query lengths) -- picks the decode KV split
//     size and writes exclusive prefix sums of work items per segment.
//   * attn_kernel is persistent: every workgroup repeatedly takes the next work
//     item from a device counter.  Chunk tiles come first (long, MFMA bound),
//     decode splits fill in behind them (short, HBM bound), so both kinds share
//     the CUs in one launch -- the fused single kernel the kwkr.cn article
//     argues for (section on the hybrid batch), with no host synchronisation.
//       - chunk role: 128 query rows x one head; 4 waves x 32 rows; K and V
//         tiles of 64 keys staged in LDS; S^T = K Q^T and O^T += V^T P^T on
//         32x32 MFMA (bf16 inputs, fp32 accumulate); the mask is evaluated only
//         on tiles that cross the causal diagonal.
//       - decode role (bf16): 4 heads of one (segment, KV split); each 16-lane
//         row of a wave owns one head, so a 16-byte load instruction reads one
//         key row of the 4 heads, and the 4 waves take a quarter of the keys
//         each, streamed 16 keys per step with non-temporal loads; 16-lane
//         butterfly reduce-scatter of the partial dot products, fp32 (m, l, acc)
//         per lane, merged across the waves through LDS.  (fp32: one head per
//         wave.)  Splits of a segment write partial (m, l, acc) rows that
//         combine_kernel merges.
#include <atomic>
#include <mutex>

#include "ha_common.hpp"
#include "ha_internal.hpp"

namespace ha {

// ==================================================================== plan
struct PlanArgs {
  const int32_t* cu;
  const int32_t* sk;
  int num_seqs, total_q, max_q, max_k, max_blocks, num_heads, head_groups, parts_cap,
      target_items, grid, tiles_cap, chunk_slots_cap;
  // workgroups that start on the chunk queues / on the decode queue (their first
  // items are assigned statically, so the counters start past them)
  int chunk_first_wgs, dec_first_wgs;
  int split_items;  // most chunk items splitting may create
  // rough cost of one 64-key step of a chunk tile, in units of one decode
  // (key, head) pair: decides whether long chunk tiles are split along the keys
  int chunk_step_cost;
  // contiguous K/V: segment b's keys are rows cu_k[b] .. cu_k[b+1] of a buffer of
  // total_k rows; the planner writes Lk_b into sk_out for the other kernels
  const int32_t* cu_k;
  int total_k;
  int32_t* sk_out;
  PlanHeader* hdr;
  int32_t* tile_prefix;
  int32_t* dec_prefix;
  int32_t* part_prefix;
  int32_t* tail_prefix;
  int chunk_gsub;  // queue groups per head (chunk_group_items)
  // decode-first workgroups left without a decode item take their first chunk
  // item statically as well (fused fp32 launches, see attn_kernel)
  int spare_chunk;
};

constexpr int kPlanThreads = 1024;

// Segment shape and whether it meets the documented preconditions; segments
// that do not are skipped (no work items, output rows untouched).
__device__ __forceinline__ bool plan_segment(const PlanArgs& a, int b, int& lq, int& lk) {
  const int c0 = a.cu[b], c1 = a.cu[b + 1];
  lq = c1 - c0;
  bool rows_ok = true;
  if (a.cu_k) {
    const int k0 = a.cu_k[b], k1 = a.cu_k[b + 1];
    lk = k1 - k0;
    rows_ok = k0 >= 0 && k1 <= a.total_k;
  } else {
    lk = a.sk[b];
  }
  return rows_ok && c0 >= 0 && c1 >= c0 && c1 <= a.total_q && lq <= lk && lk <= a.max_k &&
         lq <= a.max_q && ((lk + kPage - 1) / kPage) <= a.max_blocks;
}

// Chunk tiles are split along the keys when the longest one alone would outlast
// an even share of the whole step's work; then every chunk tile is cut into S
// ranges, within the item, slot and minimum-length limits.
__device__ int chunk_split_count(const PlanArgs& a, long long csteps, long long dkeys,
                                 long long n_ct, long long steps_max, bool cap_items = true) {
  int S = 1;
  if (n_ct > 0 && n_ct <= a.tiles_cap && a.chunk_slots_cap >= 2) {
    const double work = (static_cast<double>(csteps) * a.chunk_step_cost +
                         static_cast<double>(dkeys)) * a.num_heads;
    const double share = work / a.grid;
    const double longest = static_cast<double>(steps_max) * a.chunk_step_cost;
    if (longest > share) {
      long long want = static_cast<long long>(ceil(longest / share));
      if (cap_items) {  // every (tile, range) pair counted as an item
        want = min(want, static_cast<long long>(a.split_items) / (n_ct * a.num_heads));
        want = min(want, static_cast<long long>(kChunkSplitItems) / (n_ct * a.num_heads));
      }
      want = min(want, static_cast<long long>(a.chunk_slots_cap) / n_ct);
      want = min(want, steps_max * 64 / kChunkSplitMinKeys);
      S = static_cast<int>(max(want, 1LL));
    }
  }
  return S;
}

// Header fields and queue counters once the totals are known: the attention
// kernel hands out the first item of every workgroup statically (chunk-first
// workgroup b takes item b / 8 of chunk group b % 8, decode-first workgroup b
// takes decode item b - chunk_first_wgs); the counters start past those items.
__device__ void write_plan_header(const PlanArgs& a, int chunk_pairs, int dec_full, int parts,
                                  int dec_tail, int split, int csplit, int bad) {
  const int dec_items = dec_full + dec_tail;
  a.tile_prefix[a.num_seqs] = chunk_pairs;
  a.dec_prefix[a.num_seqs] = dec_full;
  a.part_prefix[a.num_seqs] = parts;
  a.tail_prefix[a.num_seqs] = dec_tail;
  a.hdr->n_chunk_tiles = chunk_pairs;
  a.hdr->n_dec_items = dec_items;
  a.hdr->n_dec_full = dec_full;
  a.hdr->n_parts = parts;
  a.hdr->split = split;
  a.hdr->chunk_split = csplit;
  a.hdr->chunk_gsub = a.chunk_gsub;
  a.hdr->bad_segments = bad;
  const int cw = a.chunk_first_wgs;
  const int dec_static = min(dec_items, a.dec_first_wgs);
  for (int x = 0; x < kXcdGroups; ++x) {
    const int items = chunk_group_items(a.num_heads, a.chunk_gsub, chunk_pairs, x);
    const int first = static_chunk_ranks(cw, dec_static, a.grid, a.spare_chunk != 0, x);
    a.hdr->chunk_counter[x] = static_cast<uint32_t>(min(items, first));
  }
  a.hdr->dec_counter = static_cast<uint32_t>(min(dec_items, a.dec_first_wgs));
}

// Planner for steps of at most one wave of segments: lane b owns segment b;
// every total, the split choice and the prefix sums are wave operations, with
// no barrier.  Same results as plan_kernel.
constexpr int kPlanSmallSegments = kWave;

__device__ __forceinline__ void plan_small(const PlanArgs& a) {  // the 64 lanes of one wave
  const int b = threadIdx.x & (kWave - 1);
  int lq = -1, lk = 0;
  if (b < a.num_seqs) {
    int q, k;
    if (plan_segment(a, b, q, k)) {
      lq = q;
      lk = k;
    }
  }
  const bool bad = b < a.num_seqs && lq < 0;
  // decode split: the smallest candidate whose whole splits stay within the
  // item target and whose partial slots (tail pieces counted) fit
  int pick = kSplitCandidates - 1;
  for (int k = 0; k < kSplitCandidates; ++k) {
    const int sh = kSplitMinLog2 + k;
    long long full = 0, tail = 0;
    if (lq == 1) decode_pieces(lk, sh, full, tail);
    long long items = lq == 1 ? (lk + (1LL << sh) - 1) >> sh : 0, parts = full + tail > 1 ? full + tail : 0;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      items += __shfl_xor(items, m);
      parts += __shfl_xor(parts, m);
    }
    if (parts <= a.parts_cap && items * a.head_groups <= static_cast<long long>(a.target_items)) {
      pick = k;
      break;
    }
  }
  // chunk work estimate (as in plan_kernel)
  long long csteps = 0, dkeys = lq == 1 ? lk : 0, ctiles = 0, cmax = 0;
  if (lq >= 2) {
    const long long nt = (lq + kChunkRows - 1) / kChunkRows;
    const long long h0_steps = (static_cast<long long>(lk - lq) + 63) >> 6;
    const long long last = (static_cast<long long>(lk) + 63) >> 6;
    csteps = (nt - 1) * h0_steps + (nt - 1) * nt + last;
    ctiles = nt;
    cmax = last;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    csteps += __shfl_xor(csteps, m);
    dkeys += __shfl_xor(dkeys, m);
    ctiles += __shfl_xor(ctiles, m);
    cmax = max(cmax, __shfl_xor(cmax, m));
  }
  // chunk split: the largest count whose non-empty (tile, range) items fit the
  // item limits; ranges of a segment are of equal length (chunk_key_range), so
  // tiles with fewer keys have fewer non-empty ranges
  int csplit = chunk_split_count(a, csteps, dkeys, ctiles, cmax, false);
  while (csplit > 1) {
    long long n = 0;
    if (lq >= 2) {
      // sum over tiles of ceil(kend / ck): the full tiles' ends step by 128,
      // so the quotient is carried along instead of divided out per tile
      const int ck = chunk_range_keys(lk, csplit);
      const int full = (lq - 1) / kChunkRows;  // tiles before the last
      int q = (lk - lq + kChunkRows + ck - 1) / ck, rr = (lk - lq + kChunkRows + ck - 1) - q * ck;
      for (int t = 0; t < full; ++t) {
        n += q;
        rr += kChunkRows;
        while (rr >= ck) {
          rr -= ck;
          ++q;
        }
      }
      n += (lk + ck - 1) / ck;  // the last tile ends at lk
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) n += __shfl_xor(n, m);
    if (n * a.num_heads <= min(static_cast<long long>(a.split_items), static_cast<long long>(kChunkSplitItems)))
      break;
    --csplit;
  }
  const int split_log = kSplitMinLog2 + pick;
  const int split = 1 << split_log;
  // exclusive prefix sums over the lanes: chunk (tile, range) pairs, decode
  // full-split items, partial slots, decode tail-piece items
  int v[4] = {0, 0, 0, 0};
  if (b < a.num_seqs) {
    if (a.sk_out) a.sk_out[b] = lq < 0 ? 0 : lk;
    if (lq >= 2) {
      v[0] = (lq + kChunkRows - 1) / kChunkRows * csplit;
    } else if (lq == 1) {
      long long full, tail;
      decode_pieces(lk, split_log, full, tail);
      v[1] = static_cast<int>(full) * a.head_groups;
      v[2] = full + tail > 1 ? static_cast<int>(full + tail) : 0;
      v[3] = static_cast<int>(tail) * a.head_groups;
    }
  }
  int incl[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int o = __shfl_up(incl[c], off);
      if (b >= off) incl[c] += o;
    }
  }
  if (b < a.num_seqs) {
    a.tile_prefix[b] = incl[0] - v[0];
    a.dec_prefix[b] = incl[1] - v[1];
    a.part_prefix[b] = incl[2] - v[2];
    a.tail_prefix[b] = incl[3] - v[3];
  }
  const int tot0 = __shfl(incl[0], kWave - 1), tot1 = __shfl(incl[1], kWave - 1);
  const int tot2 = __shfl(incl[2], kWave - 1), tot3 = __shfl(incl[3], kWave - 1);
  const int nbad = __popcll(__ballot(bad));
  if (b == 0) write_plan_header(a, tot0, tot1, tot2, tot3, split, csplit, nbad);
}

__global__ __launch_bounds__(kWave) void plan_kernel_small(PlanArgs a) { plan_small(a); }

// A step's append and the small planner in one launch (hybrid_step_fwd):
// workgroup 0 plans with its first wave while the other workgroups copy the
// new token rows into the pools (one workgroup per token for rows of at least
// half a workgroup of 16-byte chunks, else one thread per chunk), so the
// planner's latency hides behind the copy instead of running as a launch of
// its own between the append and the attention.  The planner reads only
// metadata, none of the pools.
__global__ __launch_bounds__(kThreads) void append_plan_kernel(PlanArgs pa, AppendRows rows) {
  if (blockIdx.x == 0) {
    if (threadIdx.x < kWave) plan_small(pa);
    return;
  }
  if (rows.chunks_per_row >= kThreads / 2)
    append_row(rows, static_cast<int>(blockIdx.x) - 1);
  else
    append_chunk(rows, static_cast<long long>(blockIdx.x - 1) * kThreads + threadIdx.x);
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ int s_lq[kPlanThreads], s_lk[kPlanThreads];  // shapes of the first segments; lq -1: skipped
  __shared__ long long s_items[32][32];
  __shared__ long long s_parts[32][32];
  __shared__ long long s_cstat[32][4];  // per group: chunk steps, decode keys, chunk tiles, max steps
  __shared__ int s_split_log, s_csplit;
  __shared__ int s_wave_tot[kPlanThreads / kWave][4];
  __shared__ int s_carry[4];
  __shared__ int s_pass_tot[4];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const bool cached = a.num_seqs <= kPlanThreads;

  // 0. every thread reads the shape of segment tid once
  int my_lq = -1, my_lk = 0;
  if (tid < a.num_seqs) {
    int lq, lk;
    if (plan_segment(a, tid, lq, lk)) {
      my_lq = lq;
      my_lk = lk;
    }
  }
  s_lq[tid] = my_lq;
  s_lk[tid] = my_lk;
  if (tid == 0) s_bad = 0;
  __syncthreads();

  // 1. decode work and partial-slot counts for every candidate split size
  // (power-of-two sizes, so the divisions are shifts); the candidate-0 lanes
  // also total the work estimate used for chunk splits.  Tile t of a chunk
  // with history H0 covers keys [0, min(Lk, H0 + 128 (t + 1))), so every tile
  // but the last takes ceil(H0 / 64) + 2 (t + 1) steps of 64 keys.
  {
    const int k = tid & 31, grp = tid >> 5;
    long long items = 0, parts = 0, csteps = 0, dkeys = 0, ctiles = 0, cmax = 0;
    if (k < kSplitCandidates) {
      const int sh = kSplitMinLog2 + k;
      for (int b = grp; b < a.num_seqs; b += 32) {
        int lq, lk;
        if (cached) {
          lq = s_lq[b];
          lk = s_lk[b];
        } else if (!plan_segment(a, b, lq, lk)) {
          lq = -1;
        }
        if (lq == 1) {
          long long full, tail;
          decode_pieces(lk, sh, full, tail);
          items += (lk + (1LL << sh) - 1) >> sh;  // whole splits: the item target ignores tail pieces
          parts += full + tail > 1 ? full + tail : 0;
          dkeys += lk;
        } else if (lq >= 2) {
          const long long nt = (lq + kChunkRows - 1) / kChunkRows;
          const long long h0_steps = (static_cast<long long>(lk - lq) + 63) >> 6;
          const long long last = (static_cast<long long>(lk) + 63) >> 6;
          csteps += (nt - 1) * h0_steps + (nt - 1) * nt + last;
          ctiles += nt;
          cmax = max(cmax, last);
        }
      }
    }
    s_items[grp][k] = items;
    s_parts[grp][k] = parts;
    if (k == 0) {
      s_cstat[grp][0] = csteps;
      s_cstat[grp][1] = dkeys;
      s_cstat[grp][2] = ctiles;
      s_cstat[grp][3] = cmax;
    }
  }
  __syncthreads();
  // Wave 0 totals the groups: lanes 0..31 one candidate each, lanes 32..35 the
  // chunk statistics; the split is the smallest candidate that fits the
  // partial slots and keeps the decode whole-split count near the target (the largest
  // candidate, 2^30 keys, always fits).
  if (tid < kWave) {
    long long items = 0, parts = 0, stat = 0;
    if (tid < 32) {
      for (int g = 0; g < 32; ++g) {
        items += s_items[g][tid];
        parts += s_parts[g][tid];
      }
    } else if (tid < 36) {
      const int c = tid - 32;
      for (int g = 0; g < 32; ++g) stat = c == 3 ? max(stat, s_cstat[g][c]) : stat + s_cstat[g][c];
    }
    const bool fits = tid < kSplitCandidates && parts <= a.parts_cap &&
                      items * a.head_groups <= static_cast<long long>(a.target_items);
    const unsigned long long fit_mask = __ballot(fits);
    const long long csteps = __shfl(stat, 32), dkeys = __shfl(stat, 33);
    const long long n_ct = __shfl(stat, 34), steps_max = __shfl(stat, 35);
    if (tid == 0) {
      s_split_log = fit_mask ? __ffsll(static_cast<long long>(fit_mask)) - 1 : kSplitCandidates - 1;
      for (int c = 0; c < 4; ++c) s_carry[c] = 0;
      s_csplit = chunk_split_count(a, csteps, dkeys, n_ct, steps_max);
    }
  }
  __syncthreads();
  const int split_log = kSplitMinLog2 + s_split_log;
  const int split = 1 << split_log;
  const int csplit = s_csplit;

  // 2. exclusive prefix sums of chunk tiles, decode full-split items, partial
  // slots and decode tail-piece items.
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  for (int base = 0; base < a.num_seqs; base += kPlanThreads) {
    const int b = base + tid;
    int v[4] = {0, 0, 0, 0};
    if (b < a.num_seqs) {
      int lq = my_lq, lk = my_lk;
      if (base > 0 && !plan_segment(a, b, lq, lk)) lq = -1;
      if (a.sk_out) a.sk_out[b] = lq < 0 ? 0 : lk;
      if (lq < 0) {
        atomicAdd(&s_bad, 1);
      } else if (lq >= 2) {
        v[0] = (lq + kChunkRows - 1) / kChunkRows * csplit;  // (query tile, split) pairs per head
      } else if (lq == 1) {
        long long full, tail;
        decode_pieces(lk, split_log, full, tail);
        v[1] = static_cast<int>(full) * a.head_groups;
        v[2] = full + tail > 1 ? static_cast<int>(full + tail) : 0;
        v[3] = static_cast<int>(tail) * a.head_groups;
      }
    }
    int incl[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int o = __shfl_up(incl[c], off);
        if (lane >= off) incl[c] += o;
      }
    }
    if (lane == kWave - 1)
      for (int c = 0; c < 4; ++c) s_wave_tot[wave][c] = incl[c];
    __syncthreads();
    if (tid < 4) {
      int run = 0;
      for (int w = 0; w < kPlanThreads / kWave; ++w) {
        const int t = s_wave_tot[w][tid];
        s_wave_tot[w][tid] = run;  // exclusive offset of wave w within this pass
        run += t;
      }
      s_pass_tot[tid] = run;
    }
    __syncthreads();
    if (b < a.num_seqs) {
      a.tile_prefix[b] = s_carry[0] + s_wave_tot[wave][0] + incl[0] - v[0];
      a.dec_prefix[b] = s_carry[1] + s_wave_tot[wave][1] + incl[1] - v[1];
      a.part_prefix[b] = s_carry[2] + s_wave_tot[wave][2] + incl[2] - v[2];
      a.tail_prefix[b] = s_carry[3] + s_wave_tot[wave][3] + incl[3] - v[3];
    }
    __syncthreads();
    if (tid < 4) s_carry[tid] += s_pass_tot[tid];
    __syncthreads();
  }
  if (tid == 0)
    write_plan_header(a, s_carry[0], s_carry[1], s_carry[2], s_carry[3], split, csplit, s_bad);
}

// ==================================================================== attention
struct MainArgs {
  const void* q;
  const void* kc;
  const void* vc;
  void* out;
  const int32_t* cu;
  const int32_t* sk;
  const int32_t* bt;
  int num_seqs, num_heads, num_kv_heads, group, num_blocks, max_blocks, part_stride;
  float scale_log2;  // sm_scale * log2(e): softmax runs in base 2
  PlanHeader* hdr;
  const int32_t* tile_prefix;
  const int32_t* dec_prefix;
  const int32_t* part_prefix;
  const int32_t* tail_prefix;
  float* partials;
  float* chunk_partials;  // [slot][head][128 rows][part_stride] of split chunk tiles
  const int32_t* cu_k;  // contiguous K/V: first row of each segment's keys (else null)
  int roles;      // bit 0: this launch runs chunk items, bit 1: decode items
  int chunk_wgs;  // workgroups of this launch that prefer the chunk queues (the first ones)
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// Lanes l and l ^ 32 combined with one VALU lane swap (v_permlane32_swap)
// instead of an LDS permute, whose result would wait behind every LDS read
// issued before it.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Position of the largest entry of the non-decreasing prefix[0..n] that is
// <= x, i.e. the segment owning item x.
__device__ __forceinline__ int find_segment(const int32_t* prefix, int n, int x) {
  int lo = 0, hi = n;  // invariant: prefix[lo] <= x < prefix[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// Row of the A operand that wave lane (l % 32) loads so that, in the MFMA
// accumulator, the 8 values a lane holds for u = v / 8 are 8 CONSECUTIVE keys
// 16u + 8 * (l / 32) + (v % 8): then P^T feeds the P.V MFMA straight from
// registers and V^T is read from LDS with one 16-byte load per MFMA.
__device__ __forceinline__ int key_perm(int r) {
  return ((r >> 4) << 4) | (((r >> 2) & 1) << 3) | (((r >> 3) & 1) << 2) | (r & 3);
}

// Where the keys of a segment live.  Paged: key j is in page
// block_table[seg][j / 16] of the pool.  Contiguous (varlen_attn_fwd): the
// segment's keys are rows cu_k[seg] .. of a packed [total_k, Hkv, D] buffer;
// a run of 16 keys then starts at row cu_k[seg] + 16 * (j / 16).  A "page"
// below is a block id (paged) or that first row (contiguous), -1 for none, and
// page_base turns it into the address of the run's first key, so both layouts
// share every role's code.
template <bool kContig>
__device__ __forceinline__ int segment_page(const_i32_t* btrow, int row0, int idx, int last_page,
                                            int num_blocks) {
  if constexpr (kContig) {
    return idx <= last_page ? row0 + idx * kPage : -1;
  } else {
    const int id = btrow[min(idx, last_page)];  // scalar load, always inside the row
    return (idx <= last_page && static_cast<unsigned>(id) < static_cast<unsigned>(num_blocks)) ? id : -1;
  }
}
template <bool kContig>
__device__ __forceinline__ unsigned char* page_base(const void* pool, int page, uint32_t slot_bytes,
                                                    uint32_t page_bytes) {
  unsigned char* p = const_cast<unsigned char*>(static_cast<const unsigned char*>(pool));
  return p + static_cast<size_t>(page < 0 ? 0 : page) * (kContig ? slot_bytes : page_bytes);
}
template <bool kContig>
__device__ __forceinline__ int segment_row0(const MainArgs& a, int seg) {
  if constexpr (kContig) return a.cu_k[seg];
  else return 0;
}

// s_waitcnt operand (gfx9 encoding) that waits for every outstanding vector
// memory load and nothing else: vmcnt 0, expcnt 7, lgkmcnt 15.
constexpr int kWaitVmcnt0 = 0x0F70;
// ... and the one that waits until at most n vector memory loads are
// outstanding (vmcnt is split: bits 3:0 and 15:14)
constexpr int wait_vmcnt(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
// ... and the one that waits for LDS (and scalar memory) operations only:
// vmcnt 63, expcnt 7, lgkmcnt 0
constexpr int kWaitLgkmcnt0 = 0xC07F;

constexpr uint32_t kBf16PairOne = 0x3f803f80u;  // (1.0, 1.0) as a bf16 pair

template <typename T> struct ChunkCfg;
// bf16: a stage holds a 64-key step of K and of V, both key-major (rows of 2D
// bytes, no padding).  Two stages, each a __shared__ array of its own (the
// kernel's `smem` is the first): as distinct objects the compiler can tell
// that reads of one stage do not alias the loads streaming into the other, and
// puts no wait for those loads in front of them.
template <> struct ChunkCfg<bf16_t> {
  template <int D> struct Sizes {
    static constexpr int BN = 64;
    static constexpr int ROW = D * 2;                    // bytes per key row
    static constexpr int POOL = BN * ROW;                // one pool's step
    static constexpr int STAGE = 2 * POOL;               // K, then V
    static constexpr int BYTES = STAGE;                  // the first stage
  };
};
template <> struct ChunkCfg<float> {
  template <int D> struct Sizes {
    static constexpr int BN = D == 128 ? 32 : 64;  // 4 keys x 4 channels staged per thread
    static constexpr int ROWF = D + 4;             // floats per key row of the K tile
    static constexpr int STAGE = (BN * ROWF + D * BN) * 4;  // K natural + V^T
    static constexpr int BYTES = 2 * STAGE;        // double buffered
  };
};
// 16-byte chunk swizzle of row d of the fp32 V^T tile (rows of NCH chunks of 4
// keys): the transposed writes (rows 4c + i, c over the lanes) and the MFMA
// operand reads (consecutive rows) both land on distinct bank groups.
template <int NCH>
__device__ __forceinline__ int vt_swz_f32(int d) { return (d ^ (d >> 2)) & (NCH - 1); }

// ---------------------------------------------------------------- chunk KV splits
// Keys [kb0, kb1) of range `split` out of `nsplit` of a chunk tile whose keys
// are [0, kend) in a segment of lk keys: the segment's ranges cut at the
// tile's end, so the late ranges of tiles with fewer keys are empty.
__device__ __forceinline__ void chunk_key_range(int lk, int kend, int split, int nsplit, int& kb0, int& kb1) {
  if (nsplit == 1) {
    kb0 = 0;
    kb1 = kend;
    return;
  }
  const int ck = chunk_range_keys(lk, nsplit);
  kb0 = min(split * ck, kend);
  kb1 = min(kb0 + ck, kend);
}

// A split chunk tile: each (tile, head, key range) item leaves fp32 rows
// (m in log2 units, l, acc[D]) in its slot of chunk_partials; combine_kernel
// merges the ranges of every row after the attention launch.
template <int D>
__device__ __forceinline__ void chunk_store_partial(const MainArgs& a, int seg, int h, int tile,
                                                    int split, int nsplit, float m_log2, float l_tot,
                                                    const f32x16_t (&acc)[D / 32]) {
  constexpr int NM = D / 32;
  const int lane = threadIdx.x & 63, w = wave_id(), qc = lane & 31, g = lane >> 5;
  const int slot = a.tile_prefix[seg] + tile * nsplit + split;
  float* pp = a.chunk_partials +
              ((static_cast<size_t>(slot) * a.num_heads + h) * kChunkRows + w * 32 + qc) * a.part_stride;
  if (g == 0) *reinterpret_cast<float2*>(pp) = float2{m_log2, l_tot};
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4)
      *reinterpret_cast<f32x4_t*>(pp + 4 + m * 32 + i4 * 8 + g * 4) =
          f32x4_t{acc[m][4 * i4], acc[m][4 * i4 + 1], acc[m][4 * i4 + 2], acc[m][4 * i4 + 3]};
}

// ---------------------------------------------------------------- chunk role, bf16
// LDS layout of a stage (row R = key of the 64-key step, 2D bytes per row):
// the 16-byte chunks of a row are stored at swizzled positions, chunk c of
// row R at c ^ swz(R), with one swizzle for K and one for V, chosen so that the
// MFMA operand reads below hit distinct LDS banks:
//   K: 8 or 16 consecutive lanes read chunk c of the rows key_perm(0..15); at
//      D = 128 (256-byte rows, every row starting at bank 0) swz = R & 15; at
//      D = 64 (128-byte rows, odd rows on the other half of the banks) swz =
//      (R >> 1) & 7.
//   V: a transposing read (ds_read_b64_tr_b16) of one 16-lane group covers 4
//      consecutive rows and 2 adjacent chunks; swz shifts those rows' chunk
//      pairs apart: (R & 3) << 1 at D = 128, ((R >> 1) & 1) << 1 at D = 64.
template <int D> __device__ __forceinline__ int kswz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D> __device__ __forceinline__ int vswz(int r) {
  return D == 128 ? ((r & 3) << 1) : (((r >> 1) & 1) << 1);
}

// kSplit: the tile is one of nsplit key ranges (else nsplit == 1, split == 0);
// kContig: keys in a packed buffer instead of pages
//
// Data movement: each 64-key step of K and V goes from the pool straight into
// an LDS stage (buffer loads with the LDS bit: lane i of a wave instruction
// writes bytes 16 i .. 16 i + 15 of a 1 KB block, from whatever source offset
// the lane gives, so the swizzle is applied on the source side; lanes whose
// offset is out of range, or whose page descriptor is empty, write zeros).
// Wave w loads the step's keys 16 w .. 16 w + 15, one page.  Two stages: the
// next step's loads are issued as soon as the barrier closing the previous
// step has freed its stage, and waited for (vmcnt) before the barrier closing
// this step.  No registers hold staged data and no VALU work transposes V:
// the P.V operand V^T (32 channels x 8 keys per lane) is read with two
// transposing LDS reads per MFMA.
template <int D, bool kSplit, bool kContig, bool kQWait>
__device__ void chunk_tile_bf16(const MainArgs& a, int seg, int h, int tile, int split, int nsplit,
                                unsigned char* stage_a, unsigned char* stage_b) {
  if constexpr (!kSplit) {
    split = 0;
    nsplit = 1;
  }
  using Cfg = ChunkCfg<bf16_t>::Sizes<D>;
  constexpr int BN = Cfg::BN, NKB = BN / 32, KS = D / 16, NM = D / 32;
  constexpr int ROW = Cfg::ROW, POOL = Cfg::POOL;
  constexpr int CPR = D / 8;          // 16-byte chunks per key row
  constexpr int RPI = kWave / CPR;    // rows per wave load instruction (1 KB)
  constexpr int KPW = BN / 4;         // keys of a step each wave loads (one page)
  constexpr int IPW = KPW / RPI;      // load instructions per wave, per pool and step
  static_assert(KPW == kPage && KPW % RPI == 0, "each wave loads one page per step");

  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int qc = lane & 31, g = lane >> 5;
  const int q0 = a.cu[seg], Lq = a.cu[seg + 1] - q0, Lk = a.sk[seg], H0 = Lk - Lq;
  const int kvh = h / a.group;
  const int row0 = tile * kChunkRows;
  const int rows_end = min(row0 + kChunkRows, Lq);
  const int kend = H0 + rows_end;  // keys [0, kend) are visible to some row of the tile
  int kb0, kb1;                    // this item's keys
  chunk_key_range(Lk, kend, split, nsplit, kb0, kb1);
  const int wrow0 = row0 + w * 32;
  const int my_row = wrow0 + qc;
  const bool wave_active = wrow0 < rows_end;
  const int pi = key_perm(qc);

  // Q^T operand: lane supplies Q[my_row][s*16 + g*8 .. +8]
  u32x4_t qf[KS];
  {
    const bool ok = my_row < Lq;
    const bf16_t* qp = static_cast<const bf16_t*>(a.q) +
                       (static_cast<size_t>(q0 + (ok ? my_row : 0)) * a.num_heads + h) * D + g * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = ok ? ld16(qp + s * 16) : u32x4_t{0, 0, 0, 0};
  }
  // kQWait: wait for the Q loads here, once per tile, instead of at the first
  // MFMA of every key step (where the wait would also cover the step's loads)
  if constexpr (kQWait) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  f32x16_t acc[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) acc[m] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;

  const_i32_t* btrow = (const_i32_t*)(a.bt) + static_cast<size_t>(seg) * a.max_blocks;
  const int last_page = (max(kb1, 1) - 1) >> 4;
  const uint32_t slot_bytes = static_cast<uint32_t>(a.num_kv_heads) * D * 2;
  const uint32_t page_bytes = slot_bytes * kPage;
  const uint32_t head_off = static_cast<uint32_t>(kvh) * D * 2;
  const int krow0 = segment_row0<kContig>(a, seg);  // first key row (contiguous K/V)
  // A wave's page of the step at key k0: page index and the raw block-table
  // entry (scalar load).  The entry is checked only where it is used, a step
  // later, so the load's latency is not waited out right after issuing it.
  struct PageRef { int idx, raw; };
  auto page_ref = [&](int k0) -> PageRef {
    const int idx = (k0 >> 4) + w;
    if constexpr (kContig) return {idx, krow0 + idx * kPage};
    else return {idx, btrow[min(idx, last_page)]};  // always inside the row
  };
  auto page_id = [&](PageRef r) {  // -1 past the range or outside the pool
    if constexpr (kContig) return r.idx <= last_page ? r.raw : -1;
    else return (r.idx <= last_page && static_cast<unsigned>(r.raw) < static_cast<unsigned>(a.num_blocks)) ? r.raw : -1;
  };
  // this lane's part of every load: row (within its wave's page) and chunk
  const int lrow = lane / CPR, lpos = lane % CPR;
  // loads of the step at key k0 into stage st (past the range the descriptor
  // is empty and the loads write zeros)
  auto issue_step = [&](int k0, PageRef pr, unsigned char* st) {
    const int id = page_id(pr);
    const int range = id >= 0 ? static_cast<int>(page_bytes) : 0;
    const auto rk = __builtin_amdgcn_make_buffer_rsrc(page_base<kContig>(a.kc, id, slot_bytes, page_bytes), 0,
                                                      range, kRawBufferWord3);
    const auto rv = __builtin_amdgcn_make_buffer_rsrc(page_base<kContig>(a.vc, id, slot_bytes, page_bytes), 0,
                                                      range, kRawBufferWord3);
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int r = RPI * j + lrow;  // key within the page
      const int row = KPW * w + r;   // row within the step
      const bool in = k0 + row < kb1;
      const uint32_t base = static_cast<uint32_t>(r) * slot_bytes + head_off;
      const uint32_t ok_ = in ? base + static_cast<uint32_t>(lpos ^ kswz<D>(row)) * 16 : kOffsetOutOfRange;
      const uint32_t ov_ = in ? base + static_cast<uint32_t>(lpos ^ vswz<D>(row)) * 16 : kOffsetOutOfRange;
      unsigned char* dk = st + (KPW * w + RPI * j) * ROW;
      load_lds16(rk, dk, ok_);
      load_lds16(rv, dk + POOL, ov_);
    }
  };
  PageRef nref{0, -1};  // this wave's page of the next step to load
  if (kb0 < kb1) {
    issue_step(kb0, page_ref(kb0), stage_a);
    nref = page_ref(kb0 + BN);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  }
  // One step: the next step streams into the other stage while this one is
  // computed from `cur`.
  auto step = [&](int k0, const unsigned char* cur, unsigned char* nxt) {
    const unsigned char* Ks = cur;
    const unsigned char* Vs = cur + POOL;
    issue_step(k0 + BN, nref, nxt);
    if (wave_active && k0 <= H0 + wrow0 + 31) {  // else the step is invisible to this wave
      const bool need_mask = (k0 + BN - 1) > (H0 + wrow0);
      // S^T = K Q^T, the 32-key blocks interleaved so the matrix pipe never
      // waits on the previous accumulator of one chain
      f32x16_t sacc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sacc[kb] = f32x16_t{};
#pragma unroll
      for (int s = 0; s < KS; s += 2) {
        u32x4_t kf[NKB][2];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int r = kb * 32 + pi;
#pragma unroll
          for (int t = 0; t < 2; ++t) kf[kb][t] = ld16(Ks + r * ROW + (((s + t) * 2 + g) ^ kswz<D>(r)) * 16);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) sacc[kb] = mfma_bf16(kf[kb][t], qf[s + t], sacc[kb]);
      }
      // causal mask on diagonal steps, running max of the raw scores (the
      // positive scale preserves order), weights exp2(scale * (s - max))
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float x = sacc[kb][v];
          if (need_mask) {
            const int kp = k0 + kb * 32 + ((v >> 3) << 4) + (g << 3) + (v & 7);
            if (kp > H0 + my_row) x = -INFINITY;
          }
          sacc[kb][v] = x;
          tmax = fmaxf(tmax, x);
        }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float m_new = fmaxf(m_run, tmax);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2((m_run - m_use) * a.scale_log2);
      const float neg_m = -m_use * a.scale_log2;
      m_run = m_new;
      float psum = 0.f;
      u32x4_t pk[NKB][2];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const float p0 = fast_exp2(fmaf(sacc[kb][8 * u + 2 * e2], a.scale_log2, neg_m));
            const float p1 = fast_exp2(fmaf(sacc[kb][8 * u + 2 * e2 + 1], a.scale_log2, neg_m));
            const uint32_t w2 = pack_bf16x2(p0, p1);
            pk[kb][u][e2] = w2;
            psum = dot2_bf16(w2, kBf16PairOne, psum);  // the same rounded weights P.V uses
          }
        }
      }
      l_run = l_run * alpha + psum;
      if (__any(alpha != 1.f)) {  // no row max moved: the accumulators need no rescale
#pragma unroll
        for (int m = 0; m < NM; ++m) acc[m] *= alpha;
      }
      // O^T += V^T P^T for each 16-key slice: lane l of the A operand holds
      // channel 32 m + l % 32 for keys 8 (l / 32) .. + 7 of the slice, gathered
      // by two transposing reads (4 keys each): in the 16-lane group q = l / 16,
      // lane 4 x + y reads the 4 channels 32 m + 16 (q % 2) + 4 y .. + 3 of key
      // 8 (q / 2) + 4 r + x, and the read hands lane 4 a + b channel
      // 32 m + 16 (q % 2) + 4 a + b of those 4 keys.
      const int tq = lane >> 4, tc = lane & 15, tx = tc >> 2, ty = tc & 3;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          u32x4_t vf[NM];
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            const int d0 = 32 * m + 16 * (tq & 1) + 4 * ty;  // first channel this lane reads
#pragma unroll
            for (int r = 0; r < 2; ++r) {
              const int row = kb * 32 + 16 * u + 8 * (tq >> 1) + 4 * r + tx;
              const unsigned char* src =
                  Vs + row * ROW + (((d0 >> 3) ^ vswz<D>(row)) << 4) + ((d0 & 7) << 1);
              const u32x2_t t2 = lds_read_tr16(src);
              vf[m][2 * r] = t2[0];
              vf[m][2 * r + 1] = t2[1];
            }
          }
#pragma unroll
          for (int m = 0; m < NM; ++m) acc[m] = mfma_bf16(vf[m], pk[kb][u], acc[m]);
        }
      }
    }
    // the block-table entry of the step after next, loaded only now: scalar
    // loads share the LDS wait counter and complete out of order, so any LDS
    // wait of this step's compute would have waited for it as well
    __builtin_amdgcn_sched_barrier(0);
    nref = page_ref(k0 + 2 * BN);
    // this wave's loads of the next step have landed; after the barrier every
    // wave's have, and the stage just read is free for the step after
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  };
  // two steps per trip, so that each step's stages are fixed objects
  for (int k0 = kb0; k0 < kb1; k0 += 2 * BN) {
    step(k0, stage_a, stage_b);
    if (k0 + BN < kb1) step(k0 + BN, stage_b, stage_a);
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);  // lanes l and l^32 share a row
  const bool row_ok = wave_active && my_row < Lq;
  if (!row_ok) return;
  if constexpr (kSplit) {
    chunk_store_partial<D>(a, seg, h, tile, split, nsplit, m_run * a.scale_log2, l_tot, acc);
    return;
  }
  const float inv = 1.f / l_tot;
  bf16_t* op = static_cast<bf16_t*>(a.out) + (static_cast<size_t>(q0 + my_row) * a.num_heads + h) * D;
#pragma unroll
  for (int m = 0; m < NM; ++m) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = m * 32 + i4 * 8 + g * 4;
      st8(op + d, u32x2_t{pack_bf16x2(acc[m][4 * i4] * inv, acc[m][4 * i4 + 1] * inv),
                          pack_bf16x2(acc[m][4 * i4 + 2] * inv, acc[m][4 * i4 + 3] * inv)});
    }
  }
}

// ---------------------------------------------------------------- chunk role, fp32
// Same tile and online softmax as the bf16 role on v_mfma_f32_32x32x2f32.  The
// contraction of S^T = K Q^T pairs channel s (half-wave 0) with channel D/2 + s
// (half-wave 1) in MFMA step s, so a lane's K and Q operands are D/2
// consecutive floats, read 4 at a time.  V is staged transposed (V^T[d][key],
// swizzled 16-byte chunks of 4 keys) so that the P.V operand of 8 consecutive
// keys is two 16-byte reads.  Two LDS stages, one barrier per key step.
template <int D, bool kSplit, bool kContig>
__device__ void chunk_tile_f32(const MainArgs& a, int seg, int h, int tile, int split, int nsplit,
                               unsigned char* smem) {
  if constexpr (!kSplit) {
    split = 0;
    nsplit = 1;
  }
  using Cfg = ChunkCfg<float>::Sizes<D>;
  constexpr int BN = Cfg::BN, NKB = BN / 32, KS = D / 2, NM = D / 32, ROWF = Cfg::ROWF;
  constexpr int STAGE = Cfg::STAGE;
  constexpr int CPR = D / 4;   // 16-byte chunks per key row
  constexpr int NCH = BN / 4;  // 16-byte chunks per V^T row
  static_assert(BN * CPR == 4 * kThreads, "each thread stages 4 keys x 4 channels of a tile");
  static_assert((kWave / CPR) * 4 <= kPage, "a wave's tile loads stay inside one page");

  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int qc = lane & 31, g = lane >> 5;
  const int q0 = a.cu[seg], Lq = a.cu[seg + 1] - q0, Lk = a.sk[seg], H0 = Lk - Lq;
  const int kvh = h / a.group;
  const int row0 = tile * kChunkRows;
  const int rows_end = min(row0 + kChunkRows, Lq);
  const int kend = H0 + rows_end;
  int kb0, kb1;  // this item's keys
  chunk_key_range(Lk, kend, split, nsplit, kb0, kb1);
  const int wrow0 = row0 + w * 32;
  const int my_row = wrow0 + qc;
  const bool wave_active = wrow0 < rows_end;
  const int pi = key_perm(qc);

  // lane supplies Q[my_row][g * KS + s] * scale * log2(e): the scores come out
  // of the MFMAs already in the base-2 units of the softmax
  float qf[KS];
  {
    const bool ok = my_row < Lq;
    const float* qp = static_cast<const float*>(a.q) +
                      (static_cast<size_t>(q0 + (ok ? my_row : 0)) * a.num_heads + h) * D + g * KS;
#pragma unroll
    for (int s = 0; s < KS; s += 4) {
      const f32x4_t v = ok ? *reinterpret_cast<const f32x4_t*>(qp + s) : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[s + e] = v[e] * a.scale_log2;
    }
  }
  f32x16_t acc[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) acc[m] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;

  // Tile loads: thread (j4, c4) reads channels [4 c4, 4 c4 + 4) of keys
  // 4 j4 .. 4 j4 + 3; a wave's keys lie in one page, so the page id is one
  // scalar block-table read and the gathers are buffer loads; keys at or past
  // kb1 read 0 (offset out of range, or an empty descriptor past the pages).
  const_i32_t* btrow = (const_i32_t*)(a.bt) + static_cast<size_t>(seg) * a.max_blocks;
  const int last_page = (max(kb1, 1) - 1) >> 4;
  const uint32_t slot_bytes = static_cast<uint32_t>(a.num_kv_heads) * D * 4;
  const uint32_t page_bytes = slot_bytes * kPage;
  const uint32_t head_off = static_cast<uint32_t>(kvh) * D * 4;
  const int krow0 = segment_row0<kContig>(a, seg);  // first key row (contiguous K/V)
  const int c4 = tid % CPR, j4 = tid / CPR;
  const int pidx = (w * kWave / CPR) * 4 / kPage;  // page of this wave's keys within a tile
  u32x4_t kreg[4], vreg[4];
  auto issue_tile = [&](int k0) {
    const int id = segment_page<kContig>(btrow, krow0, (k0 >> 4) + pidx, last_page, a.num_blocks);
    const int range = id >= 0 ? static_cast<int>(page_bytes) : 0;
    const auto kr = __builtin_amdgcn_make_buffer_rsrc(page_base<kContig>(a.kc, id, slot_bytes, page_bytes),
                                                      0, range, kRawBufferWord3);
    const auto vr = __builtin_amdgcn_make_buffer_rsrc(page_base<kContig>(a.vc, id, slot_bytes, page_bytes),
                                                      0, range, kRawBufferWord3);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int key = 4 * j4 + it;
      const uint32_t off = (k0 + key < kb1) ? (key & 15) * slot_bytes + head_off + c4 * 16
                                            : kOffsetOutOfRange;
      kreg[it] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0));
      vreg[it] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 0));
    }
  };
  // registers -> one LDS stage: K natural Ks[key][d], V transposed Vt[d][key]
  // (the 4 x 4 block transposed in registers, one 16-byte write per channel)
  auto store_tile = [&](unsigned char* st) {
    float* Ks = reinterpret_cast<float*>(st);
    float* Vt = Ks + BN * ROWF;
#pragma unroll
    for (int it = 0; it < 4; ++it) st16(Ks + (4 * j4 + it) * ROWF + 4 * c4, kreg[it]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 4 * c4 + i;
      st16(Vt + d * BN + 4 * (j4 ^ vt_swz_f32<NCH>(d)),
           u32x4_t{vreg[0][i], vreg[1][i], vreg[2][i], vreg[3][i]});
    }
  };

  if (kb0 < kb1) {
    issue_tile(kb0);
    store_tile(smem);
    issue_tile(kb0 + BN);
    __syncthreads();
  }
  for (int k0 = kb0, i = 0; k0 < kb1; k0 += BN, ++i) {
    const float* Ks = reinterpret_cast<const float*>(smem + (i & 1) * STAGE);
    const float* Vt = Ks + BN * ROWF;
    if (wave_active && k0 <= H0 + wrow0 + 31) {  // else the tile is invisible to this wave
      const bool need_mask = (k0 + BN - 1) > (H0 + wrow0);
      f32x16_t sacc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        sacc[kb] = f32x16_t{};
        const float* kr = Ks + (kb * 32 + pi) * ROWF + g * KS;
        // all of the block's K operands first: the reads overlap each other and
        // the previous block's MFMAs instead of one read latency per 4 MFMAs
        f32x4_t kf[KS / 4];
#pragma unroll
        for (int s4 = 0; s4 < KS / 4; ++s4) kf[s4] = *reinterpret_cast<const f32x4_t*>(kr + 4 * s4);
        // keep the reads ahead of the MFMAs (at D = 128 the held operands would spill)
        if constexpr (D == 64) __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);  // MFMA clusters issue ahead of the other wave's softmax
#pragma unroll
        for (int s4 = 0; s4 < KS / 4; ++s4)
#pragma unroll
          for (int e = 0; e < 4; ++e) sacc[kb] = mfma_f32(kf[s4][e], qf[4 * s4 + e], sacc[kb]);
        __builtin_amdgcn_s_setprio(0);
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float x = sacc[kb][v];
          if (need_mask) {
            const int kp = k0 + kb * 32 + ((v >> 3) << 4) + (g << 3) + (v & 7);
            if (kp > H0 + my_row) x = -INFINITY;
          }
          sacc[kb][v] = x;
          tmax = fmaxf(tmax, x);
        }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float m_new = fmaxf(m_run, tmax);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = fast_exp2(sacc[kb][v] - m_use);
          sacc[kb][v] = p;
          psum += p;
        }
      }
      l_run = l_run * alpha + psum;
      if (__any(alpha != 1.f)) {  // no row max moved: the accumulators need no rescale
#pragma unroll
        for (int m = 0; m < NM; ++m) acc[m] *= alpha;
      }
      // O^T += V^T P^T: value n of sacc[kb] is key kb*32 + 16 (n/8) + 8 g + n % 8,
      // i.e. 16-byte V^T chunk kb*8 + 4 (n/8) + 2 g + (n % 8) / 4
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        // the block's V^T operands first (2 halves x NM channel blocks x 2 chunks)
        f32x4_t vf[2][NM][2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            const int d = m * 32 + qc;
            const float* vrow = Vt + d * BN;
            const int ch = kb * 8 + 4 * u + 2 * g, sw = vt_swz_f32<NCH>(d);
            vf[u][m][0] = *reinterpret_cast<const f32x4_t*>(vrow + 4 * (ch ^ sw));
            vf[u][m][1] = *reinterpret_cast<const f32x4_t*>(vrow + 4 * ((ch + 1) ^ sw));
          }
        if constexpr (D == 64) __builtin_amdgcn_sched_barrier(0);  // as for K
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                acc[m] = mfma_f32(vf[u][m][h2][e], sacc[kb][8 * u + 4 * h2 + e], acc[m]);
        __builtin_amdgcn_s_setprio(0);
      }
    }
    if (k0 + BN < kb1) {
      store_tile(smem + ((i + 1) & 1) * STAGE);  // tile i+1, loaded during tile i
      issue_tile(k0 + 2 * BN);                   // tile i+2 streams in
    }
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);  // lanes l and l^32 share a row
  const bool row_ok = wave_active && my_row < Lq;
  if (!row_ok) return;
  if constexpr (kSplit) {
    chunk_store_partial<D>(a, seg, h, tile, split, nsplit, m_run, l_tot, acc);
    return;
  }
  const float inv = 1.f / l_tot;
  float* op = static_cast<float*>(a.out) + (static_cast<size_t>(q0 + my_row) * a.num_heads + h) * D;
#pragma unroll
  for (int m = 0; m < NM; ++m) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = m * 32 + i4 * 8 + g * 4;
      *reinterpret_cast<f32x4_t*>(op + d) =
          f32x4_t{acc[m][4 * i4] * inv, acc[m][4 * i4 + 1] * inv, acc[m][4 * i4 + 2] * inv,
                  acc[m][4 * i4 + 3] * inv};
    }
  }
}

// Work item codes of the persistent kernel: chunk item i of group x is
// x << 24 | i, decode item d is kDecodeTag | d.
constexpr int kDecodeTag = 1 << 28, kDone = 0x7fffffff;
// scheduler state: the next item is to be claimed at the top of the item loop
constexpr int kPending = 0x7ffffffe;

// ---------------------------------------------------------------- decode role
// One wave = one head of one (segment, KV split).  Lane l = 16 r + c covers
// channels [c * EPL, (c + 1) * EPL) of key rows 4u + r of each 64-key step.
template <typename T, int EPL> struct RowFrag {
  static constexpr int kWords = EPL * static_cast<int>(sizeof(T)) / 4;
  uint32_t w[kWords];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < kWords; ++i) w[i] = 0;
  }
  __device__ __forceinline__ void load(const T* p) {
    if constexpr (kWords == 8) {
      const u32x4_t a = ld16(p), b = ld16(reinterpret_cast<const unsigned char*>(p) + 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) { w[i] = a[i]; w[4 + i] = b[i]; }
    } else if constexpr (kWords == 4) {
      const u32x4_t a = ld16(p);
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = a[i];
    } else {
      const u32x2_t a = ld8(p);
      w[0] = a[0];
      w[1] = a[1];
    }
  }
  __device__ __forceinline__ float elem(int e) const {
    if constexpr (sizeof(T) == 2) {
      return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
    } else {
      return __uint_as_float(w[e]);
    }
  }
};

template <typename T, int EPL>
__device__ __forceinline__ void store_row(T* p, const float* v) {
  if constexpr (sizeof(T) == 2) {
    uint32_t w[EPL / 2];
#pragma unroll
    for (int i = 0; i < EPL / 2; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    if constexpr (EPL == 8) st16(p, u32x4_t{w[0], w[1], w[2], w[3]});
    else st8(p, u32x2_t{w[0], w[1]});
  } else {
#pragma unroll
    for (int i = 0; i < EPL; i += 4)
      *reinterpret_cast<f32x4_t*>(p + i) = f32x4_t{v[i], v[i + 1], v[i + 2], v[i + 3]};
  }
}

// An item covers keys [kbeg, min(Lk, kbeg + klen)) of 4 query heads of a decode
// segment; slot < 0: the segment's only item, which writes the output row;
// else its partial result goes to partial slot part_prefix[seg] + slot.
template <typename T, int D, bool kContig>
__device__ void decode_item(const MainArgs& a, int seg, int hg, int kbeg, int klen, int slot) {
  constexpr int EPL = D / 16;  // channels per lane
  using Frag = RowFrag<T, EPL>;
  constexpr bool kLateV = Frag::kWords > 4;  // fp32 D=128: load V after the scores
  const int lane = threadIdx.x & 63, w = wave_id();
  const int h = hg * kHeadsPerDecodeItem + w;
  if (h >= a.num_heads) return;
  const int row = a.cu[seg], Lk = a.sk[seg];
  const int kfin = min(Lk, kbeg + klen);
  const int r = lane >> 4, c = lane & 15;
  const int kvh = h / a.group;
  const int32_t* btrow = a.bt + static_cast<size_t>(seg) * a.max_blocks;
  const size_t slot_elems = static_cast<size_t>(a.num_kv_heads) * D;
  const T* kbase = static_cast<const T*>(a.kc) + static_cast<size_t>(kvh) * D + c * EPL;
  const T* vbase = static_cast<const T*>(a.vc) + static_cast<size_t>(kvh) * D + c * EPL;
  const int row0 = segment_row0<kContig>(a, seg);
  const int nb_ok = kContig ? 0x7fffffff : a.num_blocks;  // contiguous: any first row >= 0

  float qv[EPL];
  {
    Frag f;
    f.load(static_cast<const T*>(a.q) + (static_cast<size_t>(row) * a.num_heads + h) * D + c * EPL);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[e] = f.elem(e) * a.scale_log2;
  }
  float m_run = -INFINITY, l_lane = 0.f, acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;

  for (int kb = kbeg; kb < kfin; kb += 64) {
    int pages[4];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp)
      pages[pp] = (kb + pp * 16 < kfin) ? (kContig ? row0 + kb + pp * 16 : btrow[(kb >> 4) + pp]) : -1;
    Frag kf[16], vf[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int pg = pages[u >> 2];
      const bool ok = (kb + 4 * u + r < kfin) &&
                      static_cast<unsigned>(pg) < static_cast<unsigned>(nb_ok);
      const size_t off = (static_cast<size_t>(ok ? pg : 0) * (kContig ? 1 : kPage) + 4 * (u & 3) + r) * slot_elems;
      if (ok) kf[u].load(kbase + off); else kf[u].zero();
      if constexpr (!kLateV) {
        if (ok) vf[u].load(vbase + off); else vf[u].zero();
      }
    }
    // partial dot products of this lane's channels with 16 key rows
    float pu[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) s = fmaf(qv[e], kf[u].elem(e), s);
      pu[u] = s;
    }
    // butterfly reduce-scatter over the 16 lanes of a row group: afterwards
    // lane c holds the full score of key row u = c, i.e. key kb + 4c + r.
#pragma unroll
    for (int half = 8; half >= 1; half >>= 1) {
      const bool upper = (c & half) != 0;
#pragma unroll
      for (int i = 0; i < half; ++i) {
        const float send = upper ? pu[i] : pu[i + half];
        const float keep = upper ? pu[i + half] : pu[i];
        pu[i] = keep + __shfl_xor(send, half);
      }
    }
    const int my_key = kb + 4 * c + r;
    const float s = my_key < kfin ? pu[0] : -INFINITY;
    const float m_new = fmaxf(m_run, wave_max(s));  // finite: key kb is in range
    const float alpha = fast_exp2(m_run - m_new);
    const float p = fast_exp2(s - m_new);
    m_run = m_new;
    l_lane = l_lane * alpha + p;
    if constexpr (kLateV) {
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int pg = pages[u >> 2];
        const bool ok = (kb + 4 * u + r < kfin) &&
                        static_cast<unsigned>(pg) < static_cast<unsigned>(nb_ok);
        const size_t off = (static_cast<size_t>(ok ? pg : 0) * (kContig ? 1 : kPage) + 4 * (u & 3) + r) * slot_elems;
        if (ok) vf[u].load(vbase + off); else vf[u].zero();
      }
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const float pv = __shfl(p, (r << 4) | u);  // weight of key row 4u + r
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(pv, vf[u].elem(e), acc[e]);
    }
  }

  const float l_tot = wave_sum(l_lane);
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    acc[e] += __shfl_xor(acc[e], 16);
    acc[e] += __shfl_xor(acc[e], 32);
  }
  if (slot < 0) {
    if (r == 0) {
      const float inv = 1.f / l_tot;
      float o[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = acc[e] * inv;
      store_row<T, EPL>(static_cast<T*>(a.out) + (static_cast<size_t>(row) * a.num_heads + h) * D + c * EPL, o);
    }
  } else {
    float* pp = a.partials +
                (static_cast<size_t>(a.part_prefix[seg] + slot) * a.num_heads + h) * a.part_stride;
    if (r == 0) store_row<float, EPL>(pp + 4 + c * EPL, acc);
    if (lane == 0) {
      pp[0] = m_run;
      pp[1] = l_tot;
    }
  }
}

// ---------------------------------------------------------------- decode role, bf16
// An item is (segment, KV split, 4 query heads).  Lane 16r + c of every wave
// works on head 4 hg + r, channels [2 WPL c, 2 WPL c + 2 WPL), so one load
// instruction of a wave reads the 4 heads' slices of one key row -- for
// MHA with D = 128, 1 KB contiguous -- instead of 256-byte pieces of 4 rows:
// on MI355X a pure read in the sliced pattern peaks near 5.4 TB/s, in 1 KB
// pieces near 6.35 TB/s.  Wave w takes the w-th quarter of the split's keys
// (rounded to whole 16-key steps, so every step lies in one page), keeps a
// running (max, sum, acc) per head, and the 4 waves merge through LDS at the
// end.  Scores with v_dot2_f32_bf16 on the
// raw bf16 pairs and a 16-lane DPP reduce-scatter (lane c ends with key c of
// the step); weights rounded to bf16, the sum taken from the same rounded
// values, P.V with row_newbcast broadcasts of weight pairs; the next step's K
// is loaded as soon as the dot products have consumed the current K, the next
// V after P.V.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<kDppRowMirror>(v));
  v = fmaxf(v, dpp_f32<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppQuadReverse>(v));
  v = fmaxf(v, dpp_f32<kDppQuadSwap>(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<kDppRowMirror>(v);
  v += dpp_f32<kDppRowHalfMirror>(v);
  v += dpp_f32<kDppQuadReverse>(v);
  v += dpp_f32<kDppQuadSwap>(v);
  return v;
}

template <int WPL>
struct KvStep {  // one 16-key step of one pool: 16 key rows x WPL words per lane
  uint32_t w[16][WPL];
};

// Loads one 16-key step (keys t0 .. t0 + 15, t0 a multiple of 16, so all in
// one page) of one pool for this lane.  The page is addressed through a buffer
// descriptor (base in SGPRs, 32-bit lane offset, key u at scalar offset
// u * slot_bytes): the hardware range check returns zeros for a page past the
// split or a block id outside the pool (descriptor of size 0) and for keys
// past the end of the split (offset moved out of range), without branches.
// The loads are non-temporal: each decode key is read once per item, and on
// MI355X streaming it through L2 with normal priority evicted the chunk
// tiles' shared K/V (a step of 2 chunks of 512 and 30 decodes: 246.7 -> 225.2 us
// with the hint).
template <int WPL, bool kContig>
__device__ __forceinline__ void load_step16(KvStep<WPL>& dst, const void* pool, const_i32_t* btrow,
                                            int row0, int t0, int kfin, int num_blocks,
                                            uint32_t slot_bytes, uint32_t page_bytes,
                                            uint32_t lane_off) {
  const int idx = t0 >> 4, last_page = (kfin - 1) >> 4;
  int pg;
  bool ok;
  if constexpr (kContig) {
    pg = idx <= last_page ? row0 + idx * kPage : -1;
    ok = pg >= 0;
  } else {
    const int id = btrow[min(idx, last_page)];  // scalar load, always inside the row
    pg = idx <= last_page ? id : -1;
    ok = static_cast<unsigned>(pg) < static_cast<unsigned>(num_blocks);
  }
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      page_base<kContig>(pool, ok ? pg : 0, slot_bytes, page_bytes), 0,
      ok ? static_cast<int>(page_bytes) : 0, kRawBufferWord3);
  const int lim = kfin - t0;  // keys u < lim are in the split
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const uint32_t vo = u < lim ? lane_off : kOffsetOutOfRange;
    const uint32_t so = u * slot_bytes;
    if constexpr (WPL == 4) {
      const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, vo, so, kLoadNonTemporal));
#pragma unroll
      for (int i = 0; i < 4; ++i) dst.w[u][i] = v[i];
    } else {
      const u32x2_t v = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rs, vo, so, kLoadNonTemporal));
      dst.w[u][0] = v[0];
      dst.w[u][1] = v[1];
    }
  }
}

template <int D, bool kContig>
__device__ void decode_item_bf16(const MainArgs& a, int seg, int hg, int kbeg, int klen, int slot,
                                 unsigned char* smem) {
  constexpr int WPL = D / 32;  // bf16 pairs per lane per key row (8 or 4 channels)
  constexpr int EPL = 2 * WPL;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int r = lane >> 4, c = lane & 15;
  // rows past the last head (num_heads not a multiple of 4) read the group's
  // first head and are dropped at the end
  const int h = hg * kHeadsPerDecodeItem + r;
  const int hq = h < a.num_heads ? h : hg * kHeadsPerDecodeItem;
  const int row = a.cu[seg], Lk = a.sk[seg];
  const int kfin = min(Lk, kbeg + klen);
  const int kvh = hq / a.group;
  const_i32_t* btrow = (const_i32_t*)(a.bt) + static_cast<size_t>(seg) * a.max_blocks;
  const uint32_t slot_bytes = static_cast<uint32_t>(a.num_kv_heads) * D * 2;
  const uint32_t page_bytes = slot_bytes * kPage;
  const uint32_t lane_off = static_cast<uint32_t>(kvh) * D * 2 + c * WPL * 4;
  const void* kpool = a.kc;
  const void* vpool = a.vc;
  const int row0 = segment_row0<kContig>(a, seg);

  uint32_t qw[WPL];
  {
    const unsigned char* qp = static_cast<const unsigned char*>(a.q) +
                              (static_cast<size_t>(row) * a.num_heads + hq) * D * 2 + c * WPL * 4;
    if constexpr (WPL == 4) {
      const u32x4_t v = ld16(qp);
#pragma unroll
      for (int i = 0; i < 4; ++i) qw[i] = v[i];
    } else {
      const u32x2_t v = ld8(qp);
      qw[0] = v[0];
      qw[1] = v[1];
    }
  }
  float m_run = -INFINITY, l_lane = 0.f, acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;

  const int quarter = ((kfin - kbeg + 63) >> 6) << 4;  // keys per wave, a multiple of 16
  const int t_first = kbeg + quarter * w;
  const int kend = min(kfin, t_first + quarter);      // this wave's keys: [t_first, kend)
  KvStep<WPL> kst, vst;
  load_step16<WPL, kContig>(kst, kpool, btrow, row0, t_first, kend, a.num_blocks, slot_bytes, page_bytes, lane_off);
  load_step16<WPL, kContig>(vst, vpool, btrow, row0, t_first, kend, a.num_blocks, slot_bytes, page_bytes, lane_off);
  for (int t0 = t_first; t0 < kend; t0 += 16) {
    // partial dot products: this lane's channels of keys t0 + u
    float pu[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      float sdot = 0.f;
#pragma unroll
      for (int i = 0; i < WPL; ++i) sdot = dot2_bf16(kst.w[u][i], qw[i], sdot);
      pu[u] = sdot;
    }
    // K registers are free: start the next step's K (past the split every
    // descriptor is empty and the loads return zeros without touching memory)
    load_step16<WPL, kContig>(kst, kpool, btrow, row0, t0 + 16, kend, a.num_blocks, slot_bytes, page_bytes,
                              lane_off);
    // reduce-scatter over the 16 lanes of the row: lane c ends with key u = c
    {
      const bool up8 = (c & 8) != 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float send = up8 ? pu[i] : pu[i + 8];
        const float keep = up8 ? pu[i + 8] : pu[i];
        pu[i] = keep + dpp_f32<kDppRowMirror>(send);
      }
      const bool up4 = (c & 4) != 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float send = up4 ? pu[i] : pu[i + 4];
        const float keep = up4 ? pu[i + 4] : pu[i];
        pu[i] = keep + dpp_f32<kDppRowHalfMirror>(send);
      }
      const bool up2 = (c & 2) != 0;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float send = up2 ? pu[i] : pu[i + 2];
        const float keep = up2 ? pu[i + 2] : pu[i];
        pu[i] = keep + dpp_f32<kDppQuadReverse>(send);
      }
      const bool up1 = (c & 1) != 0;
      const float send = up1 ? pu[0] : pu[1];
      const float keep = up1 ? pu[1] : pu[0];
      pu[0] = keep + dpp_f32<kDppQuadSwap>(send);
    }
    const float s = t0 + c < kend ? pu[0] * a.scale_log2 : -INFINITY;
    const float m_new = fmaxf(m_run, row16_max(s));  // finite: key t0 is in range
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    // this lane's weight rounded to bf16; pairs (keys 2t, 2t+1) formed on even lanes
    const uint32_t pbits = pack_bf16x2(fast_exp2(s - m_new), 0.f) & 0xffffu;
    l_lane = l_lane * alpha + __uint_as_float(pbits << 16);
    const uint32_t pair = pbits | (dpp_u32<kDppQuadSwap>(pbits) << 16);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      uint32_t pw;
      switch (t) {  // row_newbcast needs a compile-time lane
        case 0: pw = dpp_u32<kDppRowBcast0 + 0>(pair); break;
        case 1: pw = dpp_u32<kDppRowBcast0 + 2>(pair); break;
        case 2: pw = dpp_u32<kDppRowBcast0 + 4>(pair); break;
        case 3: pw = dpp_u32<kDppRowBcast0 + 6>(pair); break;
        case 4: pw = dpp_u32<kDppRowBcast0 + 8>(pair); break;
        case 5: pw = dpp_u32<kDppRowBcast0 + 10>(pair); break;
        case 6: pw = dpp_u32<kDppRowBcast0 + 12>(pair); break;
        default: pw = dpp_u32<kDppRowBcast0 + 14>(pair); break;
      }
#pragma unroll
      for (int i = 0; i < WPL; ++i) {
        const uint32_t v0 = vst.w[2 * t][i], v1 = vst.w[2 * t + 1][i];
        acc[2 * i] = dot2_bf16(pw, pair_lo(v0, v1), acc[2 * i]);
        acc[2 * i + 1] = dot2_bf16(pw, pair_hi(v0, v1), acc[2 * i + 1]);
      }
    }
    load_step16<WPL, kContig>(vst, vpool, btrow, row0, t0 + 16, kend, a.num_blocks, slot_bytes, page_bytes,
                              lane_off);
  }

  // merge the 4 waves' (max, sum, acc) of each head through LDS: wave w writes
  // its rows, then wave w finishes head 4 hg + w over all 4 waves
  float* s_acc = reinterpret_cast<float*>(smem);  // [wave][lane][EPL]
  float* s_ml = s_acc + kThreads * EPL;           // [wave][row][2]
  const float l_row = row16_sum(l_lane);
#pragma unroll
  for (int e = 0; e < EPL; ++e) s_acc[threadIdx.x * EPL + e] = acc[e];
  if (c == 0) {
    s_ml[(w * 4 + r) * 2] = m_run;
    s_ml[(w * 4 + r) * 2 + 1] = l_row;
  }
  __syncthreads();
  constexpr int CPL = D / kWave;  // channels per lane in the merge
  const int hm = hg * kHeadsPerDecodeItem + w;
  if (hm < a.num_heads) {
    float mw[4], mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      mw[v] = s_ml[(v * 4 + w) * 2];
      mx = fmaxf(mx, mw[v]);
    }
    float l_tot = 0.f, o[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) o[e] = 0.f;
    const int ch = lane * CPL;               // first channel of this lane
    const int src_lane = 16 * w + ch / EPL;  // lane of the compute layout holding it
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float f = mw[v] == -INFINITY ? 0.f : fast_exp2(mw[v] - mx);  // a wave with no keys adds nothing
      l_tot = fmaf(s_ml[(v * 4 + w) * 2 + 1], f, l_tot);
      const float* src = s_acc + (v * kWave + src_lane) * EPL + ch % EPL;
#pragma unroll
      for (int e = 0; e < CPL; ++e) o[e] = fmaf(src[e], f, o[e]);
    }
    if (slot < 0) {
      const float inv = 1.f / l_tot;
      bf16_t* op = static_cast<bf16_t*>(a.out) + (static_cast<size_t>(row) * a.num_heads + hm) * D + ch;
      if constexpr (CPL == 2) {
        *reinterpret_cast<uint32_t*>(op) = pack_bf16x2(o[0] * inv, o[1] * inv);
      } else {
        *op = static_cast<bf16_t>(pack_bf16x2(o[0] * inv, 0.f) & 0xffffu);
      }
    } else {
      float* pp = a.partials +
                  (static_cast<size_t>(a.part_prefix[seg] + slot) * a.num_heads + hm) * a.part_stride;
#pragma unroll
      for (int e = 0; e < CPL; ++e) pp[4 + ch + e] = o[e];
      if (lane == 0) {
        pp[0] = mx;
        pp[1] = l_tot;
      }
    }
  }
}

// ---------------------------------------------------------------- persistent kernel
constexpr int kLdsSegments = 512;  // item prefix sums of up to this many segments live in LDS

__device__ __forceinline__ int find_segment_lds(const int* prefix, int n, int x) {
  int lo = 0, hi = n;  // invariant: prefix[lo] <= x < prefix[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// kSplit: this launch may meet split chunk tiles (the planner was allowed to
// split); the instance without it keeps the unsplit roles' register allocation.
// kDefer: a chunk item, or a decode item of at least kLateClaimKeys keys, claims
// its successor only when it is done; other items claim it at their start,
// which hides the atomic's latency behind the item.  An item reserved at the
// start of a long one waits behind it while other workgroups run out of work,
// so long items reserve nothing.
template <typename T, int D, bool kSplit, bool kContig, bool kDefer>
__global__ __launch_bounds__(kThreads, 2) void attn_kernel(MainArgs a) {
  constexpr int kSmem = ChunkCfg<T>::template Sizes<D>::BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kSmem];
  // the bf16 chunk role's second stage (an object of its own)
  constexpr bool kBf16 = sizeof(T) == 2;
  __shared__ __attribute__((aligned(16))) unsigned char smem_b[kBf16 ? ChunkCfg<bf16_t>::Sizes<D>::STAGE : 16];
  __shared__ int s_prefix[3][kLdsSegments + 1];  // chunk pairs, decode full splits, decode tail pieces
  __shared__ int s_work[6];
  // scheduler state, touched by thread 0 only; kept in LDS so no register holds
  // it across work items
  __shared__ int s_next;           // item claimed for the next iteration
  __shared__ unsigned s_chunk_open;  // bit x: chunk group x may still have items
  __shared__ int s_dec_open;
  const int n_tiles = a.hdr->n_chunk_tiles;
  const int n_dec = a.hdr->n_dec_items;
  const int n_dec_full = a.hdr->n_dec_full;
  const int split_keys = a.hdr->split;
  const int head_groups = (a.num_heads + kHeadsPerDecodeItem - 1) / kHeadsPerDecodeItem;
  const int csplit = kSplit ? a.hdr->chunk_split : 1;
  const int gsub = sizeof(T) == 4 ? a.hdr->chunk_gsub : 1;  // bf16 planners always write 1
  const bool lds_lookup = a.num_seqs <= kLdsSegments;
  if (lds_lookup) {
    for (int i = threadIdx.x; i <= a.num_seqs; i += kThreads) {
      s_prefix[0][i] = a.tile_prefix[i];
      s_prefix[1][i] = a.dec_prefix[i];
      s_prefix[2][i] = a.tail_prefix[i];
    }
  }
  // Work distribution.  Decode splits come from one queue; chunk tiles from
  // kXcdGroups queues (tiles of head h in group h % kXcdGroups).  The first
  // chunk_wgs workgroups (half of the grid in the fused launch) take chunk tiles
  // while any are left -- their own XCD's group first, then the others -- the
  // rest decode splits; each falls back to the other kind when its own is empty,
  // so both roles run side by side on every CU.  A launch for one role only
  // (roles) never opens the other kind's queues.  The first item of every workgroup is assigned statically (the planner
  // starts the counters past those items); afterwards the next item is claimed
  // with an atomic at the start of the current one, hiding the claim's latency
  // (fp32 chunk items: at their end).
  const int half = a.chunk_wgs;
  const bool chunk_first = static_cast<int>(blockIdx.x) < half;
  const int my_group = blockIdx.x % kXcdGroups;
  auto claim_chunk = [&]() -> int {
    if (!s_chunk_open) return kDone;
    // one round of independent (relaxed, device-scope) counter reads closes the
    // groups already drained, so at most one atomic is spent on a likely winner
    // instead of a chain of failing atomics
    unsigned seen[kXcdGroups];
#pragma unroll
    for (int x = 0; x < kXcdGroups; ++x)
      seen[x] = __hip_atomic_load(&a.hdr->chunk_counter[x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned open = s_chunk_open;
#pragma unroll
    for (int x = 0; x < kXcdGroups; ++x)
      if (seen[x] >= static_cast<unsigned>(chunk_group_items(a.num_heads, gsub, n_tiles, x))) open &= ~(1u << x);
    if constexpr (sizeof(T) == 4) {
      // fp32 steps have few heads, so most groups are empty and most
      // workgroups claim from another group: after its own group, a workgroup
      // tries the open groups starting at an offset that differs between the
      // workgroups of a group, which spreads the atomics over every open
      // counter instead of queueing them on the first.  (Kept out of the bf16
      // instances, where the extra state costs register spills.)  Each pass
      // closes one group: at most kXcdGroups passes.
      while (open) {
        int x = my_group;
        if (!(open & (1u << my_group))) {
          unsigned m = open;
          for (int j = (static_cast<int>(blockIdx.x) / kXcdGroups) % __popc(open); j > 0; --j) m &= m - 1;
          x = __ffs(m) - 1;
        }
        const int n = chunk_group_items(a.num_heads, gsub, n_tiles, x);
        const int c = static_cast<int>(atomicAdd(&a.hdr->chunk_counter[x], 1u));
        if (c < n) {
          s_chunk_open = open;
          return (x << 24) | c;
        }
        open &= ~(1u << x);
      }
    } else {
      for (int k = 0; k < kXcdGroups && open; ++k) {
        const int x = (my_group + k) % kXcdGroups;
        if (!(open & (1u << x))) continue;
        const int n = chunk_group_items(a.num_heads, gsub, n_tiles, x);
        const int c = static_cast<int>(atomicAdd(&a.hdr->chunk_counter[x], 1u));
        if (c < n) {
          s_chunk_open = open;
          return (x << 24) | c;
        }
        open &= ~(1u << x);
      }
    }
    s_chunk_open = open;
    return kDone;
  };
  auto claim_dec = [&]() -> int {
    if (!s_dec_open) return kDone;
    // fp32: a relaxed read first closes a drained queue without an atomic --
    // with few decode items (the worked example has 2), hundreds of workgroups
    // would otherwise queue failing atomics on this one counter before they
    // look at the chunk queues.  (Not in the bf16 instances, whose compiled
    // code it would change; their steps have many decode items.)
    if (sizeof(T) == 4 &&
        __hip_atomic_load(&a.hdr->dec_counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >=
            static_cast<unsigned>(n_dec)) {
      s_dec_open = 0;
      return kDone;
    }
    const int d = static_cast<int>(atomicAdd(&a.hdr->dec_counter, 1u));
    if (d < n_dec) return kDecodeTag | d;
    s_dec_open = 0;
    return kDone;
  };
  auto claim = [&]() -> int {
    int it = chunk_first ? claim_chunk() : claim_dec();
    if (it == kDone) it = chunk_first ? claim_dec() : claim_chunk();
    return it;
  };
  if (threadIdx.x == 0) {
    s_chunk_open = (a.roles & 1) ? (1u << kXcdGroups) - 1 : 0u;
    s_dec_open = (a.roles & 2) ? 1 : 0;
    const int rank = blockIdx.x / kXcdGroups;  // among chunk-first workgroups of this group
    if (chunk_first && rank < chunk_group_items(a.num_heads, gsub, n_tiles, my_group))
      s_next = (my_group << 24) | rank;
    else if (!chunk_first && static_cast<int>(blockIdx.x) - half < n_dec)
      s_next = kDecodeTag | (blockIdx.x - half);
    else if constexpr (sizeof(T) == 4) {
      // fused launch: a decode-first workgroup with no decode item takes the
      // next static rank of its own group, after the chunk-first ones (the
      // planner starts the counters past these too), instead of queueing an
      // atomic on the shared counters (the worked example's 254 such
      // workgroups started their first item 8 us late)
      int it = kDone;
      if (!chunk_first && a.roles == 3) {
        const int r = spare_chunk_rank(static_cast<int>(blockIdx.x), half, n_dec);
        if (r < chunk_group_items(a.num_heads, gsub, n_tiles, my_group)) it = (my_group << 24) | r;
      }
      s_next = it == kDone ? claim() : it;
    } else
      s_next = claim();
  }
  __syncthreads();  // LDS prefix copy complete
  // Thread-0-only code belongs in the block at the top of this loop or right
  // after the barriers, never between the work and the back edge: there it let
  // the compiler split the loop so that thread 0 left the inner part through
  // the exec mask while the other lanes went round the barriers without it (a
  // hang; tests/test_kernel_structure.py checks the compiled loops).
  for (;;) {
    if (threadIdx.x == 0) {
      if (kDefer && s_next == kPending) s_next = claim();  // claim deferred by a chunk item
      const int cur = s_next;
      int kind = 0, seg = 0, p1 = 0, p2 = 0, p3 = 0, p4 = 0;  // kind: 0 done, 1 chunk, 2 decode
      if (cur != kDone && (cur & kDecodeTag)) {
        // full splits first (dec_prefix), then the tail pieces (tail_prefix),
        // both segment by segment with the head groups innermost: item ->
        // head group p1, keys [p2, p2 + p3), partial slot p4 (-1: the segment's
        // only item writes the output row)
        const int d = cur & (kDecodeTag - 1);
        const bool tail = d >= n_dec_full;
        const int e = tail ? d - n_dec_full : d;
        auto resolve = [&](const int* dp, const int* tp) {  // LDS copies or the workspace arrays
          const int* ep = tail ? tp : dp;
          int lo = 0, hi = a.num_seqs;  // segment owning item e: ep[lo] <= e < ep[hi]
          while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (ep[mid] <= e) lo = mid; else hi = mid;
          }
          seg = lo;
          const int local = e - ep[seg];
          const int piece = local / head_groups;
          const int nfull = (dp[seg + 1] - dp[seg]) / head_groups;
          const int ntail = (tp[seg + 1] - tp[seg]) / head_groups;
          const int tail_keys = split_keys >> kTailLog2;
          p1 = local - piece * head_groups;
          p2 = tail ? nfull * split_keys + piece * tail_keys : piece * split_keys;
          p3 = tail ? tail_keys : split_keys;
          p4 = nfull + ntail == 1 ? -1 : (tail ? nfull + piece : piece);
        };
        if (lds_lookup) resolve(s_prefix[1], s_prefix[2]);
        else resolve(a.dec_prefix, a.tail_prefix);
        kind = 2;
      } else if (cur != kDone) {
        // group x holds, segment by segment, (head x + 8k, tile, split) for its
        // heads; tile_prefix counts (tile, split) pairs.  With gsub > 1 group x
        // holds pairs x / H, x / H + gsub, ... of head x % H.
        const int x = cur >> 24, i = cur & ((1 << 24) - 1);
        const int nh = gsub > 1 ? 1 : chunk_group_heads(a.num_heads, x);
        // pair rank over all segments (scaled down by the group's heads)
        const int t = gsub > 1 ? i * gsub + x / a.num_heads : i / nh;
        seg = lds_lookup ? find_segment_lds(s_prefix[0], a.num_seqs, t)
                         : find_segment(a.tile_prefix, a.num_seqs, t);
        const int t0 = lds_lookup ? s_prefix[0][seg] : a.tile_prefix[seg];
        const int nts = (lds_lookup ? s_prefix[0][seg + 1] : a.tile_prefix[seg + 1]) - t0;
        const int local = gsub > 1 ? t - t0 : i - nh * t0, r = local % nts;
        p1 = gsub > 1 ? x % a.num_heads : x + kXcdGroups * (local / nts);  // query head
        if (csplit == 1) {
          p2 = nts - 1 - r;                   // query tile, longest first
        } else {
          // range-major: the first range of every tile before any second
          // range, so the short and empty last ranges are handed out last
          const int ntl = nts / csplit;
          p3 = r / ntl;                       // key range of the tile
          p2 = ntl - 1 - (r - p3 * ntl);      // query tile, longest first
        }
        kind = 1;
      }
      s_work[0] = kind;
      s_work[1] = seg;
      s_work[2] = p1;
      s_work[3] = p2;
      s_work[4] = p3;
      s_work[5] = p4;
    }
    __syncthreads();
    // the work item is uniform across the workgroup: keep it in scalar registers so
    // every address derived from it (segment row, block-table row, pages) is scalar
    const int kind = __builtin_amdgcn_readfirstlane(s_work[0]);
    const int seg = __builtin_amdgcn_readfirstlane(s_work[1]);
    const int p1 = __builtin_amdgcn_readfirstlane(s_work[2]);
    const int p2 = __builtin_amdgcn_readfirstlane(s_work[3]);
    const int p3 = __builtin_amdgcn_readfirstlane(s_work[4]);
    const int p4 = __builtin_amdgcn_readfirstlane(s_work[5]);
    __syncthreads();
    if (kind == 0) break;
    // the next item, claimed while this one runs (hides the atomic's latency),
    // or with kDefer, after a chunk item or a long decode item only once it is
    // done: an item reserved at the start of a long item waits behind it while
    // other workgroups run dry
    if (threadIdx.x == 0) s_next = (kDefer && (kind == 1 || p3 >= kLateClaimKeys)) ? kPending : claim();
    if (kind == 1) {
      if (csplit == 1) {
        if constexpr (sizeof(T) == 2) chunk_tile_bf16<D, false, kContig, kDefer>(a, seg, p1, p2, 0, 1, smem, smem_b);
        else chunk_tile_f32<D, false, kContig>(a, seg, p1, p2, 0, 1, smem);
      } else if constexpr (kSplit) {
        if constexpr (sizeof(T) == 2) chunk_tile_bf16<D, true, kContig, kDefer>(a, seg, p1, p2, p3, csplit, smem, smem_b);
        else chunk_tile_f32<D, true, kContig>(a, seg, p1, p2, p3, csplit, smem);
      }
    } else {
      if constexpr (sizeof(T) == 2) decode_item_bf16<D, kContig>(a, seg, p1, p2, p3, p4, smem);
      else decode_item<T, D, kContig>(a, seg, p1, p2, p3, p4);
    }
  }
}

// ---------------------------------------------------------------- combine
// Workgroups past the decode ones merge split chunk tiles: each takes
// (tile, head, 16-row group) units in turn; 16 threads per query row, D / 16
// channels each.
constexpr int kChunkMergeBlocks = 256;

template <typename T, int D>
__device__ void merge_chunk_tiles(const MainArgs& a, int blk) {
  const int S = a.hdr->chunk_split;
  if (S <= 1) return;
  constexpr int QPR = 16, CPT = D / QPR, NV = CPT / 4;
  constexpr int RPB = kThreads / QPR;       // rows of a tile merged by one workgroup pass
  constexpr int GROUPS = kChunkRows / RPB;  // row groups per (tile, head)
  constexpr int BATCH = 16;                 // key ranges whose partials are loaded together
  const int n_pairs = a.hdr->n_chunk_tiles / S * a.num_heads;
  const size_t sstep = static_cast<size_t>(a.num_heads) * kChunkRows * a.part_stride;
  const int c0 = (threadIdx.x % QPR) * CPT;
  for (int u = blk; u < n_pairs * GROUPS; u += kChunkMergeBlocks) {
    const int p = u / GROUPS, grp = u - p * GROUPS;
    const int ti = p / a.num_heads, h = p - ti * a.num_heads;  // tile over all chunk segments
    const int seg = find_segment(a.tile_prefix, a.num_seqs, ti * S);
    const int tile = ti - a.tile_prefix[seg] / S;
    const int q0 = a.cu[seg], Lq = a.cu[seg + 1] - q0;
    const size_t slot0 = static_cast<size_t>(a.tile_prefix[seg] + tile * S);
    const int rr = grp * RPB + static_cast<int>(threadIdx.x) / QPR;
    const int row = tile * kChunkRows + rr;
    if (row >= Lq) continue;
    const float* base = a.chunk_partials + ((slot0 * a.num_heads + h) * kChunkRows + rr) * a.part_stride;
    // one online pass over the ranges, BATCH at a time: the loads of a batch are
    // independent, so a row waits for S / BATCH round trips instead of 2 S; an
    // empty range (max -inf) weighs 0, and range 0 holds key 0, which every row
    // sees, so the running max is finite after the first batch
    float mx = -INFINITY, l = 0.f;
    f32x4_t o[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += BATCH) {
      float mv[BATCH], lv[BATCH];
      f32x4_t ov[BATCH][NV];
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
        const bool in = s0 + j < S;
        const float* pp = base + static_cast<size_t>(in ? s0 + j : 0) * sstep;
        mv[j] = in ? pp[0] : -INFINITY;
        lv[j] = in ? pp[1] : 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i)
          ov[j][i] = in ? *reinterpret_cast<const f32x4_t*>(pp + 4 + c0 + 4 * i) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
      float bm = mx;
#pragma unroll
      for (int j = 0; j < BATCH; ++j) bm = fmaxf(bm, mv[j]);
      const float sc = mx == -INFINITY ? 0.f : fast_exp2(mx - bm);
      l *= sc;
#pragma unroll
      for (int i = 0; i < NV; ++i) o[i] *= sc;
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
        const float wgt = mv[j] == -INFINITY ? 0.f : fast_exp2(mv[j] - bm);
        l = fmaf(lv[j], wgt, l);
#pragma unroll
        for (int i = 0; i < NV; ++i) o[i] += wgt * ov[j][i];
      }
      mx = bm;
    }
    const float inv = 1.f / l;
    T* op = static_cast<T*>(a.out) + (static_cast<size_t>(q0 + row) * a.num_heads + h) * D + c0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const f32x4_t v = o[i] * inv;
      if constexpr (sizeof(T) == 2) {
        st8(op + 4 * i, u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
      } else {
        *reinterpret_cast<f32x4_t*>(op + 4 * i) = v;
      }
    }
  }
}

// One wave per (decode segment, head) that was split: lanes first reduce the
// split maxima, then every lane owns D / 64 channels and sums the rescaled
// partial accumulators of all splits.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void combine_kernel(MainArgs a) {
  const int head_groups = (a.num_heads + kHeadsPerDecodeItem - 1) / kHeadsPerDecodeItem;
  const int n_dec_blocks = a.num_seqs * head_groups;
  if (static_cast<int>(blockIdx.x) >= n_dec_blocks) {
    merge_chunk_tiles<T, D>(a, blockIdx.x - n_dec_blocks);
    return;
  }
  const int seg = blockIdx.x / head_groups, hg = blockIdx.x - seg * head_groups;
  const int p0 = a.part_prefix[seg], np = a.part_prefix[seg + 1] - p0;
  if (np <= 0) return;
  constexpr int EPL = D / kWave;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int h = hg * kHeadsPerDecodeItem + w;
  if (h >= a.num_heads) return;
  const int row = a.cu[seg];
  const size_t step = static_cast<size_t>(a.num_heads) * a.part_stride;
  const float* base = a.partials + (static_cast<size_t>(p0) * a.num_heads + h) * a.part_stride;
  float mx = -INFINITY;
  for (int sp = lane; sp < np; sp += kWave) mx = fmaxf(mx, base[sp * step]);
  mx = wave_max(mx);
  float l = 0.f, o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;
  for (int s0 = 0; s0 < np; s0 += kWave) {
    const int sp = s0 + lane;
    float wgt = 0.f;  // weight of split s0 + lane (0 past the last split)
    if (sp < np) {
      wgt = fast_exp2(base[sp * step] - mx);
      l = fmaf(base[sp * step + 1], wgt, l);
    }
    const int n = min(kWave, np - s0);
    for (int t0 = 0; t0 < n; t0 += 8) {  // 8 independent partial loads in flight
      float v[8][EPL];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int t = t0 + jj;
        const float* pp = base + (s0 + min(t, n - 1)) * step + 4 + lane * EPL;
#pragma unroll
        for (int e = 0; e < EPL; ++e) v[jj][e] = pp[e];
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const float wt = t0 + jj < n ? __shfl(wgt, t0 + jj) : 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] = fmaf(v[jj][e], wt, o[e]);
      }
    }
  }
  const float inv = 1.f / wave_sum(l);
  T* op = static_cast<T*>(a.out) + (static_cast<size_t>(row) * a.num_heads + h) * D + lane * EPL;
  if constexpr (sizeof(T) == 2) {
    if constexpr (EPL == 2) {
      *reinterpret_cast<uint32_t*>(op) = pack_bf16x2(o[0] * inv, o[1] * inv);
    } else {
      *op = static_cast<bf16_t>(pack_bf16x2(o[0] * inv, 0.f) & 0xffffu);
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) op[e] = o[e] * inv;
  }
}

// ---------------------------------------------------------------- prefill helpers
// Pool-to-LDS 16-byte load (as load_lds16) written as inline asm, so that the
// compiler does not see it write LDS: with dozens of these in flight its alias
// tracking of such loads runs out of slots, and it then waits for all of them
// in front of LDS reads of other stages.  The caller waits (vmcnt) for the
// loads it needs; the instruction has no register result.  An LDS-DMA load
// needs one wait state after the SALU write of M0 that it reads, which the
// compiler inserts for its own such loads but cannot see here: hence the
// s_nop.  (A VALU write of one of its SGPR operands needs five; the compiler
// builds the descriptor and M0 with SALU instructions, and a kernel-structure
// test checks both distances in the compiled code.)
__device__ __forceinline__ void load_lds16_async(__amdgpu_buffer_rsrc_t rsrc, unsigned char* dst, uint32_t off) {
  const auto lp = (__attribute__((address_space(3))) unsigned char*)dst;
  const uint32_t lds = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lp)));
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(off), "s"(rsrc), "{m0}"(lds)
               : "memory");
}
// Workgroup barrier that leaves the pool-to-LDS loads in flight.  A
// __syncthreads() fences LDS at workgroup scope, and since those loads write
// LDS it waits for every one of them, including the steps loaded ahead.  Here
// each wave only finishes its own LDS reads (a stage is overwritten after the
// barrier that follows its last read) and the caller waits (vmcnt) for the
// loads of the steps it needs.  The empty asm statements keep the compiler
// from moving LDS accesses across the barrier, the scheduling barriers keep
// every other instruction (the MFMAs above all) on its side of it.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// ==================================================================== one-segment prefill, bf16
// A step that is a single prefill chunk (one segment) has no decode work to
// share the CUs with, so it runs a kernel shaped for the matrix cores alone:
// each wave owns 64 query rows (two 32-row blocks that share every K and V
// operand read, so a step's LDS reads serve twice the MFMA work of the fused
// kernel's 32-row waves), a tile is 256 rows x one head, a workgroup holds a
// whole CU (one wave per SIMD: 256 VGPRs, with AGPRs as spill space) and four
// LDS stages keep K/V loads two steps ahead.  With one wave per SIMD nothing
// else hides the softmax, so the key loop is software pipelined: each row
// block's softmax is scheduled among the MFMAs of the other phase.  Same data
// layout, swizzles and masks as chunk_tile_bf16; the softmax moves its
// reference max lazily (see below).
constexpr int kPrefillBlocks = 2;                          // 32-row blocks per wave
constexpr int kPrefillRows = 4 * 32 * kPrefillBlocks;      // query rows per tile

struct PrefillArgs {
  MainArgs m;
  int total_q, max_q, max_k, total_k, ntiles;
};

// Keys [0, Lk) of segment 0 and whether it meets the documented preconditions
// (the planner's test for every segment); a segment that does not is skipped.
template <bool kContig>
__device__ __forceinline__ bool prefill_segment(const PrefillArgs& p, int& q0, int& lq, int& lk) {
  const MainArgs& a = p.m;
  const int c0 = a.cu[0], c1 = a.cu[1];
  q0 = c0;
  lq = c1 - c0;
  bool rows_ok = true;
  if constexpr (kContig) {
    const int k0 = a.cu_k[0], k1 = a.cu_k[1];
    lk = k1 - k0;
    rows_ok = k0 >= 0 && k1 <= p.total_k;
  } else {
    lk = a.sk[0];
  }
  return rows_ok && c0 >= 0 && c1 >= c0 && c1 <= p.total_q && lq <= lk && lk <= p.max_k && lq <= p.max_q &&
         ((lk + kPage - 1) / kPage) <= a.max_blocks;
}

template <int D, bool kContig>
__device__ void prefill_tile_bf16(const MainArgs& a, int h, int tile, int q0, int Lq, int Lk,
                                  unsigned char* st0, unsigned char* st1, unsigned char* st2,
                                  unsigned char* st3) {
  using Cfg = ChunkCfg<bf16_t>::Sizes<D>;
  constexpr int BN = Cfg::BN, KS = D / 16, NM = D / 32, RB = kPrefillBlocks;
  static_assert(RB == 2, "the pipeline below pairs the two row blocks");
  constexpr int ROW = Cfg::ROW, POOL = Cfg::POOL;
  constexpr int CPR = D / 8;          // 16-byte chunks per key row
  constexpr int RPI = kWave / CPR;    // rows per wave load instruction (1 KB)
  constexpr int KPW = BN / 4;         // keys of a step each wave loads (one page)
  constexpr int IPW = KPW / RPI;      // load instructions per wave, per pool and step
  static_assert(KPW == kPage && KPW % RPI == 0, "each wave loads one page per step");
  // s_waitcnt operands: all vector loads but the last one / two steps' landed
  constexpr int kWaitOneStep = wait_vmcnt(2 * IPW);
  constexpr int kWaitTwoSteps = wait_vmcnt(4 * IPW);

  const int lane = threadIdx.x & 63, w = wave_id();
  const int qc = lane & 31, g = lane >> 5;
  const int H0 = Lk - Lq;
  const int kvh = h / a.group;
  // Tiles are aligned to the chunk's end: tile t holds rows
  // [256 t - shift, 256 (t + 1) - shift) with shift = 256 ceil(Lq / 256) - Lq,
  // so the one partial tile is the first, which sees the fewest keys (every
  // wave runs every step of its tile, rows or not).  Rows below 0 take zero
  // queries and the keys the causal rule gives them (none without history);
  // they are never stored.
  const int shift = (Lq + kPrefillRows - 1) / kPrefillRows * kPrefillRows - Lq;
  const int row0 = tile * kPrefillRows - shift;
  const int rows_end = row0 + kPrefillRows;
  const int kb1 = H0 + rows_end;  // keys [0, kb1) are visible to some row of the tile
  const int nsteps = (kb1 + BN - 1) / BN;
  const int wrow0 = row0 + w * 32 * RB;
  const int pi = key_perm(qc);

  // Q^T operands: for row block r, lane supplies Q[wrow0 + 32 r + qc][s*16 + g*8 .. +8]
  u32x4_t qf[RB][KS];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int row = wrow0 + 32 * r + qc;
    const bool ok = row >= 0 && row < Lq;
    const bf16_t* qp = static_cast<const bf16_t*>(a.q) +
                       (static_cast<size_t>(q0 + (ok ? row : 0)) * a.num_heads + h) * D + g * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[r][s] = ok ? ld16(qp + s * 16) : u32x4_t{0, 0, 0, 0};
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  f32x16_t acc[RB][NM];
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[r][m] = f32x16_t{};
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
  }

  const_i32_t* btrow = (const_i32_t*)(a.bt);  // segment 0's row of the block table
  const int last_page = (max(kb1, 1) - 1) >> 4;
  const uint32_t slot_bytes = static_cast<uint32_t>(a.num_kv_heads) * D * 2;
  const uint32_t page_bytes = slot_bytes * kPage;
  const uint32_t head_off = static_cast<uint32_t>(kvh) * D * 2;
  const int krow0 = kContig ? a.cu_k[0] : 0;
  struct PageRef { int idx, raw; };
  auto page_ref = [&](int k0) -> PageRef {
    const int idx = (k0 >> 4) + w;
    if constexpr (kContig) return {idx, krow0 + idx * kPage};
    else return {idx, btrow[min(idx, last_page)]};  // always inside the row
  };
  auto page_id = [&](PageRef r) {  // -1 past the range or outside the pool
    if constexpr (kContig) return r.idx <= last_page ? r.raw : -1;
    else return (r.idx <= last_page && static_cast<unsigned>(r.raw) < static_cast<unsigned>(a.num_blocks)) ? r.raw : -1;
  };
  const int lrow = lane / CPR, lpos = lane % CPR;
  auto issue_step = [&](int k0, PageRef pr, unsigned char* st) {
    const int id = page_id(pr);
    const int range = id >= 0 ? static_cast<int>(page_bytes) : 0;
    const auto rk = __builtin_amdgcn_make_buffer_rsrc(page_base<kContig>(a.kc, id, slot_bytes, page_bytes), 0,
                                                      range, kRawBufferWord3);
    const auto rv = __builtin_amdgcn_make_buffer_rsrc(page_base<kContig>(a.vc, id, slot_bytes, page_bytes), 0,
                                                      range, kRawBufferWord3);
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int r = RPI * j + lrow;  // key within the page
      const int row = KPW * w + r;   // row within the step
      const bool in = k0 + row < kb1;
      const uint32_t base = static_cast<uint32_t>(r) * slot_bytes + head_off;
      const uint32_t ok_ = in ? base + static_cast<uint32_t>(lpos ^ kswz<D>(row)) * 16 : kOffsetOutOfRange;
      const uint32_t ov_ = in ? base + static_cast<uint32_t>(lpos ^ vswz<D>(row)) * 16 : kOffsetOutOfRange;
      unsigned char* dk = st + (KPW * w + RPI * j) * ROW;
      load_lds16_async(rk, dk, ok_);
      load_lds16_async(rv, dk + POOL, ov_);
    }
  };

  // ---- the pieces of the pipeline, per half step (32 keys, key block kb)
  // LDS operand addresses.  K: chunk (2s + g) of step row 32 kb + pi sits at
  // chunk (2s + g) ^ z, z = kswz(pi), i.e. at byte
  //   32 kb ROW + (kofs ^ 32 s),  kofs = pi ROW + 16 (g ^ (z & 1)) + 32 (z >> 1)
  // (32 s and 32 (z >> 1) share bits 5..7, which nothing else uses).  V: the
  // transposing read of (kb, u, r, m) is at
  //   (32 kb + 16 u + 4 r) ROW + (vofs ^ 64 m)
  // with vofs the lane's part (see pv).  Both offsets pass through an empty asm
  // statement at every use, so the compiler recomputes the few XORs instead of
  // keeping an address register per (stage, s) or (stage, m).
  const int kz = kswz<D>(pi);
  const uint32_t kofs0 = static_cast<uint32_t>(pi * ROW + 16 * (g ^ (kz & 1)) + 32 * (kz >> 1));
  const int tq = lane >> 4, tc = lane & 15, tx = tc >> 2, ty = tc & 3;
  const int vz = vswz<D>(8 * (tq >> 1) + tx);
  const int vx = 2 * (tq & 1) + (ty >> 1);
  const uint32_t vofs0 = static_cast<uint32_t>((8 * (tq >> 1) + tx) * ROW + 16 * (vx ^ (vz & 3)) +
                                               8 * (ty & 1) + 64 * (vz >> 2));
  // the K operands of one key block, into registers
  auto load_k = [&](const unsigned char* Ks, int kb, u32x4_t (&kf)[KS]) {
    uint32_t kofs = kofs0;
    asm volatile("" : "+v"(kofs));
#pragma unroll
    for (int s = 0; s < KS; ++s) kf[s] = ld16(Ks + kb * 32 * ROW + (kofs ^ static_cast<uint32_t>(32 * s)));
  };
  // S_r = K Q_r^T of one key block for both row blocks, each K operand used
  // by both
  auto qk = [&](const u32x4_t (&kf)[KS], f32x16_t& s0, f32x16_t& s1) {
    s0 = s1 = f32x16_t{};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      s0 = mfma_bf16(kf[s], qf[0][s], s0);
      s1 = mfma_bf16(kf[s], qf[1][s], s1);
    }
  };
  // causal mask of the key block starting at key kbase (value v is key
  // kbase + 16 (v / 8) + 8 g + v % 8), for blocks past this wave's first
  // diagonal; it also blanks blocks past the wave's (or the tile's) last row
  auto mask = [&](int kbase, f32x16_t& sc, int r) {
    const int lim = H0 + wrow0 + 32 * r + qc - kbase - (g << 3);
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if (((v >> 3) << 4) + (v & 7) > lim) sc[v] = -INFINITY;
  };
  // online softmax of row block r over one key block: weights as bf16 pairs
  // (P^T operands), the reference max and the running sum; returns the
  // accumulator rescale factor.  The reference max moves only when a score
  // passes it by more than 2^8 in weight terms (weights up to 256 are exact
  // enough in bf16 and fp32, and O / l is unchanged by the choice of
  // reference), so the accumulator rescale -- 64 multiplies per row block,
  // behind a branch -- is left for the rare large jumps instead of every new
  // maximum (on N(0,1) data a wave saw one in about three half steps).
  // moved[r]: whether any row of block r moved its reference max in the last
  // softmax, a wave-wide vote taken right after the max, so the rescale
  // branch does not wait for the exponential that gives the factor.
  // The softmax is cut into kSmPieces pieces -- 4 of the row max, the
  // reference decision, 8 pairs of weights, the running sum -- so that one
  // region can spread it between its MFMAs in source order (qk_softmax).
  bool moved[RB] = {};
  struct SmState { float tmax, alpha, neg_m, psum; };
  constexpr int kSmPieces = 14;
  auto sm_piece = [&](int i, const f32x16_t& sc, int r, u32x4_t (&pk)[2], SmState& st) {
    if (i < 4) {
#pragma unroll
      for (int v = 4 * i; v < 4 * i + 4; ++v) st.tmax = fmaxf(st.tmax, sc[v]);
    } else if (i == 4) {
      const float tmax = max_xor32(st.tmax);  // lanes l and l^32 hold one row: same decision
      const float m_old = m_run[r];
      const float m_new = fmaxf(m_old, tmax);
      const bool move = !(m_new * a.scale_log2 - m_old * a.scale_log2 <= 8.f);  // also from -inf
      moved[r] = __any(move);
      const float m_ref = move ? m_new : m_old;
      const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
      st.alpha = move ? fast_exp2((m_old - m_use) * a.scale_log2) : 1.f;
      st.neg_m = -m_use * a.scale_log2;
      m_run[r] = m_ref;
    } else if (i < 13) {
      const int e = i - 5;  // weights of values 2e, 2e + 1
      const float p0 = fast_exp2(fmaf(sc[2 * e], a.scale_log2, st.neg_m));
      const float p1 = fast_exp2(fmaf(sc[2 * e + 1], a.scale_log2, st.neg_m));
      const uint32_t w2 = pack_bf16x2(p0, p1);
      pk[e >> 2][e & 3] = w2;
      st.psum = dot2_bf16(w2, kBf16PairOne, st.psum);  // the same rounded weights P.V uses
    } else {
      l_run[r] = l_run[r] * st.alpha + st.psum;
    }
  };
  auto softmax = [&](const f32x16_t& sc, int r, u32x4_t (&pk)[2]) -> float {
    SmState st{-INFINITY, 1.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kSmPieces; ++j) sm_piece(j, sc, r, pk, st);
    return st.alpha;
  };
  // S = K Q^T of the next key block (both row blocks, MFMAs alternating
  // between them) with the softmax of row block r of the current block spread
  // between the MFMAs.  Written out in this order because the compiler's
  // scheduler, asked to interleave the two (as for the P.V region below),
  // put the whole softmax after the last MFMA at D = 128, where registers
  // are tightest.
  auto qk_softmax = [&](const u32x4_t (&kf)[KS], f32x16_t& s0, f32x16_t& s1, const f32x16_t& sc, int r,
                        u32x4_t (&pk)[2]) -> float {
    SmState st{-INFINITY, 1.f, 0.f, 0.f};
    s0 = s1 = f32x16_t{};
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) {
      if (i & 1) s1 = mfma_bf16(kf[i >> 1], qf[1][i >> 1], s1);
      else s0 = mfma_bf16(kf[i >> 1], qf[0][i >> 1], s0);
#pragma unroll
      for (int j = i * kSmPieces / (2 * KS); j < (i + 1) * kSmPieces / (2 * KS); ++j) sm_piece(j, sc, r, pk, st);
    }
    return st.alpha;
  };
  auto rescale = [&](int r, float alpha) {
    if (moved[r]) {  // no row max moved: the accumulators need no rescale
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[r][m] *= alpha;
    }
  };
  // O_r += V^T P_r^T over one key block for both row blocks; lane l of the A
  // operand holds channel 32 m + l % 32 for keys 8 (l / 32) .. + 7 of a
  // 16-key slice, gathered by two transposing reads (as in chunk_tile_bf16):
  // in the 16-lane group tq, lane 4 tx + ty reads channels
  // 32 m + 16 (tq % 2) + 4 ty .. + 3 of step row 32 kb + 16 u + 8 (tq / 2) +
  // 4 r + tx, whose 16-byte chunk 4 m + vx sits at chunk (4 m + vx) ^ vswz(row)
  auto load_v = [&](const unsigned char* Vs, int kb, u32x4_t (&vf)[NM][2]) {
    uint32_t vofs = vofs0;
    asm volatile("" : "+v"(vofs));
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const uint32_t o = vofs ^ static_cast<uint32_t>(64 * m);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const u32x2_t t2 = lds_read_tr16(Vs + (kb * 32 + 16 * u + 4 * rr) * ROW + o);
          vf[m][u][2 * rr] = t2[0];
          vf[m][u][2 * rr + 1] = t2[1];
        }
    }
  };
  auto pv = [&](const u32x4_t (&vf)[NM][2], const u32x4_t (&p0)[2], const u32x4_t (&p1)[2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        acc[0][m] = mfma_bf16(vf[m][u], p0[u], acc[0][m]);
        acc[1][m] = mfma_bf16(vf[m][u], p1[u], acc[1][m]);
      }
  };
  // order of the P.V region: its 2 KS MFMAs, each followed by up to five VALU
  // instructions of the softmax that runs under them (the region's K operand
  // reads are left where the compiler puts them)
  auto interleave = [&]() {
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 0, 0);  // no LDS read
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // VALU
    }
  };

  // ---- the pipeline over half steps h (key block h % 2 of step h / 2).
  // Unit h: S(h+1) = K(h+1) Q^T under the softmax of row block 1 of h, then
  // O += V(h) P(h)^T under the softmax of row block 0 of h + 1.  Every wave
  // runs every half step of the tile: blocks past the wave's rows are masked
  // to nothing (m, l and O unchanged), which costs only time the wave would
  // otherwise wait at the barrier.  Four LDS stages, step j in stage j % 4:
  // step j's iteration reads stages j and j + 1 and loads step j + 3 into
  // the stage step j - 1 was the last to read.
  issue_step(0, page_ref(0), st0);
  issue_step(BN, page_ref(BN), st1);
  issue_step(2 * BN, page_ref(2 * BN), st2);
  PageRef nref = page_ref(3 * BN);
  __builtin_amdgcn_s_waitcnt(kWaitTwoSteps);  // step 0 landed
  stage_barrier();
  f32x16_t sa, sb;  // S of the next half step, row blocks 0 and 1
  u32x4_t p0[2], p1[2];
  u32x4_t kf[KS];     // K operands of the next half step
  u32x4_t vf[NM][2];  // V^T operands of the current half step
  load_k(st0, 0, kf);
  qk(kf, sa, sb);
  if (31 > H0 + wrow0) {
    mask(0, sa, 0);
    mask(0, sb, 1);
  }
  rescale(0, softmax(sa, 0, p0));
  load_k(st0, 1, kf);
  __builtin_amdgcn_s_waitcnt(kWaitOneStep);  // step 1 landed
  stage_barrier();

  // unit h = 2 j + kb (cur holds step j, nxt step j + 1).  Operand reads run
  // one region ahead: region 1 reads V(h) for region 2, region 2 reads
  // K(h+2) -- key block kb of step j + 1 -- for the next unit's region 1.
  // An empty asm use of a region's softmax results ends the region: the
  // compiler would otherwise sink the weights' arithmetic to their first use,
  // past the MFMAs it is meant to run under.
  auto pin = [](u32x4_t (&pk)[2], float& alpha) {
    asm volatile("" : "+v"(pk[0]), "+v"(pk[1]), "+v"(alpha));
  };
  auto unit = [&](int h, const unsigned char* cur, const unsigned char* nxt, int kb) {
    const f32x16_t sc = sb;  // S of half step h, row block 1
    load_v(cur + POOL, kb, vf);
    float alpha1 = qk_softmax(kf, sa, sb, sc, 1, p1);
    pin(p1, alpha1);
    const int kn = (h + 1) * 32;  // first key of half step h + 1
    if (kn + 31 > H0 + wrow0) {
      mask(kn, sa, 0);
      mask(kn, sb, 1);
    }
    rescale(1, alpha1);
    u32x4_t pn[2];
    load_k(nxt, kb, kf);
    pv(vf, p0, p1);
    float alpha0 = softmax(sa, 0, pn);
    interleave();
    pin(pn, alpha0);
    rescale(0, alpha0);
    p0[0] = pn[0];
    p0[1] = pn[1];
  };
  auto iteration = [&](int j, const unsigned char* cur, const unsigned char* nxt, unsigned char* ld) {
    const int k0 = j * BN;
    issue_step(k0 + 3 * BN, nref, ld);
    unit(2 * j, cur, nxt, 0);
    unit(2 * j + 1, cur, nxt, 1);
    __builtin_amdgcn_sched_barrier(0);
    nref = page_ref(k0 + 4 * BN);
    // step j + 2 has landed (j + 3 may still stream); after the barrier every
    // wave's has, and stage j is free
    __builtin_amdgcn_s_waitcnt(kWaitOneStep);
    stage_barrier();
  };
  // four steps per trip, so that each step's stages are fixed objects
  for (int j = 0; j < nsteps; j += 4) {
    iteration(j, st0, st1, st3);
    if (j + 1 < nsteps) iteration(j + 1, st1, st2, st0);
    if (j + 2 < nsteps) iteration(j + 2, st2, st3, st1);
    if (j + 3 < nsteps) iteration(j + 3, st3, st0, st2);
  }
  // no load may still write into LDS when the workgroup ends
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int my_row = wrow0 + 32 * r + qc;
    const float l_tot = sum_xor32(l_run[r]);  // lanes l and l^32 share a row
    if (my_row < 0 || my_row >= Lq) continue;
    const float inv = 1.f / l_tot;
    bf16_t* op = static_cast<bf16_t*>(a.out) + (static_cast<size_t>(q0 + my_row) * a.num_heads + h) * D;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = m * 32 + i4 * 8 + g * 4;
        st8(op + d, u32x2_t{pack_bf16x2(acc[r][m][4 * i4] * inv, acc[r][m][4 * i4 + 1] * inv),
                            pack_bf16x2(acc[r][m][4 * i4 + 2] * inv, acc[r][m][4 * i4 + 3] * inv)});
      }
    }
  }
}

// One workgroup per (tile, head), tiles with the most keys first (the last
// tiles of a causal chunk, which are all whole); with Hq a multiple of 8 the tiles of one head all
// run on one XCD (workgroups go to XCDs round robin), sharing its L2.
template <int D, bool kContig>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(PrefillArgs p) {
  using Cfg = ChunkCfg<bf16_t>::Sizes<D>;
  __shared__ __attribute__((aligned(16))) unsigned char st0[Cfg::STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st1[Cfg::STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st2[Cfg::STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st3[Cfg::STAGE];
  const int b = blockIdx.x;
  const int tile = p.ntiles - 1 - b / p.m.num_heads;
  const int h = b - (b / p.m.num_heads) * p.m.num_heads;
  int q0, lq, lk;
  if (!prefill_segment<kContig>(p, q0, lq, lk)) return;
  if (tile * kPrefillRows >= lq) return;
  prefill_tile_bf16<D, kContig>(p.m, h, tile, q0, lq, lk, st0, st1, st2, st3);
}


// ==================================================================== launch
namespace {

// Per-device attributes, queried on first use.  Calls from several host
// threads may query them at once: each writes the same value, through an
// atomic, so the race is benign.
struct DeviceInfo {
  std::atomic<int> cus{0};
  std::atomic<int> slots[2][2][2] = {};  // [dtype][D == 128][split-capable] resident workgroups per CU
};

DeviceInfo g_info[64];

hipError_t occupancy(DeviceInfo& info, int dt, int di, int ds, const void* kernel, int& grid) {
  int n = info.slots[dt][di][ds].load(std::memory_order_relaxed);
  if (n == 0) {
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kThreads, 0);
    if (e != hipSuccess) return e;
    n = n > 0 ? n : 1;
    info.slots[dt][di][ds].store(n, std::memory_order_relaxed);
  }
  grid = info.cus.load(std::memory_order_relaxed) * n;
  return hipSuccess;
}

// Second stream and fork/join events of the two-stream baseline, per device,
// created on first use (default priority) under the device's lock.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  std::mutex lock;  // creation, then the record / wait / launch sequence of each call
};
SideStream g_side[64];

// Returns the device's side stream with its lock held by `held`.
hipError_t side_stream(int dev, SideStream*& out, std::unique_lock<std::mutex>& held) {
  SideStream& s = g_side[dev];
  held = std::unique_lock<std::mutex>(s.lock);
  if (!s.stream) {
    hipError_t e = hipStreamCreateWithFlags(&s.stream, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&s.fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&s.join, hipEventDisableTiming);
    if (e != hipSuccess) return e;
  }
  out = &s;
  return hipSuccess;
}

template <typename T, int D, bool kSplit, bool kContig, bool kDefer>
void launch_attn(const MainArgs& ma, int grid, hipStream_t st) {
  hipLaunchKernelGGL((attn_kernel<T, D, kSplit, kContig, kDefer>), dim3(grid), dim3(kThreads), 0, st, ma);
}

// A bf16 step that is one prefill chunk with at least one (256-row tile, head)
// pair per CU: the append (hybrid_step_fwd), then prefill_kernel -- no
// planner, no combine.  Returns false when the step is not of that kind.
template <int D, bool kContig>
bool run_prefill(const AttnLaunch& L, int cus, hipError_t& e) {
  if (L.launch_mode != kLaunchFused || L.num_seqs != 1 || L.max_seqlen_q < 2) return false;
  const long long ntiles = (static_cast<long long>(L.max_seqlen_q) + kPrefillRows - 1) / kPrefillRows;
  const long long wgs = ntiles * L.num_heads;
  if (wgs < cus || wgs > 0x7fffffffLL) return false;
  if (L.append_key) {
    e = launch_kv_append(L.append_key, L.append_value, L.slot_mapping, const_cast<void*>(L.k_cache),
                         const_cast<void*>(L.v_cache), L.total_q, L.num_kv_heads, L.head_dim,
                         L.num_blocks, 1, L.stream);
    if (e != hipSuccess) return true;
  }
  PrefillArgs p{};
  p.m.q = L.q;
  p.m.kc = L.k_cache;
  p.m.vc = L.v_cache;
  p.m.out = L.out;
  p.m.cu = L.cu_seqlens_q;
  p.m.sk = L.seqlens_k;
  p.m.bt = L.block_table;
  p.m.num_seqs = 1;
  p.m.num_heads = L.num_heads;
  p.m.num_kv_heads = L.num_kv_heads;
  p.m.group = L.num_heads / L.num_kv_heads;
  p.m.num_blocks = L.num_blocks;
  p.m.max_blocks = L.max_blocks;
  p.m.scale_log2 = L.sm_scale * kLog2e;
  p.m.cu_k = kContig ? L.cu_seqlens_k : nullptr;
  p.total_q = L.total_q;
  p.max_q = L.max_seqlen_q;
  p.max_k = L.max_seqlen_k;
  p.total_k = L.total_k;
  p.ntiles = static_cast<int>(ntiles);
  hipLaunchKernelGGL((prefill_kernel<D, kContig>), dim3(static_cast<unsigned>(wgs)), dim3(kThreads), 0,
                     L.stream, p);
  e = hipGetLastError();
  return true;
}

template <typename T, int D, bool kContig>
hipError_t run(const AttnLaunch& L, DeviceInfo& info, int dev, int dt, int di) {
  constexpr bool kF32 = sizeof(T) == 4;
  if constexpr (!kF32) {
    hipError_t e = hipSuccess;
    if (run_prefill<D, kContig>(L, info.cus.load(std::memory_order_relaxed), e)) return e;
  }
  // Chunk tiles may be split only when even the largest number of them the
  // bounds allow (tiles_cap per head) fills at most half of split_items; every
  // other step runs the instance without the split code.
  int grid = 0;
  hipError_t e = occupancy(info, dt, di, 0,
                           reinterpret_cast<const void*>(attn_kernel<T, D, false, kContig, kF32>), grid);
  if (e != hipSuccess) return e;
  // For bf16, splitting pays only while it brings idle CUs into use: a second
  // item on a CU shares its MFMA and LDS with the first (measured: a bf16 chunk
  // of 8 tiles x 32 heads split in two ran 40 % slower), so splits stop at one
  // item per CU.  fp32 tiles leave a CU underused with one workgroup (long
  // fp32 MFMA chains): there they go up to one item per resident workgroup
  // (worked example: 238 us against 308 us with one item per CU).
  const int split_items = sizeof(T) == 4 ? grid : info.cus.load(std::memory_order_relaxed);
  const bool split_ok = L.ws.chunk_slots_cap >= 2 &&
                        2LL * L.ws.tiles_cap * L.num_heads <= static_cast<long long>(split_items);
  if (split_ok) {
    e = occupancy(info, dt, di, 1, reinterpret_cast<const void*>(attn_kernel<T, D, true, kContig, kF32>), grid);
    if (e != hipSuccess) return e;
  }
  SideStream* side = nullptr;
  std::unique_lock<std::mutex> side_held;  // held until the call has enqueued its launches
  if (L.launch_mode == kLaunchTwoStreams) {
    e = side_stream(dev, side, side_held);
    if (e != hipSuccess) return e;
  }
  // workgroups per launch and how many of them start on the chunk queues
  const int half = (grid + 1) / 2;
  int chunk_first_wgs = half, dec_first_wgs = grid - half;  // fused
  if (L.launch_mode == kLaunchSerial) {
    chunk_first_wgs = grid;
    dec_first_wgs = grid;
  } else if (L.launch_mode == kLaunchTwoStreams) {
    chunk_first_wgs = half;
    dec_first_wgs = grid - half;
  }
  unsigned char* ws = L.workspace;
  PlanHeader* hdr = reinterpret_cast<PlanHeader*>(ws);
  int32_t* tile_prefix = reinterpret_cast<int32_t*>(ws + L.ws.tile_prefix);
  int32_t* dec_prefix = reinterpret_cast<int32_t*>(ws + L.ws.dec_prefix);
  int32_t* part_prefix = reinterpret_cast<int32_t*>(ws + L.ws.part_prefix);
  int32_t* tail_prefix = reinterpret_cast<int32_t*>(ws + L.ws.tail_prefix);
  int32_t* seqlens = reinterpret_cast<int32_t*>(ws + L.ws.seqlens);
  const int head_groups = (L.num_heads + kHeadsPerDecodeItem - 1) / kHeadsPerDecodeItem;

  // cost of a 64-key chunk step in decode (key, head) pairs, measured roughly on
  // MI355X: a bf16 step at D = 128 takes about as long as streaming 128 decode
  // keys of one head; fp32 and D = 64 steps cost relatively more
  const int chunk_step_cost = (sizeof(T) == 4 || D == 64) ? 192 : 128;
  PlanArgs pa{L.cu_seqlens_q, L.seqlens_k, L.num_seqs, L.total_q, L.max_seqlen_q, L.max_seqlen_k,
              L.max_blocks, L.num_heads, head_groups, L.ws.parts_cap, grid * kItemsPerSlot,
              grid, L.ws.tiles_cap, split_ok ? L.ws.chunk_slots_cap : 0, chunk_first_wgs,
              dec_first_wgs, split_items, chunk_step_cost, kContig ? L.cu_seqlens_k : nullptr,
              L.total_k, kContig ? seqlens : nullptr, hdr, tile_prefix, dec_prefix, part_prefix,
              tail_prefix, chunk_group_sub(sizeof(T) == 4, L.num_heads),
              sizeof(T) == 4 && L.launch_mode == kLaunchFused ? 1 : 0};
  // hybrid_step_fwd: the append first -- with the small planner in the same
  // launch when the step has few segments, else on its own
  const long long chunks_per_row = static_cast<long long>(L.num_kv_heads) * L.head_dim * sizeof(T) / 16;
  const long long append_wgs = chunks_per_row >= kThreads / 2
                                   ? L.total_q
                                   : (L.total_q * chunks_per_row + kThreads - 1) / kThreads;
  const bool fused_append = L.append_key && L.num_seqs <= kPlanSmallSegments &&
                            append_wgs < 0x7fffffffLL;
  if (L.append_key && !fused_append) {
    e = launch_kv_append(L.append_key, L.append_value, L.slot_mapping, const_cast<void*>(L.k_cache),
                         const_cast<void*>(L.v_cache), L.total_q, L.num_kv_heads, L.head_dim,
                         L.num_blocks, sizeof(T) == 4 ? 0 : 1, L.stream);
    if (e != hipSuccess) return e;
  }
  if (fused_append) {
    const AppendRows rows{static_cast<const uint4*>(L.append_key), static_cast<const uint4*>(L.append_value),
                          L.slot_mapping, static_cast<uint4*>(const_cast<void*>(L.k_cache)),
                          static_cast<uint4*>(const_cast<void*>(L.v_cache)),
                          static_cast<int>(chunks_per_row), static_cast<long long>(L.num_blocks) * kPage,
                          L.total_q};
    hipLaunchKernelGGL(append_plan_kernel, dim3(static_cast<unsigned>(append_wgs) + 1), dim3(kThreads), 0,
                       L.stream, pa, rows);
  } else if (L.num_seqs <= kPlanSmallSegments) {
    hipLaunchKernelGGL(plan_kernel_small, dim3(1), dim3(kWave), 0, L.stream, pa);
  } else {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, L.stream, pa);
  }

  MainArgs ma{L.q, L.k_cache, L.v_cache, L.out, L.cu_seqlens_q,
              kContig ? seqlens : L.seqlens_k, L.block_table,
              L.num_seqs, L.num_heads, L.num_kv_heads, L.num_heads / L.num_kv_heads,
              L.num_blocks, L.max_blocks, L.ws.part_stride, L.sm_scale * kLog2e, hdr,
              tile_prefix, dec_prefix, part_prefix, tail_prefix,
              reinterpret_cast<float*>(ws + L.ws.partials),
              reinterpret_cast<float*>(ws + L.ws.chunk_partials), L.cu_seqlens_k, 3, half};
  // Unsplit steps run the instance with deferred claims (kDefer): a chunk item,
  // or a long decode item, does not reserve its successor while it runs.  With
  // early claims a 1984-token chunk + 64 decodes (64 heads) ran 3157 us against
  // 3035 (chunk items reserved behind chunk items), and the steps with long
  // decode histories ended on workgroups that had reserved a full split behind
  // a full split (130K-token chunk + 64 decodes, 256 decodes of up to 32K
  // keys: 0.6-0.8 % slower); the two-chunk mixed step measures the same
  // either way.  The split instance keeps early claims for bf16.
  auto attn = split_ok ? launch_attn<T, D, true, kContig, kF32> : launch_attn<T, D, false, kContig, true>;
  if (L.launch_mode == kLaunchFused) {
    attn(ma, grid, L.stream);
  } else {
    MainArgs mc = ma, md = ma;
    mc.roles = 1;
    md.roles = 2;
    md.chunk_wgs = 0;
    if (L.launch_mode == kLaunchSerial) {
      mc.chunk_wgs = grid;
      attn(mc, grid, L.stream);
      attn(md, grid, L.stream);
    } else {
      mc.chunk_wgs = half;
      e = hipEventRecord(side->fork, L.stream);
      if (e == hipSuccess) e = hipStreamWaitEvent(side->stream, side->fork, 0);
      if (e != hipSuccess) return e;
      attn(mc, half, side->stream);
      e = hipEventRecord(side->join, side->stream);
      if (e != hipSuccess) return e;
      attn(md, grid - half, L.stream);
      e = hipStreamWaitEvent(L.stream, side->join, 0);
      if (e != hipSuccess) return e;
    }
  }
  const int merge_blocks = split_ok ? kChunkMergeBlocks : 0;
  hipLaunchKernelGGL((combine_kernel<T, D>), dim3(L.num_seqs * head_groups + merge_blocks),
                     dim3(kThreads), 0, L.stream, ma);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnLaunch& L) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  DeviceInfo& info = g_info[dev];
  if (info.cus.load(std::memory_order_relaxed) == 0) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    info.cus.store(cus, std::memory_order_relaxed);
  }
  if (L.cu_seqlens_k) {
    if (L.dtype == 1) {
      return L.head_dim == 128 ? run<bf16_t, 128, true>(L, info, dev, 1, 1)
                               : run<bf16_t, 64, true>(L, info, dev, 1, 0);
    }
    return L.head_dim == 128 ? run<float, 128, true>(L, info, dev, 0, 1)
                             : run<float, 64, true>(L, info, dev, 0, 0);
  }
  if (L.dtype == 1) {
    return L.head_dim == 128 ? run<bf16_t, 128, false>(L, info, dev, 1, 1)
                             : run<bf16_t, 64, false>(L, info, dev, 1, 0);
  }
  return L.head_dim == 128 ? run<float, 128, false>(L, info, dev, 0, 1)
                           : run<float, 64, false>(L, info, dev, 0, 0);
}

}  // namespace ha
