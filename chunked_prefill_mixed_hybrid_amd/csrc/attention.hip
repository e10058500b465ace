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
//       - decode role: 4 waves = 4 heads of one (segment, KV split); each wave
//         streams its head's rows of 64 keys per step with 16-byte loads,
//         reduces the 16-lane partial dot products with a butterfly
//         reduce-scatter, and keeps fp32 (m, l, acc) per lane.  Splits of a
//         segment write partial (m, l, acc) rows that combine_kernel merges.
#include "ha_common.hpp"
#include "ha_internal.hpp"

namespace ha {

// ==================================================================== plan
struct PlanArgs {
  const int32_t* cu;
  const int32_t* sk;
  int num_seqs, total_q, max_q, max_k, max_blocks, num_heads, head_groups, parts_cap,
      target_items;
  PlanHeader* hdr;
  int32_t* chunk_prefix;
  int32_t* dec_prefix;
  int32_t* part_prefix;
};

constexpr int kPlanThreads = 1024;

// Segment shape and whether it meets the documented preconditions; segments
// that do not are skipped (no work items, output rows untouched).
__device__ __forceinline__ bool plan_segment(const PlanArgs& a, int b, int& lq, int& lk) {
  const int c0 = a.cu[b], c1 = a.cu[b + 1];
  lq = c1 - c0;
  lk = a.sk[b];
  return c0 >= 0 && c1 >= c0 && c1 <= a.total_q && lq <= lk && lk <= a.max_k &&
         lq <= a.max_q && ((lk + kPage - 1) / kPage) <= a.max_blocks;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ long long s_items[32][32];
  __shared__ long long s_parts[32][32];
  __shared__ int s_split_log;
  __shared__ int s_wave_tot[kPlanThreads / kWave][3];
  __shared__ int s_carry[3];
  __shared__ int s_pass_tot[3];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  if (tid == 0) s_bad = 0;

  // 1. decode work and partial-slot counts for every candidate split size.
  {
    const int k = tid & 31, grp = tid >> 5;
    long long items = 0, parts = 0;
    if (k < kSplitCandidates) {
      const long long split = static_cast<long long>(kSplitMin) << k;
      for (int b = grp; b < a.num_seqs; b += 32) {
        int lq, lk;
        if (!plan_segment(a, b, lq, lk) || lq != 1) continue;
        const long long n = (lk + split - 1) / split;
        items += n;
        parts += n > 1 ? n : 0;
      }
    }
    s_items[grp][k] = items;
    s_parts[grp][k] = parts;
  }
  __syncthreads();
  if (tid < 32) {
    long long items = 0, parts = 0;
    for (int g = 0; g < 32; ++g) {
      items += s_items[g][tid];
      parts += s_parts[g][tid];
    }
    s_items[0][tid] = items;
    s_parts[0][tid] = parts;
  }
  __syncthreads();
  if (tid == 0) {
    // smallest split that fits the partial slots and keeps the decode item
    // count near the target; the largest candidate (2^30 keys) always fits.
    int pick = kSplitCandidates - 1;
    for (int k = 0; k < kSplitCandidates; ++k) {
      if (s_parts[0][k] <= a.parts_cap &&
          s_items[0][k] * a.head_groups <= static_cast<long long>(a.target_items)) {
        pick = k;
        break;
      }
    }
    s_split_log = pick;
    for (int c = 0; c < 3; ++c) s_carry[c] = 0;
  }
  __syncthreads();
  const int split = kSplitMin << s_split_log;

  // 2. exclusive prefix sums of chunk items, decode items and partial slots.
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  for (int base = 0; base < a.num_seqs; base += kPlanThreads) {
    const int b = base + tid;
    int v[3] = {0, 0, 0};
    if (b < a.num_seqs) {
      int lq, lk;
      if (!plan_segment(a, b, lq, lk)) {
        atomicAdd(&s_bad, 1);
      } else if (lq >= 2) {
        v[0] = ((lq + kChunkRows - 1) / kChunkRows) * a.num_heads;
      } else if (lq == 1) {
        const int n = (lk + split - 1) / split;
        v[1] = n * a.head_groups;
        v[2] = n > 1 ? n : 0;
      }
    }
    int incl[3] = {v[0], v[1], v[2]};
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
#pragma unroll
      for (int c = 0; c < 3; ++c) {
        const int o = __shfl_up(incl[c], off);
        if (lane >= off) incl[c] += o;
      }
    }
    if (lane == kWave - 1)
      for (int c = 0; c < 3; ++c) s_wave_tot[wave][c] = incl[c];
    __syncthreads();
    if (tid < 3) {
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
      a.chunk_prefix[b] = s_carry[0] + s_wave_tot[wave][0] + incl[0] - v[0];
      a.dec_prefix[b] = s_carry[1] + s_wave_tot[wave][1] + incl[1] - v[1];
      a.part_prefix[b] = s_carry[2] + s_wave_tot[wave][2] + incl[2] - v[2];
    }
    __syncthreads();
    if (tid < 3) s_carry[tid] += s_pass_tot[tid];
    __syncthreads();
  }
  if (tid == 0) {
    a.chunk_prefix[a.num_seqs] = s_carry[0];
    a.dec_prefix[a.num_seqs] = s_carry[1];
    a.part_prefix[a.num_seqs] = s_carry[2];
    a.hdr->n_chunk_items = s_carry[0];
    a.hdr->n_dec_items = s_carry[1];
    a.hdr->n_parts = s_carry[2];
    a.hdr->split = split;
    a.hdr->bad_segments = s_bad;
    a.hdr->counter = 0;
  }
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
  const int32_t* chunk_prefix;
  const int32_t* dec_prefix;
  const int32_t* part_prefix;
  float* partials;
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

template <typename T> struct ChunkCfg;
template <> struct ChunkCfg<bf16_t> {
  template <int D> struct Sizes {
    static constexpr int BN = 64;
    static constexpr int KROW = (D + 8) * 2;   // bytes per key row of the K tile
    static constexpr int VROW = (BN + 8) * 2;  // bytes per channel row of V^T
    static constexpr int BYTES = BN * KROW + D * VROW;
  };
};
template <> struct ChunkCfg<float> {
  template <int D> struct Sizes {
    static constexpr int BN = D == 128 ? 32 : 64;
    static constexpr int ROWF = D + 4;  // floats per key row (K and V)
    static constexpr int BYTES = 2 * BN * ROWF * 4;
  };
};

// ---------------------------------------------------------------- chunk role, bf16
template <int D>
__device__ void chunk_tile_bf16(const MainArgs& a, int seg, int j, unsigned char* smem) {
  using Cfg = ChunkCfg<bf16_t>::Sizes<D>;
  constexpr int BN = Cfg::BN, NKB = BN / 32, KS = D / 16, NM = D / 32;
  constexpr int KROW = Cfg::KROW, VROW = Cfg::VROW;
  constexpr int CPR = D * 2 / 16;            // 16-byte chunks per key row
  constexpr int KLOADS = BN * CPR / kThreads;  // K chunks per thread per tile
  constexpr int VKG = BN * CPR / kThreads;     // keys per thread in the V transpose
  static_assert(KLOADS * kThreads == BN * CPR, "tile load must divide evenly");
  unsigned char* Ks = smem;
  unsigned char* Vt = smem + BN * KROW;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int qc = lane & 31, g = lane >> 5;
  const int q0 = a.cu[seg], Lq = a.cu[seg + 1] - q0, Lk = a.sk[seg], H0 = Lk - Lq;
  const int ntiles = (Lq + kChunkRows - 1) / kChunkRows;
  const int h = j / ntiles, tile = ntiles - 1 - (j - h * ntiles);
  const int kvh = h / a.group;
  const int row0 = tile * kChunkRows;
  const int rows_end = min(row0 + kChunkRows, Lq);
  const int kend = H0 + rows_end;  // keys [0, kend) are visible to some row of the tile
  const int wrow0 = row0 + w * 32;
  const int my_row = wrow0 + qc;
  const bool wave_active = wrow0 < rows_end;
  const int32_t* btrow = a.bt + static_cast<size_t>(seg) * a.max_blocks;
  const bf16_t* kc = static_cast<const bf16_t*>(a.kc);
  const bf16_t* vc = static_cast<const bf16_t*>(a.vc);
  const size_t slot_elems = static_cast<size_t>(a.num_kv_heads) * D;
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

  f32x16_t acc[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) acc[m] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;

  for (int k0 = 0; k0 < kend; k0 += BN) {
    __syncthreads();  // previous tile fully consumed
    // K tile, natural layout Ks[key][d]
#pragma unroll
    for (int it = 0; it < KLOADS; ++it) {
      const int idx = it * kThreads + tid;
      const int key = idx / CPR, c = idx % CPR, kp = k0 + key;
      u32x4_t v = {0, 0, 0, 0};
      if (kp < Lk) {
        const int page = btrow[kp >> 4];
        if (static_cast<unsigned>(page) < static_cast<unsigned>(a.num_blocks))
          v = ld16(kc + (static_cast<size_t>(page) * kPage + (kp & 15)) * slot_elems +
                   static_cast<size_t>(kvh) * D + c * 8);
      }
      st16(Ks + key * KROW + c * 16, v);
    }
    // V tile, transposed: Vt[d][key]; thread owns chunk c (8 channels) of VKG keys
    {
      const int c = tid % CPR, kg = tid / CPR;
      u32x4_t v[VKG];
#pragma unroll
      for (int t = 0; t < VKG; ++t) {
        const int kp = k0 + kg * VKG + t;
        v[t] = u32x4_t{0, 0, 0, 0};
        if (kp < Lk) {
          const int page = btrow[kp >> 4];
          if (static_cast<unsigned>(page) < static_cast<unsigned>(a.num_blocks))
            v[t] = ld16(vc + (static_cast<size_t>(page) * kPage + (kp & 15)) * slot_elems +
                        static_cast<size_t>(kvh) * D + c * 8);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t hv[VKG];
#pragma unroll
        for (int t = 0; t < VKG; ++t) {
          const uint32_t word = v[t][e >> 1];
          hv[t] = (e & 1) ? (word >> 16) : (word & 0xffffu);
        }
        unsigned char* dst = Vt + (c * 8 + e) * VROW + kg * VKG * 2;
        if constexpr (VKG == 4) {
          st8(dst, u32x2_t{hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16)});
        } else {
          static_assert(VKG == 2, "V transpose handles 2 or 4 keys per thread");
          *reinterpret_cast<uint32_t*>(dst) = hv[0] | (hv[1] << 16);
        }
      }
    }
    __syncthreads();
    if (!wave_active || k0 > H0 + wrow0 + 31) continue;  // tile invisible to this wave
    const bool need_mask = (k0 + BN - 1) > (H0 + wrow0);

    // S^T = K Q^T, two 32-key blocks
    f32x16_t sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sacc[kb] = f32x16_t{};
      const unsigned char* kr = Ks + (kb * 32 + pi) * KROW + g * 16;
#pragma unroll
      for (int s = 0; s < KS; ++s) sacc[kb] = mfma_bf16(ld16(kr + s * 32), qf[s], sacc[kb]);
    }
    // scale (base 2), causal mask on diagonal tiles, running max
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = sacc[kb][v] * a.scale_log2;
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
    u32x4_t pk[NKB][2];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const float p0 = fast_exp2(sacc[kb][8 * u + 2 * e2] - m_use);
          const float p1 = fast_exp2(sacc[kb][8 * u + 2 * e2 + 1] - m_use);
          psum += p0 + p1;
          pk[kb][u][e2] = pack_bf16x2(p0, p1);
        }
      }
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[m] *= alpha;
    // O^T += V^T P^T
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const unsigned char* vr = Vt + (m * 32 + qc) * VROW + g * 16;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int u = 0; u < 2; ++u) acc[m] = mfma_bf16(ld16(vr + (kb * 32 + u * 16) * 2), pk[kb][u], acc[m]);
      }
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);  // lanes l and l^32 share a row
  if (!wave_active || my_row >= Lq) return;
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
template <int D>
__device__ void chunk_tile_f32(const MainArgs& a, int seg, int j, unsigned char* smem) {
  using Cfg = ChunkCfg<float>::Sizes<D>;
  constexpr int BN = Cfg::BN, NKB = BN / 32, KS = D / 2, NM = D / 32, ROWF = Cfg::ROWF;
  constexpr int CPR = D / 4;
  constexpr int LOADS = BN * CPR / kThreads;
  static_assert(LOADS * kThreads == BN * CPR, "tile load must divide evenly");
  float* Ks = reinterpret_cast<float*>(smem);
  float* Vs = Ks + BN * ROWF;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int qc = lane & 31, g = lane >> 5;
  const int q0 = a.cu[seg], Lq = a.cu[seg + 1] - q0, Lk = a.sk[seg], H0 = Lk - Lq;
  const int ntiles = (Lq + kChunkRows - 1) / kChunkRows;
  const int h = j / ntiles, tile = ntiles - 1 - (j - h * ntiles);
  const int kvh = h / a.group;
  const int row0 = tile * kChunkRows;
  const int rows_end = min(row0 + kChunkRows, Lq);
  const int kend = H0 + rows_end;
  const int wrow0 = row0 + w * 32;
  const int my_row = wrow0 + qc;
  const bool wave_active = wrow0 < rows_end;
  const int32_t* btrow = a.bt + static_cast<size_t>(seg) * a.max_blocks;
  const float* kc = static_cast<const float*>(a.kc);
  const float* vc = static_cast<const float*>(a.vc);
  const size_t slot_elems = static_cast<size_t>(a.num_kv_heads) * D;
  const int pi = key_perm(qc);

  float qf[KS];  // lane supplies Q[my_row][2s + g]
  {
    const bool ok = my_row < Lq;
    const float* qp = static_cast<const float*>(a.q) +
                      (static_cast<size_t>(q0 + (ok ? my_row : 0)) * a.num_heads + h) * D + g;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = ok ? qp[2 * s] : 0.f;
  }
  f32x16_t acc[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) acc[m] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;

  for (int k0 = 0; k0 < kend; k0 += BN) {
    __syncthreads();
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int idx = it * kThreads + tid;
      const int key = idx / CPR, c = idx % CPR, kp = k0 + key;
      u32x4_t kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
      if (kp < Lk) {
        const int page = btrow[kp >> 4];
        if (static_cast<unsigned>(page) < static_cast<unsigned>(a.num_blocks)) {
          const size_t off = (static_cast<size_t>(page) * kPage + (kp & 15)) * slot_elems +
                             static_cast<size_t>(kvh) * D + c * 4;
          kv = ld16(kc + off);
          vv = ld16(vc + off);
        }
      }
      st16(Ks + key * ROWF + c * 4, kv);
      st16(Vs + key * ROWF + c * 4, vv);
    }
    __syncthreads();
    if (!wave_active || k0 > H0 + wrow0 + 31) continue;
    const bool need_mask = (k0 + BN - 1) > (H0 + wrow0);

    f32x16_t sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sacc[kb] = f32x16_t{};
      const float* kr = Ks + (kb * 32 + pi) * ROWF + g;
#pragma unroll
      for (int s = 0; s < KS; ++s) sacc[kb] = mfma_f32(kr[2 * s], qf[s], sacc[kb]);
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = sacc[kb][v] * a.scale_log2;
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
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[m] *= alpha;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int n = 0; n < 16; ++n) {
          const int key = kb * 32 + ((n >> 3) << 4) + (g << 3) + (n & 7);
          acc[m] = mfma_f32(Vs[key * ROWF + m * 32 + qc], sacc[kb][n], acc[m]);
        }
      }
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);  // lanes l and l^32 share a row
  if (!wave_active || my_row >= Lq) return;
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

template <typename T, int D>
__device__ void decode_item(const MainArgs& a, int seg, int j, int split_keys) {
  constexpr int EPL = D / 16;  // channels per lane
  using Frag = RowFrag<T, EPL>;
  constexpr bool kLateV = Frag::kWords > 4;  // fp32 D=128: load V after the scores
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int head_groups = (a.num_heads + kHeadsPerDecodeItem - 1) / kHeadsPerDecodeItem;
  const int split = j / head_groups, hg = j - split * head_groups;
  const int h = hg * kHeadsPerDecodeItem + w;
  if (h >= a.num_heads) return;
  const int row = a.cu[seg], Lk = a.sk[seg];
  const int nsplit = (Lk + split_keys - 1) / split_keys;
  const int kbeg = split * split_keys, kfin = min(Lk, kbeg + split_keys);
  const int r = lane >> 4, c = lane & 15;
  const int kvh = h / a.group;
  const int32_t* btrow = a.bt + static_cast<size_t>(seg) * a.max_blocks;
  const size_t slot_elems = static_cast<size_t>(a.num_kv_heads) * D;
  const T* kbase = static_cast<const T*>(a.kc) + static_cast<size_t>(kvh) * D + c * EPL;
  const T* vbase = static_cast<const T*>(a.vc) + static_cast<size_t>(kvh) * D + c * EPL;

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
    for (int pp = 0; pp < 4; ++pp) pages[pp] = (kb + pp * 16 < kfin) ? btrow[(kb >> 4) + pp] : -1;
    Frag kf[16], vf[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int pg = pages[u >> 2];
      const bool ok = (kb + 4 * u + r < kfin) &&
                      static_cast<unsigned>(pg) < static_cast<unsigned>(a.num_blocks);
      const size_t off = (static_cast<size_t>(ok ? pg : 0) * kPage + 4 * (u & 3) + r) * slot_elems;
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
                        static_cast<unsigned>(pg) < static_cast<unsigned>(a.num_blocks);
        const size_t off = (static_cast<size_t>(ok ? pg : 0) * kPage + 4 * (u & 3) + r) * slot_elems;
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
  if (nsplit == 1) {
    if (r == 0) {
      const float inv = 1.f / l_tot;
      float o[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = acc[e] * inv;
      store_row<T, EPL>(static_cast<T*>(a.out) + (static_cast<size_t>(row) * a.num_heads + h) * D + c * EPL, o);
    }
  } else {
    float* pp = a.partials +
                (static_cast<size_t>(a.part_prefix[seg] + split) * a.num_heads + h) * a.part_stride;
    if (r == 0) store_row<float, EPL>(pp + 4 + c * EPL, acc);
    if (lane == 0) {
      pp[0] = m_run;
      pp[1] = l_tot;
    }
  }
}

// ---------------------------------------------------------------- persistent kernel
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void attn_kernel(MainArgs a) {
  constexpr int kSmem = ChunkCfg<T>::template Sizes<D>::BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kSmem];
  __shared__ int s_work[3];
  const int n_chunk = a.hdr->n_chunk_items;
  const int n_total = n_chunk + a.hdr->n_dec_items;
  const int split_keys = a.hdr->split;
  for (;;) {
    if (threadIdx.x == 0) {
      const int it = static_cast<int>(atomicAdd(&a.hdr->counter, 1u));
      int seg = 0, local = 0;
      if (it < n_chunk) {
        seg = find_segment(a.chunk_prefix, a.num_seqs, it);
        local = it - a.chunk_prefix[seg];
      } else if (it < n_total) {
        seg = find_segment(a.dec_prefix, a.num_seqs, it - n_chunk);
        local = it - n_chunk - a.dec_prefix[seg];
      }
      s_work[0] = it;
      s_work[1] = seg;
      s_work[2] = local;
    }
    __syncthreads();
    const int it = s_work[0], seg = s_work[1], local = s_work[2];
    __syncthreads();
    if (it >= n_total) break;
    if (it < n_chunk) {
      if constexpr (sizeof(T) == 2) chunk_tile_bf16<D>(a, seg, local, smem);
      else chunk_tile_f32<D>(a, seg, local, smem);
    } else {
      decode_item<T, D>(a, seg, local, split_keys);
    }
  }
}

// ---------------------------------------------------------------- combine
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void combine_kernel(MainArgs a) {
  const int seg = blockIdx.x;
  const int p0 = a.part_prefix[seg], np = a.part_prefix[seg + 1] - p0;
  if (np <= 0) return;
  constexpr int EPL = D / kWave;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row = a.cu[seg];
  for (int h = w; h < a.num_heads; h += kThreads / kWave) {
    const float* base = a.partials + (static_cast<size_t>(p0) * a.num_heads + h) * a.part_stride;
    const size_t step = static_cast<size_t>(a.num_heads) * a.part_stride;
    float mx = -INFINITY;
    for (int s = 0; s < np; ++s) mx = fmaxf(mx, base[s * step]);
    float l = 0.f, o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = 0.f;
    for (int s = 0; s < np; ++s) {
      const float* pp = base + s * step;
      const float wgt = fast_exp2(pp[0] - mx);
      l = fmaf(pp[1], wgt, l);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = fmaf(pp[4 + lane * EPL + e], wgt, o[e]);
    }
    const float inv = 1.f / l;
    T* op = static_cast<T*>(a.out) + (static_cast<size_t>(row) * a.num_heads + h) * D + lane * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      if constexpr (sizeof(T) == 2) op[e] = static_cast<bf16_t>(f32_to_bf16_rne(o[e] * inv));
      else op[e] = o[e] * inv;
    }
  }
}

// ==================================================================== launch
namespace {

struct DeviceInfo {
  int cus = 0;
  int slots[2][2] = {{0, 0}, {0, 0}};  // [dtype][D == 128] resident workgroups per CU
};

DeviceInfo g_info[64];

template <typename T, int D>
hipError_t run(const AttnLaunch& L, DeviceInfo& info, int dt, int di) {
  if (info.slots[dt][di] == 0) {
    int n = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_kernel<T, D>, kThreads, 0);
    if (e != hipSuccess) return e;
    info.slots[dt][di] = n > 0 ? n : 1;
  }
  const int grid = info.cus * info.slots[dt][di];
  unsigned char* ws = L.workspace;
  PlanHeader* hdr = reinterpret_cast<PlanHeader*>(ws);
  int32_t* chunk_prefix = reinterpret_cast<int32_t*>(ws + L.ws.chunk_prefix);
  int32_t* dec_prefix = reinterpret_cast<int32_t*>(ws + L.ws.dec_prefix);
  int32_t* part_prefix = reinterpret_cast<int32_t*>(ws + L.ws.part_prefix);
  const int head_groups = (L.num_heads + kHeadsPerDecodeItem - 1) / kHeadsPerDecodeItem;

  PlanArgs pa{L.cu_seqlens_q, L.seqlens_k, L.num_seqs, L.total_q, L.max_seqlen_q, L.max_seqlen_k,
              L.max_blocks, L.num_heads, head_groups, L.ws.parts_cap, grid * kItemsPerSlot,
              hdr, chunk_prefix, dec_prefix, part_prefix};
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, L.stream, pa);

  MainArgs ma{L.q, L.k_cache, L.v_cache, L.out, L.cu_seqlens_q, L.seqlens_k, L.block_table,
              L.num_seqs, L.num_heads, L.num_kv_heads, L.num_heads / L.num_kv_heads,
              L.num_blocks, L.max_blocks, L.ws.part_stride, L.sm_scale * kLog2e, hdr,
              chunk_prefix, dec_prefix, part_prefix,
              reinterpret_cast<float*>(ws + L.ws.partials)};
  hipLaunchKernelGGL((attn_kernel<T, D>), dim3(grid), dim3(kThreads), 0, L.stream, ma);
  hipLaunchKernelGGL((combine_kernel<T, D>), dim3(L.num_seqs), dim3(kThreads), 0, L.stream, ma);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnLaunch& L) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  DeviceInfo& info = g_info[dev];
  if (info.cus == 0) {
    e = hipDeviceGetAttribute(&info.cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
  }
  if (L.dtype == 1) {
    return L.head_dim == 128 ? run<bf16_t, 128>(L, info, 1, 1) : run<bf16_t, 64>(L, info, 1, 0);
  }
  return L.head_dim == 128 ? run<float, 128>(L, info, 0, 1) : run<float, 64>(L, info, 0, 0);
}

}  // namespace ha
