// Device-side building blocks shared by the gfx950 kernels of libhybridattn:
// element types, 16-byte vector loads, MFMA wrappers and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ha {

constexpr int kWave = 64;         // CDNA wavefront width
constexpr int kPage = 16;         // tokens per KV page (the only page size supported)
constexpr float kLog2e = 1.4426950408889634f;

typedef uint16_t bf16_t;  // storage type of bfloat16 (upper half of an fp32)
// int32 data the kernels only read (block tables): viewed through the constant
// address space so uniform reads become scalar loads.
typedef const __attribute__((address_space(4))) int32_t const_i32_t;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// Two fp32 -> packed bf16 pair (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
// a.lo * b.lo + a.hi * b.hi + c on bf16 pairs, fp32 accumulate (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}
// Bytes [a.lo16, b.lo16] and [a.hi16, b.hi16] of two bf16 pairs.
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// ---- DPP lane exchanges inside rows of 16 lanes ---------------------------------------
constexpr int kDppRowMirror = 0x140;      // lane c <- lane 15 - c
constexpr int kDppRowHalfMirror = 0x141;  // lane c <- lane (c & 8) | (7 - (c & 7))
constexpr int kDppQuadReverse = 0x1B;     // quad_perm [3,2,1,0]
constexpr int kDppQuadSwap = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppRowBcast0 = 0x150;      // row_newbcast:n -> every lane gets lane n of its row
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kCtrl, 0xf, 0xf, false));
}
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<kCtrl>(__float_as_uint(v)));
}

// Element traits: T is float (fp32 storage) or bf16_t.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kBytes = 4;
  __device__ static float to_f32(float x) { return x; }
};
template <> struct Elem<bf16_t> {
  static constexpr int kBytes = 2;
  __device__ static float to_f32(bf16_t x) { return bf16_to_f32(x); }
};

// ---- buffer descriptors ---------------------------------------------------------------
// Word 3 of a raw (untyped, stride 0) buffer descriptor on the gfx9 family.
constexpr int kRawBufferWord3 = 0x00020000;
// A buffer offset past every descriptor's range: loads return 0.
constexpr uint32_t kOffsetOutOfRange = 0x80000000u;
// Cache-policy operand of a buffer load: nt (non-temporal) on gfx950 -- the
// lines are marked for early eviction, so a stream read once does not push
// reused data (chunk tiles' K/V shared through L2, partials) out of the caches.
constexpr int kLoadNonTemporal = 2;

// ---- 16-byte global / LDS accesses ------------------------------------------------
__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }
__device__ __forceinline__ u32x2_t ld8(const void* p) { return *reinterpret_cast<const u32x2_t*>(p); }
__device__ __forceinline__ void st8(void* p, u32x2_t v) { *reinterpret_cast<u32x2_t*>(p) = v; }

// ---- gfx950 LDS instructions ----------------------------------------------------------
// (The host compilation pass does not know these builtins; it sees the bodies
// only on the device pass.)
typedef short i16x4_t __attribute__((ext_vector_type(4)));
// Transposing 8-byte LDS read (ds_read_b64_tr_b16): within each group of 16
// lanes, lane 4x + y names 8 bytes (4 bf16 values); the read hands lane 4a + b
// value b of the 8-byte pieces named by lanes a, a + 4, a + 8, a + 12, in that
// order.
__device__ __forceinline__ u32x2_t lds_read_tr16(const unsigned char* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p));
#else
  (void)p;
  return u32x2_t{0, 0};
#endif
}
// Pool-to-LDS 16-byte load (buffer_load_dwordx4 ... lds): lane i writes LDS
// bytes dst + 16 i .. + 15 (dst uniform across the wave) with the 16 bytes at
// buffer offset off of rsrc; an offset past the descriptor's range writes zeros.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rsrc, unsigned char* dst, uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
#else
  (void)rsrc; (void)dst; (void)off;
#endif
}

// Index of this wave in its workgroup, as a scalar (uniform) value.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
}

// ---- wave reductions (64 lanes) --------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// ---- MFMA ---------------------------------------------------------------------------
// 32x32 output tiles.  For every 32x32xK MFMA used here the accumulator lane
// layout is: lane l holds column (l % 32); value v (0..15) sits in row
// 8 * (v / 4) + 4 * (l / 32) + (v % 4).  A and B operands are symmetric:
// lane l supplies row (A) / column (B) l % 32 and the K-slice owned by the
// half-wave l / 32.
__device__ __forceinline__ f32x16_t mfma_bf16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma_f32(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

}  // namespace ha
