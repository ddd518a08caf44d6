// Device helpers shared by the gfx950 kernels of libgqa_rope: bf16 packing, MFMA operand types,
// cross-lane reductions, and the launch descriptors the C-ABI layer fills in.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint64_t u64x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
// Initial running maximum: finite, so exp2(m_old - m_new) never sees inf - inf.
constexpr float kNegBig = -1.0e30f;

// ---- bf16 <-> fp32 (bit level; bf16 is the top half of an fp32) ------------------------------
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Round-to-nearest-even pack of two floats into one dword of bf16 (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

// ---- wave-level reductions (64 lanes) ----------------------------------------------------------
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}
// Value held by lane (l ^ 32).
__device__ __forceinline__ float swap_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- launch descriptors ------------------------------------------------------------------------
// Fields are element strides; the C-ABI layer derives them from the documented layouts.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  int64_t q_b, q_i, q_h;     // q element (b, i, h, 0)
  int64_t k_b, k_j, k_h;     // k and v element (b, j, g, 0)
  int64_t o_b, o_i, o_h;
  const int32_t* qpos;       // null: decode mode, the query sits at lens[b] - 1
  int64_t qpos_b;
  const int32_t* kpos;       // null: key j sits at position j
  int64_t kpos_b;
  const int32_t* lens;       // decode: keys per sequence; null: S for every sequence
  int32_t B, L, S, Hq, Hkv, G, D, R;
  int32_t style;             // 0 half-split, 1 interleaved
  int32_t n_cached;          // keys j < n_cached are used as stored
  int32_t window;
  int32_t qk_norm;
  float eps;
  const void* qw;
  const void* kw;
  const float* cos_t;
  const float* sin_t;
  int32_t table_len;
  float scale;               // score scale (natural units)
  float softcap;             // 0 = off
};


}  // namespace gqa
