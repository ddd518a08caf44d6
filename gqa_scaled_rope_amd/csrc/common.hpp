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
  const float* sinks;        // [Hq] logits in scaled-score units; null = none
  int32_t chunk;             // chunk length in positions; 0 = no chunking
  int32_t chunk_lb;          // visible chunks before the query's own
  uint32_t chunk_m_lo, chunk_m_hi;  // ceil(2^64 / chunk) for chunk >= 2 (set by set_chunk)

  // true when some key position below the query's can be masked (window or chunks)
  __host__ __device__ bool has_floor() const { return window > 0 || chunk > 0; }
};

// floor(u / chunk) for any 32-bit u, by multiplication: with M = ceil(2^64 / chunk) = 2^64/chunk + e
// (0 <= e < 1), u*M / 2^64 exceeds u/chunk by less than 2^-32, and the fraction of u/chunk is at
// most 1 - 1/chunk, so the floor is exact for chunk < 2^32.  The 96-bit product is formed from the
// two 32-bit halves of M.
__host__ __device__ inline uint32_t chunk_div(const AttnArgs& a, uint32_t u) {
  if (a.chunk == 1) return u;
  const uint64_t t = (uint64_t)u * a.chunk_m_hi + (((uint64_t)u * a.chunk_m_lo) >> 32);
  return (uint32_t)(t >> 32);
}

// Sets the chunk fields (chunk 0: off).
inline void set_chunk(AttnArgs& a, int32_t chunk, int32_t lookback) {
  a.chunk = chunk > 0 ? chunk : 0;
  a.chunk_lb = chunk > 0 ? lookback : 0;
  const uint64_t m = chunk >= 2 ? UINT64_MAX / (uint64_t)chunk + 1 : 0;
  a.chunk_m_lo = (uint32_t)m;
  a.chunk_m_hi = (uint32_t)(m >> 32);
}

// Smallest key position a query at position p (an int32 value) may see ([Models] "Sliding windows": p - w + 1;
// chunked attention: the first position of the chunk chunk_lb chunks before p's own, chunks
// counted by floor division).  Nondecreasing in p, so over a block of queries the smallest
// floor is the first query's and the largest the last one's.  Without window and chunks the
// result is far below every int32 position.
__host__ __device__ inline int64_t key_floor(const AttnArgs& a, int64_t p) {
  int64_t lo = -((int64_t)1 << 40);
  if (a.window > 0) lo = p - a.window + 1;
  if (a.chunk > 0) {
    // floor(p / chunk) for an int32 p: |p| (+ chunk - 1 when negative) stays below 2^32
    const int32_t p32 = (int32_t)p;
    const int64_t idx = p32 >= 0 ? (int64_t)chunk_div(a, (uint32_t)p32)
                                 : -(int64_t)chunk_div(a, 0u - (uint32_t)p32 + (uint32_t)(a.chunk - 1));
    const int64_t first = (idx - a.chunk_lb) * (int64_t)a.chunk;
    lo = lo > first ? lo : first;
  }
  return lo;
}


}  // namespace gqa
