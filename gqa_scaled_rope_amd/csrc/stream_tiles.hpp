// Pieces shared by the two streaming prefill attention kernels -- attn_prefill_stream.hip (eight
// wavefronts per workgroup, one workgroup per CU, for long key bands) and attn_prefill_short.hip
// (four wavefronts, two workgroups per CU, for short ones): tile geometry, buffer descriptors,
// the HBM -> LDS tile copies and the counted-wait barriers that hand tiles to their readers,
// the LDS swizzles, the key-band search and the argument block.
#pragma once

#include "launch.hpp"

namespace gqa {
namespace stream {

constexpr int HD = 128;
constexpr int BN = 32;
constexpr int TILE_ELEMS = BN * HD;
constexpr float kRescaleThreshold = 8.0f;
constexpr int kBufFlags = 0x00020000;  // raw buffer, 32-bit dwords, range checked

constexpr int kXcds = 8;               // MI355X: 8 accelerator complex dies, one L2 each

typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor as four words (base, stride 0, num_records, flags) for tile_dma16.
__device__ __forceinline__ i32x4 rsrc_words(const void* base, int nrec) {
  const uint64_t p = (uint64_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(p >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane(nrec);
  r[3] = kBufFlags;
  return r;
}

// One HBM -> LDS copy of 16 bytes per lane (buffer_load_dwordx4 ... lds: lane l's bytes land at
// dst + 16 l).  Written as assembly on purpose: the compiler's wait-count pass cannot tell these
// asynchronous LDS writes apart from the reads of the other tile buffers and would make the
// next LDS read wait for every tile load just issued, which removes the prefetch.  Correctness
// rests on the explicit full wait before each barrier that hands a buffer to its readers; the
// compiler's own memory waits stay correct because loads retire in issue order.
// The five wait states before the load cover the m0 write (one needed) and a descriptor word
// written by a VALU instruction just before (five needed before a memory instruction reads it);
// the compiler does not look inside the statement for either hazard.
__device__ __forceinline__ void tile_dma16(i32x4 rsrc, const lds_void* dst, uint32_t voff) {
  uint32_t saved;  // m0 is the LDS address operand; it is restored for the compiler
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 4\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane((int)(uintptr_t)dst)), "v"(voff), "s"(rsrc));
}
// The same with the LDS address given as a constant part (a buffer's address, materialised where
// used) plus a per-wavefront part held in one scalar register, so that no per-buffer address
// stays live across the loop.
__device__ __forceinline__ void tile_dma16_at(i32x4 rsrc, const lds_void* base, uint32_t woff,
                                              uint32_t voff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_add_u32 m0, %1, %2\n\ts_nop 4\n\t"
      "buffer_load_dwordx4 %3, %4, 0 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"((uint32_t)(uintptr_t)base), "s"(woff), "v"(voff), "s"(rsrc)
      : "scc");
}

// One HBM -> LDS copy of 4 bytes per lane (buffer_load_dword ... lds: lane l's dword lands at
// dst + 4 l).  Same hazards as tile_dma16.
__device__ __forceinline__ void tile_dma4(i32x4 rsrc, const lds_void* dst, uint32_t voff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 4\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"((uint32_t)(uintptr_t)dst), "v"(voff), "s"(rsrc));
}

// Workgroup barrier ordering LDS accesses only (the fences wait for this wavefront's LDS
// operations, not for its buffer loads); scheduling barriers keep the two phases apart.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  __builtin_amdgcn_sched_barrier(0);
}
// The same after waiting until at most N of this wavefront's buffer loads are outstanding (they
// retire in order): every wavefront's share of the tile due has then landed.
template <int N>
__device__ __forceinline__ void barrier_after_loads() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N));
  phase_barrier();
}

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *(const u32x4*)p; }
__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& w) { return __builtin_bit_cast(bf16x8, w); }

__device__ __forceinline__ void unpack8(const u32x4& w, float* x) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = bf16lo(w[e]);
    x[2 * e + 1] = bf16hi(w[e]);
  }
}
__device__ __forceinline__ u32x4 pack8(const float* x) {
  u32x4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
  return w;
}


// LDS layout of a tile: row r's 16-byte chunk c sits at chunk position c ^ swz(r).  K tiles use
// swz = r & 15, measured free of bank conflicts for the operand reads (ds_read_b128, 32 rows).
// V tiles: ds_read_b64_tr_b16 serves lanes 0-31 and 32-63 as two passes of 256 bytes over the
// 64 four-byte banks (measured on gfx950); each pass here reads four chunks of each of four
// consecutive rows, 256-byte rows, so the rows' 64-byte chunk quads must land in four different
// quarters of the bank array: swz = (r & 3) << 2 moves row r's quad by r & 3 quarters.
__device__ __forceinline__ int kswz(int r) { return r & 15; }
__device__ __forceinline__ int vswz(int r) { return (r & 3) << 2; }

// First index j in [0, n) with kp[j] >= x for a nondecreasing kp, found by the whole wavefront:
// each round samples 64 evenly spaced entries and keeps the one segment that contains the
// boundary, so n keys take ceil(log64 n) dependent loads instead of log2 n.
__device__ __forceinline__ int wave_lower_bound(const int32_t* kp, int n, int64_t x) {
  const int lane = threadIdx.x & 63;
  int lo = 0, hi = n;  // answer in [lo, hi]
  while (hi > lo) {
    const int stride = (hi - lo + 63) >> 6;
    const int idx = lo + lane * stride;
    const bool below = idx < hi && (int64_t)kp[idx] < x;
    const int cnt = __popcll(__ballot(below));
    if (cnt == 0) {
      hi = lo;
    } else {
      const int nlo = lo + (cnt - 1) * stride + 1;
      hi = min(lo + cnt * stride, hi);
      lo = nlo;
    }
  }
  return lo;
}

struct StreamArgs {
  AttnArgs a;
  const uint16_t* kprep;   // [B, S - w0, Hkv, D] keys from row w0 = max(n_cached - (BN-1), 0) on,
                           // new ones prepared (null if nothing needs preparing)
  float* part;             // split partials (eight-wavefront kernel; null: no item is split)
  int32_t nqb;             // query blocks per (b, g)
  int32_t nfull;           // items walked whole; workgroups past them take half an item each
  int32_t grid;            // workgroups of the launch
};

// The four-wavefront kernel over the same prepared keys (attn_prefill_short.hip).
hipError_t launch_attn_short(const StreamArgs& sa, hipStream_t stream);

}  // namespace stream
}  // namespace gqa
