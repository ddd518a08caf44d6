// Absorbed multi-head latent attention decode core, bf16, gfx950.
//
// [Models] "Multi-head latent attention" (paged_forward): each query is mapped into latent space
// once (W_uk^T q_nope) and attends, together with its rotated q_rope, over the cached [c, k_rope]
// rows -- multi-query attention with ONE key/value head 576 wide (kv_lora_rank 512 +
// qk_rope_head_dim 64) whose values are the first 512 features of the same rows.  This file is
// that attention core for one new token per sequence: q [B, H, 576] (absorbed and rotated by the
// caller, as the page does before its backend call), cache [B, Smax, 576], out [B, H, 512]
// (before W_uv).
//
// The step reads every cached row once per 64 query heads (HBM-bound for 16 heads, balanced
// against the matrix cores for 128):
//   mla_split_kernel      grid (split of 2048 keys, group of 64 heads, sequence); 4 wavefronts,
//                         16 heads each; the split's rows stream HBM -> LDS in blocks of 32 keys
//                         (buffer_load ... lds, two LDS stages, one barrier per block) and all
//                         four wavefronts read them:
//                           S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (K from LDS, the wave's Q
//                           operands -- q as given, not rounded again -- in registers, 18 k-steps
//                           over 576 features), times scale * log2(e) in fp32;
//                           online softmax in log2 units, lazily rescaled;
//                           O = P V on the same MFMA, V (the rows' first 512 features) read with
//                           transposing LDS reads, O for 16 heads x 512 features in registers;
//                         one partial (m, l, O) per (sequence, split, head);
//   mla_combine_kernel    log-sum-exp merge of a sequence's splits -> bf16.
#include <algorithm>
#include <type_traits>

#include "launch.hpp"

namespace gqa {
namespace {

constexpr int QKD = 576;               // row width: latent 512 + rotary 64
constexpr int LAT = 512;               // value width
constexpr int KB = 32;                 // keys per block
constexpr int LROW = 73;               // LDS row stride in 16-byte chunks (72 + 1 pad: no swizzle)
constexpr int NDMA = (KB * LROW + 63) / 64;  // 1 KB DMA instructions per block
constexpr int BUF_BYTES = NDMA * 1024;        // what they write (the tail past row 31 is zero)
constexpr int NWM = 4;                 // wavefronts per workgroup
constexpr int HPW = 16;                // query heads per wavefront
constexpr int SPLITM = 2048;           // keys per split
constexpr int kMlaFlags = 0x00020000;  // raw buffer, range checked

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& w) { return __builtin_bit_cast(bf16x8, w); }

__device__ __forceinline__ i32x4 rsrc_words(const void* base, int nrec) {
  const uint64_t p = (uint64_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(p >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane(nrec);
  r[3] = kMlaFlags;
  return r;
}

// HBM -> LDS copy of 16 bytes per lane (lane l's bytes land at dst + 16 l), as assembly so that
// the compiler's wait counts do not make LDS reads wait for it (correctness rests on the explicit
// full wait before each barrier that hands a block to its readers; compiler-visible loads retire
// in issue order, so its own waits stay correct).  Five wait states cover the m0 write and a
// descriptor word written by a VALU instruction just before.
__device__ __forceinline__ void dma16(i32x4 rsrc, const lds_void* dst, int voff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 4\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane((int)(uintptr_t)dst)), "v"(voff), "s"(rsrc));
}

struct MlaArgs {
  const uint16_t* q;      // [B, H, 576]
  const uint16_t* cache;  // [B, Smax, 576]
  const int32_t* lens;    // [B]
  uint16_t* out;          // [B, H, 512]
  float* part_o;          // [B, nsplit, H, 512]
  float* part_ml;         // [B, nsplit, H, 2]
  int32_t B, H, Smax, nsplit;
  float qscale;           // scale * log2(e)
};

__shared__ __attribute__((aligned(16))) uint16_t g_m0[BUF_BYTES / 2];
__shared__ __attribute__((aligned(16))) uint16_t g_m1[BUF_BYTES / 2];

template <int BUF>
__device__ __forceinline__ uint16_t* mbuf() { return BUF == 0 ? g_m0 : g_m1; }

__global__ __launch_bounds__(NWM * 64, 2) void mla_split_kernel(MlaArgs m) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sp = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
  const int n = min(max(m.lens[b], 0), m.Smax);
  const int ks = sp * SPLITM;
  if (ks >= n) return;  // uniform over the workgroup: no barrier is skipped by part of it
  const int ke = min(ks + SPLITM, n);
  const int nblk = (ke - ks + KB - 1) / KB;
  const int h0 = hq * (NWM * HPW) + w * HPW;  // this wavefront's first head
  const bool active = h0 < m.H;                // (H is a multiple of 16)

  // DMA lane offsets: instruction i of the block fills LDS chunks 64 i .. 64 i + 63, i.e. row
  // L / 73, chunk L % 73 for L = 64 i + lane; chunk 72 is padding and rows past the block are
  // out of range (zero).
  int doff[(NDMA + NWM - 1) / NWM];
#pragma unroll
  for (int k = 0; k < (NDMA + NWM - 1) / NWM; ++k) {
    const int L = 64 * (w + NWM * k) + lane;
    const int r = L / LROW, c = L - r * LROW;
    doff[k] = (r < KB && c < QKD / 8) ? r * (QKD * 2) + c * 16 : 0x7ffffff0;
  }
  auto issue = [&](int blk, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int kb0 = ks + blk * KB;
    const i32x4 rs = rsrc_words(m.cache + ((int64_t)b * m.Smax + kb0) * QKD,
                                min(max(ke - kb0, 0), KB) * QKD * 2);
#pragma unroll
    for (int k = 0; k < (NDMA + NWM - 1) / NWM; ++k) {
      const int i = w + NWM * k;
      if (i < NDMA) dma16(rs, (const lds_void*)(mbuf<buf>() + i * 512), doff[k]);
    }
  };

  // query operands: head h0 + (lane & 15), features 32 s + 8 (lane >> 4) .. + 7
  u32x4 qop[QKD / 32];
  {
    const int hh = active ? h0 + (lane & 15) : 0;
    const uint16_t* qr = m.q + ((int64_t)b * m.H + hh) * QKD + 8 * (lane >> 4);
#pragma unroll
    for (int s = 0; s < QKD / 32; ++s) qop[s] = *(const u32x4*)(qr + 32 * s);
  }

  f32x4 o[LAT / 16];
#pragma unroll
  for (int db = 0; db < LAT / 16; ++db) o[db] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float mx = kNegBig, lsum = 0.f;
  const int gi = lane >> 4, si = lane & 15;

  auto compute = [&](int blk, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const uint16_t* rows = mbuf<buf>();
    const int kb0 = ks + blk * KB;
    // S^T = K Q^T: lane holds head si, keys 16 kq + 4 gi + r
    f32x4 sk[2];
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {
      sk[kq] = (f32x4){0.f, 0.f, 0.f, 0.f};
      const uint16_t* kr = rows + (kq * 16 + si) * (LROW * 8) + 8 * gi;
#pragma unroll
      for (int s = 0; s < QKD / 32; ++s) {
        const u32x4 ka = *(const u32x4*)(kr + 32 * s);
        sk[kq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka), as_bf16x8(qop[s]), sk[kq],
                                                         0, 0, 0);
      }
    }
#pragma unroll
    for (int kq = 0; kq < 2; ++kq)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sk[kq][r] = kb0 + kq * 16 + 4 * gi + r < ke ? sk[kq][r] * m.qscale : -INFINITY;
    float mt = fmaxf(fmaxf(fmaxf(sk[0][0], sk[0][1]), fmaxf(sk[0][2], sk[0][3])),
                     fmaxf(fmaxf(sk[1][0], sk[1][1]), fmaxf(sk[1][2], sk[1][3])));
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    if (__ballot(mt > mx + 8.0f) != 0) {  // lazy rescale: the reference moves by more than 8
      const float m_new = fmaxf(mx, mt);
      const float alpha = fast_exp2(mx - m_new);
      lsum *= alpha;
      // O rows are heads 4 gi + r; their alpha lives in lane 4 gi + r
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, 4 * gi + r, 64);
#pragma unroll
        for (int db = 0; db < LAT / 16; ++db) o[db][r] *= ar;
      }
      mx = m_new;
    }
    float p[8];
#pragma unroll
    for (int kq = 0; kq < 2; ++kq)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[4 * kq + r] = fast_exp2(sk[kq][r] - mx);
        lsum += p[4 * kq + r];
      }
    u32x4 pw;
#pragma unroll
    for (int e = 0; e < 4; ++e) pw[e] = pack_bf16x2(p[2 * e], p[2 * e + 1]);
    const bf16x8 pa = as_bf16x8(pw);
    // O = P V: B operand = V[32 keys][16 features] via transposing LDS reads (key order matching
    // the one P's operand holds)
    const int row1 = 4 * gi + (si >> 2);
    const int row2 = row1 + 16;
#pragma unroll
    for (int db = 0; db < LAT / 16; ++db) {
      const int col = 16 * db + 4 * (si & 3);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(rows + row1 * (LROW * 8) + col));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(rows + row2 * (LROW * 8) + col));
      const i16x8 vb = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(bf16x8, vb), o[db],
                                                      0, 0, 0);
    }
  };

  issue(0, std::integral_constant<int, 0>());
  for (int blk = 0; blk < nblk; blk += 2) {
    __builtin_amdgcn_s_waitcnt(0);  // block blk's rows are in (and every earlier load)
    __syncthreads();                // ... for every wavefront; buffer 1 is free again
    if (blk + 1 < nblk) issue(blk + 1, std::integral_constant<int, 1>());
    if (active) compute(blk, std::integral_constant<int, 0>());
    if (blk + 1 < nblk) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (blk + 2 < nblk) issue(blk + 2, std::integral_constant<int, 0>());
      if (active) compute(blk + 1, std::integral_constant<int, 1>());
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load into LDS outstanding when the workgroup ends

  if (!active) return;
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  const int64_t pbase = ((int64_t)b * m.nsplit + sp) * m.H;
  if (lane < HPW) {
    float* ml = m.part_ml + (pbase + h0 + lane) * 2;
    ml[0] = mx;
    ml[1] = lsum;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float* po = m.part_o + (pbase + h0 + 4 * gi + r) * LAT + si;
#pragma unroll
    for (int db = 0; db < LAT / 16; ++db) po[16 * db] = o[db][r];
  }
}

// out[b, h, :] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over the splits that hold keys.
__global__ __launch_bounds__(LAT) void mla_combine_kernel(MlaArgs m) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int n = min(max(m.lens[b], 0), m.Smax);
  const int nsp = (n + SPLITM - 1) / SPLITM;
  const int64_t base = (int64_t)b * m.nsplit * m.H + h;
  float M = kNegBig;
  for (int s = 0; s < nsp; ++s) M = fmaxf(M, m.part_ml[(base + (int64_t)s * m.H) * 2]);
  float acc = 0.f, lt = 0.f;
  for (int s = 0; s < nsp; ++s) {
    const int64_t it = base + (int64_t)s * m.H;
    const float wgt = fast_exp2(m.part_ml[it * 2] - M);
    lt += wgt * m.part_ml[it * 2 + 1];
    acc += wgt * m.part_o[it * LAT + d];
  }
  m.out[((int64_t)b * m.H + h) * LAT + d] = f32_to_bf16(lt > 0.f ? acc / lt : 0.f);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t mla_decode_workspace_bytes(int B, int H, int Smax) {
  const int64_t nsplit = (Smax + SPLITM - 1) / SPLITM;
  return align256((size_t)B * nsplit * H * LAT * 4) + (size_t)B * nsplit * H * 2 * 4;
}

hipError_t launch_mla_decode(const void* q, const void* cache, const int32_t* lens, int B, int H,
                             int Smax, float scale, void* out, void* workspace,
                             hipStream_t stream) {
  if (B == 0) return hipSuccess;
  MlaArgs m;
  m.q = (const uint16_t*)q;
  m.cache = (const uint16_t*)cache;
  m.lens = lens;
  m.out = (uint16_t*)out;
  m.B = B;
  m.H = H;
  m.Smax = Smax;
  m.nsplit = (Smax + SPLITM - 1) / SPLITM;
  m.qscale = scale * kLog2e;
  char* ws = (char*)workspace;
  m.part_o = (float*)ws;
  m.part_ml = (float*)(ws + align256((size_t)B * m.nsplit * H * LAT * 4));
  hipLaunchKernelGGL(mla_split_kernel, dim3(m.nsplit, (H + NWM * HPW - 1) / (NWM * HPW), B),
                     dim3(NWM * 64), 0, stream, m);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_combine_kernel, dim3(H, B), dim3(LAT), 0, stream, m);
  return hipGetLastError();
}

}  // namespace gqa
