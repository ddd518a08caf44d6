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
// Every cached row is read from HBM once per 128 query heads.  The batch's rows, cut into blocks
// of 32 keys per sequence and laid end to end, are dealt out in equal contiguous shares, one per
// workgroup (grid: kMlaWorkgroups shares x groups of 128 heads), so every compute unit gets the
// same work whatever the length mix; a share may span the end of one sequence and the start of
// the next.  A share's blocks stream HBM -> LDS (buffer_load ... lds, four LDS stages, one barrier
// per block) and every wavefront of the workgroup reads them.  One partial (m, l, O) per (share,
// sequence) piece and head goes to slot share + sequence (unique: along the pieces both indices
// only grow).
//   mla_split32_kernel   4 wavefronts (one per SIMD), 32 heads each:
//                          S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (32 keys x 32 heads; K from
//                          LDS, the wave's Q operands -- q as given -- in registers, 36 k-steps
//                          over 576 features), scaled by scale * log2(e) in fp32;
//                          weights 2^(s - r) against a reference r fixed at the piece's first
//                          block (its maximum), never moved: O^T is not rescaled, so it stays in
//                          the 256 accumulation registers per lane, which hold nothing else;
//                          O^T += V^T P^T on the same MFMA, V (the rows' first 512 features) read
//                          with transposing LDS reads.
//                        Each 1 KB operand read from LDS feeds a 32x32x16 product: half the LDS
//                        bytes per multiply of 16-head wavefronts, whose operand reads bound
//                        their block rate.  A weight above 2^64 (a score more than 64 log2 units
//                        over the reference) could overflow the sums: then the wavefront flags
//                        its share, and the share is computed again by
//   mla_split16_kernel   8 wavefronts, 16 heads each, on v_mfma_f32_16x16x32_bf16, O in registers
//                        with the lazy rescale (reference moved when a score passes it by 8): a
//                        workgroup whose share is not flagged leaves at once;
//   mla_combine_kernel   log-sum-exp merge of a sequence's pieces -> bf16.
//
// LDS layout of a block: row r (key) holds its 72 16-byte chunks at r * 74 + chunk.  Of the row
// strides near 72 chunks, 74 is the one measured free of LDS bank conflicts (on gfx950, with the
// bank-conflict counter) for 16-byte reads of one chunk from each of consecutive rows (the K
// operand) and for transposing reads of 32 bytes from each of 4 consecutive rows (the V operand);
// 72 costs those 12 and 6 extra cycles per instruction, 73 4 and 2.
#include <algorithm>
#include <type_traits>

#include "launch.hpp"

namespace gqa {
namespace {

constexpr int QKD = 576;                 // row width: latent 512 + rotary 64
constexpr int LAT = 512;                 // value width
constexpr int CPR = QKD / 8;             // 16-byte chunks per row
constexpr int LROW = 74;                 // LDS row stride in chunks (2 of padding)
constexpr int KB = 32;                   // keys per block
constexpr int NDMA = KB * LROW / 64;     // 1 KB DMA instructions per block (37)
constexpr int BUF_BYTES = NDMA * 1024;
constexpr int HPG = 128;                 // query heads per workgroup
constexpr int NSTM = 4;                  // LDS stages
constexpr int kMlaWorkgroups = 256;      // shares of the batch: one per compute unit
constexpr int kMlaFlags = 0x00020000;    // raw buffer, range checked
constexpr float kRefLimit = 64.0f;       // largest score - reference (log2 units) taken in place
static_assert(KB * LROW % 64 == 0, "whole 1 KB loads per block");

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
// wait before each barrier that hands a block to its readers; vector memory loads retire in issue
// order, so the compiler's own waits stay correct).  Five wait states cover the m0 write and a
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
  float* part_o;          // [kMlaWorkgroups + B, H, 512]
  float* part_ml;         // [kMlaWorkgroups + B, H, 2]
  int32_t* flags;         // [groups of 128 heads, kMlaWorkgroups, 4]: share to compute again
  int32_t B, H, Smax;
  float qscale;           // scale * log2(e)
};

// lengths through the constant address space: scalar loads where b is uniform (a vector load would
// bring a full vector-memory wait, and with it every block in flight, at each sequence change)
__device__ __forceinline__ int seq_len(const MlaArgs& m, int b) {
  const __attribute__((address_space(4))) int32_t* lens =
      (const __attribute__((address_space(4))) int32_t*)m.lens;
  return b < m.B ? min(max(lens[b], 0), m.Smax) : 0;
}
__device__ __forceinline__ int seq_blocks(const MlaArgs& m, int b) {
  return (seq_len(m, b) + KB - 1) / KB;
}
__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
  return x;
}
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}
// total blocks of the batch
__device__ __forceinline__ int total_blocks(const MlaArgs& m, int lane) {
  int u = 0;
  for (int base = 0; base < m.B; base += 64) u += wave_sum(seq_blocks(m, base + lane));
  return u;
}
// first block of share c
__device__ __forceinline__ int share_lo(int c, int U) {
  return (int)((int64_t)c * U / kMlaWorkgroups);
}
// the share that holds block u (the last c with share_lo(c) <= u)
__device__ __forceinline__ int share_of(int u, int U) {
  return (int)(((int64_t)(u + 1) * kMlaWorkgroups - 1) / U);
}

// s_waitcnt immediate that waits for vector memory count <= n only (gfx9 layout: vmcnt bits 3:0
// and 15:14; expcnt and lgkmcnt at their maxima)
constexpr int vm_wait(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
// wait until this wavefront's loads of the block about to be read are in: `later` blocks were
// issued after it, PER + 1 loads each (`extra`) or PER
template <int PER>
__device__ __forceinline__ void wait_block(int later, bool extra) {
  if (later >= 2) {
    if (extra)
      __builtin_amdgcn_s_waitcnt(vm_wait(2 * (PER + 1)));
    else
      __builtin_amdgcn_s_waitcnt(vm_wait(2 * PER));
  } else if (later == 1) {
    if (extra)
      __builtin_amdgcn_s_waitcnt(vm_wait(PER + 1));
    else
      __builtin_amdgcn_s_waitcnt(vm_wait(PER));
  } else {
    __builtin_amdgcn_s_waitcnt(0);
  }
}

// the stages, one block each (a runtime stage index: per-stage constant addresses would not fit
// the LDS instructions' 16-bit offsets and would cost a register set each)
__shared__ __attribute__((aligned(16))) uint16_t g_mla[NSTM * BUF_BYTES / 2];

// position in the batch: sequence b, its block j, its length n and block count nb
struct Cursor {
  int b, j, n, nb;
};

// The share of workgroup c: its block count (0: nothing to do) and the cursor at its first block
// (uniform over the wavefront; every wavefront computes it).
__device__ __forceinline__ int share_start(const MlaArgs& m, int c, int lane, Cursor& cc) {
  const int U = __builtin_amdgcn_readfirstlane(total_blocks(m, lane));
  const int lo = share_lo(c, U), hi = share_lo(c + 1, U);
  const int nu = hi - lo;
  if (nu <= 0) return 0;
  cc.b = m.B;
  cc.j = 0;
  int acc = 0;
  for (int base = 0; base < m.B; base += 64) {  // lo < U: some sequence holds block lo
    const int nb = seq_blocks(m, base + lane);
    const int incl = acc + wave_incl_scan(nb, lane);
    const uint64_t hit = __ballot(nb > 0 && incl - nb <= lo && lo < incl);
    if (hit != 0) {
      const int l = __builtin_ctzll(hit);
      cc.b = base + l;
      cc.j = lo - __builtin_amdgcn_readfirstlane(__shfl(incl - nb, l, 64));
      break;
    }
    acc = __builtin_amdgcn_readfirstlane(__shfl(incl, 63, 64));
  }
  cc.b = __builtin_amdgcn_readfirstlane(cc.b);
  cc.j = __builtin_amdgcn_readfirstlane(cc.j);
  if (cc.b >= m.B) return 0;  // (not reached)
  cc.n = seq_len(m, cc.b);
  cc.nb = (cc.n + KB - 1) / KB;
  return nu;
}
__device__ __forceinline__ void cursor_advance(const MlaArgs& m, Cursor& u) {
  if (++u.j < u.nb) return;
  u.j = 0;
  do {
    ++u.b;
    u.n = seq_len(m, u.b);
    u.nb = (u.n + KB - 1) / KB;
  } while (u.nb == 0 && u.b + 1 < m.B);
}
// DMA lane offsets: instruction i of a block fills LDS chunks 64 i .. 64 i + 63; chunk P holds
// chunk P % 74 of row P / 74 (chunks 72 and 73 are padding: out of range, never read)
__device__ __forceinline__ int dma_off(int i, int lane) {
  const int P = 64 * i + lane;
  const int r = P / LROW, c = P - r * LROW;
  return c < CPR ? r * (QKD * 2) + c * 16 : 0x7ffffff0;
}
// block u into stage st: NW wavefronts, wave w issuing loads w, w + NW, ...
template <int NW>
__device__ __forceinline__ void issue_block(const MlaArgs& m, const Cursor& u, int st, int w,
                                            int lane) {
  constexpr int PER = NDMA / NW;
  uint16_t* dst = g_mla + st * (BUF_BYTES / 2);
  const int k0 = u.j * KB;
  const i32x4 rs = rsrc_words(m.cache + ((int64_t)u.b * m.Smax + k0) * QKD,
                              min(u.n - k0, KB) * QKD * 2);
  // (the lane offsets are recomputed here rather than kept in registers across the loop)
  int lz = lane;
  asm volatile("" : "+v"(lz));
#pragma unroll
  for (int k = 0; k < PER; ++k)
    dma16(rs, (const lds_void*)(dst + (w + NW * k) * 512), dma_off(w + NW * k, lz));
  if (w < NDMA - PER * NW)
    dma16(rs, (const lds_void*)(dst + (w + NW * PER) * 512), dma_off(w + NW * PER, lz));
}

__global__ __launch_bounds__(4 * 64, 1) void mla_split32_kernel(MlaArgs m) {
  constexpr int NW = 4, HPW = 32;
  constexpr int KLA = 8, VLA = 8;  // operand reads ahead of their MFMAs: K, V
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = blockIdx.x;
  int32_t* flag = m.flags + ((int64_t)blockIdx.y * kMlaWorkgroups + c) * NW + w;
  Cursor cc;
  const int nu = share_start(m, c, lane, cc);
  if (nu <= 0) {  // uniform over the workgroup: no barrier is skipped by part of it
    if (lane == 0) *flag = 0;
    return;
  }

  const int h0 = blockIdx.y * HPG + w * HPW;  // this wavefront's first head
  const bool active = h0 < m.H;              // (H is a multiple of 16: a wave may hold 16 heads)
  const bool extra = w < NDMA - (NDMA / NW) * NW;  // waves issuing one more load per block

  // lane (ql, hg): head h0 + ql (clamped to a real head for the loads), key half hg
  const int ql = lane & 31, hg = lane >> 5;
  const int hq = h0 + ql;
  const bool hvalid = active && hq < m.H;
  // query operands (B of S^T = K Q^T): head hq, features 16 s + 8 hg .. + 7
  u32x4 qop[QKD / 16];
  auto load_q = [&](int bq) __attribute__((always_inline)) {
    const uint16_t* qr = m.q + ((int64_t)bq * m.H + min(hq, m.H - 1)) * QKD + 8 * hg;
#pragma unroll
    for (int s = 0; s < QKD / 16; ++s) qop[s] = *(const u32x4*)(qr + 16 * s);
    // wait here (once per sequence) so that no wait for q is left pending into the block loop,
    // where the compiler would place one before each score MFMA and, not counting the blocks in
    // flight, drain them all
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  };

  // O^T, 512 features x 32 heads in 16 blocks of 32 features: lane (ql, hg) holds head h0 + ql,
  // features 32 db + 8 (r / 4) + 4 hg + r % 4 in o[db][r]
  f32x16 o[LAT / 32];
#pragma unroll
  for (int db = 0; db < LAT / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float mr = kNegBig, lsum = 0.f;  // per head: the piece's reference (log2 units), this lane's sum
  bool over = false;               // a weight of this wavefront would have passed 2^64
  const int gi = lane >> 4, s16 = lane & 15;

  // LDS read positions (bf16 elements).  K operand (A of S^T): row ql, chunk 2 s + hg.  V^T
  // operand (A of O^T, by transposing reads): lane (gi, s16) names row 4 hg + s16 / 4 (+ 8 for
  // the second half, + 16 u for keys 16 u ..), columns 32 db + 16 (gi & 1) + 4 (s16 & 3) .. + 3;
  // each lane then holds feature 32 db + (lane & 31) of keys 16 u + 4 hg + {0..3, 8..11}, the key
  // order in which the scores' lane holds the weights.
  const int kbase = ql * (LROW * 8) + 8 * hg;
  const int vbase = (4 * hg + (s16 >> 2)) * (LROW * 8) + 16 * (gi & 1) + 4 * (s16 & 3);
  int doff[NDMA / NW + 1];  // lane offsets of this wavefront's block loads
#pragma unroll
  for (int k = 0; k <= NDMA / NW; ++k) doff[k] = dma_off(w + NW * k, lane);

  auto compute = [&](const Cursor& u, int st, bool more, i32x4 rs, uint16_t* dst)
      __attribute__((always_inline)) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const uint16_t* rows = g_mla + st * (BUF_BYTES / 2);
    const int kb0 = u.j * KB;
    // S^T = K Q^T: lane holds head h0 + ql, keys 8 (r / 4) + 4 hg + r % 4
    f32x16 sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
    const uint16_t* kr = rows + kbase;
    // Operand reads KLA MFMAs ahead of their use (one wavefront per SIMD: nothing else hides
    // their latency), in a ring of KLA registers; scheduling fences keep each read in its step.
    u32x4 kring[KLA];
#pragma unroll
    for (int s = 0; s < KLA; ++s) kring[s] = *(const u32x4*)(kr + 16 * s);
#pragma unroll
    for (int s = 0; s < QKD / 16; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      const u32x4 ka = kring[s % KLA];
      if (s + KLA < QKD / 16) kring[s % KLA] = *(const u32x4*)(kr + 16 * (s + KLA));
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka), as_bf16x8(qop[s]), sc, 0, 0, 0);
      // the next block's loads: load k after score MFMA 3 k + 2
      if (s % 3 == 2 && s / 3 <= NDMA / NW) {
        const int k = s / 3;
        if (more && (k < NDMA / NW || extra))
          dma16(rs, (const lds_void*)(dst + (w + NW * k) * 512), doff[k]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // keys past the sequence's end (only in its last block) take no weight
    if (kb0 + KB > u.n) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kb0 + 8 * (r >> 2) + 4 * hg + (r & 3) >= u.n) sc[r] = -INFINITY;
    }
    // the block's maximum scaled score (the scale is positive); the other 16 keys of the head
    // are in lane l ^ 32.  It sets the reference at the piece's first block.
    float mt = sc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sc[r]);
    mt = fmaxf(mt, swap_halves(mt)) * m.qscale;
    if (mr == kNegBig) mr = mt;
    over |= mt > mr + kRefLimit;
    // weights of keys 0-15 now; those of keys 16-31 beside the first P V MFMAs, which use only
    // the first half
    bf16x8 pw[2];
    float p1[8];
    {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = fast_exp2(__builtin_fmaf(sc[e], m.qscale, -mr));
        lsum += p[e];
      }
      u32x4 w4;
#pragma unroll
      for (int e = 0; e < 4; ++e) w4[e] = pack_bf16x2(p[2 * e], p[2 * e + 1]);
      pw[0] = as_bf16x8(w4);
    }
    // O^T += V^T P^T over keys 16 uh .. 16 uh + 15 (step i = 16 uh + db); operands VLA steps
    // ahead in a ring, as above
    auto vread = [&](int i) __attribute__((always_inline)) {
      const uint16_t* vp = rows + vbase + (i >> 4) * 16 * (LROW * 8) + 32 * (i & 15);
      const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp));
      const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp + 8 * (LROW * 8)));
      return i16x8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
    };
    i16x8 vring[VLA];
#pragma unroll
    for (int i = 0; i < VLA; ++i) vring[i] = vread(i);
#pragma unroll
    for (int i = 0; i < LAT / 16; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      const i16x8 vv = vring[i % VLA];
      if (i + VLA < LAT / 16) vring[i % VLA] = vread(i + VLA);
      o[i & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv),
                                                          pw[i >> 4], o[i & 15], 0, 0, 0);
      if (i < 8) {  // weight 8 + i of this lane
        p1[i] = fast_exp2(__builtin_fmaf(sc[8 + i], m.qscale, -mr));
        lsum += p1[i];
      } else if (i == 8) {
        u32x4 w4;
#pragma unroll
        for (int e = 0; e < 4; ++e) w4[e] = pack_bf16x2(p1[2 * e], p1[2 * e + 1]);
        pw[1] = as_bf16x8(w4);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // the piece of sequence bq this share holds is done: write its partial and start afresh
  auto finish = [&](int bq) __attribute__((always_inline)) {
    const float l = lsum + swap_halves(lsum);
    const int64_t prow = (int64_t)(c + bq) * m.H + hq;
    if (hvalid) {
      if (hg == 0) {
        float* ml = m.part_ml + prow * 2;
        ml[0] = mr;
        ml[1] = l;
      }
      float* po = m.part_o + prow * LAT + 4 * hg;
#pragma unroll
      for (int db = 0; db < LAT / 32; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq)
          *(f32x4*)(po + 32 * db + 8 * rq) =
              (f32x4){o[db][4 * rq], o[db][4 * rq + 1], o[db][4 * rq + 2], o[db][4 * rq + 3]};
    }
#pragma unroll
    for (int db = 0; db < LAT / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
    mr = kNegBig;
    lsum = 0.f;
  };

  // Four stages: when block t is read, blocks t + 1 and t + 2 are in flight and t + 3 goes into
  // the stage that held t - 1 (every wavefront is past its reads of it: they precede this
  // barrier).
  // The loads of block t + 3 are issued inside block t's score chain, one after every third
  // MFMA (issued back to back, the wavefront waits for them about as long as for the chain).
  Cursor ic = cc;
  issue_block<NW>(m, ic, 0, w, lane);
  if (nu > 1) {
    cursor_advance(m, ic);
    issue_block<NW>(m, ic, 1, w, lane);
  }
  if (nu > 2) {
    cursor_advance(m, ic);
    issue_block<NW>(m, ic, 2, w, lane);
  }
  if (active) load_q(cc.b);
  for (int t = 0; t < nu; ++t) {
    wait_block<NDMA / NW>(min(nu - 1 - t, 2), extra);
    __syncthreads();
    const bool more = t + 3 < nu;
    if (more) cursor_advance(m, ic);
    const i32x4 rs = rsrc_words(m.cache + ((int64_t)ic.b * m.Smax + ic.j * KB) * QKD,
                                more ? min(ic.n - ic.j * KB, KB) * QKD * 2 : 0);
    uint16_t* dst = g_mla + ((t + 3) % NSTM) * (BUF_BYTES / 2);
    if (active) {
      compute(cc, t % NSTM, more, rs, dst);
    } else if (more) {
#pragma unroll
      for (int k = 0; k < NDMA / NW; ++k)
        dma16(rs, (const lds_void*)(dst + (w + NW * k) * 512), doff[k]);
      if (extra) dma16(rs, (const lds_void*)(dst + (w + NW * (NDMA / NW)) * 512), doff[NDMA / NW]);
    }
    const bool last = t + 1 == nu;
    if (cc.j + 1 == cc.nb || last) {
      if (active) finish(cc.b);
      if (!last) {
        cursor_advance(m, cc);
        if (active) load_q(cc.b);
      }
    } else {
      ++cc.j;
    }
  }
  // every wavefront writes its flag: 1 when its weights may have overflowed (the share is then
  // computed again by mla_split16_kernel), else 0
  const bool any_over = __ballot(over) != 0;
  if (lane == 0) *flag = any_over ? 1 : 0;
  __builtin_amdgcn_s_waitcnt(0);  // no load into LDS outstanding when the workgroup ends
}

__global__ __launch_bounds__(8 * 64, 1) void mla_split16_kernel(MlaArgs m) {
  constexpr int NW = 8, HPW = 16;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = blockIdx.x;
  // only a share that the 32-head kernel flagged is computed here
  const int32_t* flags = m.flags + ((int64_t)blockIdx.y * kMlaWorkgroups + c) * 4;
  const __attribute__((address_space(4))) int32_t* fl =
      (const __attribute__((address_space(4))) int32_t*)flags;
  if ((fl[0] | fl[1] | fl[2] | fl[3]) == 0) return;  // uniform over the workgroup
  Cursor cc;
  const int nu = share_start(m, c, lane, cc);
  if (nu <= 0) return;

  const int h0 = blockIdx.y * HPG + w * HPW;  // this wavefront's first head
  const bool active = h0 < m.H;              // (H is a multiple of 16)
  const bool extra = w < NDMA - (NDMA / NW) * NW;  // waves issuing one more load per block

  // query operands: head h0 + (lane & 15), features 32 s + 8 (lane >> 4) .. + 7
  u32x4 qop[QKD / 32];
  const int hh = active ? h0 + (lane & 15) : 0;
  auto load_q = [&](int bq) {
    const uint16_t* qr = m.q + ((int64_t)bq * m.H + hh) * QKD + 8 * (lane >> 4);
#pragma unroll
    for (int s = 0; s < QKD / 32; ++s) qop[s] = *(const u32x4*)(qr + 32 * s);
    // wait here (once per sequence) so that no wait for q is left pending into the block loop,
    // where the compiler would place one before each score MFMA and, not counting the blocks in
    // flight, drain them all
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  };

  f32x4 o[LAT / 16];
#pragma unroll
  for (int db = 0; db < LAT / 16; ++db) o[db] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float mx = kNegBig, lsum = 0.f;
  const int gi = lane >> 4, si = lane & 15;

  // LDS read positions (in bf16 elements).  K operand: row 16 kq + si, chunk 4 s + gi.  V
  // operand: rows 4 gi + (si >> 2) (+ 16), bytes 32 db + 8 (si & 3).
  const int kbase = si * (LROW * 8) + 8 * gi;
  const int vbase = (4 * gi + (si >> 2)) * (LROW * 8) + 4 * (si & 3);

  auto compute = [&](const Cursor& u, int st) {
    const uint16_t* rows = g_mla + st * (BUF_BYTES / 2);
    const int kb0 = u.j * KB;
    // S^T = K Q^T: lane holds head si, keys 16 kq + 4 gi + r
    f32x4 sk[2];
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {
      sk[kq] = (f32x4){0.f, 0.f, 0.f, 0.f};
      const uint16_t* kr = rows + kq * 16 * (LROW * 8) + kbase;
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
        sk[kq][r] = kb0 + kq * 16 + 4 * gi + r < u.n ? sk[kq][r] * m.qscale : -INFINITY;
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
#pragma unroll
    for (int db = 0; db < LAT / 16; ++db) {
      const uint16_t* vp = rows + vbase + 16 * db;
      const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vp));
      const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vp + 16 * (LROW * 8)));
      const i16x8 vv = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(bf16x8, vv), o[db],
                                                      0, 0, 0);
    }
  };

  // the piece of sequence bq this share holds is done: write its partial and start afresh
  auto finish = [&](int bq) {
    float l = lsum + __shfl_xor(lsum, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int64_t pbase = (int64_t)(c + bq) * m.H + h0;
    if (lane < HPW) {
      float* ml = m.part_ml + (pbase + lane) * 2;
      ml[0] = mx;
      ml[1] = l;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float* po = m.part_o + (pbase + 4 * gi + r) * LAT + si;
#pragma unroll
      for (int db = 0; db < LAT / 16; ++db) po[16 * db] = o[db][r];
    }
#pragma unroll
    for (int db = 0; db < LAT / 16; ++db) o[db] = (f32x4){0.f, 0.f, 0.f, 0.f};
    mx = kNegBig;
    lsum = 0.f;
  };

  // Four stages: when block t is read, blocks t + 1 and t + 2 are in flight and t + 3 goes into
  // the stage that held t - 1 (every wavefront is past its reads of it: they precede this
  // barrier).
  Cursor ic = cc;
  issue_block<NW>(m, ic, 0, w, lane);
  if (nu > 1) {
    cursor_advance(m, ic);
    issue_block<NW>(m, ic, 1, w, lane);
  }
  if (nu > 2) {
    cursor_advance(m, ic);
    issue_block<NW>(m, ic, 2, w, lane);
  }
  if (active) load_q(cc.b);
  for (int t = 0; t < nu; ++t) {
    wait_block<NDMA / NW>(min(nu - 1 - t, 2), extra);
    __syncthreads();
    if (t + 3 < nu) {
      cursor_advance(m, ic);
      issue_block<NW>(m, ic, (t + 3) % NSTM, w, lane);
    }
    if (active) compute(cc, t % NSTM);
    const bool last = t + 1 == nu;
    if (cc.j + 1 == cc.nb || last) {
      if (active) finish(cc.b);
      if (!last) {
        cursor_advance(m, cc);
        if (active) load_q(cc.b);
      }
    } else {
      ++cc.j;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load into LDS outstanding when the workgroup ends
}

// out[b, h, :] = sum_p 2^(m_p - M) O_p / sum_p 2^(m_p - M) l_p over the pieces p of sequence b;
// 4 heads per workgroup, 8 features per lane.
__global__ __launch_bounds__(256) void mla_combine_kernel(MlaArgs m) {
  const int b = blockIdx.x, lane = threadIdx.x & 63;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (h >= m.H) return;
  int U = 0, first = 0;  // the batch's blocks, and those of the sequences before b
  for (int base = 0; base < m.B; base += 64) {
    const int nb = seq_blocks(m, base + lane);
    U += wave_sum(nb);
    first += wave_sum(base + lane < b ? nb : 0);
  }
  const int nb = seq_blocks(m, b);
  uint16_t* dst = m.out + ((int64_t)b * m.H + h) * LAT + 8 * lane;
  if (nb == 0) {  // no cached row: zeros
    *(u32x4*)dst = (u32x4){0u, 0u, 0u, 0u};
    return;
  }
  const int c0 = share_of(first, U), c1 = share_of(first + nb - 1, U);
  float M = kNegBig;
  for (int c = c0; c <= c1; ++c)
    if (share_lo(c, U) < share_lo(c + 1, U))
      M = fmaxf(M, m.part_ml[((int64_t)(c + b) * m.H + h) * 2]);
  f32x4 a0 = (f32x4){0.f, 0.f, 0.f, 0.f}, a1 = a0;
  float lt = 0.f;
  for (int c = c0; c <= c1; ++c) {
    if (share_lo(c, U) == share_lo(c + 1, U)) continue;
    const int64_t it = (int64_t)(c + b) * m.H + h;
    const float wgt = fast_exp2(m.part_ml[it * 2] - M);
    lt += wgt * m.part_ml[it * 2 + 1];
    const f32x4* po = (const f32x4*)(m.part_o + it * LAT + 8 * lane);
    a0 += wgt * po[0];
    a1 += wgt * po[1];
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const u32x4 v = {pack_bf16x2(a0[0] * inv, a0[1] * inv), pack_bf16x2(a0[2] * inv, a0[3] * inv),
                   pack_bf16x2(a1[0] * inv, a1[1] * inv), pack_bf16x2(a1[2] * inv, a1[3] * inv)};
  *(u32x4*)dst = v;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t mla_decode_workspace_bytes(int B, int H, int Smax) {
  (void)Smax;
  const size_t slots = (size_t)kMlaWorkgroups + B;
  const size_t groups = (size_t)(H + HPG - 1) / HPG;
  return align256(slots * H * LAT * 4) + align256(slots * H * 2 * 4) +
         groups * kMlaWorkgroups * 4 * sizeof(int32_t);
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
  m.qscale = scale * kLog2e;
  char* ws = (char*)workspace;
  const size_t slots = (size_t)kMlaWorkgroups + B;
  m.part_o = (float*)ws;
  m.part_ml = (float*)(ws + align256(slots * H * LAT * 4));
  m.flags = (int32_t*)(ws + align256(slots * H * LAT * 4) + align256(slots * H * 2 * 4));
  const dim3 grid(kMlaWorkgroups, (H + HPG - 1) / HPG);
  hipLaunchKernelGGL(mla_split32_kernel, grid, dim3(4 * 64), 0, stream, m);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_split16_kernel, grid, dim3(8 * 64), 0, stream, m);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_combine_kernel, dim3(B, (H + 3) / 4), dim3(256), 0, stream, m);
  return hipGetLastError();
}

}  // namespace gqa
