// bf16 MFMA prefill, head_dim 128, gfx950 -- streaming variant used when the caller provides a
// workspace for the prepared keys.
//
// Two launches:
//  1. rows_prep_kernel: every NEW key row (index >= n_cached) is RMS-normed and rotated once
//     ([Models] "What differs": q/k norm then rotation; [Guide] section 3.2 and section 4) and
//     written, rounded to bf16, to the workspace; the workspace also holds the last 31 cached rows
//     (copied as stored) so that every key tile reads a single source.  Other cached rows are
//     used in place.  This is the cache-append step of the page's flow (rotate,
//     then cache.update) and costs one read and one write of the new keys, instead of redoing the
//     norm and rotation each time a key tile is revisited by another query block.
//  2. prefill_stream_kernel: the attention proper.  Same tiling and math as the fused kernel
//     (4 wavefronts x 32 query rows of one KV head, 32-key tiles, S^T = K Q^T and O^T = V^T P^T on
//     v_mfma_f32_32x32x16_bf16, online softmax in log2 units with lazy rescaling), but K and V
//     tiles travel from HBM straight into LDS with buffer_load ... lds: no VGPR staging, no LDS
//     store instructions, 32-bit offsets from a buffer descriptor, and the descriptor's range check
//     returns zeros past the last key, which handles the ragged tail.  Each wave instruction fills
//     1 KB of LDS in lane order; choosing the source chunk per lane produces the XOR-swizzled
//     layout the MFMA operand reads want.
#include <type_traits>

#include "launch.hpp"

namespace gqa {
namespace {

constexpr int HD = 128;
constexpr int NW = 4;
constexpr int NT = NW * 64;
constexpr int ROWS = NW * 32;
constexpr int BN = 32;
constexpr int TILE_ELEMS = BN * HD;
constexpr int kTileRounds = BN / (4 * NW);  // 1 KB loads per wave per K (or V) tile
static_assert(BN % (4 * NW) == 0 && BN <= 64, "tile loader and key-position loader layout");
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
__device__ __forceinline__ void tile_dma16(i32x4 rsrc, const lds_void* dst, int voff) {
  uint32_t saved;  // m0 is the LDS address operand; it is restored for the compiler
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 4\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane((int)(uintptr_t)dst)), "v"(voff), "s"(rsrc));
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

// ---------------------------------------------------------------------------------------------
// 1. key preparation: 16 lanes per key row (8 features each), 16 rows per 256-thread block
// ---------------------------------------------------------------------------------------------
// Rows j0 .. S-1 of k are visited; row (b, j, g) lands at kout + b*ob + (j - jofs)*oj + g*D: the
// compact workspace [B, S - j0, Hkv, D] (jofs = j0) or a full [B, S, Hkv, D] buffer such as a KV
// cache (jofs = 0), which may be k itself (each row is read completely before it is written).
// Rows below n_cached are copied as stored, rows from n_cached on are normed and rotated.
struct PrepOut {
  uint16_t* p;
  int64_t ob, oj;
  int32_t jofs;
  int32_t j0;
};

// Lane exchanges within a row of 16 lanes by data-parallel-primitive moves (no LDS traffic).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppShl4 = 0x104;       // lane i reads lane i + 4
constexpr int kDppShr4 = 0x114;       // lane i reads lane i - 4
constexpr int kDppRor8 = 0x128;       // lane i reads lane i ^ 8 (rotate by half a row)
constexpr int kDppHalfMirror = 0x141; // lane i reads lane 7 - i within its 8
constexpr int kDppMirror = 0x140;     // lane i reads lane 15 - i

// Sum over the 16 lanes of a row, in every lane.
__device__ __forceinline__ float row16_sum(float s) {
  s += dpp_mov<kDppXor1>(s);
  s += dpp_mov<kDppXor2>(s);
  s += dpp_mov<kDppHalfMirror>(s);
  s += dpp_mov<kDppMirror>(s);
  return s;
}

// Rows (b, p, h) for position indices p in [p0, pend) of a [B, *, H, 128] bf16 source are normed
// (gain w), rotated at pos[b * pos_b + p] and multiplied by mul, then stored as bf16 at
// dst + b*db + (p - pofs)*dp + h*128 -- or, with a block table, at slot slot0[b] + p - p0 of a
// paged pool dst [num_blocks, H, 2^log2bs, 128].  Rows with p < fresh_from are copied as stored.
struct RowJob {
  const int32_t* ptable;  // paged destination when non-null
  const int32_t* slot0;
  int32_t pmax_blocks, plog2bs, pnum_blocks;
  const uint16_t* src;
  int64_t sb, sp, sh;
  uint16_t* dst;
  int64_t db, dp;
  const int32_t* pos;
  int64_t pos_b;
  const uint16_t* w;
  int32_t H, p0, pend, pofs, fresh_from;
  float mul;
};

// 16 lanes per row, 8 features per lane (lane c: features 8c .. 8c + 7).  Each 16-lane group takes
// up to kHeadsPerGroup heads of one position, so the position's table entries are loaded once
// for all of them; 16 groups per block, blockIdx.y is the sequence.  (pend - p0) * H < 2^31 (the
// host checks the sizes).
constexpr int kHeadsPerGroup = 8;

template <int ROT, bool NORM>
__global__ __launch_bounds__(256) void rows_prep_kernel(AttnArgs a, RowJob jb) {
  constexpr int HG = kHeadsPerGroup;
  const int b = blockIdx.y;
  const int c = threadIdx.x & 15;
  const uint32_t nch = (uint32_t)(jb.H + HG - 1) / HG;  // head chunks per position
  const uint32_t gi = blockIdx.x * 16u + (threadIdx.x >> 4);
  const bool valid = gi < (uint32_t)(jb.pend - jb.p0) * nch;
  const uint32_t gg = valid ? gi : 0u;
  const uint32_t pi = gg / nch;
  const int h0 = (int)(gg - pi * nch) * HG;
  const int p = jb.p0 + (int)pi;
  const bool fresh = p >= jb.fresh_from;  // uniform over the group's 16 lanes
  const uint16_t* src = jb.src + (int64_t)b * jb.sb + (int64_t)p * jb.sp + 8 * c;
  u32x4 raw[HG];
#pragma unroll
  for (int k = 0; k < HG; ++k) raw[k] = ld16(src + (int64_t)min(h0 + k, jb.H - 1) * jb.sh);
  // this lane's table entries at the row position: 8 (half-split) or 4 (adjacent pairs) pairs
  float cs[8], sn[8];
  const bool rot = ROT != 0 && fresh && 8 * c < a.R;
  if (ROT != 0) {
    const int32_t pp = jb.pos[(int64_t)b * jb.pos_b + p];
    const int64_t tp = min<int64_t>(max<int64_t>(pp, 0), a.table_len - 1);
    const int halfp = a.R >> 1;
    const int d0 = rot ? 8 * c : 0;
    const int q0 = ROT == 1 ? (d0 < halfp ? d0 : d0 - halfp) : d0 >> 1;
    const float* cr = a.cos_t + tp * halfp + q0;
    const float* sr = a.sin_t + tp * halfp + q0;
    const f32x4 c0 = *(const f32x4*)cr, s0 = *(const f32x4*)sr;
    f32x4 c1 = c0, s1 = s0;
    if (ROT == 1) {
      c1 = *(const f32x4*)(cr + 4);
      s1 = *(const f32x4*)(sr + 4);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      cs[e] = c0[e];
      sn[e] = s0[e];
      cs[e + 4] = c1[e];
      sn[e + 4] = s1[e];
    }
  }
  float wv[8];
  if (NORM) unpack8(ld16(jb.w + 8 * c), wv);
  const bool first = 8 * c < (a.R >> 1);
  const int P = a.R >> 4;  // half-split: the partner chunk is P = R/16 chunks away (lane c ^ P)
#pragma unroll
  for (int k = 0; k < HG; ++k) {
    float x[8];
    unpack8(raw[k], x);
    if (NORM && fresh) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
      ss = row16_sum(ss);
      const float rs = rsqrtf(ss * (1.0f / HD) + a.eps);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= rs * wv[e];
    }
    if (ROT == 1 && fresh) {
      float y[8];
      if (P == 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = dpp_mov<kDppXor1>(x[e]);
      } else if (P == 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = dpp_mov<kDppXor2>(x[e]);
      } else if (P == 4) {
        const bool up = (c & 4) != 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float l = dpp_mov<kDppShl4>(x[e]), rgt = dpp_mov<kDppShr4>(x[e]);
          y[e] = up ? rgt : l;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = dpp_mov<kDppRor8>(x[e]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float r = first ? (x[e] * cs[e] - y[e] * sn[e]) : (y[e] * sn[e] + x[e] * cs[e]);
        x[e] = rot ? r : x[e];
      }
    } else if (ROT == 2 && fresh) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float u = x[2 * e], v = x[2 * e + 1];
        x[2 * e] = rot ? u * cs[e] - v * sn[e] : u;
        x[2 * e + 1] = rot ? u * sn[e] + v * cs[e] : v;
      }
    }
    if (jb.mul != 1.0f) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= jb.mul;
    }
    if (valid && h0 + k < jb.H) {
      uint16_t* dst;
      if (jb.ptable) {
        // slot and table index clamped into the table: a violated precondition writes wrong
        // slots, never outside the pool
        const int64_t cap = (int64_t)jb.pmax_blocks << jb.plog2bs;
        const int64_t slot = min<int64_t>(max<int64_t>((int64_t)jb.slot0[b] + (p - jb.p0), 0),
                                          cap - 1);
        int phys = jb.ptable[(int64_t)b * jb.pmax_blocks + (slot >> jb.plog2bs)];
        phys = min(max(phys, 0), jb.pnum_blocks - 1);
        const int64_t row = ((((int64_t)phys * jb.H + h0 + k) << jb.plog2bs) |
                             (slot & ((1 << jb.plog2bs) - 1)));
        dst = jb.dst + row * HD;
      } else {
        dst = jb.dst + (int64_t)b * jb.db + (int64_t)(p - jb.pofs) * jb.dp + (int64_t)(h0 + k) * HD;
      }
      *(u32x4*)(dst + 8 * c) = pack8(x);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// 2. attention over prepared keys
// ---------------------------------------------------------------------------------------------
// Triple-buffered K/V/key-position tiles.  Each buffer is its own LDS object and the step loop
// is unrolled over the buffer cycle, so every access names its buffer at compile time: the
// compiler can then see that reads of the current tiles never alias the asynchronous HBM->LDS
// loads of a later one and does not make them wait for those loads.
constexpr int NBUF = 3;
__shared__ __attribute__((aligned(16))) uint16_t g_k0[TILE_ELEMS];
__shared__ __attribute__((aligned(16))) uint16_t g_k1[TILE_ELEMS];
__shared__ __attribute__((aligned(16))) uint16_t g_k2[TILE_ELEMS];
__shared__ __attribute__((aligned(16))) uint16_t g_v0[TILE_ELEMS];
__shared__ __attribute__((aligned(16))) uint16_t g_v1[TILE_ELEMS];
__shared__ __attribute__((aligned(16))) uint16_t g_v2[TILE_ELEMS];
__shared__ __attribute__((aligned(16))) int32_t g_p0[BN];
__shared__ __attribute__((aligned(16))) int32_t g_p1[BN];
__shared__ __attribute__((aligned(16))) int32_t g_p2[BN];

template <int BUF>
__device__ __forceinline__ uint16_t* kbuf() { return BUF == 0 ? g_k0 : BUF == 1 ? g_k1 : g_k2; }
template <int BUF>
__device__ __forceinline__ uint16_t* vbuf() { return BUF == 0 ? g_v0 : BUF == 1 ? g_v1 : g_v2; }
template <int BUF>
__device__ __forceinline__ int32_t* pbuf() { return BUF == 0 ? g_p0 : BUF == 1 ? g_p1 : g_p2; }

struct StreamArgs {
  AttnArgs a;
  const uint16_t* kprep;   // [B, S - w0, Hkv, D] keys from row w0 = max(n_cached - (BN-1), 0) on,
                           // new ones prepared (null if nothing needs preparing)
};

template <int ROT, bool NORM, bool CAP>
// Two workgroups per CU (3 x 16 KB tiles of LDS and up to 256 VGPRs each): one's query prep and
// first tiles overlap the other's loop, and each barrier holds only the four waves of one group.
__global__ __launch_bounds__(NT, 2) void prefill_stream_kernel(StreamArgs sa, int nqb) {
  const AttnArgs& a = sa.a;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int ql = lane & 31, hg = lane >> 5;
  // Work item of this workgroup.  Workgroups are dealt to the 8 XCDs round-robin by id; map ids
  // so that every query block of one (b, g) lands on the same XCD (its K/V then stay in that
  // XCD's L2), heaviest (latest) query blocks first within each XCD.
  int qb, g, b;
  {
    const int L = blockIdx.x;
    const int npairs = a.B * a.Hkv;
    int pair, rank;
    if (npairs % kXcds == 0) {
      const int per = npairs / kXcds;
      const int x = L % kXcds, k = L / kXcds;
      pair = x + kXcds * (k % per);
      rank = k / per;
    } else {
      pair = L % npairs;
      rank = L / npairs;
    }
    qb = nqb - 1 - rank;
    b = pair / a.Hkv;
    g = pair % a.Hkv;
  }
  const int G = a.G;
  const int64_t nrows = (int64_t)a.L * G;
  const int64_t f0 = (int64_t)qb * ROWS;

  // ---- this lane's query row (flattened position-major (position, head) index) ----
  const int64_t f = f0 + w * 32 + ql;
  const bool qvalid = f < nrows;
  const int qi = qvalid ? (int)(f / G) : 0;
  const int qh = g * G + (qvalid ? (int)(f % G) : 0);
  const int32_t* qpos_b = a.qpos + (int64_t)b * a.qpos_b;
  const int32_t qp_raw = qpos_b[qi];  // qi is a valid index even for rows past the end
  const int32_t qp = qvalid ? qp_raw : 0;

  // ---- key band of the workgroup's query positions (loads issued here, used after Q prep) ----
  const int32_t* kpos_b = a.kpos + (int64_t)b * a.kpos_b;
  const int i_lo = (int)(f0 / G);
  const int i_hi = (int)min<int64_t>((f0 + ROWS - 1) / G, (int64_t)a.L - 1);
  // (at most ROWS positions; every load is issued, at a clamped index, before any is used)
  int32_t prange[ROWS / 64];
#pragma unroll
  for (int k = 0; k < ROWS / 64; ++k) prange[k] = qpos_b[min(i_lo + lane + 64 * k, i_hi)];
  int32_t pmn = INT32_MAX, pmx = INT32_MIN;
#pragma unroll
  for (int k = 0; k < ROWS / 64; ++k) {
    const bool in = i_lo + lane + 64 * k <= i_hi;
    pmn = min(pmn, in ? prange[k] : INT32_MAX);
    pmx = max(pmx, in ? prange[k] : INT32_MIN);
  }
  const int32_t kp0 = kpos_b[0];

  // ---- buffer descriptors of this (b, g): cached keys, prepared keys, values ----
  const int row_bytes = (int)(a.k_j * 2);  // bytes between consecutive keys of one head
  const int64_t kv_base = (int64_t)b * a.k_b + (int64_t)g * a.k_h;
  // Without a workspace nothing needs preparing and every key comes from k.  With one, a tile
  // whose keys all lie below nc comes from k as stored and any other from the workspace, which
  // starts at row w0 <= (first row of any tile reaching past nc).  The choice is uniform per
  // tile, so each load names one descriptor.
  const int nc = sa.kprep ? a.n_cached : a.S;
  const int w0 = nc > BN - 1 ? nc - (BN - 1) : 0;
  const int nws = a.S - w0;
  const i32x4 rk = rsrc_words((const uint16_t*)a.k + kv_base,
                              nc > 0 ? (nc - 1) * row_bytes + HD * 2 : 0);
  const i32x4 rw = rsrc_words(
      sa.kprep ? sa.kprep + (int64_t)b * nws * a.k_j + (int64_t)g * a.k_h : nullptr,
      (sa.kprep && nws > 0) ? (nws - 1) * row_bytes + HD * 2 : 0);
  const i32x4 rv = rsrc_words((const uint16_t*)a.v + kv_base, (a.S - 1) * row_bytes + HD * 2);
  const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.kpos + (int64_t)b * a.kpos_b), (short)0, a.S * 4, kBufFlags);

  uint32_t kp_pend = 0;
  bool kp_pend_ok = false;
  // Tile loader: wave w, round i fills LDS rows 4*(w + NW i) .. +3 (1 KB); lane -> row
  // 4(w + NW i) + lane/16, LDS chunk lane%16, which holds source chunk (lane%16) ^ swz(row).
  // Lane constants of the tile loader (offset of the lane's 16 bytes within a tile); a tile adds
  // jt rows.  Rows at or past S fall outside the descriptors' ranges and read as zero.
  int lk[kTileRounds], lv[kTileRounds];
#pragma unroll
  for (int i = 0; i < kTileRounds; ++i) {
    const int r = 4 * (w + NW * i) + (lane >> 4);
    lk[i] = r * row_bytes + (((lane & 15) ^ kswz(r)) << 4);
    lv[i] = r * row_bytes + (((lane & 15) ^ vswz(r)) << 4);
  }
  auto issue_tile = [&](int jt, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int tb = jt * row_bytes;  // values (and cached keys): rows from 0
    const bool from_k = sa.kprep == nullptr || jt + BN <= nc;
    const i32x4 rks = from_k ? rk : rw;
    const int kb0 = from_k ? tb : (jt - w0) * row_bytes;
#pragma unroll
    for (int i = 0; i < kTileRounds; ++i) {
      lds_void* kdst = (lds_void*)(kbuf<buf>() + 4 * (w + NW * i) * HD);
      lds_void* vdst = (lds_void*)(vbuf<buf>() + 4 * (w + NW * i) * HD);
      tile_dma16(rv, vdst, lv[i] + tb);
      tile_dma16(rks, kdst, lk[i] + kb0);
    }
    // key positions of the tile: loaded by wave 0 into a register and written to LDS by
    // commit_kpos once the tile's loads are complete, with INT32_MAX past the last key so that the
    // position test alone masks the ragged tail
    if (w == 0) {
      kp_pend = __builtin_amdgcn_raw_buffer_load_b32(rp, (jt + lane) * 4, 0, 0);
      kp_pend_ok = lane < BN && jt + lane < a.S;
    }
  };
  auto commit_kpos = [&](auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    if (w == 0 && lane < BN) pbuf<buf>()[lane] = kp_pend_ok ? (int32_t)kp_pend : INT32_MAX;
  };


  // ---- band guesses: with consecutive key positions the band edges are known from the query
  // positions; the two keys around each guess are loaded now (clamped indices) and checked below
  int32_t qmn = pmn, qmx = pmx;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    qmn = min(qmn, __shfl_xor(qmn, off, 64));
    qmx = max(qmx, __shfl_xor(qmx, off, 64));
  }
  // wave-uniform from here on: scalar registers
  const int64_t qmin = __builtin_amdgcn_readfirstlane(qmn), qmax = __builtin_amdgcn_readfirstlane(qmx);
  const int64_t x_hi = qmax + 1, x_lo = key_floor(a, qmin);
  // a tile needs no mask when every query may see its first key (and its last is causal for all)
  const int32_t floor_max = (int32_t)max<int64_t>(key_floor(a, qmax), INT32_MIN);
  const int g_hi = (int)min<int64_t>(max<int64_t>(x_hi - kp0, 0), a.S);
  const int g_lo = (int)min<int64_t>(max<int64_t>(x_lo - kp0, 0), a.S);
  // The first tile's loads go out now -- at key 0 without a window or chunks, else at the guessed
  // band start (loaded again below if the guess is wrong) -- after the waits for the position
  // loads above (a wait for those placed behind the tile's loads would wait for the tile too) and
  // beside the band and query-prep loads below.
  const int j_first = a.has_floor() ? g_lo : 0;
  __builtin_amdgcn_sched_barrier(0);
  issue_tile(j_first, std::integral_constant<int, 0>());
  const int32_t hi_l = kpos_b[max(g_hi - 1, 0)], hi_r = kpos_b[min(g_hi, a.S - 1)];
  const int32_t lo_l = kpos_b[max(g_lo - 1, 0)], lo_r = kpos_b[min(g_lo, a.S - 1)];
  // smallest key position the row may see (window, chunks); INT32_MAX for rows past the end
  const int32_t qlo32 = !qvalid ? INT32_MAX
                        : a.has_floor() ? (int32_t)max<int64_t>(key_floor(a, qp), INT32_MIN)
                                        : INT32_MIN;

  // ---- query prep, per wavefront and in registers: lane (ql, hg) loads, for its row, exactly the
  // features its MFMA operands hold -- 16 s + 8 hg .. + 7 for s = 0..7 -- RMS-norms the row (the
  // other 64 features are in lane ql + 32), rotates it at its position and scales it into log2
  // units.  With half-split rotation at R = 32, 64 or 128 a feature's partner (R/2 further on)
  // lies R/32 operand chunks further in the same lane; at R = 16 it is in lane l ^ 32.
  // Interleaved pairs are adjacent.  No LDS and no barrier: the waves prep independently, in two
  // memory round trips (rows, gains and the position; then the table entries at the position).
  bf16x8 qop[8];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + (int64_t)b * a.q_b + (int64_t)qi * a.q_i +
                           (int64_t)qh * a.q_h + 8 * hg;
    u32x4 xw[8], ww[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) xw[s] = ld16(qrow + 16 * s);
    if (NORM) {
#pragma unroll
      for (int s = 0; s < 8; ++s) ww[s] = ld16((const uint16_t*)a.qw + 16 * s + 8 * hg);
    }
    const int P = a.R >> 4;  // half-split: partner distance in 8-feature chunks
    const int halfp = a.R >> 1;
    const int64_t tp = min<int64_t>(max<int64_t>(qp, 0), a.table_len - 1);
    const float* crow = a.cos_t + tp * halfp;
    const float* srow = a.sin_t + tp * halfp;
    // table entries: half-split -- for each first-half chunk c = 2 s + hg < P (so s < 4), its 8
    // pairs (at R = 16 both lanes load pairs 0..7); interleaved -- for each rotated chunk, its 4
    f32x4 tc[8][2], ts[8][2];
    if (ROT == 1) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int cch = 2 * s + hg;
        const bool ld = P == 1 ? s == 0 : cch < P;
        const int pb = P == 1 ? 0 : 8 * cch;
        if (ld) {
          tc[s][0] = *(const f32x4*)(crow + pb);
          tc[s][1] = *(const f32x4*)(crow + pb + 4);
          ts[s][0] = *(const f32x4*)(srow + pb);
          ts[s][1] = *(const f32x4*)(srow + pb + 4);
        }
      }
    } else if (ROT == 2) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int cch = 2 * s + hg;
        if (8 * cch < a.R) {
          tc[s][0] = *(const f32x4*)(crow + 4 * cch);
          ts[s][0] = *(const f32x4*)(srow + 4 * cch);
        }
      }
    }
    float x[8][8];
#pragma unroll
    for (int s = 0; s < 8; ++s) unpack8(xw[s], x[s]);
    if (NORM) {
      float ss = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += x[s][e] * x[s][e];
      ss += swap_halves(ss);
      const float rs = rsqrtf(ss * (1.0f / HD) + a.eps);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        float wv[8];
        unpack8(ww[s], wv);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[s][e] *= rs * wv[e];
      }
    }
    if (ROT == 1) {
      if (P == 1) {
        // chunk 0 (lane hg = 0, first half) and chunk 1 (lane hg = 1, second half) pair up
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float y = swap_halves(x[0][e]);
          const float cs = tc[0][e >> 2][e & 3], sn = ts[0][e >> 2][e & 3];
          x[0][e] = hg == 0 ? x[0][e] * cs - y * sn : y * sn + x[0][e] * cs;
        }
      } else {
        const int hs = P >> 1;  // partner distance in this lane's chunk index: 1, 2 or 4
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if (2 * s + hg < P) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float cs = tc[s][e >> 2][e & 3], sn = ts[s][e >> 2][e & 3];
              const float lo = x[s][e];
              // (the partner chunk is picked without dynamic register indexing)
              const float hi = hs == 1 ? x[s + 1][e] : hs == 2 ? x[s + 2][e] : x[s + 4][e];
              x[s][e] = lo * cs - hi * sn;
              const float nhi = hi * cs + lo * sn;
              if (hs == 1) x[s + 1][e] = nhi;
              else if (hs == 2) x[s + 2][e] = nhi;
              else x[s + 4][e] = nhi;
            }
          }
        }
      }
    } else if (ROT == 2) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if (8 * (2 * s + hg) < a.R) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float cs = tc[s][0][e], sn = ts[s][0][e];
            const float u = x[s][2 * e], v = x[s][2 * e + 1];
            x[s][2 * e] = u * cs - v * sn;
            x[s][2 * e + 1] = u * sn + v * cs;
          }
        }
      }
    }
    const float qscale = a.scale * kLog2e;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[s][e] = qvalid ? x[s][e] * qscale : 0.f;
      qop[s] = as_bf16x8(pack8(x[s]));
    }
  }

  // ---- band: first key past the newest query, first key the oldest query may see ----
  // (a guess is right when the key before it is below the target and the key at it is not; if
  // positions are not consecutive the wavefront searches)
  const bool ok_hi = (g_hi == 0 || (int64_t)hi_l < x_hi) && (g_hi == a.S || (int64_t)hi_r >= x_hi);
  const bool ok_lo = (g_lo == 0 || (int64_t)lo_l < x_lo) && (g_lo == a.S || (int64_t)lo_r >= x_lo);
  int j_hi = ok_hi ? g_hi : wave_lower_bound(kpos_b, a.S, x_hi);
  int j_lo = !a.has_floor() ? 0 : ok_lo ? g_lo : wave_lower_bound(kpos_b, a.S, x_lo);
  j_lo = min(j_lo, j_hi);
  const int n_tiles = (j_hi - j_lo + BN - 1) / BN;

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  // Running max m (log2 units; kNegBig until the row has seen an allowed key) and sum.  Scores
  // are kept relative to m_eff = (m set ? m : 0): the S^T accumulators start at -m_eff, so the
  // MFMAs deliver s - m_eff directly.  (Soft-capping needs the raw score: there they start at 0
  // and m_eff is subtracted after the cap.)
  float m = kNegBig, lsum = 0.f;
  const float cap2 = a.softcap * kLog2e;
  const float inv_cap2 = CAP ? 1.0f / cap2 : 0.f;

  // per-lane LDS read offsets (elements).  K: row ql, chunk 2s + hg.  V^T (transposing reads):
  // rows 4*hgv + s16/4 (+8 for items 4..7) of each 16-key group, columns db*32 + 16*(gi&1) +
  // 4*(s16&3); both swizzles only see the row's low 4 bits, which the 16-key group offset leaves
  // unchanged.
  const int gi = lane >> 4, s16 = lane & 15;
  const int hgv = gi >> 1;
  int koff[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) koff[s] = ql * HD + (((2 * s + hg) ^ kswz(ql)) << 3);
  int voff[2][4];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int row = 4 * hgv + (s16 >> 2) + 8 * h2;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int col = db * 32 + 16 * (gi & 1) + 4 * (s16 & 3);
      voff[h2][db] = row * HD + (((col >> 3) ^ vswz(row)) << 3) + (col & 7);
    }
  }
  // mask bounds in int32: allowed <=> qlo32 <= key position <= qp32 (key positions past the last
  // key read INT32_MAX, so the ragged tail fails the first test)
  // (qlo32, the window/chunk bound, is computed once the band loads are out: earlier it would
  // wait for this row's position before any other load is issued, later it costs registers)
  const int32_t qp32 = qvalid ? (int32_t)qp : INT32_MIN;

  // S^T - m_eff for the 32 keys of a buffered tile
  auto qk = [&](auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const uint16_t* ks = kbuf<buf>();
    u32x4 kop[8];
#pragma unroll
    for (int st = 0; st < 8; ++st) kop[st] = *(const u32x4*)(ks + koff[st]);
    // all eight operand reads in flight before the first MFMA waits on one
    __builtin_amdgcn_sched_barrier(0);
    const float init = (CAP || m == kNegBig) ? 0.f : -m;
    const uint64_t init2 = ((uint64_t)__float_as_uint(init) << 32) | __float_as_uint(init);
    const u64x8 seed = {init2, init2, init2, init2, init2, init2, init2, init2};
    f32x16 acc = __builtin_bit_cast(f32x16, seed);
#pragma unroll
    for (int st = 0; st < 8; ++st)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kop[st]), qop[st], acc, 0, 0, 0);
    return acc;
  };

  // One step = one 32-key tile, software-pipelined: the step's own S^T was computed by the
  // previous step; here the mask and running max come first, then the NEXT tile's S^T MFMAs are
  // issued, then this step's exponentials and P V.  In program order the next S^T MFMAs therefore
  // sit beside this step's exponentials, and this step's P V MFMAs beside the next step's mask and
  // max, so the matrix unit and the vector ALU work at the same time.
  // Tiles live in NBUF = 3 buffers: the barrier before the S^T of tile t+1 waits for tile t+1's
  // loads, and once every wavefront is past it the buffer of tile t-1 is free for tile t+2's.
  const int nsteps = n_tiles;
  // two score sets that trade roles every step (a step reads one and fills the other), so no
  // copy of the next step's scores has to wait for its MFMAs
  f32x16 s_a, s_b;
  auto step = [&](int s, auto phc, f32x16& sc, f32x16& s_next) {
    constexpr int PH = decltype(phc)::value;  // position in the 6-step cycle (buffers x score sets)
    constexpr int buf = PH % NBUF;
    constexpr int nbuf = (buf + 1) % NBUF;
    const int t = s;
    const int jt = j_lo + t * BN;
    const int32_t* kpt = pbuf<buf>();
    const int32_t kfirst = kpt[0];
    const int32_t klast = kpt[BN - 1];
    const bool full = (jt + BN <= j_hi) && ((int64_t)klast <= qmin) &&
                      (kfirst >= floor_max);

    // ---- soft-cap, mask, running max ----
    const bool unset = m == kNegBig;
    if (CAP) {
      const float meff = unset ? 0.f : m;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = sc[r] * inv_cap2;
        const float e = fast_exp2(-2.0f * kLog2e * fabsf(x));
        sc[r] = copysignf(cap2 * (1.0f - e) * __builtin_amdgcn_rcpf(1.0f + e), x) - meff;
      }
    }
    if (!full) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int32_t kp = kpt[8 * (r >> 2) + 4 * hg + (r & 3)];
        if (!(kp <= qp32 && kp >= qlo32)) sc[r] = -INFINITY;
      }
    }
    float mt = sc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sc[r]);
    mt = fmaxf(mt, swap_halves(mt));
    // lazy rescale: the reference moves only when a score exceeds it by more than the threshold
    // (or on the row's first allowed key)
    const bool upd = unset ? (mt > -INFINITY) : (mt > kRescaleThreshold);
    if (__ballot(upd) != 0) {
      const float delta = unset ? (mt > -INFINITY ? mt : 0.f) : fmaxf(mt, 0.f);
      const float alpha = unset ? 1.f : fast_exp2(-delta);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      m = unset ? (mt > -INFINITY ? mt : kNegBig) : m + delta;
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] -= delta;
    }

    // ---- the next tile's S^T, after the crossing into it ----
    if (s + 1 < nsteps) {
      __builtin_amdgcn_s_waitcnt(0);
      commit_kpos(std::integral_constant<int, nbuf>());
      __syncthreads();
      if (t + 2 < n_tiles) issue_tile(jt + 2 * BN, std::integral_constant<int, (buf + 2) % NBUF>());
    }
    // Issued unconditionally so that it shares one basic block with the exponentials and P V
    // below (the scheduler interleaves only within a block); after the last step it reads a
    // stale buffer and its result is unused.
    s_next = qk(std::integral_constant<int, nbuf>());

    // ---- P = exp2(s - m); row sums of the bf16 weights the P V product uses, two per
    // v_dot2_f32_bf16 against (1, 1) ----
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones2 = {(__bf16)1.0f, (__bf16)1.0f};
    bf16x8 pb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = fast_exp2(sc[8 * u + e]);
      pb[u] = as_bf16x8(pack8(p));
      // (each pair is built from its two floats: taking it out of the packed vector with a bit
      // cast made the compiler feed the first pair to all four dot products)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2 pr = {(__bf16)p[2 * e], (__bf16)p[2 * e + 1]};
        lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2, lsum, false);
      }
    }

    // ---- O^T += V^T P^T ----
    const uint16_t* vs = vbuf<buf>();
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int base = 16 * u * HD;
        const i16x4 vlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vs + base + voff[0][db]));
        const i16x4 vhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vs + base + voff[1][db]));
        const i16x8 va = {vlo[0], vlo[1], vlo[2], vlo[3], vhi[0], vhi[1], vhi[2], vhi[3]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va), pb[u],
                                                        o[db], 0, 0, 0);
      }
  };

  if (j_lo != j_first && n_tiles > 0) {
    __builtin_amdgcn_s_waitcnt(0);  // the guessed tile's loads land before the right tile's
    issue_tile(j_lo, std::integral_constant<int, 0>());
  }
  __builtin_amdgcn_s_waitcnt(0);  // also retires the early first-tile loads when n_tiles == 0
  commit_kpos(std::integral_constant<int, 0>());
  __syncthreads();  // the first tile and its key positions are visible to every wave
  if (n_tiles > 1) issue_tile(j_lo + BN, std::integral_constant<int, 1>());
  if (nsteps > 0) s_a = qk(std::integral_constant<int, 0>());
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  using P3 = std::integral_constant<int, 3>;
  using P4 = std::integral_constant<int, 4>;
  using P5 = std::integral_constant<int, 5>;
  for (int s = 0; s < nsteps; s += 6) {
    step(s, P0(), s_a, s_b);
    if (s + 1 < nsteps) step(s + 1, P1(), s_b, s_a);
    if (s + 2 < nsteps) step(s + 2, P2(), s_a, s_b);
    if (s + 3 < nsteps) step(s + 3, P3(), s_b, s_a);
    if (s + 4 < nsteps) step(s + 4, P4(), s_a, s_b);
    if (s + 5 < nsteps) step(s + 5, P5(), s_b, s_a);
  }

  const float ltot = lsum + swap_halves(lsum);
  // a learned sink joins the denominator only (log2 units, relative to the running max m, which
  // is set whenever ltot > 0)
  const float lden =
      (a.sinks != nullptr && ltot > 0.f) ? ltot + fast_exp2(a.sinks[qh] * kLog2e - m) : ltot;
  const float inv = ltot > 0.f ? 1.0f / lden : 0.f;
  if (qvalid) {
    uint16_t* orow = (uint16_t*)a.out + (int64_t)b * a.o_b + (int64_t)qi * a.o_i +
                     (int64_t)qh * a.o_h;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d = db * 32 + 8 * rq + 4 * hg;
        u32x2 w2;
        w2[0] = pack_bf16x2(o[db][4 * rq + 0] * inv, o[db][4 * rq + 1] * inv);
        w2[1] = pack_bf16x2(o[db][4 * rq + 2] * inv, o[db][4 * rq + 3] * inv);
        *(u32x2*)(orow + d) = w2;
      }
  }
}

template <int ROT, bool NORM, bool CAP>
hipError_t launch_attn(const StreamArgs& sa, hipStream_t stream) {
  const AttnArgs& a = sa.a;
  const int64_t nrows = (int64_t)a.L * a.G;
  const int nqb = (int)((nrows + ROWS - 1) / ROWS);
  hipLaunchKernelGGL((prefill_stream_kernel<ROT, NORM, CAP>), dim3(nqb * a.Hkv * a.B), dim3(NT),
                     0, stream, sa, nqb);
  return hipGetLastError();
}
template <int ROT, bool NORM>
hipError_t launch_attn_cap(const StreamArgs& sa, hipStream_t s) {
  return sa.a.softcap > 0.f ? launch_attn<ROT, NORM, true>(sa, s) : launch_attn<ROT, NORM, false>(sa, s);
}
template <int ROT>
hipError_t launch_attn_norm(const StreamArgs& sa, hipStream_t s) {
  return sa.a.qk_norm ? launch_attn_cap<ROT, true>(sa, s) : launch_attn_cap<ROT, false>(sa, s);
}

template <int ROT, bool NORM>
hipError_t launch_rows(const AttnArgs& a, const RowJob& jb, int B, hipStream_t stream) {
  const int64_t ng = (int64_t)(jb.pend - jb.p0) * ((jb.H + kHeadsPerGroup - 1) / kHeadsPerGroup);
  if (ng <= 0 || B == 0) return hipSuccess;
  hipLaunchKernelGGL((rows_prep_kernel<ROT, NORM>), dim3((unsigned)((ng + 15) / 16), (unsigned)B),
                     dim3(256), 0, stream, a, jb);
  return hipGetLastError();
}

hipError_t dispatch_rows(const AttnArgs& a, const RowJob& jb, bool norm, hipStream_t stream) {
  const int rot = a.R == 0 ? 0 : (a.style == 0 ? 1 : 2);
  switch (rot * 2 + (norm ? 1 : 0)) {
    case 0: return launch_rows<0, false>(a, jb, a.B, stream);
    case 1: return launch_rows<0, true>(a, jb, a.B, stream);
    case 2: return launch_rows<1, false>(a, jb, a.B, stream);
    case 3: return launch_rows<1, true>(a, jb, a.B, stream);
    case 4: return launch_rows<2, false>(a, jb, a.B, stream);
    default: return launch_rows<2, true>(a, jb, a.B, stream);
  }
}

// Keys j0 .. S-1: the new ones (j >= n_cached) normed and rotated, the others copied as stored.
hipError_t dispatch_prep(const AttnArgs& a, const PrepOut& po, hipStream_t stream) {
  if (a.R == 0 && !a.qk_norm && po.p == (uint16_t*)a.k) return hipSuccess;  // nothing to do
  RowJob jb{};
  jb.src = (const uint16_t*)a.k;
  jb.sb = a.k_b;
  jb.sp = a.k_j;
  jb.sh = a.k_h;
  jb.dst = po.p;
  jb.db = po.ob;
  jb.dp = po.oj;
  jb.pos = a.kpos;
  jb.pos_b = a.kpos_b;
  jb.w = (const uint16_t*)a.kw;
  jb.H = a.Hkv;
  jb.p0 = po.j0;
  jb.pend = a.S;
  jb.pofs = po.jofs;
  jb.fresh_from = a.n_cached;
  jb.mul = 1.0f;
  return dispatch_rows(a, jb, a.qk_norm != 0, stream);
}

}  // namespace

hipError_t launch_paged_append(const AttnArgs& a, const PagedKV& kv, void* k_pool, void* v_pool,
                               const int32_t* start, hipStream_t stream) {
  RowJob jb{};
  jb.ptable = kv.table;
  jb.slot0 = start;
  jb.pmax_blocks = kv.max_blocks;
  jb.plog2bs = kv.log2bs;
  jb.pnum_blocks = kv.num_blocks;
  jb.pos = a.kpos;
  jb.pos_b = a.kpos_b;
  jb.w = (const uint16_t*)a.kw;
  jb.H = a.Hkv;
  jb.p0 = 0;
  jb.pend = a.L;
  jb.pofs = 0;
  jb.fresh_from = 0;
  jb.mul = 1.0f;
  // keys: norm and rotation; values: copied
  jb.src = (const uint16_t*)a.k;
  jb.sb = a.k_b;
  jb.sp = a.k_j;
  jb.sh = a.k_h;
  jb.dst = (uint16_t*)k_pool;
  hipError_t e = dispatch_rows(a, jb, a.qk_norm != 0, stream);
  if (e != hipSuccess) return e;
  AttnArgs av = a;
  av.R = 0;
  jb.src = (const uint16_t*)a.v;
  jb.dst = (uint16_t*)v_pool;
  return dispatch_rows(av, jb, false, stream);
}

bool prep_keys_supported(const AttnArgs& a) {
  if (a.D != HD) return false;
  if (a.R == 0 || a.style == 1) return a.R % 8 == 0;
  const int P = a.R / 16;
  return a.R % 16 == 0 && (P == 1 || P == 2 || P == 4 || P == 8);
}

hipError_t launch_prep_keys(const AttnArgs& a, void* k_out, hipStream_t stream) {
  PrepOut po;
  po.p = (uint16_t*)k_out;
  po.oj = a.k_j;
  po.ob = a.k_b;
  po.jofs = 0;
  po.j0 = a.n_cached;
  return dispatch_prep(a, po, stream);
}

bool prefill_needs_kprep(const AttnArgs& a) { return (a.qk_norm || a.R > 0) && a.n_cached < a.S; }

// First key row of the prepared-key workspace: it also holds the last BN - 1 cached rows (as
// stored), so that a tile starting below n_cached but reaching past it comes whole from the
// workspace and every tile reads one source.
static int kprep_first_row(const AttnArgs& a) { return a.n_cached > BN - 1 ? a.n_cached - (BN - 1) : 0; }

size_t prefill_stream_workspace_bytes(const AttnArgs& a) {
  if (!prefill_needs_kprep(a)) return 0;
  return (size_t)a.B * (a.S - kprep_first_row(a)) * a.Hkv * HD * sizeof(uint16_t);
}

bool prefill_stream_supported(const AttnArgs& a) {
  // 32-bit buffer offsets: every key row of one sequence must be addressable
  return prefill_mfma_supported(a) && ((int64_t)a.S + BN) * a.k_j * 2 < (int64_t)INT32_MAX;
}

hipError_t launch_prefill_stream(const AttnArgs& a, void* workspace, hipStream_t stream) {
  if (a.B == 0 || a.L == 0) return hipSuccess;
  StreamArgs sa;
  sa.a = a;
  sa.kprep = nullptr;
  if (prefill_needs_kprep(a)) {
    PrepOut po;
    po.p = (uint16_t*)workspace;
    po.oj = a.k_j;
    po.j0 = kprep_first_row(a);
    po.ob = (int64_t)(a.S - po.j0) * a.k_j;
    po.jofs = po.j0;
    hipError_t e = dispatch_prep(a, po, stream);
    if (e != hipSuccess) return e;
    sa.kprep = po.p;
  }
  switch (a.R == 0 ? 0 : (a.style == 0 ? 1 : 2)) {
    case 0: return launch_attn_norm<0>(sa, stream);
    case 1: return launch_attn_norm<1>(sa, stream);
    default: return launch_attn_norm<2>(sa, stream);
  }
}

}  // namespace gqa
