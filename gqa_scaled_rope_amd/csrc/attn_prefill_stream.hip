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
//  2. prefill_stream_kernel: the attention proper.  The same math as the fused kernel (32-key
//     tiles, S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_bf16, online softmax in log2
//     units with lazy rescaling), on 8 wavefronts x 32 query rows of one KV head in two groups
//     that alternate matrix and softmax phases; K and V
//     tiles travel from HBM straight into LDS with buffer_load ... lds: no VGPR staging, no LDS
//     store instructions, 32-bit offsets from a buffer descriptor, and the descriptor's range check
//     returns zeros past the last key, which handles the ragged tail.  Each wave instruction fills
//     1 KB of LDS in lane order; choosing the source chunk per lane produces the XOR-swizzled
//     layout the MFMA operand reads want.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "stream_tiles.hpp"

namespace gqa {
namespace {

using namespace stream;

constexpr int NW = 8;                 // wavefronts per workgroup, two per SIMD
constexpr int NT = NW * 64;
constexpr int WROWS = 32;             // query rows per wavefront
constexpr int ROWS = NW * WROWS;      // 256 query rows per workgroup
constexpr int kTileRounds = BN / (4 * NW);  // 1 KB loads per wave per K (or V) tile
static_assert(BN % (4 * NW) == 0 && BN <= 64, "tile loader and key-position loader layout");

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
// A workgroup is eight wavefronts of 32 query rows (256 rows of one KV head), one workgroup per
// CU, so each SIMD holds two wavefronts: w and w + 4 (waves are dealt to the SIMDs in turn).  On
// gfx950 a wavefront's own vector instructions do not overlap its 32x32x16 MFMAs (each MFMA
// holds the wavefront for about 28 of its 32 cycles), but another wavefront's do.  So the two
// wavefronts of a SIMD take turns: while one issues its matrix phase the other runs its
// softmax phase, and a workgroup barrier after every phase swaps them.  Per 32-key tile t a
// wavefront runs
//   matrix phase M(t):   S(t+1) = K(t+1) Q^T and O^T += V(t)^T P(t)^T (16 MFMAs, K and V read
//                        from LDS)
//   softmax phase V(t):  mask (edge tiles only), row max, rare rescale, exp2, bf16 P(t+1), row
//                        sums
// group 0 (waves 0-3) in the order M(0) V(0) M(1) V(1) ..., group 1 (waves 4-7) one phase later:
// [idle] M(0) V(0) M(1) ...  Scores arrive relative to the row's running reference m (log2 units):
// the first MFMA of each S^T chain starts from a template holding -m, and m moves only when a
// score exceeds it by more than kRescaleThreshold (exact, rare), when O, the sum, the scores and
// the template are corrected.
//
// K, V and key positions travel HBM -> LDS by buffer_load ... lds through eight buffers; tile
// t+7 is issued (by every wavefront, 1/8 of the tile each) at the start of the softmax phase that
// follows M(t), about six tiles before its keys are needed.  Tiles past the band are issued with an
// out-of-range offset (no memory access, zeros written), so every wavefront issues the same
// number of loads per tile and fixed vmcnt waits retire exactly the tiles that must have landed.
constexpr int NBUF = 8;
constexpr int kDmaPerTile = 2 * kTileRounds + 1; // per wavefront: K, V and the key positions
constexpr uint32_t kNullOfs = 0x7FFFF000u;       // a buffer offset past every descriptor's range
// The K tiles come first, so that every K operand read reaches its buffer with a constant offset
// below 64 KB from one per-lane address; the V reads get their own per-lane base 64 KB on.
// Key positions: wave 0 loads the tile's; the other wavefronts' loads (out of range, same count)
// write zeros into their own rows, never into the one that is read.  144 KB in all.
struct StreamLds {
  uint16_t k[NBUF][TILE_ELEMS];
  uint16_t v[NBUF][TILE_ELEMS];
  int32_t kp[NBUF][NW][64];
};
__shared__ __attribute__((aligned(16))) StreamLds g_lds;


// Query block, KV head and sequence of work item L.  Workgroups are dealt to the 8 XCDs
// round-robin by id; items are numbered so that every query block of one (b, g) lands on the
// same XCD (its K/V then stay in that XCD's L2), heaviest (latest) query blocks first.
struct WorkItem {
  int qb, g, b;
};
__device__ __forceinline__ WorkItem work_item(const AttnArgs& a, int L, int nqb) {
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
  return WorkItem{nqb - 1 - rank, pair % a.Hkv, pair / a.Hkv};
}

// Split key walks.  When the query blocks leave a last, partial round of the GPU (R items over
// C CUs, 2R <= C), each of those R items is walked by two workgroups, one per half of its key
// tiles; each writes its partial (O relative to its reference m, m, and each lane's share of the
// row sum) to the workspace and prefill_split_combine_kernel merges the two ([Guide] 3.4's
// softmax is a ratio of sums, so halves merge exactly up to rounding).  A partial is kept
// thread-major: value v of thread t at v * NT + t.
constexpr int kSplitMax = 128;                         // items that may be split
constexpr int kPartialVals = 66;                       // 64 of O, m, the lane's sum
constexpr size_t kPartialFloats = (size_t)kPartialVals * NT;
constexpr size_t kSplitBytes = (size_t)kSplitMax * 2 * kPartialFloats * sizeof(float);

template <int ROT, bool NORM, bool CAP, bool WS>
__global__ __launch_bounds__(NT, 1) void prefill_stream_kernel(StreamArgs sa, int nqb) {
  const AttnArgs& a = sa.a;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = w >> 2;  // 0: matrix phase first; 1: one phase later
  const int ql = lane & 31, hg = lane >> 5;
  // Work item of this workgroup; past the first nfull workgroups, two per item, one per half of
  // its key tiles (half 0 or 1; -1: the whole walk).
  int item = blockIdx.x, half = -1;
  if (item >= sa.nfull) {
    half = (item - sa.nfull) & 1;
    item = sa.nfull + ((item - sa.nfull) >> 1);
  }
  const WorkItem wi = work_item(a, item, nqb);
  const int qb = wi.qb, g = wi.g, b = wi.b;
  const int G = a.G;
  const int64_t nrows = (int64_t)a.L * G;
  const int64_t f0 = (int64_t)qb * ROWS;

  // ---- this lane's query row (flattened position-major (position, head) index) ----
  const int64_t f = f0 + WROWS * w + ql;
  const bool qvalid = f < nrows;
  const int qi = qvalid ? (int)(f / G) : 0;
  const int qh = g * G + (qvalid ? (int)(f % G) : 0);
  const int32_t* qpos_b = a.qpos + (int64_t)b * a.qpos_b;
  const int32_t qp_raw = qpos_b[qi];  // qi is a valid index even for rows past the end
  const int32_t qp = qvalid ? qp_raw : 0;
  // The row's query features (and the norm weights) do not depend on any position: their loads
  // go out now, beside the position loads, and land while the band is worked out.
  u32x4 xw[8], ww[8];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + (int64_t)b * a.q_b + (int64_t)qi * a.q_i +
                           (int64_t)qh * a.q_h + 8 * hg;
#pragma unroll
    for (int s = 0; s < 8; ++s) xw[s] = ld16(qrow + 16 * s);
    if (NORM) {
#pragma unroll
      for (int s = 0; s < 8; ++s) ww[s] = ld16((const uint16_t*)a.qw + 16 * s + 8 * hg);
    }
  }

  // ---- key band of the workgroup's query positions (loads issued here, used after Q prep) ----
  const int32_t* kpos_b = a.kpos + (int64_t)b * a.kpos_b;
  const int i_lo = (int)(f0 / G);
  const int i_hi = (int)min<int64_t>((f0 + ROWS - 1) / G, (int64_t)a.L - 1);
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

  // ---- buffer descriptors of this (b, g): cached keys, prepared keys, values, key positions ----
  const int row_bytes = (int)(a.k_j * 2);  // bytes between consecutive keys of one head
  const int64_t kv_base = (int64_t)b * a.k_b + (int64_t)g * a.k_h;
  // Without a workspace (WS false) nothing needs preparing and every key comes from k.  With
  // one, a tile whose keys all lie below nc comes from k as stored and any other from the
  // workspace, which starts at row w0 <= (first row of any tile reaching past nc).  The choice is
  // uniform per tile, so each load names one descriptor.
  const int nc = WS ? a.n_cached : a.S;
  const int w0 = nc > BN - 1 ? nc - (BN - 1) : 0;
  const int nws = a.S - w0;
  const i32x4 rk = rsrc_words((const uint16_t*)a.k + kv_base,
                              nc > 0 ? (nc - 1) * row_bytes + HD * 2 : 0);
  const i32x4 rw = rsrc_words(
      WS ? sa.kprep + (int64_t)b * nws * a.k_j + (int64_t)g * a.k_h : nullptr,
      (WS && nws > 0) ? (nws - 1) * row_bytes + HD * 2 : 0);
  const i32x4 rv = rsrc_words((const uint16_t*)a.v + kv_base, (a.S - 1) * row_bytes + HD * 2);
  const i32x4 rp = rsrc_words(kpos_b, a.S * 4);

  // Tile loader: wave w, round i fills LDS rows 4*(w + NW i) .. +3 (1 KB); lane -> row
  // 4(w + NW i) + lane/16, LDS chunk lane%16, which holds source chunk (lane%16) ^ swz(row).
  // Rows at or past S fall outside the descriptors' ranges and read as zero.  Wave 0 also loads
  // the tile's key positions (64 entries: the tile's 32 and the next 32, unused).
  const uint32_t lds_w = (uint32_t)(4 * w * HD * sizeof(uint16_t));  // this wave's rows of a tile
  uint32_t lk[kTileRounds], lv[kTileRounds];
#pragma unroll
  for (int i = 0; i < kTileRounds; ++i) {
    const int r = 4 * (w + NW * i) + (lane >> 4);
    lk[i] = r * row_bytes + (((lane & 15) ^ kswz(r)) << 4);
    lv[i] = r * row_bytes + (((lane & 15) ^ vswz(r)) << 4);
  }
  // the tile starting at key jt (live) or an out-of-range one (no memory access) into buffer buf
  auto issue_tile = [&](int jt, bool live, auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    const bool from_k = !WS || jt + BN <= nc;
    const i32x4 rks = from_k ? rk : rw;
    const uint32_t tb = live ? (uint32_t)(jt * row_bytes) : kNullOfs;
    const uint32_t kb0 = live ? (uint32_t)((from_k ? jt : jt - w0) * row_bytes) : kNullOfs;
#pragma unroll
    for (int i = 0; i < kTileRounds; ++i) {
      tile_dma16_at(rv, (lds_void*)(g_lds.v[buf] + 4 * NW * i * HD), lds_w, lv[i] + tb);
      tile_dma16_at(rks, (lds_void*)(g_lds.k[buf] + 4 * NW * i * HD), lds_w, lk[i] + kb0);
    }
    // (the other wavefronts issue it with an out-of-range offset: same count of loads everywhere)
    tile_dma4(rp, (lds_void*)g_lds.kp[buf][w],
              live && w == 0 ? (uint32_t)((jt + lane) * 4) : kNullOfs + 4 * lane);
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
  const int32_t qmin32 = (int32_t)qmin;
  const int g_hi = (int)min<int64_t>(max<int64_t>(x_hi - kp0, 0), a.S);
  const int g_lo = (int)min<int64_t>(max<int64_t>(x_lo - kp0, 0), a.S);
  // The first tile's loads go out now -- at key 0 without a window or chunks, else at the guessed
  // band start (loaded again below if the guess is wrong) -- beside the band and query-prep loads.
  int j_first = a.has_floor() ? g_lo : 0;
  if (half == 1) {  // the second half starts after the first ceil(n/2) tiles of the guessed band
    const int gt = (max(g_hi, j_first) - j_first + BN - 1) / BN;
    j_first += ((gt + 1) >> 1) * BN;
  }
  __builtin_amdgcn_sched_barrier(0);
  issue_tile(j_first, true, std::integral_constant<int, 0>());
  const int32_t hi_l = kpos_b[max(g_hi - 1, 0)], hi_r = kpos_b[min(g_hi, a.S - 1)];
  const int32_t lo_l = kpos_b[max(g_lo - 1, 0)], lo_r = kpos_b[min(g_lo, a.S - 1)];
  // smallest key position the row may see (window, chunks); INT32_MAX for rows past the end
  const int32_t qlo32 = !qvalid ? INT32_MAX
                        : a.has_floor() ? (int32_t)max<int64_t>(key_floor(a, qp), INT32_MIN)
                                        : INT32_MIN;
  const int32_t qp32 = qvalid ? qp : INT32_MIN;

  // ---- query prep, per wavefront and in registers: lane (ql, hg) loads, for its row, exactly the
  // features its MFMA operands hold -- 16 s + 8 hg .. + 7 for s = 0..7 -- RMS-norms the row (the
  // other 64 features are in lane ql + 32), rotates it at its position and scales it into log2
  // units.  With half-split rotation at R = 32, 64 or 128 a feature's partner (R/2 further on)
  // lies R/32 operand chunks further in the same lane; at R = 16 it is in lane l ^ 32.
  // Interleaved pairs are adjacent.
  bf16x8 qop[8];
  {
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
    // log2 units; with the soft cap the rows also carry the cap's factor k (below), so the
    // products arrive as k s, ready for the cap's exp2
    const float qscale = CAP ? -2.0f * a.scale * kLog2e / a.softcap : a.scale * kLog2e;
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
  int n_tiles = (j_hi - j_lo + BN - 1) / BN;
  if (half >= 0) {  // this workgroup's half of the walk
    const int n0 = (n_tiles + 1) >> 1;
    if (half == 0) {
      n_tiles = n0;
    } else {
      j_lo += n0 * BN;
      n_tiles -= n0;
    }
  }
  // first key index past this walk: the band's end, or the first half's last tile.  Key indices
  // from j_end on are masked (the walk's last tile may reach past it).
  const int j_end = min(j_hi, j_lo + n_tiles * BN);

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  // Running reference m (log2 units; kNegBig until the row has seen an allowed key) and sum.  The
  // S^T chains start from -m_eff (m_eff = m once set, else 0), so the scores arrive relative to
  // the reference: between a softmax phase and the next S^T the score registers hold that start
  // value.  (Soft-capping needs the raw score: there the chains start from 0 and m_eff is
  // subtracted with the cap.)
  float m = kNegBig, lsum = 0.f;
  // The row's rescale threshold and chain start value, changed only when the reference moves:
  // -inf and 0 until the row has a reference, then kRescaleThreshold and -m.  tmpl holds the start
  // value in all 16 places, ready as the first MFMA's accumulator input.
  float thr = -INFINITY, mstart = 0.f;
  const f32x16 zero16 = {};
  f32x16 tmpl = zero16;
  const float cap2 = a.softcap * kLog2e;
  // cap2 tanh(s / cap2) = 2 cap2 / (1 + 2^(k s)) - cap2 with k = -2 log2(e) / cap2: one exp2, one
  // reciprocal and one fma per score, with the limits +-cap2 reached exactly for large |s|.  The
  // query rows are scaled by k as well, so the S^T chains deliver k s.

  // per-lane LDS read offsets (elements).  K: row ql, chunk 2s + hg.  V^T (transposing reads):
  // rows 4*hgv + s16/4 (+8 for items 4..7) of each 16-key group, columns db*32 + 16*(gi&1) +
  // 4*(s16&3); both swizzles only see the row's low 4 bits, which the 16-key group offset leaves
  // unchanged.
  const int gi = lane >> 4, s16 = lane & 15;
  const int hgv = gi >> 1;
  int koff[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) koff[s] = ql * HD + (((2 * s + hg) ^ kswz(ql)) << 3);
  // V reads: LDS byte addresses in buffer 0, hidden from the compiler so that each read adds a
  // constant (buffer and key half) below 64 KB to one of these eight registers
  uint32_t vaddr[2][4];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int row = 4 * hgv + (s16 >> 2) + 8 * h2;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int col = db * 32 + 16 * (gi & 1) + 4 * (s16 & 3);
      const int voff = row * HD + (((col >> 3) ^ vswz(row)) << 3) + (col & 7);
      vaddr[h2][db] = (uint32_t)(uintptr_t)(lds_void*)(g_lds.v[0] + voff);
      asm volatile("" : "+v"(vaddr[h2][db]));
    }
  }

  // The mask's key positions are read from one per-lane base address, hidden from the compiler,
  // plus a constant below 64 KB, so that no address per buffer is kept.
  uint32_t kpaddr = (uint32_t)(uintptr_t)(lds_void*)(g_lds.kp[0][0] + 4 * hg);
  asm volatile("" : "+v"(kpaddr));

  // Without the soft cap the softmax phase is much shorter than the matrix phase, so the V^T
  // operands of the next P V's first four MFMAs are read at its end and the matrix phase starts
  // on MFMAs at once.  With the cap both phases take about as long, and the reads would lengthen
  // the softmax one: there all operands are read in the matrix phase.
  constexpr bool kPrefetchV = !CAP;
  i16x8 vpre[4];       // (kPrefetchV) V^T operands of the first four MFMAs of the next P V
  f32x16 sc = zero16;  // the next tile's scores (S^T), or the start value of their chain
  bf16x8 pw[2];       // the current tile's weights P, as the B operand of P V
  // S^T of the K tile in buffer buf
  auto qk = [&](auto bufc, const f32x16& c0) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    const uint16_t* ks = g_lds.k[buf];
    u32x4 kop[8];
#pragma unroll
    for (int st = 0; st < 8; ++st) kop[st] = *(const u32x4*)(ks + koff[st]);
    f32x16 acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kop[0]), qop[0], c0, 0, 0, 0);
#pragma unroll
    for (int st = 1; st < 8; ++st)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kop[st]), qop[st], acc, 0, 0, 0);
    return acc;
  };
  // O^T += V^T P^T over the V tile in buffer buf
  auto pv = [&](auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        i16x8 va;
        if (kPrefetchV && u == 0) {
          va = vpre[db];
        } else {
          const uint32_t ofs = (uint32_t)((buf * TILE_ELEMS + 16 * u * HD) * sizeof(uint16_t));
          const i16x4 vlo =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(vaddr[0][db] + ofs));
          const i16x4 vhi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(vaddr[1][db] + ofs));
          va = i16x8{vlo[0], vlo[1], vlo[2], vlo[3], vhi[0], vhi[1], vhi[2], vhi[3]};
        }
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va), pw[u],
                                                        o[db], 0, 0, 0);
      }
  };
  // The V^T operands of the first four P V MFMAs (keys 0-15) of the V tile in buffer buf, read
  // ahead into vpre.  That tile has been visible to every wavefront since the barrier before the
  // matrix phase that scored its K, and its buffer is refilled only several phases later.
  auto vprefetch = [&](auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const uint32_t ofs = (uint32_t)(buf * TILE_ELEMS * sizeof(uint16_t));
      const i16x4 vlo =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(vaddr[0][db] + ofs));
      const i16x4 vhi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(vaddr[1][db] + ofs));
      vpre[db] = i16x8{vlo[0], vlo[1], vlo[2], vlo[3], vhi[0], vhi[1], vhi[2], vhi[3]};
    }
  };
  // The tile starting at key jt needs no mask when all its keys are in range, none is newer than
  // the oldest query, and every query may see its first key.
  auto tile_full = [&](int jt, auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    const int32_t kfirst = g_lds.kp[buf][0][0], klast = g_lds.kp[buf][0][BN - 1];
    return (jt + BN <= j_end) & (klast <= qmin32) & (kfirst >= floor_max);
  };
  // Softmax of the freshly computed scores of the tile at key jt (buffer buf): soft-cap, mask
  // (allowed <=> key index < j_end and qlo32 <= key position <= qp32), row max, rare rescale,
  // exp2, bf16 weights P into pw and the row sum of those weights.
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  // soft cap of score r (the products arrive as k s, see cap_k's note)
  auto cap_score = [&](int r) __attribute__((always_inline)) {
    const float e = fast_exp2(sc[r]);
    sc[r] = __builtin_fmaf(__builtin_amdgcn_rcpf(1.0f + e), 2.0f * cap2, mstart - cap2);
  };
  // (lo_capped: the matrix phase has already capped scores 0-7)
  auto softmax = [&](int jt, auto bufc, bool full, bool lo_capped = false)
      __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    if (CAP) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (lo_capped && r < 8) continue;
        const float e = fast_exp2(sc[r]);
        sc[r] = __builtin_fmaf(__builtin_amdgcn_rcpf(1.0f + e), 2.0f * cap2, mstart - cap2);
      }
    }
    if (!full) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int idx0 = 8 * gq + 4 * hg;
        typedef __attribute__((address_space(3))) i32x4 lds_i32x4;
        const i32x4 k4 = *(const lds_i32x4*)(uintptr_t)(
            kpaddr + (uint32_t)((buf * NW * 64 + 8 * gq) * sizeof(int32_t)));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = jt + idx0 + e < j_end && k4[e] <= qp32 && k4[e] >= qlo32;
          if (!ok) sc[4 * gq + e] = -INFINITY;
        }
      }
    }
    // row max (scores relative to m_eff); the reference moves only when a score exceeds it by
    // more than the threshold, or on the row's first allowed key
    float mt = sc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sc[r]);
    mt = fmaxf(mt, swap_halves(mt));
    if (__ballot(mt > thr) != 0) {
      const bool upd = mt > thr;
      const bool unset = m == kNegBig;
      const float meff = -mstart;
      const float mnew = upd ? meff + mt : m;
      const float alpha = unset ? 1.f : fast_exp2(m - mnew);
      const bool set_new = mnew != kNegBig;
      const float meff_new = set_new ? mnew : 0.f;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] += meff - meff_new;
      m = mnew;
      mstart = -meff_new;
      thr = set_new ? kRescaleThreshold : -INFINITY;
      if (!CAP) {
#pragma unroll
        for (int r = 0; r < 16; ++r) tmpl[r] = mstart;
      }
    }
    // P = exp2(s); row sums of the bf16 weights the P V product uses, two per v_dot2_f32_bf16
    const bf16x2 ones2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = fast_exp2(sc[8 * u + e]);
      pw[u] = as_bf16x8(pack8(p));
      // (each pair is built from its two floats: taking it out of the packed vector with a bit
      // cast made the compiler feed the first pair to all four dot products)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2 pr = {(__bf16)p[2 * e], (__bf16)p[2 * e + 1]};
        lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2, lsum, false);
      }
    }
  };
  // Matrix phase: O^T += V(buffer b0)^T P^T and S^T of the K tile in buffer b1.  The LDS operand
  // reads run a few MFMAs ahead of their use (four with the soft cap; two S^T/P V step pairs
  // without it, where the first four V operands were read in the softmax phase), and no further,
  // so that only a few operands are live at a time (two wavefronts share each SIMD's registers).
  // The phase also reads the next tile's first and last key positions and decides whether its
  // softmax needs the mask (that tile's loads have landed: its K is read here).  It runs at raised
  // wavefront priority, so that when both wavefronts of a SIMD have an instruction ready the
  // MFMA issue of this one goes before the softmax arithmetic of the other.
  auto mphase = [&](auto b0c, auto b1c, int jt1, bool& full1) __attribute__((always_inline)) {
    constexpr int b1 = decltype(b1c)::value;
    __builtin_amdgcn_s_setprio(3);
    const int32_t kfirst = g_lds.kp[b1][0][0], klast = g_lds.kp[b1][0][BN - 1];
    if (CAP) {
      // With the soft cap the softmax phase is the longer one: S^T goes first here, and the cap
      // of its first eight scores runs beside the P V MFMAs (the rest in the softmax phase).
      sc = qk(b1c, zero16);
      pv(b0c);
#pragma unroll
      for (int r = 0; r < 8; ++r) cap_score(r);
    } else {
      static_assert(kPrefetchV == !CAP, "the matrix phase without the cap starts from vpre");
      // S^T step i and P V step i+3 alternate (P V 0-2 first: their operands are in registers),
      // so that each MFMA of the dependent S^T chain has an independent one before it.  Each
      // step is fenced, with the operand reads two steps ahead in the step before.
      constexpr int b0 = decltype(b0c)::value;
      typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
      const uint16_t* ks = g_lds.k[b1];
      auto kread = [&](int st) __attribute__((always_inline)) {
        return *(const u32x4*)(ks + koff[st]);
      };
      auto vread = [&](int db) __attribute__((always_inline)) {  // key half 1, feature block db
        const uint32_t ofs = (uint32_t)((b0 * TILE_ELEMS + 16 * HD) * sizeof(uint16_t));
        const i16x4 vlo =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(vaddr[0][db] + ofs));
        const i16x4 vhi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(vaddr[1][db] + ofs));
        return i16x8{vlo[0], vlo[1], vlo[2], vlo[3], vhi[0], vhi[1], vhi[2], vhi[3]};
      };
      auto pvs = [&](int i, const i16x8& v) __attribute__((always_inline)) {
        o[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v),
                                                            pw[i >> 2], o[i & 3], 0, 0, 0);
      };
      u32x4 kop[8];
      i16x8 va[4];
      kop[0] = kread(0);
      kop[1] = kread(1);
      __builtin_amdgcn_sched_barrier(0);
      pvs(0, vpre[0]);
      kop[2] = kread(2);
      va[0] = vread(0);
      __builtin_amdgcn_sched_barrier(0);
      pvs(1, vpre[1]);
      kop[3] = kread(3);
      va[1] = vread(1);
      __builtin_amdgcn_sched_barrier(0);
      pvs(2, vpre[2]);
      kop[4] = kread(4);
      va[2] = vread(2);
      __builtin_amdgcn_sched_barrier(0);
      f32x16 acc = tmpl;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kop[i]), qop[i], acc, 0, 0, 0);
        if (i + 3 < 8) pvs(i + 3, i == 0 ? vpre[3] : va[i - 1]);
        if (i + 5 < 8) kop[i + 5] = kread(i + 5);
        if (i == 0) va[3] = vread(3);
        __builtin_amdgcn_sched_barrier(0);
      }
      sc = acc;
    }
    full1 = (jt1 + BN <= j_end) & (__builtin_amdgcn_readfirstlane(klast) <= qmin32) &
            (__builtin_amdgcn_readfirstlane(kfirst) >= floor_max);
    if (CAP) {
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);    // positions, K of S^T 0-3
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // S^T i
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // K of S^T 4-7, V of P V 0-5
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // P V i
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // V of P V 6-7
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // cap of the first scores
      }
    }  // (without the cap each step is fenced above)
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  };
  // ---- first tiles: 0 .. NBUF-2 issued, 0 and 1 landed; S(0) and its weights ----
  if (j_lo != j_first && n_tiles > 0) {
    asm volatile("s_waitcnt vmcnt(0)");  // the guessed tile's loads land before the right tile's
    issue_tile(j_lo, true, std::integral_constant<int, 0>());
  }
  issue_tile(j_lo + 1 * BN, 1 < n_tiles, std::integral_constant<int, 1>());
  issue_tile(j_lo + 2 * BN, 2 < n_tiles, std::integral_constant<int, 2>());
  issue_tile(j_lo + 3 * BN, 3 < n_tiles, std::integral_constant<int, 3>());
  issue_tile(j_lo + 4 * BN, 4 < n_tiles, std::integral_constant<int, 4>());
  issue_tile(j_lo + 5 * BN, 5 < n_tiles, std::integral_constant<int, 5>());
  issue_tile(j_lo + 6 * BN, 6 < n_tiles, std::integral_constant<int, 6>());
  barrier_after_loads<(NBUF - 3) * kDmaPerTile>();
  sc = qk(std::integral_constant<int, 0>(), zero16);
  softmax(j_lo, std::integral_constant<int, 0>(), tile_full(j_lo, std::integral_constant<int, 0>()));
  if (kPrefetchV) vprefetch(std::integral_constant<int, 0>());

  // Tile t sits in buffer t mod NBUF.  Both groups run the same sequence -- M(t), barrier, refill
  // of tile t-1's buffer with tile t+NBUF-1, V(t+1), barrier -- group 1 one phase behind group 0:
  // it passes one extra barrier before its first phase, group 0 one after its last.  So group 0's
  // M(t) and group 1's V(t) share a phase, as do group 0's V(t+1) and group 1's M(t).  Tile t-1
  // was last read by group 1's M(t-1), which ended before either group passes M(t)'s barrier;
  // the refill is issued in the softmax phase, off the matrix path.  Before a barrier each
  // wavefront waits until at most its newest NBUF-4 (after M) or NBUF-3 (after V) tiles'
  // loads are outstanding: its share of the tile that the next phase's S^T reads has then landed
  // (loads retire in issue order).
  auto iter = [&](int t, auto phc) __attribute__((always_inline)) {
    constexpr int PH = decltype(phc)::value;
    using B0 = std::integral_constant<int, PH>;
    using B1 = std::integral_constant<int, (PH + 1) % NBUF>;
    using BR = std::integral_constant<int, (PH + NBUF - 1) % NBUF>;
    const int jt1 = j_lo + (t + 1) * BN;
    bool full1;
    mphase(B0(), B1(), jt1, full1);
    barrier_after_loads<(NBUF - 4) * kDmaPerTile>();
    issue_tile(j_lo + (t + NBUF - 1) * BN, t + NBUF - 1 < n_tiles, BR());
    softmax(jt1, B1(), full1, true);
    if (kPrefetchV) vprefetch(B1());
    barrier_after_loads<(NBUF - 3) * kDmaPerTile>();
  };
  // The walk's last tile (buffer PH) has no next tile to score: its matrix phase is the P V
  // product alone, and one barrier ends it.  With group 1 one phase behind, that barrier pairs
  // with group 0's closing one below, so group 1's last V reads are done before any wavefront
  // moves on; tiles still in flight then all lie past the walk, in other buffers.
  auto tail = [&](int buf) __attribute__((always_inline)) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const uint32_t bofs = (uint32_t)(buf * TILE_ELEMS * sizeof(uint16_t));
    __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint32_t ofs = bofs + (uint32_t)(16 * u * HD * sizeof(uint16_t));
        const i16x4 vlo =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(vaddr[0][db] + ofs));
        const i16x4 vhi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(vaddr[1][db] + ofs));
        const i16x8 va = i16x8{vlo[0], vlo[1], vlo[2], vlo[3], vhi[0], vhi[1], vhi[2], vhi[3]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va), pw[u],
                                                        o[db], 0, 0, 0);
      }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    phase_barrier();
  };
  if (grp == 1) barrier_after_loads<(NBUF - 4) * kDmaPerTile>();
  // (exits after any iteration: the unrolled body stays one straight path with no joins inside)
  const int t_last = n_tiles - 1;
  for (int t = 0; t < t_last;) {
    iter(t, std::integral_constant<int, 0>());
    if (++t >= t_last) break;
    iter(t, std::integral_constant<int, 1>());
    if (++t >= t_last) break;
    iter(t, std::integral_constant<int, 2>());
    if (++t >= t_last) break;
    iter(t, std::integral_constant<int, 3>());
    if (++t >= t_last) break;
    iter(t, std::integral_constant<int, 4>());
    if (++t >= t_last) break;
    iter(t, std::integral_constant<int, 5>());
    if (++t >= t_last) break;
    iter(t, std::integral_constant<int, 6>());
    if (++t >= t_last) break;
    iter(t, std::integral_constant<int, 7>());
    ++t;
  }
  if (n_tiles > 0) tail(t_last & (NBUF - 1));
  static_assert(NBUF == 8, "the loop above is unrolled by NBUF");
  if (grp == 0) phase_barrier();
  // every wavefront's loads retire before the workgroup ends (the last ones were out of range)
  asm volatile("s_waitcnt vmcnt(0)");
  if (half >= 0) {
    float* pp = sa.part + ((size_t)(item - sa.nfull) * 2 + half) * kPartialFloats + tid;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) pp[(size_t)(db * 16 + r) * NT] = o[db][r];
    pp[(size_t)64 * NT] = m;
    pp[(size_t)65 * NT] = lsum;
    return;
  }

  const float ltot = lsum + swap_halves(lsum);
  // a learned sink joins the denominator only (log2 units, relative to the running max m, which
  // is set whenever ltot > 0)
  const float lden =
      (a.sinks != nullptr && ltot > 0.f) ? ltot + fast_exp2(a.sinks[qh] * kLog2e - m) : ltot;
  const float inv = ltot > 0.f ? 1.0f / lden : 0.f;
  // The output goes out through LDS: each wavefront writes its 32 rows (bf16, 128 features) into
  // a staging area of 264-byte rows, then stores whole rows, 16 bytes per lane, four rows per
  // store instruction (in place of 8 bytes from each of 32 rows).  The padding puts the 8-byte
  // writes of each half wavefront, and the reads of each group of 16 lanes, in distinct banks.
  // The tile buffers are free once every wavefront's last (out-of-range) tile loads have landed
  // (the wait above): one more barrier.
  phase_barrier();
  constexpr int kStagePitch = HD + 4;  // elements
  uint16_t* const stage = (uint16_t*)&g_lds + w * (WROWS * kStagePitch);
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      u32x2 w2;
      w2[0] = pack_bf16x2(o[db][4 * rq + 0] * inv, o[db][4 * rq + 1] * inv);
      w2[1] = pack_bf16x2(o[db][4 * rq + 2] * inv, o[db][4 * rq + 3] * inv);
      *(u32x2*)(stage + ql * kStagePitch + db * 32 + 8 * rq + 4 * hg) = w2;
    }
  // element offset of this lane's row in out (-1: past the end), fetched by the storing lanes
  const int64_t orow = qvalid ? (int64_t)b * a.o_b + (int64_t)qi * a.o_i + (int64_t)qh * a.o_h : -1;
  const int c16 = lane & 15;
#pragma unroll
  for (int j = 0; j < WROWS / 4; ++j) {
    const int rr = 4 * j + (lane >> 4);
    const int64_t dst = __shfl(orow, rr, 64);
    const uint16_t* src = stage + rr * kStagePitch + 8 * c16;
    const u32x2 lo = *(const u32x2*)src, hi = *(const u32x2*)(src + 4);
    if (dst >= 0) *(u32x4*)((uint16_t*)a.out + dst + 8 * c16) = u32x4{lo[0], lo[1], hi[0], hi[1]};
  }
}

// Merge of a split item's two partials (one workgroup per split item, the attention kernel's
// thread layout): O = O0 2^(m0-m) + O1 2^(m1-m), likewise the sums, m = max(m0, m1); a half that
// saw no allowed key (m = kNegBig) contributes nothing.  Then the same normalisation, sink and
// bf16 output as the attention kernel's epilogue.
__global__ __launch_bounds__(NT) void prefill_split_combine_kernel(StreamArgs sa, int nqb) {
  const AttnArgs& a = sa.a;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int ql = lane & 31, hg = lane >> 5;
  const WorkItem wi = work_item(a, sa.nfull + blockIdx.x, nqb);
  const int64_t f = (int64_t)wi.qb * ROWS + WROWS * w + ql;
  const bool qvalid = f < (int64_t)a.L * a.G;
  const float* p0 = sa.part + (size_t)blockIdx.x * 2 * kPartialFloats + tid;
  const float* p1 = p0 + kPartialFloats;
  const float m0 = p0[(size_t)64 * NT], m1 = p1[(size_t)64 * NT];
  const float mm = fmaxf(m0, m1);
  const float a0 = m0 == kNegBig ? 0.f : fast_exp2(m0 - mm);
  const float a1 = m1 == kNegBig ? 0.f : fast_exp2(m1 - mm);
  const float lsum = p0[(size_t)65 * NT] * a0 + p1[(size_t)65 * NT] * a1;
  const float ltot = lsum + swap_halves(lsum);
  if (!qvalid) return;
  const int qi = (int)(f / a.G);
  const int qh = wi.g * a.G + (int)(f % a.G);
  const float lden =
      (a.sinks != nullptr && ltot > 0.f) ? ltot + fast_exp2(a.sinks[qh] * kLog2e - mm) : ltot;
  const float inv = ltot > 0.f ? 1.0f / lden : 0.f;
  uint16_t* orow = (uint16_t*)a.out + (int64_t)wi.b * a.o_b + (int64_t)qi * a.o_i +
                   (int64_t)qh * a.o_h;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d = db * 32 + 8 * rq + 4 * hg;
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const size_t v = (size_t)(db * 16 + 4 * rq + e) * NT;
        x[e] = (p0[v] * a0 + p1[v] * a1) * inv;
      }
      u32x2 w2;
      w2[0] = pack_bf16x2(x[0], x[1]);
      w2[1] = pack_bf16x2(x[2], x[3]);
      *(u32x2*)(orow + d) = w2;
    }
}

template <int ROT, bool NORM, bool CAP, bool WS>
hipError_t launch_attn(const StreamArgs& sa, hipStream_t stream) {
  hipLaunchKernelGGL((prefill_stream_kernel<ROT, NORM, CAP, WS>), dim3(sa.grid), dim3(NT), 0,
                     stream, sa, sa.nqb);
  return hipGetLastError();
}
template <int ROT, bool NORM, bool CAP>
hipError_t launch_attn_ws(const StreamArgs& sa, hipStream_t s) {
  return sa.kprep ? launch_attn<ROT, NORM, CAP, true>(sa, s) : launch_attn<ROT, NORM, CAP, false>(sa, s);
}
template <int ROT, bool NORM>
hipError_t launch_attn_cap(const StreamArgs& sa, hipStream_t s) {
  return sa.a.softcap > 0.f ? launch_attn_ws<ROT, NORM, true>(sa, s)
                            : launch_attn_ws<ROT, NORM, false>(sa, s);
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

size_t prefill_stream_required_bytes(const AttnArgs& a) {
  if (!prefill_needs_kprep(a)) return 0;
  return (size_t)a.B * (a.S - kprep_first_row(a)) * a.Hkv * HD * sizeof(uint16_t);
}
static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }
size_t prefill_stream_workspace_bytes(const AttnArgs& a) {
  return align256(prefill_stream_required_bytes(a)) + kSplitBytes;
}

// Compute units of the current device (cached per device).
static int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

bool prefill_stream_supported(const AttnArgs& a) {
  // 32-bit buffer offsets: every key row of one sequence must be addressable
  return prefill_mfma_supported(a) && ((int64_t)a.S + BN) * a.k_j * 2 < (int64_t)INT32_MAX;
}

// Keys one workgroup of the eight-wavefront kernel visits on average, taking positions as
// consecutive with the queries at the last L of the S key positions (a fresh prefill or a chunk
// appended to a cache): its own query positions plus those below them that it may see -- the
// window, the visible chunks, or on average S - L/2 keys of the causal range.
static int64_t mean_band_keys(const AttnArgs& a) {
  const int64_t span = (ROWS + a.G - 1) / a.G;
  int64_t below = std::max<int64_t>((int64_t)a.S - a.L / 2, 0);
  if (a.window > 0) below = std::min<int64_t>(below, a.window);
  if (a.chunk > 0) below = std::min<int64_t>(below, (int64_t)a.chunk * a.chunk_lb + a.chunk / 2);
  return below + span;
}
// Below this many keys per workgroup (24 tiles) the four-wavefront kernel, two workgroups per CU,
// is faster: the eight-wavefront kernel's longer pipeline start and its one workgroup per CU cost
// more than its faster loop saves (measured: 0.25 against 0.27 ms for a 128-key window at B4,
// L 4096, Hq 64, Hkv 8; level at about 1000 keys, 6% slower at 4096).
constexpr int64_t kShortBandKeys = 24 * BN;

bool prefill_stream_short(const AttnArgs& a, StreamKernel which) {
  return which == StreamKernel::kShort ||
         (which == StreamKernel::kAuto && mean_band_keys(a) < kShortBandKeys);
}

hipError_t launch_prefill_stream(const AttnArgs& a, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream, StreamKernel which) {
  if (a.B == 0 || a.L == 0) return hipSuccess;
  StreamArgs sa;
  sa.a = a;
  sa.kprep = nullptr;
  sa.part = nullptr;
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
  if (prefill_stream_short(a, which)) return stream::launch_attn_short(sa, stream);
  // a last, partial round of query blocks has its key walks split when the workspace has room
  const int64_t nrows = (int64_t)a.L * a.G;
  const int nqb = (int)((nrows + ROWS - 1) / ROWS);
  const int64_t items = (int64_t)nqb * a.Hkv * a.B;
  const int cus = device_cus();
  const int64_t rest = items % cus;
  const bool split = workspace != nullptr && workspace_bytes >= prefill_stream_workspace_bytes(a) &&
                     rest > 0 && 2 * rest <= cus && rest <= kSplitMax;
  sa.nqb = nqb;
  sa.nfull = (int)(split ? items - rest : items);
  sa.grid = (int)(split ? items + rest : items);
  if (split) sa.part = (float*)((char*)workspace + align256(prefill_stream_required_bytes(a)));
  hipError_t e;
  switch (a.R == 0 ? 0 : (a.style == 0 ? 1 : 2)) {
    case 0: e = launch_attn_norm<0>(sa, stream); break;
    case 1: e = launch_attn_norm<1>(sa, stream); break;
    default: e = launch_attn_norm<2>(sa, stream); break;
  }
  if (e != hipSuccess || !split) return e;
  hipLaunchKernelGGL(prefill_split_combine_kernel, dim3((unsigned)rest), dim3(NT), 0, stream, sa,
                     nqb);
  return hipGetLastError();
}

}  // namespace gqa
