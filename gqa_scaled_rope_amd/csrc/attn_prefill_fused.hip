// bf16 MFMA prefill of rotary grouped-query causal attention, head_dim 128, for gfx950 -- fused
// variant, used when the caller gives no workspace: new keys are normed and rotated in registers
// each time their tile is staged.
//
// What it computes is [Models] "What differs between model families" (DecoderAttention.forward:
// q/k norm, rotation, window mask, causal attention) with [Guide] section 3.4's softmax; how:
//
//  * One workgroup = 8 wavefronts = 256 query rows of ONE KV head g of one sequence b.  Rows are
//    the flattened (position, query head) pairs of the group, position-major, so every K/V tile
//    staged in LDS is used by all G = Hq/Hkv query heads that share it (no K/V re-read per head).
//  * Each wavefront owns 32 rows.  Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K comes from LDS as the A operand, the wave's normed, rotated and
//    pre-scaled queries stay in VGPRs as the B operand.  In the accumulator each lane then holds
//    16 keys of ONE query row, so the softmax row statistics are a lane-local reduction plus one
//    v_permlane32_swap, and the probabilities are already laid out as the B operand of
//    O^T = V^T P^T: P never leaves registers.  V^T is read from row-major LDS with
//    ds_read_b64_tr_b16 (transposing LDS read), so V needs no transpose on its way into LDS.
//  * Scores are kept in log2 units (scale * log2(e) folded into q), p = exp2(s - m).  The running
//    max is only raised (and O, l rescaled) when a tile's max exceeds it by more than 8, which is
//    exact (any common shift cancels in O / l) and skips almost every rescale.
//  * K/V tiles of 64 keys are double-buffered in LDS (XOR-swizzled 16-byte chunks, conflict-free
//    for both the row reads of K and the transposing reads of V); the next tile's global loads
//    are in flight while the current tile is computed.  New keys (index >= n_cached) are RMS-normed
//    and rotated in registers between the global load and the LDS store.
//  * Only key tiles that intersect the causal/window/chunk band of the workgroup's queries are
//    visited ([Models] "Sliding windows": the loop starts at the first block the oldest query may
//    see, by window or by chunk); only tiles that straddle the band's edge evaluate the mask per
//    element.  A learned sink ([Ster] gpt_oss paragraph) enters the final denominator only.
#include "launch.hpp"

namespace gqa {
namespace {

constexpr int HD = 128;          // head_dim
constexpr int NW = 8;            // wavefronts per workgroup
constexpr int NT = NW * 64;      // threads
constexpr int ROWS = NW * 32;    // query rows per workgroup
constexpr int BN = 64;           // keys per tile
constexpr int TILE_ELEMS = BN * HD;
constexpr float kRescaleThreshold = 8.0f;  // log2 units

// Element offset of 16-byte chunk c of row r in a [BN][HD] bf16 tile.
__device__ __forceinline__ int tile_off(int r, int c) { return r * HD + ((c ^ (r & 15)) << 3); }
// V tiles: the transposing reads serve lanes 0-31 and 32-63 as two passes of 256 bytes over the
// 64 four-byte banks (measured on gfx950); a pass reads a 64-byte chunk quad of each of four
// consecutive rows, and (r & 3) << 2 puts the four quads in different quarters of the bank array.
__device__ __forceinline__ int vtile_off(int r, int c) { return r * HD + ((c ^ ((r & 3) << 2)) << 3); }

struct Smem {
  uint16_t k[2][TILE_ELEMS];
  uint16_t v[2][TILE_ELEMS];
  int32_t kpos[2][BN];
};

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *(const u32x4*)p; }

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

__device__ __forceinline__ int lower_bound_pos(const int32_t* kp, int n, int64_t x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if ((int64_t)kp[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Rotate chunk x (8 consecutive features starting at 8*c) given its rotation partner chunk y.
// half-split (ROT 1): pair index of feature d < R/2 is d, of d in [R/2, R) is d - R/2;
// interleaved (ROT 2): features (2i, 2i+1) within the chunk form pair i.
template <int ROT>
__device__ __forceinline__ void rotate_chunk(float* x, const float* y, int c, int R,
                                             const float* cos_row, const float* sin_row) {
  if (ROT == 1) {
    const int half = R >> 1;
    const int d0 = c * 8;
    if (d0 >= R) return;
    const bool first = d0 < half;
    const int p0 = first ? d0 : d0 - half;
    const f32x4 c0 = *(const f32x4*)(cos_row + p0), c1 = *(const f32x4*)(cos_row + p0 + 4);
    const f32x4 s0 = *(const f32x4*)(sin_row + p0), s1 = *(const f32x4*)(sin_row + p0 + 4);
    const float cs[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
    const float sn[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // first half: a = x, b = partner -> a c - b s;  second half: a = partner, b = x -> a s + b c
      x[e] = first ? (x[e] * cs[e] - y[e] * sn[e]) : (y[e] * sn[e] + x[e] * cs[e]);
    }
  } else if (ROT == 2) {
    const int d0 = c * 8;
    if (d0 >= R) return;
    const int p0 = d0 >> 1;
    const f32x4 cs = *(const f32x4*)(cos_row + p0);
    const f32x4 sn = *(const f32x4*)(sin_row + p0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = x[2 * e], b = x[2 * e + 1];
      x[2 * e] = a * cs[e] - b * sn[e];
      x[2 * e + 1] = a * sn[e] + b * cs[e];
    }
  }
}

struct Ctx {
  int b, g;
  int64_t k_base;  // element offset of (b, 0, g, 0)
};

// Global loads of one K/V tile into registers: thread t covers key row t/8, chunks t%8 and t%8+8.
struct TileRegs {
  u32x4 k0, k1, v0, v1;
  int32_t kp;
  bool valid;
};

__device__ __forceinline__ void load_tile(const AttnArgs& a, const Ctx& cx, int jt, int j_hi,
                                          TileRegs& tr) {
  const int t = threadIdx.x;
  const int row = t >> 3, c0 = t & 7;
  const int j = jt + row;
  tr.valid = j < j_hi;
  const u32x4 z = {0u, 0u, 0u, 0u};
  tr.k0 = tr.k1 = tr.v0 = tr.v1 = z;
  tr.kp = 0x7fffffff;
  if (tr.valid) {
    const uint16_t* kr = (const uint16_t*)a.k + cx.k_base + (int64_t)j * a.k_j;
    const uint16_t* vr = (const uint16_t*)a.v + cx.k_base + (int64_t)j * a.k_j;
    tr.k0 = ld16(kr + c0 * 8);
    tr.k1 = ld16(kr + (c0 + 8) * 8);
    tr.v0 = ld16(vr + c0 * 8);
    tr.v1 = ld16(vr + (c0 + 8) * 8);
    tr.kp = a.kpos[cx.b * a.kpos_b + j];
  }
}

// Norm and rotate the new keys of the tile in registers, then store K, V and key positions to LDS.
template <int ROT, bool NORM>
__device__ __forceinline__ void store_tile(const AttnArgs& a, int jt, TileRegs& tr, Smem& sm,
                                           int buf) {
  const int t = threadIdx.x;
  const int row = t >> 3, c0 = t & 7;
  const int j = jt + row;
  const bool tile_prep = (NORM || ROT != 0) && (jt + BN > a.n_cached);
  if (tile_prep) {
    const bool prep = tr.valid && j >= a.n_cached;
    float x0[8], x1[8];
    unpack8(tr.k0, x0);
    unpack8(tr.k1, x1);
    if (NORM) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += x0[e] * x0[e] + x1[e] * x1[e];
      ss += __shfl_xor(ss, 1, 64);
      ss += __shfl_xor(ss, 2, 64);
      ss += __shfl_xor(ss, 4, 64);
      const float rs = rsqrtf(ss * (1.0f / HD) + a.eps);
      const uint16_t* kwp = (const uint16_t*)a.kw;
      float kw0[8], kw1[8];
      unpack8(ld16(kwp + 8 * c0), kw0);
      unpack8(ld16(kwp + 8 * (c0 + 8)), kw1);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x0[e] *= rs * kw0[e];
        x1[e] *= rs * kw1[e];
      }
    }
    if (ROT != 0) {
      const int64_t tp = min<int64_t>(max<int64_t>(tr.kp, 0), a.table_len - 1);
      const int halfp = a.R >> 1;
      const float* cr = a.cos_t + tp * halfp;
      const float* sr = a.sin_t + tp * halfp;
      if (ROT == 1) {
        const int P = a.R >> 4;  // partner distance in chunks
        if (P == 8) {
          float y0[8], y1[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) { y0[e] = x1[e]; y1[e] = x0[e]; }
          if (prep) {
            rotate_chunk<1>(x0, y0, c0, a.R, cr, sr);
            rotate_chunk<1>(x1, y1, c0 + 8, a.R, cr, sr);
          }
        } else {
          float y0[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) y0[e] = __shfl_xor(x0[e], P, 64);
          if (prep) rotate_chunk<1>(x0, y0, c0, a.R, cr, sr);
        }
      } else {
        if (prep) {
          rotate_chunk<2>(x0, x0, c0, a.R, cr, sr);
          rotate_chunk<2>(x1, x1, c0 + 8, a.R, cr, sr);
        }
      }
    }
    if (prep) {
      tr.k0 = pack8(x0);
      tr.k1 = pack8(x1);
    }
  }
  *(u32x4*)(&sm.k[buf][tile_off(row, c0)]) = tr.k0;
  *(u32x4*)(&sm.k[buf][tile_off(row, c0 + 8)]) = tr.k1;
  *(u32x4*)(&sm.v[buf][vtile_off(row, c0)]) = tr.v0;
  *(u32x4*)(&sm.v[buf][vtile_off(row, c0 + 8)]) = tr.v1;
  if (c0 == 0) sm.kpos[buf][row] = tr.kp;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& w) { return __builtin_bit_cast(bf16x8, w); }

template <int ROT, bool NORM, bool CAP>
__global__ __launch_bounds__(NT, 1) void prefill_mfma_kernel(AttnArgs a, int nqb) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int ql = lane & 31, hg = lane >> 5;
  const int qb = nqb - 1 - (int)blockIdx.x;  // heaviest (latest) query blocks first
  Ctx cx;
  cx.g = blockIdx.y;
  cx.b = blockIdx.z;
  cx.k_base = (int64_t)cx.b * a.k_b + (int64_t)cx.g * a.k_h;
  const int G = a.G;
  const int64_t nrows = (int64_t)a.L * G;
  const int64_t f0 = (int64_t)qb * ROWS;

  // ---- this lane's query row ----
  const int64_t f = f0 + w * 32 + ql;
  const bool qvalid = f < nrows;
  const int qi = qvalid ? (int)(f / G) : 0;
  const int qh = cx.g * G + (qvalid ? (int)(f % G) : 0);
  const int32_t* qpos_b = a.qpos + (int64_t)cx.b * a.qpos_b;
  const int64_t qp = qvalid ? (int64_t)qpos_b[qi] : 0;

  // Query prep: load the whole row, RMS-norm, rotate, scale into log2 units, keep this lane's
  // eight 16-byte chunks (chunk 2s + hg for k-step s) as bf16 MFMA operands.
  const float qscale = a.scale * kLog2e;
  bf16x8 qop[8];
  {
    const uint16_t* qr = (const uint16_t*)a.q + (int64_t)cx.b * a.q_b + (int64_t)qi * a.q_i +
                         (int64_t)qh * a.q_h;
    float rs = 1.f;
    if (NORM) {
      float ss = 0.f;
      if (qvalid) {
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          float x[8];
          unpack8(ld16(qr + 8 * c), x);
#pragma unroll
          for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
        }
      }
      rs = rsqrtf(ss * (1.0f / HD) + a.eps);
    }
    const uint16_t* qw = (const uint16_t*)a.qw;
    const int64_t tp = ROT ? min<int64_t>(max<int64_t>(qp, 0), a.table_len - 1) : 0;
    const int halfp = a.R >> 1;
    const float* cr = ROT ? a.cos_t + tp * halfp : nullptr;
    const float* sr = ROT ? a.sin_t + tp * halfp : nullptr;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int c = 2 * s + hg;
      float x[8];
      if (qvalid) {
        unpack8(ld16(qr + 8 * c), x);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.f;
      }
      if (NORM) {
        float wv[8];
        unpack8(ld16(qw + 8 * c), wv);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= rs * wv[e];
      }
      if (ROT == 1 && qvalid && 8 * c < a.R) {
        const int P = a.R >> 4;
        const int pc = c ^ P;
        float y[8];
        if (qvalid) unpack8(ld16(qr + 8 * pc), y);
        if (NORM) {
          float wv[8];
          unpack8(ld16(qw + 8 * pc), wv);
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] *= rs * wv[e];
        }
        rotate_chunk<1>(x, y, c, a.R, cr, sr);
      } else if (ROT == 2 && qvalid) {
        rotate_chunk<2>(x, x, c, a.R, cr, sr);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= qscale;
      qop[s] = as_bf16x8(pack8(x));
    }
  }

  // ---- band of keys for the workgroup's query positions ----
  int64_t qmin = INT64_MAX, qmax = INT64_MIN;
  {
    const int i_lo = (int)(f0 / G);
    const int i_hi = (int)min<int64_t>((f0 + ROWS - 1) / G, (int64_t)a.L - 1);
    int64_t mn = INT64_MAX, mx = INT64_MIN;
    for (int i = i_lo + lane; i <= i_hi; i += 64) {
      const int64_t p = qpos_b[i];
      mn = min(mn, p);
      mx = max(mx, p);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      mn = min(mn, (int64_t)__shfl_xor(mn, off, 64));
      mx = max(mx, (int64_t)__shfl_xor(mx, off, 64));
    }
    qmin = mn;
    qmax = mx;
  }
  const int32_t* kpos_b = a.kpos + (int64_t)cx.b * a.kpos_b;
  const int j_hi = lower_bound_pos(kpos_b, a.S, qmax + 1);
  const int j_lo = a.has_floor() ? min(lower_bound_pos(kpos_b, a.S, key_floor(a, qmin)), j_hi) : 0;
  // smallest key position this lane's query may see (window, chunks)
  const int64_t qfl = key_floor(a, qp);
  const int n_tiles = (j_hi - j_lo + BN - 1) / BN;


  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m = kNegBig, lsum = 0.f;
  const float cap2 = a.softcap * kLog2e;
  const float inv_cap2 = CAP ? 1.0f / cap2 : 0.f;

  if (n_tiles > 0) {
    TileRegs tr;
    load_tile(a, cx, j_lo, j_hi, tr);
    store_tile<ROT, NORM>(a, j_lo, tr, sm, 0);
    __syncthreads();
  }

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    const int jt = j_lo + t * BN;
    const bool has_next = t + 1 < n_tiles;
    TileRegs nx;
    if (has_next) load_tile(a, cx, jt + BN, j_hi, nx);

    const int32_t kfirst = sm.kpos[buf][0];
    const int32_t klast = sm.kpos[buf][BN - 1];
    const bool full = (jt + BN <= j_hi) && ((int64_t)klast <= qmin) &&
                      (!a.has_floor() || (int64_t)kfirst >= key_floor(a, qmax));
    const uint16_t* ks = sm.k[buf];
    const uint16_t* vs = sm.v[buf];
    const int gi = lane >> 4, s16 = lane & 15;
    const int hgv = gi >> 1;

    // The tile is processed as two 32-key halves to keep the live score registers small.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // ---- S^T = K Q^T for 32 keys ----
      f32x16 sacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
      const int krow = kb * 32 + ql;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 ka = as_bf16x8(*(const u32x4*)(ks + tile_off(krow, 2 * s + hg)));
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qop[s], sacc, 0, 0, 0);
      }

      // ---- soft-cap and mask ----
      if (CAP) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          // cap * tanh(s / cap) with tanh(x) = sign(x) (1 - e^{-2|x|}) / (1 + e^{-2|x|})
          const float x = sacc[r] * inv_cap2;
          const float e = fast_exp2(-2.0f * kLog2e * fabsf(x));
          sacc[r] = copysignf(cap2 * (1.0f - e) / (1.0f + e), x);
        }
      }
      if (!full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = kb * 32 + 8 * (r >> 2) + 4 * hg + (r & 3);
          const int64_t kp = sm.kpos[buf][kk];
          const bool ok = qvalid && kp <= qp && kp >= qfl;
          if (!ok) sacc[r] = -INFINITY;
        }
      }

      // ---- online softmax (row = this lane's query; the other 16 keys live in lane ^ 32) ----
      float mt = sacc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sacc[r]);
      mt = fmaxf(mt, swap_halves(mt));
      if (__ballot(mt > m + kRescaleThreshold) != 0) {
        const float m_new = fmaxf(m, mt);
        const float alpha = fast_exp2(m - m_new);
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        m = m_new;
      }
      bf16x8 pb[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = fast_exp2(sacc[8 * u + e] - m);
          lsum += p[e];
        }
        pb[u] = as_bf16x8(pack8(p));
      }

      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int row1 = kb * 32 + 16 * u + 4 * hgv + (s16 >> 2);
        const int row2 = row1 + 8;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int col = db * 32 + 16 * (gi & 1) + 4 * (s16 & 3);
          const int off1 = row1 * HD + (((col >> 3) ^ ((row1 & 3) << 2)) << 3) + (col & 7);
          const int off2 = row2 * HD + (((col >> 3) ^ ((row2 & 3) << 2)) << 3) + (col & 7);
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(vs + off1));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(vs + off2));
          typedef short i16x8 __attribute__((ext_vector_type(8)));
          const i16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va), pb[u],
                                                          o[db], 0, 0, 0);
        }
      }
    }

    if (has_next) store_tile<ROT, NORM>(a, jt + BN, nx, sm, buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O / l, round to bf16, store row (b, qi, qh) ----
  const float ltot = lsum + swap_halves(lsum);
  // a learned sink joins the denominator only (log2 units, relative to the running max)
  const float lden =
      (a.sinks != nullptr && ltot > 0.f) ? ltot + fast_exp2(a.sinks[qh] * kLog2e - m) : ltot;
  const float inv = ltot > 0.f ? 1.0f / lden : 0.f;
  if (qvalid) {
    uint16_t* orow = (uint16_t*)a.out + (int64_t)cx.b * a.o_b + (int64_t)qi * a.o_i +
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
hipError_t launch_variant(const AttnArgs& a, hipStream_t stream) {
  const int64_t nrows = (int64_t)a.L * a.G;
  const int nqb = (int)((nrows + ROWS - 1) / ROWS);
  dim3 grid(nqb, a.Hkv, a.B);
  hipLaunchKernelGGL((prefill_mfma_kernel<ROT, NORM, CAP>), grid, dim3(NT), 0, stream, a, nqb);
  return hipGetLastError();
}

template <int ROT, bool NORM>
hipError_t launch_cap(const AttnArgs& a, hipStream_t s) {
  return a.softcap > 0.f ? launch_variant<ROT, NORM, true>(a, s) : launch_variant<ROT, NORM, false>(a, s);
}
template <int ROT>
hipError_t launch_norm(const AttnArgs& a, hipStream_t s) {
  return a.qk_norm ? launch_cap<ROT, true>(a, s) : launch_cap<ROT, false>(a, s);
}

}  // namespace

bool prefill_mfma_supported(const AttnArgs& a) {
  if (a.D != HD) return false;
  if (a.qpos == nullptr || a.kpos == nullptr) return false;
  if (a.R == 0) return true;
  if (a.style == 0) {  // half-split: partner distance R/16 chunks must be 1, 2, 4 or 8
    const int P = a.R / 16;
    return a.R % 16 == 0 && (P == 1 || P == 2 || P == 4 || P == 8);
  }
  return a.R % 8 == 0;
}

hipError_t launch_prefill_mfma(const AttnArgs& a, hipStream_t stream) {
  if (a.B == 0 || a.L == 0) return hipSuccess;
  const int rot = a.R == 0 ? 0 : (a.style == 0 ? 1 : 2);
  switch (rot) {
    case 0: return launch_norm<0>(a, stream);
    case 1: return launch_norm<1>(a, stream);
    default: return launch_norm<2>(a, stream);
  }
}

}  // namespace gqa
