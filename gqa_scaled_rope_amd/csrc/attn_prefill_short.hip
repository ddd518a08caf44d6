// bf16 MFMA prefill attention over prepared keys, head_dim 128, gfx950 -- the short-band kernel.
// Four wavefronts of 32 query rows of one KV head per workgroup and four K/V tile buffers (68 KB
// of LDS), so two workgroups share a CU: one's query preparation and first tile loads overlap the
// other's loop.  With few key tiles per workgroup (a short sliding window, early causal blocks)
// that overlap matters more than the longer pipeline of the eight-wavefront kernel in
// attn_prefill_stream.hip, which takes the long bands.  Same math: 32-key tiles, S^T = K Q^T and
// O^T = V^T P^T on v_mfma_f32_32x32x16_bf16, online softmax in log2 units with lazy rescaling, K
// and V tiles copied HBM -> LDS by buffer_load ... lds.
#include "stream_tiles.hpp"

namespace gqa {
namespace {

using namespace stream;

constexpr int NW = 4;
constexpr int NT = NW * 64;
constexpr int ROWS = NW * 32;
constexpr int kTileRounds = BN / (4 * NW);  // 1 KB loads per wave per K (or V) tile
static_assert(BN % (4 * NW) == 0 && BN <= 64, "tile loader and key-position loader layout");

// Four K/V/key-position tile buffers: while a step works on tiles t and t + 1, tiles t + 2 and
// t + 3 are in flight, so a band of a few tiles is loaded almost whole before the loop starts.
// Each buffer is its own LDS object and the step loop is unrolled over the buffer cycle, so every
// access names its buffer at compile time: the compiler can then see that reads of the current
// tiles never alias the asynchronous HBM->LDS loads of a later one and does not make them wait
// for those loads.  Every wavefront loads the tile's key positions into its own row, so each
// wavefront issues the same number of loads per tile and a counted wait retires exactly the
// tiles due.
constexpr int NBUF = 4;
constexpr int kDmaPerTile = 2 * kTileRounds + 1;  // per wavefront: K, V and the key positions
__shared__ __attribute__((aligned(16))) uint16_t g_k0[TILE_ELEMS];
__shared__ __attribute__((aligned(16))) uint16_t g_k1[TILE_ELEMS];
__shared__ __attribute__((aligned(16))) uint16_t g_k2[TILE_ELEMS];
__shared__ __attribute__((aligned(16))) uint16_t g_k3[TILE_ELEMS];
__shared__ __attribute__((aligned(16))) uint16_t g_v0[TILE_ELEMS];
__shared__ __attribute__((aligned(16))) uint16_t g_v1[TILE_ELEMS];
__shared__ __attribute__((aligned(16))) uint16_t g_v2[TILE_ELEMS];
__shared__ __attribute__((aligned(16))) uint16_t g_v3[TILE_ELEMS];
__shared__ __attribute__((aligned(16))) int32_t g_p[NBUF][NW][64];

template <int BUF>
__device__ __forceinline__ uint16_t* kbuf() {
  return BUF == 0 ? g_k0 : BUF == 1 ? g_k1 : BUF == 2 ? g_k2 : g_k3;
}
template <int BUF>
__device__ __forceinline__ uint16_t* vbuf() {
  return BUF == 0 ? g_v0 : BUF == 1 ? g_v1 : BUF == 2 ? g_v2 : g_v3;
}


template <int ROT, bool NORM, bool CAP>
// Two workgroups per CU (4 x 17 KB tiles of LDS and up to 256 VGPRs each): one's query prep and
// first tiles overlap the other's loop, and each barrier holds only the four waves of one group.
__global__ __launch_bounds__(NT, 2) void prefill_short_kernel(StreamArgs sa, int nqb) {
  const AttnArgs& a = sa.a;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: a scalar register
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
  const i32x4 rp = rsrc_words(kpos_b, a.S * 4);

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
    // the tile's key positions (and the next tile's, unused) into this wavefront's own row;
    // positions past the last key read as zero and are masked by key index
    tile_dma4(rp, (lds_void*)g_p[buf][w], (uint32_t)((jt + lane) * 4));
  };
  // tiles 0 .. n - 1 (n < NBUF) of a band starting at key j0, into buffers 0 .. n - 1
  auto issue_first = [&](int j0, int n) {
    static_assert(NBUF == 4, "first-tile loads are written out for four buffers");
    if (n > 0) issue_tile(j0, std::integral_constant<int, 0>());
    if (n > 1) issue_tile(j0 + BN, std::integral_constant<int, 1>());
    if (n > 2) issue_tile(j0 + 2 * BN, std::integral_constant<int, 2>());
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
  // The first NBUF - 1 tiles' loads go out now -- from key 0 without a window or chunks, else from
  // the guessed band start (loaded again below if the guess is wrong) -- after the waits for the
  // position loads above (a wait for those placed behind the tiles' loads would wait for the
  // tiles too) and beside the band and query-prep loads below.
  const int j_first = a.has_floor() ? g_lo : 0;
  const int n_first = min((max(g_hi, j_first) - j_first + BN - 1) / BN, NBUF - 1);
  __builtin_amdgcn_sched_barrier(0);
  issue_first(j_first, n_first);
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
  // mask bounds in int32: allowed <=> key index < j_hi and qlo32 <= key position <= qp32
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
  // Tiles live in NBUF = 4 buffers: the barrier before the S^T of tile t+1 waits for tile t+1's
  // loads (tile t+2's may still be in flight), and once every wavefront is past it the buffer of
  // tile t-1 is free for tile t+3's.
  const int nsteps = n_tiles;
  // two score sets that trade roles every step (a step reads one and fills the other), so no
  // copy of the next step's scores has to wait for its MFMAs
  f32x16 s_a, s_b;
  auto step = [&](int s, auto phc, f32x16& sc, f32x16& s_next) {
    constexpr int PH = decltype(phc)::value;  // position in the 4-step cycle (buffers x score sets)
    constexpr int buf = PH % NBUF;
    constexpr int nbuf = (buf + 1) % NBUF;
    const int t = s;
    const int jt = j_lo + t * BN;
    const int32_t* kpt = g_p[buf][w];
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
      const int lim = j_hi - jt - 4 * hg;  // this lane's key r is in the band iff 8(r/4) + r%4 < lim
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int32_t kp = kpt[8 * (r >> 2) + 4 * hg + (r & 3)];
        if (!(kp <= qp32 && kp >= qlo32 && 8 * (r >> 2) + (r & 3) < lim)) sc[r] = -INFINITY;
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
      if (t + 2 < n_tiles) barrier_after_loads<kDmaPerTile>();  // tile t+2 may stay in flight
      else barrier_after_loads<0>();
      if (t + 3 < n_tiles) issue_tile(jt + 3 * BN, std::integral_constant<int, (buf + 3) % NBUF>());
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

  // The loop's counted waits assume exactly the tiles 0 .. min(n_tiles, NBUF - 1) - 1 of the band
  // in flight: when the guess issued others, they land first and the right ones are issued.
  const int n_pre = min(n_tiles, NBUF - 1);
  if (j_lo != j_first || n_first != n_pre) {
    __builtin_amdgcn_s_waitcnt(0);
    issue_first(j_lo, n_pre);
  }
  // the first tile and its key positions are then visible to every wavefront
  if (n_pre > 2) barrier_after_loads<2 * kDmaPerTile>();
  else if (n_pre > 1) barrier_after_loads<kDmaPerTile>();
  else barrier_after_loads<0>();
  if (nsteps > 0) s_a = qk(std::integral_constant<int, 0>());
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  using P3 = std::integral_constant<int, 3>;
  for (int s = 0; s < nsteps; s += 4) {
    step(s, P0(), s_a, s_b);
    if (s + 1 < nsteps) step(s + 1, P1(), s_b, s_a);
    if (s + 2 < nsteps) step(s + 2, P2(), s_a, s_b);
    if (s + 3 < nsteps) step(s + 3, P3(), s_b, s_a);
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
  hipLaunchKernelGGL((prefill_short_kernel<ROT, NORM, CAP>), dim3(nqb * a.Hkv * a.B), dim3(NT),
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

}  // namespace

hipError_t stream::launch_attn_short(const StreamArgs& sa, hipStream_t stream) {
  switch (sa.a.R == 0 ? 0 : (sa.a.style == 0 ? 1 : 2)) {
    case 0: return launch_attn_norm<0>(sa, stream);
    case 1: return launch_attn_norm<1>(sa, stream);
    default: return launch_attn_norm<2>(sa, stream);
  }
}

}  // namespace gqa
