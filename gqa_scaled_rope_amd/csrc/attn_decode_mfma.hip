// bf16 split-KV single-token decode, head_dim 128, for gfx950.
//
// [Guide] section 3.3 (KVCache, layout [B, Hkv, Smax, D]) and section 3.7 (the decode step:
// the new query sits after every cached key, so only the window or chunks can mask: they set
// the first slot read, and a learned sink enters the final log-sum-exp merge), with the query
// normed and rotated at position lens-1 ([Models] "What differs": keys are cached already
// rotated, so they are read as stored).
//
// The step is bound by HBM: every cached K and V row is read exactly once and serves all
// G = Hq/Hkv query heads of its KV head (the grouping [Models] stretch exercise 5 asks a decode
// kernel to exploit).  Three launches:
//   decode_prep_q_kernel   every query row normed, rotated, scaled into log2 units, as bf16;
//   decode_split_kernel    a persistent grid walking a dense list of work items (sequence b,
//                          KV head g, split of 1024 keys); a workgroup's 4 wavefronts take 256
//                          keys each, in blocks of 32:
//                            S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (K straight from the loaded
//                            registers as the A operand, the G heads padded to 16 columns as B);
//                            online softmax in log2 units, lazily rescaled;
//                            O = P V on the same MFMA, P from the score accumulators, V read back
//                            from a wave-private LDS staging buffer with ds_read_b64_tr_b16;
//                          the wavefronts merge in LDS into one partial (O, max, sum) per item;
//   decode_combine_kernel  merges the partials of a sequence by their log-sum-exp weights.
//
// Why persistent: a workgroup that ends with stores in flight holds its slot until they drain,
// which under full read load costs several microseconds per item.  Here a workgroup issues the
// next item's query and first K/V block, then the previous item's stores, and only then waits
// for the new loads; the stores drain behind useful traffic.  Since the vector-memory counter
// retires loads and stores in issue order, every load and store in that sequence is
// unconditional (ranges that must not be touched are cut off by buffer descriptors), so the
// compiler's wait counts are exact and no wait ever covers the stores.
#include <algorithm>
#include <mutex>

#include "launch.hpp"

namespace gqa {
namespace {

constexpr int HD = 128;
constexpr int DWAVES = 4;
constexpr int DT = DWAVES * 64;
constexpr int SPLIT = 1024;         // keys per split; with enough work, 2 SPLIT (see split_keys)
constexpr int kLongItems = 8;       // items per resident workgroup that call for the long splits
constexpr int KBLK = 32;             // keys per block
constexpr int MAXG = 16;
constexpr int kPlanMax = 2048;       // sequences per launch of the split kernel
constexpr int kWgPerCu = 3;          // resident split workgroups per CU (LDS and VGPR budget)
constexpr float kRescaleThreshold = 8.0f;
constexpr int kRsrcFlags = 0x00020000;  // raw buffer, 32-bit elements
// Cache rows are read exactly once per call, so they are loaded non-temporally (policy bit "nt"),
// which streams measurably faster than ordinary loads on MI355X once the XCDs are evenly loaded.
constexpr int kStreamPolicy = 2;

typedef short i16x8 __attribute__((ext_vector_type(8)));

struct DecodeArgs {
  AttnArgs a;
  float* part_o;      // [B, Hkv, nsplit, G, D] unnormalised partial outputs
  float* part_ml;     // [B, Hkv, nsplit, G, 2] running max (log2 units) and sum
  uint16_t* qprep;    // [B, Hq, D] prepared queries (bf16, log2 units)
  int32_t* split_long;  // [launches] 1 when that split launch took the long splits; written by
                        // the launch's workgroup 0, read by the combine kernel
  int32_t nsplit;     // splits per (b, g) allotted in the workspace
  int32_t plan_seqs;  // sequences per launch of the split kernel (the launches' plan sets)
  int32_t resident;   // split workgroups resident on the device
  int32_t split_mode; // SplitMode: 0 chosen from the launch's sequences, 1 short, 2 long
  // paged cache (table non-null): a.k, a.v are pools [num_blocks, Hkv, 2^log2bs, D]; slot j of
  // sequence b is row j % bs of block table[b * max_blocks + j / bs]
  const int32_t* table;
  int32_t max_blocks, log2bs, num_blocks;
};

// V tile layout: row r's 16-byte chunk c at c ^ ((r & 7) << 1).  The transposing reads serve lanes
// 0-31 and 32-63 as two passes of 256 bytes over the 64 four-byte banks (measured on gfx950); a
// pass reads a 32-byte chunk pair of each of eight consecutive rows, and the XOR puts the eight
// pairs in eight different 32-byte slots of the bank array.
__device__ __forceinline__ int vt_swz(int r) { return (r & 7) << 1; }
__device__ __forceinline__ int vt_off(int r, int c) { return r * HD + ((c ^ vt_swz(r)) << 3); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, bytes, kRsrcFlags);
}

// Barrier over LDS traffic only: the fences order each wavefront's LDS accesses around
// s_barrier without waiting for its outstanding global loads and stores.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---- query preparation --------------------------------------------------------------------------
// One workgroup of HD threads per (query head h, sequence b), thread d = feature d: the row is
// RMS-normed ([Guide] section 3.2) when enabled, rotated at position lens[b]-1 ([Guide] section 4;
// half-split or adjacent pairs), multiplied by scale * log2(e) and rounded to bf16.
template <int ROT, bool NORM>
__global__ __launch_bounds__(HD) void decode_prep_q_kernel(AttnArgs a, uint16_t* qprep) {
  __shared__ float red[HD / 64];
  __shared__ float row[HD];
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const uint16_t* qr = (const uint16_t*)a.q + (int64_t)b * a.q_b + (int64_t)h * a.q_h;
  float x = bf16_to_f32(qr[d]);
  if (NORM) {
    const float ss = wave_sum(x * x);
    if ((d & 63) == 0) red[d >> 6] = ss;
    __syncthreads();
    const float rs = rsqrtf((red[0] + red[1]) * (1.0f / HD) + a.eps);
    x *= rs * bf16_to_f32(((const uint16_t*)a.qw)[d]);
  }
  if (ROT) {
    row[d] = x;
    __syncthreads();
    const int n = min(max(a.lens[b], 0), a.S);
    const int64_t tp = min<int64_t>(max<int64_t>((int64_t)n - 1, 0), a.table_len - 1);
    const int half = a.R >> 1;
    if (d < a.R) {
      if (ROT == 1) {  // pairs (i, i + R/2)
        const int p = d < half ? d : d - half;
        const float cs = a.cos_t[tp * half + p], sn = a.sin_t[tp * half + p];
        x = d < half ? x * cs - row[d + half] * sn : row[d - half] * sn + x * cs;
      } else {         // pairs (2i, 2i + 1)
        const int p = d >> 1;
        const float cs = a.cos_t[tp * half + p], sn = a.sin_t[tp * half + p];
        x = (d & 1) == 0 ? x * cs - row[d + 1] * sn : row[d - 1] * sn + x * cs;
      }
    }
  }
  const float qscale = a.scale * kLog2e;
  qprep[((int64_t)b * a.Hq + h) * HD + d] = f32_to_bf16(x * qscale);
}

// ---- split kernel -------------------------------------------------------------------------------
__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& w) { return __builtin_bit_cast(bf16x8, w); }

struct SplitSmem {
  // A wavefront's V staging buffer and, once its keys are done, its partial output share the
  // same 8 KB (LDS operations of one wavefront complete in order, so the reuse needs no barrier).
  union {
    uint16_t v[DWAVES][KBLK * HD];  // wave-private V staging
    float mo[DWAVES][MAXG][HD];     // per-wave partial outputs
  };
  float mm[DWAVES][MAXG];           // per-wave running max
  float ml[DWAVES][MAXG];           // per-wave running sum
  int plan[kPlanMax + 1];           // exclusive prefix over sequences of their work items
  int len[kPlanMax];                // clamped sequence lengths
  int wsum[DWAVES];
};
static_assert(KBLK * HD * 2 == MAXG * HD * 4, "staging and partial output share one region");

struct BlockRegs {
  u32x4 k[2][4];  // [16-key half][k-step]
  u32x4 v[8];     // rows (lane>>4) + 4e, chunk lane&15
};

// Loads the block of 32 keys starting at kb0 with buffer loads: keys at or beyond the end of the
// descriptors' range read as zero without a memory access, so no lane needs a branch.
__device__ __forceinline__ void load_block(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                           int kb0, BlockRegs& br) {
  const int lane = threadIdx.x & 63;
  // unsigned: offsets of blocks past the end may exceed INT32_MAX; they are out of range either way
  const unsigned kofs = ((unsigned)(kb0 + (lane & 15)) * HD + 8 * (lane >> 4)) * 2;
  const unsigned vofs = ((unsigned)(kb0 + (lane >> 4)) * HD + 8 * (lane & 15)) * 2;
#pragma unroll
  for (int kq = 0; kq < 2; ++kq)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      br.k[kq][s] = __builtin_amdgcn_raw_buffer_load_b128(
          rk, (int)(kofs + (kq * 16 * HD + 32 * s) * 2), 0, kStreamPolicy);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    br.v[e] = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)(vofs + 4 * e * HD * 2), 0,
                                                    kStreamPolicy);
  // keep the 16 loads together: the scheduler would otherwise start on the K operands as they
  // arrive and issue the V loads a full memory latency later
  __builtin_amdgcn_sched_barrier(0);
}

// A work item as one wavefront sees it (all fields wave-uniform).  A null item (none left) has
// we = 0 and empty descriptor ranges.  klo: first visible key (the paged walk starts below it,
// at a multiple of KBLK, and masks the keys in between).
struct Item {
  int b, g, sp, ws, we, nblk, klo;
  bool valid;
};

// First cache slot the query at position n - 1 may see: the window's and the chunk's bound
// ([Models] "Sliding windows"; chunks as in [Ster]'s llama4_text and Rnj-1.5 paragraphs); slot j
// holds position j.
__device__ __forceinline__ int first_key(const AttnArgs& a, int n) {
  return a.has_floor() ? (int)max<int64_t>(0, key_floor(a, (int64_t)n - 1)) : 0;
}

// First slot of a sequence's split walk: the first visible key, rounded down to a multiple of
// KBLK for a paged cache (so that every 16-key half of a block lies in one cache block).
__device__ __forceinline__ int walk_start(const AttnArgs& a, int n, bool paged) {
  const int f = first_key(a, n);
  return paged ? f & ~(KBLK - 1) : f;
}

// Paged loads of the block of 32 keys starting at kb0 (a multiple of KBLK) of sequence b: each
// 16-key half lies in one cache block and gets its own descriptors; keys at or past `we`, and a
// half wholly below the first visible key klo, are out of range (read as zero, no access), so a
// cache block that holds no visible key is never touched.  The table entries are wave-uniform
// scalar loads (adjacent blocks share a scalar cache line).
__device__ __forceinline__ void load_block_paged(const DecodeArgs& da, int b, int g, int we,
                                                 int klo, int kb0, BlockRegs& br) {
  const int lane = threadIdx.x & 63;
  const AttnArgs& a = da.a;
  const int bs = 1 << da.log2bs;
  const int32_t* trow = da.table + (int64_t)b * da.max_blocks;
  __amdgpu_buffer_rsrc_t rk[2], rv[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int j0 = kb0 + 16 * h;
    const int ti = min(j0 >> da.log2bs, da.max_blocks - 1);
    int phys = __builtin_amdgcn_readfirstlane(trow[ti]);
    phys = min(max(phys, 0), da.num_blocks - 1);
    const int64_t row = ((int64_t)phys * a.Hkv + g) * bs + (j0 & (bs - 1));
    const int cnt = j0 + 16 <= klo ? 0 : min(max(we - j0, 0), 16);
    rk[h] = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)a.k + row * HD), 0,
                                              cnt * HD * 2, kRsrcFlags);
    rv[h] = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)a.v + row * HD), 0,
                                              cnt * HD * 2, kRsrcFlags);
  }
  const int kofs = ((lane & 15) * HD + 8 * (lane >> 4)) * 2;
  const int vofs = ((lane >> 4) * HD + 8 * (lane & 15)) * 2;
#pragma unroll
  for (int kq = 0; kq < 2; ++kq)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      br.k[kq][s] = __builtin_amdgcn_raw_buffer_load_b128(rk[kq], kofs + 32 * s * 2, 0,
                                                          kStreamPolicy);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    br.v[e] = __builtin_amdgcn_raw_buffer_load_b128(rv[e >> 2], vofs + 4 * (e & 3) * HD * 2, 0,
                                                    kStreamPolicy);
  __builtin_amdgcn_sched_barrier(0);
}

// Keys per split of a walk of `range` keys.  When a launch's sequences hold at least kLongItems
// items (at SPLIT keys) per resident workgroup, walks longer than SPLIT take 2 SPLIT keys per
// item (fewer items, so less per-item work and fewer partials to merge); otherwise, or for short
// walks, SPLIT, so that a batch of short walks still spreads over every workgroup.  The split
// and combine kernels decide alike from the same sequences; the partials keep a stride of
// ceil(S / SPLIT) splits per (sequence, KV head).
__device__ __forceinline__ int split_keys(int range, bool longs) {
  return longs && range > SPLIT ? 2 * SPLIT : SPLIT;
}
__device__ __forceinline__ bool use_long_splits(int64_t short_items, int resident) {
  return short_items >= (int64_t)kLongItems * resident;
}

template <bool CAP, bool PAGED>
__global__ __launch_bounds__(DT, kWgPerCu) void decode_split_kernel(DecodeArgs da) {
  __shared__ SplitSmem sm;
  const AttnArgs& a = da.a;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int B = a.B, Hkv = a.Hkv, G = a.G;

  // ---- plan: items of sequence i = Hkv * (splits of its window); exclusive prefix in LDS -------
  for (int i = tid; i < B; i += DT) {
    const int n = min(max(a.lens[i], 0), a.S);
    const int start = walk_start(a, n, PAGED);
    sm.len[i] = n;
    sm.plan[i] = ((n - start + SPLIT - 1) / SPLIT) * Hkv;
  }
  __syncthreads();
  // exclusive prefix of sm.plan[0 .. B) in place, the total in sm.plan[B]
  auto scan_plan = [&]() {
    const int per = (B + DT - 1) / DT;
    const int i0 = min(tid * per, B), i1 = min(i0 + per, B);
    int loc = 0;
    for (int i = i0; i < i1; ++i) loc += sm.plan[i];
    int x = loc;  // inclusive scan over the wavefront
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63) sm.wsum[w] = x;
    __syncthreads();
    int run = x - loc;
    for (int ww = 0; ww < w; ++ww) run += sm.wsum[ww];
    for (int i = i0; i < i1; ++i) {
      const int c = sm.plan[i];
      sm.plan[i] = run;
      run += c;
    }
    if (tid == 0) sm.plan[B] = sm.wsum[0] + sm.wsum[1] + sm.wsum[2] + sm.wsum[3];
    __syncthreads();
  };
  scan_plan();
  const bool longs =
      da.split_mode == 2 ||
      (da.split_mode == 0 && use_long_splits(__builtin_amdgcn_readfirstlane(sm.plan[B]), da.resident));
  // the combine kernel takes the launch's choice from here (every workgroup decided alike)
  if (blockIdx.x == 0 && tid == 0) da.split_long[0] = longs ? 1 : 0;
  if (longs) {  // plan again with the long splits (uniform: every wave read the same total)
    __syncthreads();
    for (int i = tid; i < B; i += DT) {
      const int n = sm.len[i];
      const int start = walk_start(a, n, PAGED);
      const int sz = split_keys(n - start, true);
      sm.plan[i] = ((n - start + sz - 1) / sz) * Hkv;
    }
    __syncthreads();
    scan_plan();
  }
  const int total = __builtin_amdgcn_readfirstlane(sm.plan[B]);
  if ((int)blockIdx.x >= total) return;

  // Item t: the sequence b with plan[b] <= t < plan[b + 1], then KV head and split within it.
  // Consecutive items go to consecutive workgroups, hence round-robin over the XCDs.
  auto locate = [&](int t) {
    Item it;
    it.valid = t < total;
    if (!it.valid) {
      it.b = it.g = it.sp = it.ws = it.we = it.nblk = it.klo = 0;
      return it;
    }
    int lo = 0, hi = B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (__builtin_amdgcn_readfirstlane(sm.plan[mid]) <= t) lo = mid;
      else hi = mid;
    }
    const int p0 = __builtin_amdgcn_readfirstlane(sm.plan[lo]);
    const int p1 = __builtin_amdgcn_readfirstlane(sm.plan[lo + 1]);
    const int n = __builtin_amdgcn_readfirstlane(sm.len[lo]);
    const int nsp = (p1 - p0) / Hkv;
    const int r = t - p0;
    it.b = lo;
    it.g = r / nsp;
    it.sp = r - it.g * nsp;
    const int start = walk_start(a, n, PAGED);
    it.klo = first_key(a, n);
    const int sz = split_keys(n - start, longs), sub = sz / DWAVES;  // keys per split, per wave
    const int ks = start + it.sp * sz;
    const int ke = min(ks + sz, n);
    it.ws = ks + w * sub;
    it.we = min(it.ws + sub, ke);
    it.nblk = it.we > it.ws ? (it.we - it.ws + KBLK - 1) / KBLK : 0;
    return it;
  };
  // Descriptors of an item: its K and V rows up to this wavefront's last key, its G prepared query
  // rows, and its partial-output slots.  Empty ranges for a null item.
  auto kv_rsrc = [&](const Item& it, const void* base) {
    const int64_t off = (int64_t)it.b * a.k_b + (int64_t)it.g * a.k_h;
    return rsrc((const uint16_t*)base + off, max(it.we, 0) * HD * 2);
  };
  auto q_rsrc = [&](const Item& it) {
    return rsrc(da.qprep + ((int64_t)it.b * a.Hq + (int64_t)it.g * G) * HD,
                it.valid ? G * HD * 2 : 0);
  };
  auto part_index = [&](const Item& it) {
    return (((int64_t)it.b * Hkv + it.g) * da.nsplit + it.sp) * G;
  };

  // query operand: head slot hs = lane & 15 (zero beyond G: outside the range), chunk 4s + cg
  const int hs = lane & 15, cg = lane >> 4;
  auto load_q = [&](__amdgpu_buffer_rsrc_t rq, u32x4* qv) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qv[s] = __builtin_amdgcn_raw_buffer_load_b128(rq, (hs * HD + 8 * (4 * s + cg)) * 2, 0, 0);
  };

  uint16_t* vs = sm.v[w];
  const float cap2 = a.softcap * kLog2e;
  const float inv_cap2 = CAP ? 1.0f / cap2 : 0.f;
  f32x4 o[8];
  float m, lsum;
  bf16x8 qop[4];

  auto block = [&](const BlockRegs& cur, int kb0, int we, int klo) {
    // stage V rows of this block in the wave's LDS buffer
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = (lane >> 4) + 4 * e;
      *(u32x4*)(vs + vt_off(row, lane & 15)) = cur.v[e];
    }

    // S^T = K Q^T: lane holds head slot hs, keys kq*16 + 4*(lane>>4) + r
    f32x4 sk[2];
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {
      sk[kq] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        sk[kq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cur.k[kq][s]), qop[s], sk[kq],
                                                         0, 0, 0);
    }
#pragma unroll
    for (int kq = 0; kq < 2; ++kq)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = sk[kq][r];
        if (CAP) {  // cap * tanh(x / cap) via exp2, in log2 units
          const float y = x * inv_cap2;
          const float e = fast_exp2(-2.0f * kLog2e * fabsf(y));
          x = copysignf(cap2 * (1.0f - e) * __builtin_amdgcn_rcpf(1.0f + e), y);
        }
        const int key = kb0 + kq * 16 + 4 * (lane >> 4) + r;
        sk[kq][r] = (key < we && (!PAGED || key >= klo)) ? x : -INFINITY;
      }

    float mt = fmaxf(fmaxf(fmaxf(sk[0][0], sk[0][1]), fmaxf(sk[0][2], sk[0][3])),
                     fmaxf(fmaxf(sk[1][0], sk[1][1]), fmaxf(sk[1][2], sk[1][3])));
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    if (__ballot(mt > m + kRescaleThreshold) != 0) {
      const float m_new = fmaxf(m, mt);
      const float alpha = fast_exp2(m - m_new);
      lsum *= alpha;
      // O rows are head slots 4*(lane>>4) + r; their alpha lives in lane (4*(lane>>4) + r)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, 4 * (lane >> 4) + r, 64);
#pragma unroll
        for (int db = 0; db < 8; ++db) o[db][r] *= ar;
      }
      m = m_new;
    }
    float p[8];
#pragma unroll
    for (int kq = 0; kq < 2; ++kq)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[4 * kq + r] = fast_exp2(sk[kq][r] - m);
        lsum += p[4 * kq + r];
      }
    u32x4 pw;
#pragma unroll
    for (int e = 0; e < 4; ++e) pw[e] = pack_bf16x2(p[2 * e], p[2 * e + 1]);
    const bf16x8 pa = as_bf16x8(pw);

    // O = P V: B operand = V[32 keys][16 features] via transposing LDS reads
    const int gi = lane >> 4, si = lane & 15;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int row1 = 4 * gi + (si >> 2);
      const int row2 = row1 + 16;
      const int col = 16 * db + 4 * (si & 3);
      const int off1 = row1 * HD + (((col >> 3) ^ vt_swz(row1)) << 3) + (col & 7);
      const int off2 = row2 * HD + (((col >> 3) ^ vt_swz(row2)) << 3) + (col & 7);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vs + off1));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vs + off2));
      const i16x8 vb = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(bf16x8, vb), o[db],
                                                      0, 0, 0);
    }
  };

  // Merge the four wavefronts' partials in LDS and store them: thread tid owns column tid & 127 of
  // rows 2k + (tid >> 7), and row tid's (max, sum); rows at or beyond G fall outside the
  // descriptors' ranges and are dropped.  A fixed count of unconditional stores per thread.
  auto merge_store = [&](__amdgpu_buffer_rsrc_t ro, __amdgpu_buffer_rsrc_t rml) {
    const int d = tid & (HD - 1);
#pragma unroll
    for (int k = 0; k < MAXG * HD / DT; ++k) {
      const int row = 2 * k + (tid >> 7);
      float M = kNegBig;
#pragma unroll
      for (int ww = 0; ww < DWAVES; ++ww) M = fmaxf(M, sm.mm[ww][row]);
      float acc = 0.f;
#pragma unroll
      for (int ww = 0; ww < DWAVES; ++ww) acc += fast_exp2(sm.mm[ww][row] - M) * sm.mo[ww][row][d];
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc), ro, (row * HD + d) * 4, 0, 0);
    }
    const int row = tid & (MAXG - 1);
    float M = kNegBig;
#pragma unroll
    for (int ww = 0; ww < DWAVES; ++ww) M = fmaxf(M, sm.mm[ww][row]);
    float lt = 0.f;
#pragma unroll
    for (int ww = 0; ww < DWAVES; ++ww) lt += fast_exp2(sm.mm[ww][row] - M) * sm.ml[ww][row];
    const u32x2 mlw = {__float_as_uint(M), __float_as_uint(lt)};
    __builtin_amdgcn_raw_buffer_store_b64(mlw, rml, tid < MAXG ? row * 8 : INT32_MIN, 0, 0);
  };

  auto load_blk = [&](const Item& it, __amdgpu_buffer_rsrc_t rk_, __amdgpu_buffer_rsrc_t rv_,
                      int kb0, BlockRegs& br) {
    if (PAGED)
      load_block_paged(da, it.b, it.g, it.we, it.klo, kb0, br);
    else
      load_block(rk_, rv_, kb0, br);
  };

  // ---- the item loop ----
  int t = blockIdx.x;
  Item cur = locate(t);
  __amdgpu_buffer_rsrc_t rk = kv_rsrc(cur, a.k), rv = kv_rsrc(cur, a.v);
  u32x4 qv[4];
  load_q(q_rsrc(cur), qv);
  BlockRegs ra;
  load_blk(cur, rk, rv, cur.ws, ra);
  // partial-output descriptors of the previous item: none before the first
  __amdgpu_buffer_rsrc_t ro = rsrc(da.part_o, 0), rml = rsrc(da.part_ml, 0);
  while (true) {
    // previous item's partial (dropped on the first pass: empty ranges)
    lds_barrier();
    merge_store(ro, rml);
    lds_barrier();

    // this item
#pragma unroll
    for (int s = 0; s < 4; ++s) qop[s] = as_bf16x8(qv[s]);
#pragma unroll
    for (int db = 0; db < 8; ++db) o[db] = (f32x4){0.f, 0.f, 0.f, 0.f};
    m = kNegBig;
    lsum = 0.f;
    block(ra, cur.ws, cur.we, cur.klo);  // (all keys masked when this wavefront has none)
    for (int i = 1; i < cur.nblk; ++i) {
      load_blk(cur, rk, rv, cur.ws + i * KBLK, ra);
      block(ra, cur.ws + i * KBLK, cur.we, cur.klo);
    }
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    if (lane < MAXG) {
      sm.mm[w][lane] = m;
      sm.ml[w][lane] = lsum;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int db = 0; db < 8; ++db) sm.mo[w][4 * (lane >> 4) + r][16 * db + (lane & 15)] = o[db][r];

    const int64_t pi = part_index(cur);
    ro = rsrc(da.part_o + pi * HD, G * HD * 4);
    rml = rsrc(da.part_ml + pi * 2, G * 2 * 4);

    // next item: its loads go out before this item's stores
    t += gridDim.x;
    cur = locate(t);
    rk = kv_rsrc(cur, a.k);
    rv = kv_rsrc(cur, a.v);
    load_q(q_rsrc(cur), qv);
    load_blk(cur, rk, rv, cur.ws, ra);
    if (!cur.valid) {
      lds_barrier();
      merge_store(ro, rml);
      break;
    }
  }
}

// out[b, h, :] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over the splits of sequence b.
// The first wavefront loads the (max, sum) pairs of all splits at once, reduces them and leaves
// the split weights 2^(m_s - M) in LDS; then each thread owns one feature and sums the weighted
// partial outputs, four splits per step so that their loads overlap.
constexpr int kCombineMaxSplits = 256;  // 256K keys; longer caches use the weight formula inline
__global__ __launch_bounds__(HD) void decode_combine_kernel(DecodeArgs da) {
  const AttnArgs& a = da.a;
  __shared__ float wsc[kCombineMaxSplits];
  __shared__ float stat[2];
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int G = a.G, g = h / G, hs = h % G;
  const int n = min(max(a.lens[b], 0), a.S);
  const int start = walk_start(a, n, da.table != nullptr);
  // the split size that b's split launch chose
  const bool longs = da.split_long[b / da.plan_seqs] != 0;
  const int sz = split_keys(n - start, longs);
  const int nsp = (n - start + sz - 1) / sz;
  const int64_t item0 = (((int64_t)b * a.Hkv + g) * da.nsplit) * G + hs;
  const float* ml = da.part_ml;
  if (d < 64) {
    float M = kNegBig;
    for (int s = d; s < nsp; s += 64) M = fmaxf(M, ml[(item0 + (int64_t)s * G) * 2]);
    M = wave_max(M);
    float lt = 0.f;
    for (int s = d; s < nsp; s += 64) {
      const int64_t it = item0 + (int64_t)s * G;
      const float sc = fast_exp2(ml[it * 2] - M);
      if (s < kCombineMaxSplits) wsc[s] = sc;
      lt += sc * ml[it * 2 + 1];
    }
    lt = wave_sum(lt);
    if (d == 0) {
      stat[0] = M;
      stat[1] = lt;
    }
  }
  __syncthreads();
  const float M = stat[0], lt = stat[1];
  const float* po = da.part_o + item0 * HD + d;
  const int64_t step = (int64_t)G * HD;
  float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
  int s = 0;
  for (; s + 4 <= nsp && s + 4 <= kCombineMaxSplits; s += 4) {
    const float o0 = po[(int64_t)s * step], o1 = po[(int64_t)(s + 1) * step];
    const float o2 = po[(int64_t)(s + 2) * step], o3 = po[(int64_t)(s + 3) * step];
    acc0 += wsc[s] * o0;
    acc1 += wsc[s + 1] * o1;
    acc2 += wsc[s + 2] * o2;
    acc3 += wsc[s + 3] * o3;
  }
  for (; s < nsp; ++s) {
    const float sc = s < kCombineMaxSplits ? wsc[s] : fast_exp2(ml[(item0 + (int64_t)s * G) * 2] - M);
    acc0 += sc * po[(int64_t)s * step];
  }
  const float acc = (acc0 + acc1) + (acc2 + acc3);
  // a learned sink joins the denominator only (log2 units, relative to M)
  const float lden = (a.sinks != nullptr && lt > 0.f) ? lt + fast_exp2(a.sinks[h] * kLog2e - M) : lt;
  const float r = lt > 0.f ? acc / lden : 0.f;
  uint16_t* orow = (uint16_t*)a.out + (int64_t)b * a.o_b + (int64_t)h * a.o_h;
  orow[d] = f32_to_bf16(r);
}

template <int ROT, bool NORM>
void launch_prep(const AttnArgs& a, uint16_t* qprep, hipStream_t stream) {
  hipLaunchKernelGGL((decode_prep_q_kernel<ROT, NORM>), dim3(a.Hq, a.B), dim3(HD), 0, stream, a,
                     qprep);
}

int cu_count() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (dev >= 0 && dev < 64 && cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev >= 0 && dev < 64) cache[dev] = n;
  return n;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Sequences per split launch: at most kPlanMax, and few enough that item ids fit in int32.
int plan_seqs(int Hkv, int64_t nsplit) {
  const int64_t per_seq = (int64_t)Hkv * nsplit;
  return (int)std::min<int64_t>(kPlanMax, std::max<int64_t>(1, INT32_MAX / per_seq));
}

// Workspace: partial outputs | partial (max, sum) | prepared queries | one split flag per launch.
struct DecodeWs {
  size_t o, ml, q, flags, total;
};
DecodeWs decode_ws_layout(int B, int Hkv, int G, int Smax) {
  const int64_t nsplit = (Smax + SPLIT - 1) / SPLIT;
  const int64_t items = (int64_t)B * Hkv * nsplit * G;
  const int64_t per_launch = plan_seqs(Hkv, nsplit);
  const int64_t launches = (B + per_launch - 1) / per_launch;
  DecodeWs w;
  w.o = 0;
  w.ml = align256((size_t)items * HD * sizeof(float));
  w.q = w.ml + align256((size_t)items * 2 * sizeof(float));
  w.flags = w.q + align256((size_t)B * Hkv * G * HD * sizeof(uint16_t));
  w.total = w.flags + (size_t)std::max<int64_t>(launches, 1) * sizeof(int32_t);
  return w;
}

}  // namespace

int decode_split_keys() { return SPLIT; }

bool decode_mfma_supported(const AttnArgs& a) {
  if (a.D != HD || a.G > MAXG) return false;
  if ((int64_t)a.S * HD * 2 > INT32_MAX) return false;  // byte offsets within one (b, g) cache
  return true;
}

size_t decode_mfma_workspace_bytes(int B, int Hkv, int G, int D, int Smax) {
  (void)D;  // head_dim is 128 on this path
  return decode_ws_layout(B, Hkv, G, Smax).total;
}

// ---- fixed scratch for the entry point that allocates nothing ---------------------------------
// One array per GPU, in this module's device memory for as long as the process runs.  Host code
// never uses the array's name as an address (on the host it is only a stand-in for the symbol):
// each device's address comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address reaches kernels.
namespace {
__device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode_mfma(const AttnArgs& a, void* workspace, hipStream_t stream,
                              const PagedKV* paged, SplitMode mode) {
  if (a.B == 0) return hipSuccess;
  DecodeArgs d;
  d.a = a;
  d.table = paged ? paged->table : nullptr;
  d.max_blocks = paged ? paged->max_blocks : 0;
  d.log2bs = paged ? paged->log2bs : 0;
  d.num_blocks = paged ? paged->num_blocks : 0;
  d.nsplit = (a.S + SPLIT - 1) / SPLIT;
  d.split_mode = (int)mode;
  const DecodeWs wl = decode_ws_layout(a.B, a.Hkv, a.G, a.S);
  char* ws = (char*)workspace;
  d.part_o = (float*)(ws + wl.o);
  d.part_ml = (float*)(ws + wl.ml);
  d.qprep = (uint16_t*)(ws + wl.q);
  d.split_long = (int32_t*)(ws + wl.flags);

  const int rot = a.R == 0 ? 0 : (a.style == 0 ? 1 : 2);
  const bool norm = a.qk_norm != 0;
  switch (rot * 2 + (norm ? 1 : 0)) {
    case 0: launch_prep<0, false>(a, d.qprep, stream); break;
    case 1: launch_prep<0, true>(a, d.qprep, stream); break;
    case 2: launch_prep<1, false>(a, d.qprep, stream); break;
    case 3: launch_prep<1, true>(a, d.qprep, stream); break;
    case 4: launch_prep<2, false>(a, d.qprep, stream); break;
    default: launch_prep<2, true>(a, d.qprep, stream); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  // The split kernel plans at most kPlanMax sequences per launch (and keeps item ids in int32).
  const int64_t per_seq = (int64_t)a.Hkv * d.nsplit;
  const int chunk = plan_seqs(a.Hkv, d.nsplit);
  const int resident = cu_count() * kWgPerCu;
  d.plan_seqs = chunk;
  d.resident = resident;
  for (int b0 = 0; b0 < a.B; b0 += chunk) {
    const int nb = std::min(chunk, a.B - b0);
    DecodeArgs c = d;
    c.a.B = nb;
    c.a.k = (const uint16_t*)a.k + (int64_t)b0 * a.k_b;
    c.a.v = (const uint16_t*)a.v + (int64_t)b0 * a.k_b;
    c.a.lens = a.lens + b0;
    c.part_o = d.part_o + (int64_t)b0 * per_seq * a.G * HD;
    c.part_ml = d.part_ml + (int64_t)b0 * per_seq * a.G * 2;
    c.qprep = d.qprep + (int64_t)b0 * a.Hq * HD;
    c.split_long = d.split_long + b0 / chunk;
    const int nwg = (int)std::min<int64_t>((int64_t)nb * per_seq, resident);
    if (d.table) {
      c.a.k = a.k;  // the pools are shared by all sequences
      c.a.v = a.v;
      c.table = d.table + (int64_t)b0 * d.max_blocks;
      if (a.softcap > 0.f)
        hipLaunchKernelGGL((decode_split_kernel<true, true>), dim3(nwg), dim3(DT), 0, stream, c);
      else
        hipLaunchKernelGGL((decode_split_kernel<false, true>), dim3(nwg), dim3(DT), 0, stream, c);
    } else if (a.softcap > 0.f) {
      hipLaunchKernelGGL((decode_split_kernel<true, false>), dim3(nwg), dim3(DT), 0, stream, c);
    } else {
      hipLaunchKernelGGL((decode_split_kernel<false, false>), dim3(nwg), dim3(DT), 0, stream, c);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(decode_combine_kernel, dim3(a.Hq, a.B), dim3(HD), 0, stream, d);
  return hipGetLastError();
}

}  // namespace gqa
