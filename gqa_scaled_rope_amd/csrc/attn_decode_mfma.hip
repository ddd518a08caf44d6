// bf16 split-KV single-token decode, head_dim 128, for gfx950.
//
// [Guide] section 3.3 (KVCache, layout [B, Hkv, Smax, D]) and section 3.7 (the decode step:
// the new query sits after every cached key, so only the window can mask), with the query
// normed and rotated at position lens-1 ([Models] "What differs": keys are cached already
// rotated, so they are read as stored).
//
// The step is bound by HBM: every cached K and V row is read exactly once and serves all
// G = Hq/Hkv query heads of its KV head ([Models] stretch exercise 5's "read each row once for the
// whole head group").  Work item = (sequence b, KV head g, split of 1024 keys); a workgroup of 4
// wavefronts streams the split, 256 keys per wavefront in blocks of 32, with the next block's
// global loads in flight while the current one is computed.  Per block:
//   S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (K straight from the loaded registers as the A
//   operand; the G query heads padded to 16 columns as the B operand);
//   online softmax in log2 units, lazily rescaled as in the prefill kernel;
//   O = P V on the same MFMA, P taken lane-locally from the score accumulators as the A operand
//   and V read back from a wave-private LDS staging buffer with ds_read_b64_tr_b16.
// The four wavefronts merge (max, sum, output) in LDS and write one partial per work item; the
// combine kernel merges the partials of a sequence by their log-sum-exp weights.
#include "launch.hpp"

namespace gqa {
namespace {

constexpr int HD = 128;
constexpr int DWAVES = 4;
constexpr int DT = DWAVES * 64;
constexpr int SPLIT = 1024;
constexpr int SUB = SPLIT / DWAVES;  // keys per wavefront
constexpr int KBLK = 32;             // keys per block
constexpr int MAXG = 16;
constexpr float kRescaleThreshold = 8.0f;

typedef short i16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int vt_off(int r, int c) { return r * HD + ((c ^ (r & 15)) << 3); }

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
__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& w) { return __builtin_bit_cast(bf16x8, w); }

struct DecodeSmem {
  uint16_t v[DWAVES][KBLK * HD];        // wave-private V staging
  float mo[DWAVES][MAXG][HD];           // per-wave partial outputs
  float mm[DWAVES][MAXG];               // per-wave running max
  float ml[DWAVES][MAXG];               // per-wave running sum
};

struct BlockRegs {
  u32x4 k[2][4];  // [16-key half][k-step]
  u32x4 v[8];     // rows (lane>>4) + 4e, chunk lane&15
};

__device__ __forceinline__ void load_block(const uint16_t* kbase, const uint16_t* vbase, int kb0,
                                           int kend, BlockRegs& br) {
  const int lane = threadIdx.x & 63;
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int kq = 0; kq < 2; ++kq) {
    const int key = kb0 + kq * 16 + (lane & 15);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      br.k[kq][s] = key < kend ? ld16(kbase + (int64_t)key * HD + 8 * (4 * s + (lane >> 4))) : z;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int key = kb0 + (lane >> 4) + 4 * e;
    br.v[e] = key < kend ? ld16(vbase + (int64_t)key * HD + 8 * (lane & 15)) : z;
  }
}

template <int ROT>
__device__ __forceinline__ void rotate8(float* x, const float* y, int c, int R, const float* cr,
                                        const float* sr) {
  const int d0 = 8 * c;
  if (d0 >= R) return;
  if (ROT == 1) {
    const int half = R >> 1;
    const bool first = d0 < half;
    const int p0 = first ? d0 : d0 - half;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float cs = cr[p0 + e], sn = sr[p0 + e];
      x[e] = first ? (x[e] * cs - y[e] * sn) : (y[e] * sn + x[e] * cs);
    }
  } else if (ROT == 2) {
    const int p0 = d0 >> 1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float cs = cr[p0 + e], sn = sr[p0 + e];
      const float a = x[2 * e], b = x[2 * e + 1];
      x[2 * e] = a * cs - b * sn;
      x[2 * e + 1] = a * sn + b * cs;
    }
  }
}

template <int ROT, bool NORM, bool CAP>
__global__ __launch_bounds__(DT, 2) void decode_split_kernel(DecodeArgs da) {
  __shared__ DecodeSmem sm;
  const AttnArgs& a = da.a;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int sp = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = a.G;
  const int n = min(max(a.lens[b], 0), a.S);
  const int start = a.window > 0 ? max(0, n - a.window) : 0;
  const int nkeys = n - start;
  const int nsp = (nkeys + SPLIT - 1) / SPLIT;
  if (sp >= nsp) return;
  const int ks = start + sp * SPLIT;
  const int ke = min(ks + SPLIT, n);
  const int ws = ks + w * SUB;
  const int we = min(ws + SUB, ke);

  // ---- query operand: head slot hs = lane & 15 (zero beyond G), chunk 4s + (lane >> 4) ----
  const int hs = lane & 15, cg = lane >> 4;
  const bool hvalid = hs < G;
  bf16x8 qop[4];
  {
    const uint16_t* qr = (const uint16_t*)a.q + (int64_t)b * a.q_b +
                         (int64_t)(g * G + (hvalid ? hs : 0)) * a.q_h;
    float rs = 1.f;
    if (NORM) {
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        float x[8];
        unpack8(ld16(qr + 8 * c), x);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
      }
      rs = rsqrtf(ss * (1.0f / HD) + a.eps);
    }
    const uint16_t* qw = (const uint16_t*)a.qw;
    const int halfp = a.R >> 1;
    const int64_t tp = ROT ? min<int64_t>(max<int64_t>((int64_t)n - 1, 0), a.table_len - 1) : 0;
    const float* cr = ROT ? a.cos_t + tp * halfp : nullptr;
    const float* sr = ROT ? a.sin_t + tp * halfp : nullptr;
    const float qscale = a.scale * kLog2e;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int c = 4 * s + cg;
      float x[8];
      unpack8(ld16(qr + 8 * c), x);
      if (NORM) {
        float wv[8];
        unpack8(ld16(qw + 8 * c), wv);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= rs * wv[e];
      }
      if (ROT == 1 && 8 * c < a.R) {
        const int pc = c ^ (a.R >> 4);
        float y[8];
        unpack8(ld16(qr + 8 * pc), y);
        if (NORM) {
          float wv[8];
          unpack8(ld16(qw + 8 * pc), wv);
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] *= rs * wv[e];
        }
        rotate8<1>(x, y, c, a.R, cr, sr);
      } else if (ROT == 2) {
        rotate8<2>(x, x, c, a.R, cr, sr);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = hvalid ? x[e] * qscale : 0.f;
      qop[s] = as_bf16x8(pack8(x));
    }
  }

  const int64_t kv_base = (int64_t)b * a.k_b + (int64_t)g * a.k_h;
  const uint16_t* kbase = (const uint16_t*)a.k + kv_base;
  const uint16_t* vbase = (const uint16_t*)a.v + kv_base;
  uint16_t* vs = sm.v[w];

  f32x4 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m = kNegBig, lsum = 0.f;
  const float cap2 = a.softcap * kLog2e;
  const float inv_cap2 = CAP ? 1.0f / cap2 : 0.f;

  BlockRegs cur, nxt;
  if (ws < we) load_block(kbase, vbase, ws, we, cur);
  for (int kb0 = ws; kb0 < we; kb0 += KBLK) {
    const bool has_next = kb0 + KBLK < we;
    if (has_next) load_block(kbase, vbase, kb0 + KBLK, we, nxt);

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
        if (CAP) {
          const float y = x * inv_cap2;
          const float e = fast_exp2(-2.0f * kLog2e * fabsf(y));
          x = copysignf(cap2 * (1.0f - e) / (1.0f + e), y);
        }
        const int key = kb0 + kq * 16 + 4 * (lane >> 4) + r;
        sk[kq][r] = key < we ? x : -INFINITY;
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
    const bf16x8 pa = as_bf16x8(pack8(p));

    // O = P V: B operand = V[32 keys][16 features] via transposing LDS reads
    const int gi = lane >> 4, si = lane & 15;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int row1 = 4 * gi + (si >> 2);
      const int row2 = row1 + 16;
      const int col = 16 * db + 4 * (si & 3);
      const int off1 = row1 * HD + (((col >> 3) ^ (row1 & 15)) << 3) + (col & 7);
      const int off2 = row2 * HD + (((col >> 3) ^ (row2 & 15)) << 3) + (col & 7);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vs + off1));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vs + off2));
      const i16x8 vb = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(bf16x8, vb), o[db],
                                                      0, 0, 0);
    }
    if (has_next) cur = nxt;
  }

  // ---- merge the four wavefronts ----
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (lane < 16 && hvalid) {
    sm.mm[w][hs] = m;
    sm.ml[w][hs] = lsum;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * (lane >> 4) + r;
    if (row < G) {
#pragma unroll
      for (int db = 0; db < 8; ++db) sm.mo[w][row][16 * db + (lane & 15)] = o[db][r];
    }
  }
  __syncthreads();
  const int64_t item = (((int64_t)b * a.Hkv + g) * da.nsplit + sp) * G;
  for (int x = tid; x < G * HD; x += DT) {
    const int row = x / HD, d = x % HD;
    float M = kNegBig;
#pragma unroll
    for (int ww = 0; ww < DWAVES; ++ww) M = fmaxf(M, sm.mm[ww][row]);
    float acc = 0.f, lt = 0.f;
#pragma unroll
    for (int ww = 0; ww < DWAVES; ++ww) {
      const float sc = fast_exp2(sm.mm[ww][row] - M);
      acc += sc * sm.mo[ww][row][d];
      lt += sc * sm.ml[ww][row];
    }
    da.part_o[(item + row) * HD + d] = acc;
    if (d == 0) {
      da.part_ml[(item + row) * 2 + 0] = M;
      da.part_ml[(item + row) * 2 + 1] = lt;
    }
  }
}

// out[b, h, :] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over the splits of sequence b.
__global__ __launch_bounds__(HD) void decode_combine_kernel(DecodeArgs da) {
  const AttnArgs& a = da.a;
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int G = a.G, g = h / G, hs = h % G;
  const int n = min(max(a.lens[b], 0), a.S);
  const int start = a.window > 0 ? max(0, n - a.window) : 0;
  const int nsp = (n - start + SPLIT - 1) / SPLIT;
  const int64_t item0 = (((int64_t)b * a.Hkv + g) * da.nsplit) * G + hs;
  float M = kNegBig;
  for (int s = 0; s < nsp; ++s) M = fmaxf(M, da.part_ml[(item0 + (int64_t)s * G) * 2]);
  float acc = 0.f, lt = 0.f;
  for (int s = 0; s < nsp; ++s) {
    const int64_t it = item0 + (int64_t)s * G;
    const float sc = fast_exp2(da.part_ml[it * 2] - M);
    acc += sc * da.part_o[it * HD + d];
    lt += sc * da.part_ml[it * 2 + 1];
  }
  const float r = lt > 0.f ? acc / lt : 0.f;
  uint16_t* orow = (uint16_t*)a.out + (int64_t)b * a.o_b + (int64_t)h * a.o_h;
  orow[d] = f32_to_bf16(r);
}

template <int ROT, bool NORM, bool CAP>
hipError_t launch_variant(const DecodeArgs& d, hipStream_t stream) {
  const AttnArgs& a = d.a;
  dim3 grid(d.nsplit, a.Hkv, a.B);
  hipLaunchKernelGGL((decode_split_kernel<ROT, NORM, CAP>), grid, dim3(DT), 0, stream, d);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(a.Hq, a.B), dim3(HD), 0, stream, d);
  return hipGetLastError();
}
template <int ROT, bool NORM>
hipError_t launch_cap(const DecodeArgs& d, hipStream_t s) {
  return d.a.softcap > 0.f ? launch_variant<ROT, NORM, true>(d, s) : launch_variant<ROT, NORM, false>(d, s);
}
template <int ROT>
hipError_t launch_norm(const DecodeArgs& d, hipStream_t s) {
  return d.a.qk_norm ? launch_cap<ROT, true>(d, s) : launch_cap<ROT, false>(d, s);
}

}  // namespace

int decode_split_keys() { return SPLIT; }

bool decode_mfma_supported(const AttnArgs& a) {
  if (a.D != HD || a.G > MAXG) return false;
  if (a.R == 0) return true;
  if (a.style == 0) {
    const int P = a.R / 16;
    return a.R % 16 == 0 && (P == 1 || P == 2 || P == 4 || P == 8);
  }
  return a.R % 8 == 0;
}

size_t decode_mfma_workspace_bytes(int B, int Hkv, int G, int D, int Smax) {
  const int64_t nsplit = (Smax + SPLIT - 1) / SPLIT;
  const int64_t items = (int64_t)B * Hkv * nsplit * G;
  const size_t o = (size_t)items * D * sizeof(float);
  const size_t ml = (size_t)items * 2 * sizeof(float);
  return ((o + 255) & ~(size_t)255) + ml;
}

hipError_t launch_decode_mfma(const DecodeArgs& d, hipStream_t stream) {
  if (d.a.B == 0) return hipSuccess;
  const int rot = d.a.R == 0 ? 0 : (d.a.style == 0 ? 1 : 2);
  switch (rot) {
    case 0: return launch_norm<0>(d, stream);
    case 1: return launch_norm<1>(d, stream);
    default: return launch_norm<2>(d, stream);
  }
}

}  // namespace gqa
