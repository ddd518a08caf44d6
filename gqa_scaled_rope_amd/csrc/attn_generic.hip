// Generic rotary grouped-query attention kernel: one wavefront per (query row, query head).
//
// Covers every shape the ABI accepts (head_dim <= 256, any rotary width and pairing, any
// grouping, fp32 or bf16 storage) with fp32 arithmetic throughout.  The fp32 path runs here;
// bf16 problems run here only when the MFMA kernels do not cover their shape.
//
// Per row: the query is RMS-normed ([Guide] section 3.2) and rotated at its position ([Guide]
// section 4; [Models] "Serving it" for adjacent pairs), then scaled.  Keys in the band allowed
// by the causal/window/chunk mask ([Models] "Sliding windows"; chunks as in [Ster]'s llama4_text
// paragraph) are visited 64 at a time, one key per lane: new keys (index >= n_cached) are normed
// and rotated on the fly, cached keys are used as stored.  An online softmax (running max and
// sum, rescaled when the max grows) accumulates the values, one feature per lane; a learned sink
// adds its term to the final sum.
#include "launch.hpp"

namespace gqa {

template <typename T>
__device__ __forceinline__ float ldf(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ldf<float>(const float* p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float ldf<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}
template <typename T>
__device__ __forceinline__ void stf(T* p, int64_t i, float x);
template <>
__device__ __forceinline__ void stf<float>(float* p, int64_t i, float x) {
  p[i] = x;
}
template <>
__device__ __forceinline__ void stf<uint16_t>(uint16_t* p, int64_t i, float x) {
  p[i] = f32_to_bf16(x);
}

// First index j in [0, n) with key position >= x (key positions nondecreasing); identity when
// kp is null.
__device__ __forceinline__ int lower_bound_pos(const int32_t* kp, int n, int64_t x) {
  if (!kp) return (int)min<int64_t>(max<int64_t>(x, 0), n);
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if ((int64_t)kp[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

template <typename T>
__global__ __launch_bounds__(64) void attn_generic_kernel(AttnArgs a) {
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int g = h / a.G;
  const int D = a.D, R = a.R, half = a.R / 2;
  __shared__ float sq[256];
  __shared__ float sp[64];

  const int S = a.lens ? min(max(a.lens[b], 0), a.S) : a.S;
  const int64_t qp = a.qpos ? (int64_t)a.qpos[b * a.qpos_b + i] : (int64_t)S - 1;
  const int32_t* kp = a.kpos ? a.kpos + b * a.kpos_b : nullptr;
  const T* qrow = (const T*)a.q + b * a.q_b + i * a.q_i + h * a.q_h;
  const T* kbase = (const T*)a.k + b * a.k_b + g * a.k_h;
  const T* vbase = (const T*)a.v + b * a.k_b + g * a.k_h;
  const T* qw = (const T*)a.qw;
  const T* kw = (const T*)a.kw;

  // ---- query: norm, rotate, scale ----
  float ss = 0.f;
  for (int d = lane; d < D; d += 64) {
    float x = ldf(qrow, d);
    sq[d] = x;
    ss += x * x;
  }
  ss = wave_sum(ss);
  __syncthreads();
  if (a.qk_norm) {
    const float rs = rsqrtf(ss / D + a.eps);
    for (int d = lane; d < D; d += 64) sq[d] = sq[d] * rs * ldf(qw, d);
    __syncthreads();
  }
  if (half > 0) {
    const int64_t t = min<int64_t>(max<int64_t>(qp, 0), a.table_len - 1);
    for (int pi = lane; pi < half; pi += 64) {
      const float c = a.cos_t[t * half + pi], s = a.sin_t[t * half + pi];
      const int ix = a.style == 0 ? pi : 2 * pi, iy = a.style == 0 ? pi + half : 2 * pi + 1;
      const float x = sq[ix], y = sq[iy];
      sq[ix] = x * c - y * s;
      sq[iy] = x * s + y * c;
    }
    __syncthreads();
  }
  for (int d = lane; d < D; d += 64) sq[d] *= a.scale;
  __syncthreads();

  // ---- band of allowed keys ----
  const int hi = lower_bound_pos(kp, S, qp + 1);
  const bool floor_on = a.has_floor();
  const int64_t kfl = key_floor(a, qp);
  const int lo = floor_on ? lower_bound_pos(kp, S, kfl) : 0;

  float m = kNegBig, l = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = lo; j0 < hi; j0 += 64) {
    const int j = j0 + lane;
    bool valid = j < hi;
    int64_t kpj = 0;
    if (valid) {
      kpj = kp ? (int64_t)kp[j] : (int64_t)j;
      valid = kpj <= qp && (!floor_on || kpj >= kfl);
    }
    float s = -INFINITY;
    if (valid) {
      const T* kr = kbase + j * a.k_j;
      const bool prep = j >= a.n_cached;
      float rs = 1.f;
      if (prep && a.qk_norm) {
        float kss = 0.f;
        for (int d = 0; d < D; ++d) {
          const float x = ldf(kr, d);
          kss += x * x;
        }
        rs = rsqrtf(kss / D + a.eps);
      }
      auto kval = [&](int d) -> float {
        float x = ldf(kr, d);
        return (prep && a.qk_norm) ? x * rs * ldf(kw, d) : x;
      };
      float dot = 0.f;
      int d0 = 0;
      if (prep && half > 0) {
        const int64_t t = min<int64_t>(max<int64_t>(kpj, 0), a.table_len - 1);
        for (int pi = 0; pi < half; ++pi) {
          const float c = a.cos_t[t * half + pi], sn = a.sin_t[t * half + pi];
          const int ix = a.style == 0 ? pi : 2 * pi, iy = a.style == 0 ? pi + half : 2 * pi + 1;
          const float x = kval(ix), y = kval(iy);
          dot += sq[ix] * (x * c - y * sn) + sq[iy] * (x * sn + y * c);
        }
        d0 = R;
      }
      for (int d = d0; d < D; ++d) dot += sq[d] * kval(d);
      s = dot;
      if (a.softcap > 0.f) s = a.softcap * tanhf(s / a.softcap);
    }
    const float tmax = wave_max(s);
    const float m_new = fmaxf(m, tmax);
    const float alpha = expf(m - m_new);
    const float p = valid ? expf(s - m_new) : 0.f;
    l = l * alpha + wave_sum(p);
    sp[lane] = p;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] *= alpha;
    const int n = min(64, hi - j0);
    for (int jj = 0; jj < n; ++jj) {
      const float pj = sp[jj];
      if (pj == 0.f) continue;
      const T* vr = vbase + (int64_t)(j0 + jj) * a.k_j;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = lane + 64 * r;
        if (d < D) acc[r] += pj * ldf(vr, d);
      }
    }
    __syncthreads();
    m = m_new;
  }
  // a learned sink joins the denominator only ([Ster] gpt_oss paragraph)
  const float lt = (a.sinks != nullptr && l > 0.f) ? l + expf(a.sinks[h] - m) : l;
  const float inv = l > 0.f ? 1.f / lt : 0.f;
  T* orow = (T*)a.out + b * a.o_b + i * a.o_i + h * a.o_h;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int d = lane + 64 * r;
    if (d < D) stf(orow, d, acc[r] * inv);
  }
}

hipError_t launch_attn_generic(const AttnArgs& a, bool bf16, hipStream_t stream) {
  if (a.B == 0 || a.L == 0 || a.Hq == 0) return hipSuccess;
  dim3 grid(a.L, a.Hq, a.B);
  if (bf16)
    hipLaunchKernelGGL(attn_generic_kernel<uint16_t>, grid, dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_generic_kernel<float>, grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gqa
