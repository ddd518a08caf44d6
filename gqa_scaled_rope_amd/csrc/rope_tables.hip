// Rotary cos/sin tables ([Models] "Scaled RoPE", rope_tables): entry (p, i) holds
// a * cos(p * inv_freq[i]) and a * sin(p * inv_freq[i]), a the attention factor (1 unless the
// schedule is yarn or longrope).  The product, the sine/cosine and the scaling are evaluated
// in double precision (HIP's sincos, with its own argument reduction) and rounded once to fp32,
// so a table entry is the correctly rounded fp32 of the exact value to within one ulp even at
// positions of several hundred thousand.
#include "launch.hpp"

namespace gqa {

struct InvFreqArg {
  double f[kMaxPairs];
};

__global__ __launch_bounds__(256) void rope_tables_kernel(InvFreqArg inv, double attn, int half,
                                                          int64_t n,
                                                          float* __restrict__ cos_out,
                                                          float* __restrict__ sin_out) {
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t p = idx / half;
    const int i = (int)(idx - p * half);
    double s, c;
    sincos((double)p * inv.f[i], &s, &c);
    cos_out[idx] = (float)(attn * c);
    sin_out[idx] = (float)(attn * s);
  }
}

hipError_t launch_rope_tables(const double* inv_freq, double attention_factor, int half,
                              int table_len, float* cos_out, float* sin_out, hipStream_t stream) {
  InvFreqArg arg;
  for (int i = 0; i < kMaxPairs; ++i) arg.f[i] = i < half ? inv_freq[i] : 0.0;
  const int64_t n = (int64_t)table_len * half;
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(rope_tables_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, arg,
                     attention_factor, half, n, cos_out, sin_out);
  return hipGetLastError();
}

}  // namespace gqa
