// C-ABI of libgqa_rope: argument validation, the rotary frequency schedule, and kernel dispatch.
// Declarations and the contract of every entry point are in include/gqa_rope.h.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "gqa_rope.h"
#include "launch.hpp"

static_assert(GQA_DECODE_NOALLOC_MAX_BYTES == gqa::kDecodeScratchBytes,
              "the header states the scratch size the library holds");

namespace {

thread_local std::string g_err;

gqa_status fail(gqa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

gqa_status ok() {
  g_err.clear();
  return GQA_OK;
}

gqa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(GQA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool finite_nonneg(double x) { return std::isfinite(x) && x >= 0.0; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool finite_pos(double x) { return std::isfinite(x) && x > 0.0; }

// Frequencies of the rotated feature pairs ([Models] "Scaled RoPE", rope_inv_freq):
// base_i = theta^(-2i/R); linear divides by factor; llama3 keeps pairs with wavelength below
// original/high_freq_factor, divides pairs with wavelength above original/low_freq_factor by
// factor, and between them blends the two linearly in original/wavelength.  yarn makes the same
// split by rotation counts over the original context, with a ramp over the pair index; longrope
// ([Ster] "Overview") divides by a per-pair table chosen by the sequence length.
gqa_status check_rope(const gqa_rope_params* rp) {
  if (!rp) return fail(GQA_E_NULL, "rope params pointer is null");
  if (rp->rotary_dim < 0 || rp->rotary_dim % 2 || rp->rotary_dim > 2 * gqa::kMaxPairs)
    return fail(GQA_E_SHAPE, "rotary_dim must be even and in [0, %d], got %d", 2 * gqa::kMaxPairs,
                rp->rotary_dim);
  if (!(std::isfinite(rp->theta) && rp->theta > 0.0))
    return fail(GQA_E_VALUE, "rope theta must be finite and > 0, got %g", rp->theta);
  switch (rp->kind) {
    case GQA_ROPE_DEFAULT:
      break;
    case GQA_ROPE_LINEAR:
      if (!(std::isfinite(rp->factor) && rp->factor > 0.0))
        return fail(GQA_E_VALUE, "linear rope factor must be > 0, got %g", rp->factor);
      break;
    case GQA_ROPE_LLAMA3:
      if (!(std::isfinite(rp->factor) && rp->factor > 0.0))
        return fail(GQA_E_VALUE, "llama3 rope factor must be > 0, got %g", rp->factor);
      if (!(rp->low_freq_factor > 0.0 && rp->high_freq_factor > rp->low_freq_factor &&
            std::isfinite(rp->high_freq_factor)))
        return fail(GQA_E_VALUE, "llama3 needs 0 < low_freq_factor < high_freq_factor, got %g, %g",
                    rp->low_freq_factor, rp->high_freq_factor);
      if (!(std::isfinite(rp->original_max_pos) && rp->original_max_pos > 0.0))
        return fail(GQA_E_VALUE, "llama3 original_max_pos must be > 0, got %g", rp->original_max_pos);
      break;
    case GQA_ROPE_YARN: {
      if (!finite_pos(rp->factor))
        return fail(GQA_E_VALUE, "yarn rope factor must be > 0, got %g", rp->factor);
      if (!finite_pos(rp->original_max_pos))
        return fail(GQA_E_VALUE, "yarn original_max_pos must be > 0, got %g", rp->original_max_pos);
      const double bf = rp->beta_fast != 0.0 ? rp->beta_fast : 32.0;
      const double bs = rp->beta_slow != 0.0 ? rp->beta_slow : 1.0;
      if (!(finite_pos(bf) && finite_pos(bs) && bf > bs))
        return fail(GQA_E_VALUE, "yarn needs beta_fast > beta_slow > 0, got %g, %g", bf, bs);
      if (!finite_nonneg(rp->mscale) || !finite_nonneg(rp->mscale_all_dim))
        return fail(GQA_E_VALUE, "yarn mscale and mscale_all_dim must be finite and >= 0");
      if (!finite_nonneg(rp->attention_factor))
        return fail(GQA_E_VALUE, "attention_factor must be finite and >= 0, got %g",
                    rp->attention_factor);
      break;
    }
    case GQA_ROPE_LONGROPE: {
      if (!finite_pos(rp->original_max_pos))
        return fail(GQA_E_VALUE, "longrope original_max_pos must be > 0, got %g",
                    rp->original_max_pos);
      if (!finite_nonneg(rp->attention_factor))
        return fail(GQA_E_VALUE, "attention_factor must be finite and >= 0, got %g",
                    rp->attention_factor);
      if (rp->seq_len < 0) return fail(GQA_E_VALUE, "longrope seq_len must be >= 0");
      const bool use_long = (double)rp->seq_len > rp->original_max_pos;
      const double* table = use_long ? rp->long_factor : rp->short_factor;
      if (rp->rotary_dim > 0 && !table)
        return fail(GQA_E_NULL, "longrope needs the %s_factor table", use_long ? "long" : "short");
      for (int i = 0; i < rp->rotary_dim / 2; ++i)
        if (!finite_pos(table[i]))
          return fail(GQA_E_VALUE, "longrope factor %d must be finite and > 0, got %g", i,
                      table[i]);
      break;
    }
    default:
      return fail(GQA_E_UNSUPPORTED, "unknown rope kind %d (0 default, 1 linear, 2 llama3, 3 yarn, "
                  "4 longrope)", rp->kind);
  }
  if (rp->reserved != 0) return fail(GQA_E_VALUE, "rope params reserved field must be 0");
  return ok();
}

// YaRN's sharpening ([Models] "Scaled RoPE"): 0.1 * m * ln(s) + 1, 1 for s <= 1.
double yarn_mscale(double s, double m) { return s <= 1.0 ? 1.0 : 0.1 * m * std::log(s) + 1.0; }

// Factor multiplying cos and sin: yarn's given or derived one, longrope's given one or 1.
double attention_factor_host(const gqa_rope_params* rp) {
  if (rp->kind == GQA_ROPE_YARN) {
    if (rp->attention_factor > 0.0) return rp->attention_factor;
    if (rp->mscale > 0.0 && rp->mscale_all_dim > 0.0)
      return yarn_mscale(rp->factor, rp->mscale) / yarn_mscale(rp->factor, rp->mscale_all_dim);
    return yarn_mscale(rp->factor, 1.0);
  }
  if (rp->kind == GQA_ROPE_LONGROPE && rp->attention_factor > 0.0) return rp->attention_factor;
  return 1.0;
}

void inv_freq_host(const gqa_rope_params* rp, double* out) {
  const int R = rp->rotary_dim;
  const double two_pi = 6.283185307179586476925286766559;
  // yarn: pair index i turns original * theta^(-2i/R) / (2 pi) times over the original context,
  // fewer as i grows.  The ramp starts at the last index still turning beta_fast times and ends at
  // the first one turning at most beta_slow times (walked index by index over 0 .. R-1), or, with
  // yarn_no_truncate, at the fractional indices where the turn count equals each beta.
  double ramp_a = 0.0, ramp_b = 0.0;
  if (rp->kind == GQA_ROPE_YARN) {
    const double orig = rp->original_max_pos;
    const double fast = rp->beta_fast != 0.0 ? rp->beta_fast : 32.0;
    const double slow = rp->beta_slow != 0.0 ? rp->beta_slow : 1.0;
    auto turns_at = [&](double i) { return orig * std::pow(rp->theta, -2.0 * i / R) / two_pi; };
    if (!rp->yarn_no_truncate) {
      int a = 0;
      while (a + 1 <= R - 1 && turns_at(a + 1) >= fast) ++a;
      int b = 0;
      while (b < R - 1 && turns_at(b) > slow) ++b;
      ramp_a = a;
      ramp_b = b;
    } else {
      const double per_index = 2.0 * std::log(rp->theta) / R;  // ln(turns) drop per index
      ramp_a = std::max(std::log(turns_at(0) / fast) / per_index, 0.0);
      ramp_b = std::min(std::log(turns_at(0) / slow) / per_index, (double)(R - 1));
    }
  }
  const double* table = nullptr;
  if (rp->kind == GQA_ROPE_LONGROPE)
    table = (double)rp->seq_len > rp->original_max_pos ? rp->long_factor : rp->short_factor;
  for (int i = 0; i < R / 2; ++i) {
    const double base = std::pow(rp->theta, -2.0 * i / R);
    double f = base;
    if (rp->kind == GQA_ROPE_LINEAR) {
      f = base / rp->factor;
    } else if (rp->kind == GQA_ROPE_LLAMA3) {
      const double wavelength = two_pi / base;
      const double old = rp->original_max_pos;
      if (wavelength < old / rp->high_freq_factor) {
        f = base;
      } else if (wavelength > old / rp->low_freq_factor) {
        f = base / rp->factor;
      } else {
        const double s = (old / wavelength - rp->low_freq_factor) /
                         (rp->high_freq_factor - rp->low_freq_factor);
        f = (1.0 - s) * base / rp->factor + s * base;
      }
    } else if (rp->kind == GQA_ROPE_YARN) {
      // weight of the divided frequency: 0 up to the ramp's start, 1 from its end; where the two
      // ends meet, a step just after them
      const double w = ramp_b > ramp_a ? std::min(std::max((i - ramp_a) / (ramp_b - ramp_a), 0.0), 1.0)
                                       : (i > ramp_a ? 1.0 : 0.0);
      f = base * (1.0 - w) + (base / rp->factor) * w;
    } else if (rp->kind == GQA_ROPE_LONGROPE) {
      f = base / table[i];
    }
    out[i] = f;
  }
}

gqa_status check_cfg(const gqa_attn_cfg* c) {
  if (!c) return fail(GQA_E_NULL, "cfg pointer is null");
  if (c->dtype != GQA_F32 && c->dtype != GQA_BF16)
    return fail(GQA_E_DTYPE, "dtype must be GQA_F32 (0) or GQA_BF16 (1), got %d", c->dtype);
  if (c->head_dim < 8 || c->head_dim > 256 || c->head_dim % 8)
    return fail(GQA_E_SHAPE, "head_dim must be a multiple of 8 in [8, 256], got %d", c->head_dim);
  if (c->num_q_heads < 1 || c->num_kv_heads < 1)
    return fail(GQA_E_SHAPE, "num_q_heads and num_kv_heads must be >= 1, got %d, %d",
                c->num_q_heads, c->num_kv_heads);
  if (c->num_q_heads % c->num_kv_heads)
    return fail(GQA_E_SHAPE, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)",
                c->num_q_heads, c->num_kv_heads);
  if (c->num_q_heads > 65535) return fail(GQA_E_SHAPE, "num_q_heads must be <= 65535");
  if (c->rotary_dim < 0 || c->rotary_dim % 2 || c->rotary_dim > c->head_dim)
    return fail(GQA_E_SHAPE, "rotary_dim must be even and in [0, head_dim=%d], got %d",
                c->head_dim, c->rotary_dim);
  if (c->rot_style != GQA_ROT_HALF && c->rot_style != GQA_ROT_INTERLEAVED)
    return fail(GQA_E_VALUE, "rot_style must be GQA_ROT_HALF (0) or GQA_ROT_INTERLEAVED (1), got %d",
                c->rot_style);
  if (c->rotary_dim > 0) {
    if (!c->cos_table || !c->sin_table)
      return fail(GQA_E_NULL, "cos_table/sin_table are required when rotary_dim > 0");
    if (!aligned16(c->cos_table) || !aligned16(c->sin_table))
      return fail(GQA_E_VALUE, "cos_table/sin_table must be 16-byte aligned");
    if (c->table_len < 1) return fail(GQA_E_SHAPE, "table_len must be >= 1, got %d", c->table_len);
  }
  if (c->qk_norm != 0 && c->qk_norm != 1)
    return fail(GQA_E_VALUE, "qk_norm must be 0 or 1, got %d", c->qk_norm);
  if (c->qk_norm) {
    if (!c->q_norm_w || !c->k_norm_w)
      return fail(GQA_E_NULL, "q_norm_w and k_norm_w are required when qk_norm is set");
    if (!aligned16(c->q_norm_w) || !aligned16(c->k_norm_w))
      return fail(GQA_E_VALUE, "q_norm_w/k_norm_w must be 16-byte aligned");
    if (!finite_nonneg(c->eps)) return fail(GQA_E_VALUE, "eps must be finite and >= 0, got %g", c->eps);
  }
  if (!finite_nonneg(c->scale)) return fail(GQA_E_VALUE, "scale must be finite and >= 0, got %g", c->scale);
  if (!finite_nonneg(c->softcap))
    return fail(GQA_E_VALUE, "softcap must be finite and >= 0, got %g", c->softcap);
  if (((uintptr_t)c->sinks & 3u) != 0) return fail(GQA_E_VALUE, "sinks must be 4-byte aligned");
  if (c->chunk_size < 0 || c->chunk_lookback < 0)
    return fail(GQA_E_SHAPE, "chunk_size and chunk_lookback must be >= 0, got %d, %d",
                c->chunk_size, c->chunk_lookback);
  if (c->kernel < GQA_KERNEL_AUTO || c->kernel > GQA_KERNEL_PREFILL_SHORT)
    return fail(GQA_E_VALUE, "kernel must be a gqa_kernel_select value in [0, 5], got %d", c->kernel);
  if (c->reserved != 0) return fail(GQA_E_VALUE, "cfg reserved field must be 0");
  return ok();
}

gqa::AttnArgs base_args(const gqa_attn_cfg* c) {
  gqa::AttnArgs a{};
  a.Hq = c->num_q_heads;
  a.Hkv = c->num_kv_heads;
  a.G = c->num_q_heads / c->num_kv_heads;
  a.D = c->head_dim;
  a.R = c->rotary_dim;
  a.style = c->rot_style;
  a.qk_norm = c->qk_norm;
  a.eps = (float)c->eps;
  a.qw = c->q_norm_w;
  a.kw = c->k_norm_w;
  a.cos_t = c->cos_table;
  a.sin_t = c->sin_table;
  a.table_len = c->table_len;
  a.scale = (float)(c->scale > 0.0 ? c->scale : 1.0 / std::sqrt((double)c->head_dim));
  a.softcap = (float)c->softcap;
  a.sinks = c->sinks;
  gqa::set_chunk(a, c->chunk_size, c->chunk_lookback);
  return a;
}

}  // namespace

extern "C" {

const char* gqa_last_error(void) { return g_err.c_str(); }

const char* gqa_version(void) { return "gqa_rope 0.1.0 (gfx950)"; }

gqa_status gqa_rope_inv_freq(const gqa_rope_params* rope, double* inv_freq_out) {
  gqa_status st = check_rope(rope);
  if (st != GQA_OK) return st;
  if (rope->rotary_dim > 0 && !inv_freq_out) return fail(GQA_E_NULL, "inv_freq_out is null");
  inv_freq_host(rope, inv_freq_out);
  return ok();
}

gqa_status gqa_rope_attention_factor(const gqa_rope_params* rope, double* out) {
  gqa_status st = check_rope(rope);
  if (st != GQA_OK) return st;
  if (!out) return fail(GQA_E_NULL, "out is null");
  *out = attention_factor_host(rope);
  return ok();
}

gqa_status gqa_rope_softmax_scale(const gqa_rope_params* rope, int32_t qk_dim, double* out) {
  gqa_status st = check_rope(rope);
  if (st != GQA_OK) return st;
  if (!out) return fail(GQA_E_NULL, "out is null");
  if (qk_dim < 1) return fail(GQA_E_SHAPE, "qk_dim must be >= 1, got %d", qk_dim);
  double sc = 1.0 / std::sqrt((double)qk_dim);
  if (rope->kind == GQA_ROPE_YARN && rope->mscale_all_dim > 0.0) {
    const double m = yarn_mscale(rope->factor, rope->mscale_all_dim);
    sc *= m * m;
  }
  *out = sc;
  return ok();
}

gqa_status gqa_rope_tables(const gqa_rope_params* rope, int32_t table_len, float* cos_out,
                           float* sin_out, hipStream_t stream) {
  gqa_status st = check_rope(rope);
  if (st != GQA_OK) return st;
  if (table_len < 1) return fail(GQA_E_SHAPE, "table_len must be >= 1, got %d", table_len);
  if (rope->rotary_dim == 0) return ok();
  if (!cos_out || !sin_out) return fail(GQA_E_NULL, "cos_out/sin_out are null");
  double f[gqa::kMaxPairs];
  inv_freq_host(rope, f);
  return hip_status(gqa::launch_rope_tables(f, attention_factor_host(rope), rope->rotary_dim / 2,
                                            table_len, cos_out, sin_out, stream),
                    "rope_tables launch");
}

static gqa::AttnArgs prefill_args(const gqa_attn_cfg* cfg, int32_t B, int32_t L, int32_t S,
                                  int32_t n_cached) {
  gqa::AttnArgs a = base_args(cfg);
  const int64_t D = cfg->head_dim;
  a.q_h = D;
  a.q_i = (int64_t)a.Hq * D;
  a.q_b = (int64_t)L * a.q_i;
  a.o_h = a.q_h;
  a.o_i = a.q_i;
  a.o_b = a.q_b;
  a.k_h = D;
  a.k_j = (int64_t)a.Hkv * D;
  a.k_b = (int64_t)S * a.k_j;
  a.B = B;
  a.L = L;
  a.S = S;
  a.n_cached = n_cached;
  return a;
}

// Stream path (key preparation pass + streaming attention) applies to bf16 MFMA shapes; it needs
// workspace only when some keys must be normed or rotated.
static bool prefill_stream_applies(const gqa_attn_cfg* cfg, const gqa::AttnArgs& a) {
  gqa::AttnArgs t = a;
  // support checks look at the position pointers; any non-null stand-in will do here
  static const int32_t dummy = 0;
  t.qpos = &dummy;
  t.kpos = &dummy;
  return cfg->dtype == GQA_BF16 && cfg->kernel != GQA_KERNEL_GENERIC && a.S > 0 &&
         gqa::prefill_stream_supported(t);
}

static gqa::StreamKernel stream_kernel(const gqa_attn_cfg* cfg) {
  return cfg->kernel == GQA_KERNEL_PREFILL_LONG    ? gqa::StreamKernel::kLong
         : cfg->kernel == GQA_KERNEL_PREFILL_SHORT ? gqa::StreamKernel::kShort
                                                   : gqa::StreamKernel::kAuto;
}

size_t gqa_prefill_workspace_bytes(const gqa_attn_cfg* cfg, int32_t B, int32_t S, int32_t n_cached) {
  if (check_cfg(cfg) != GQA_OK) return 0;
  if (B < 0 || S < 0 || n_cached < 0 || n_cached > S) {
    fail(GQA_E_SHAPE, "need B >= 0 and 0 <= n_cached <= S, got B=%d S=%d n_cached=%d", B, S,
         n_cached);
    return 0;
  }
  gqa::AttnArgs a = prefill_args(cfg, B, 1, S, n_cached);
  if (!prefill_stream_applies(cfg, a)) return 0;
  const size_t n = gqa::prefill_stream_workspace_bytes(a);
  return (n + 255) & ~(size_t)255;
}

gqa_status gqa_attn_prefill(const gqa_attn_cfg* cfg, const void* q, const void* k, const void* v,
                            const int32_t* positions, int64_t pos_batch_stride,
                            const int32_t* key_positions, int64_t kpos_batch_stride, int32_t B,
                            int32_t L, int32_t S, int32_t n_cached, int32_t window, void* out,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  gqa_status st = check_cfg(cfg);
  if (st != GQA_OK) return st;
  if (B < 0 || L < 0 || S < 0)
    return fail(GQA_E_SHAPE, "B, L, S must be >= 0, got %d, %d, %d", B, L, S);
  if (B > 65535) return fail(GQA_E_SHAPE, "B must be <= 65535, got %d", B);
  if (n_cached < 0 || n_cached > S)
    return fail(GQA_E_SHAPE, "n_cached must be in [0, S=%d], got %d", S, n_cached);
  if (window < 0) return fail(GQA_E_SHAPE, "window must be >= 0, got %d", window);
  if (pos_batch_stride < 0 || kpos_batch_stride < 0)
    return fail(GQA_E_SHAPE, "position batch strides must be >= 0");
  if (B == 0 || L == 0) return ok();
  if (!q || !out || !positions) return fail(GQA_E_NULL, "q, out and positions are required");
  if (S > 0 && (!k || !v || !key_positions))
    return fail(GQA_E_NULL, "k, v and key_positions are required when S > 0");
  if (!aligned16(q) || !aligned16(out) || (S > 0 && (!aligned16(k) || !aligned16(v))))
    return fail(GQA_E_VALUE, "q, k, v and out must be 16-byte aligned");
  if ((int64_t)L * cfg->num_q_heads > INT32_MAX)
    return fail(GQA_E_SHAPE, "L * num_q_heads exceeds 2^31");
  if (workspace_bytes > 0 && !workspace)
    return fail(GQA_E_WORKSPACE, "workspace is null but workspace_bytes is %zu", workspace_bytes);
  if (workspace && ((uintptr_t)workspace & 255u) != 0)
    return fail(GQA_E_WORKSPACE, "workspace must be 256-byte aligned");
  gqa::AttnArgs a = prefill_args(cfg, B, L, S, n_cached);
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.qpos = positions;
  a.qpos_b = pos_batch_stride;
  a.kpos = key_positions;
  a.kpos_b = kpos_batch_stride;
  a.lens = nullptr;
  a.window = window;
  const bool bf16 = cfg->dtype == GQA_BF16;
  if (prefill_stream_applies(cfg, a)) {
    const size_t need = gqa::prefill_stream_required_bytes(a);
    if (need == 0 || (workspace && workspace_bytes >= need))
      return hip_status(gqa::launch_prefill_stream(a, workspace, workspace ? workspace_bytes : 0,
                                                   stream, stream_kernel(cfg)),
                        "prefill (stream) launch");
    if (workspace)
      return fail(GQA_E_WORKSPACE, "prefill workspace needs %zu bytes, got %zu", need,
                  workspace_bytes);
  }
  if (bf16 && cfg->kernel != GQA_KERNEL_GENERIC && S > 0 && gqa::prefill_mfma_supported(a))
    return hip_status(gqa::launch_prefill_mfma(a, stream), "prefill (fused) launch");
  return hip_status(gqa::launch_attn_generic(a, bf16, stream), "prefill (generic) launch");
}

gqa_status gqa_prefill_kernel(const gqa_attn_cfg* cfg, int32_t B, int32_t L, int32_t S,
                              int32_t n_cached, int32_t window, int32_t with_workspace,
                              int32_t* which) {
  gqa_status st = check_cfg(cfg);
  if (st != GQA_OK) return st;
  if (which == nullptr) return fail(GQA_E_NULL, "which must not be null");
  if (B < 0 || L < 0 || S < 0 || n_cached < 0 || n_cached > S || window < 0)
    return fail(GQA_E_SHAPE, "need B, L, S, window >= 0 and 0 <= n_cached <= S, got B=%d L=%d "
                "S=%d n_cached=%d window=%d", B, L, S, n_cached, window);
  gqa::AttnArgs a = prefill_args(cfg, B, L, S, n_cached);
  a.window = window;
  static const int32_t dummy = 0;  // the support checks look at the position pointers only
  a.qpos = &dummy;
  a.kpos = &dummy;
  const bool bf16 = cfg->dtype == GQA_BF16;
  if (prefill_stream_applies(cfg, a) &&
      (gqa::prefill_stream_required_bytes(a) == 0 || with_workspace)) {
    *which = gqa::prefill_stream_short(a, stream_kernel(cfg)) ? GQA_PREFILL_STREAM_SHORT
                                                              : GQA_PREFILL_STREAM_LONG;
  } else if (bf16 && cfg->kernel != GQA_KERNEL_GENERIC && S > 0 && gqa::prefill_mfma_supported(a)) {
    *which = GQA_PREFILL_FUSED;
  } else {
    *which = GQA_PREFILL_GENERIC;
  }
  return ok();
}

gqa_status gqa_prep_keys(const gqa_attn_cfg* cfg, const void* k, const int32_t* key_positions,
                         int64_t kpos_batch_stride, int32_t B, int32_t S, int32_t n_cached,
                         void* k_out, hipStream_t stream) {
  gqa_status st = check_cfg(cfg);
  if (st != GQA_OK) return st;
  if (B < 0 || S < 0 || n_cached < 0 || n_cached > S)
    return fail(GQA_E_SHAPE, "need B >= 0 and 0 <= n_cached <= S, got B=%d S=%d n_cached=%d", B,
                S, n_cached);
  if (B > 65535) return fail(GQA_E_SHAPE, "B must be <= 65535, got %d", B);
  if (kpos_batch_stride < 0) return fail(GQA_E_SHAPE, "kpos_batch_stride must be >= 0");
  gqa::AttnArgs a = prefill_args(cfg, B, 1, S, n_cached);
  if (cfg->dtype != GQA_BF16 || !gqa::prep_keys_supported(a))
    return fail(GQA_E_UNSUPPORTED, "prep_keys covers bf16 with head_dim 128 and the MFMA rotary "
                "widths only");
  if (B == 0 || S == n_cached) return ok();
  if (!k || !k_out || !key_positions) return fail(GQA_E_NULL, "k, key_positions and k_out are required");
  if (!aligned16(k) || !aligned16(k_out)) return fail(GQA_E_VALUE, "k and k_out must be 16-byte aligned");
  a.k = k;
  a.kpos = key_positions;
  a.kpos_b = kpos_batch_stride;
  return hip_status(gqa::launch_prep_keys(a, k_out, stream), "prep_keys launch");
}

// Decode split-size choice of a call: automatic, or forced by the kernel selector.
static gqa::SplitMode decode_split_mode(const gqa_attn_cfg* cfg) {
  return cfg->kernel == GQA_KERNEL_DECODE_SHORT  ? gqa::SplitMode::kShort
         : cfg->kernel == GQA_KERNEL_DECODE_LONG ? gqa::SplitMode::kLong
                                                 : gqa::SplitMode::kAuto;
}

static bool decode_uses_mfma(const gqa_attn_cfg* cfg) {
  gqa::AttnArgs a = base_args(cfg);
  return cfg->dtype == GQA_BF16 && cfg->kernel != GQA_KERNEL_GENERIC &&
         gqa::decode_mfma_supported(a);
}

size_t gqa_decode_workspace_bytes(const gqa_attn_cfg* cfg, int32_t B, int32_t Smax) {
  if (check_cfg(cfg) != GQA_OK) return 0;
  if (B < 0 || Smax < 1) {
    fail(GQA_E_SHAPE, "B must be >= 0 and Smax >= 1, got %d, %d", B, Smax);
    return 0;
  }
  if (!decode_uses_mfma(cfg)) return 0;
  return gqa::decode_mfma_workspace_bytes(B, cfg->num_kv_heads,
                                          cfg->num_q_heads / cfg->num_kv_heads, cfg->head_dim,
                                          Smax);
}

// gqa_attn_decode, with the split partials either in the caller's workspace or, for the entry
// point that allocates nothing (noalloc), in the library's fixed per-GPU scratch array.
static gqa_status decode_impl(const gqa_attn_cfg* cfg, const void* q, const void* kcache,
                              const void* vcache, const int32_t* lens, int32_t B, int32_t Smax,
                              int32_t window, void* out, void* workspace, size_t workspace_bytes,
                              hipStream_t stream, bool noalloc) {
  gqa_status st = check_cfg(cfg);
  if (st != GQA_OK) return st;
  if (B < 0 || Smax < 1) return fail(GQA_E_SHAPE, "B must be >= 0 and Smax >= 1, got %d, %d", B, Smax);
  if (B > 65535) return fail(GQA_E_SHAPE, "B must be <= 65535, got %d", B);
  if (window < 0) return fail(GQA_E_SHAPE, "window must be >= 0, got %d", window);
  if (B == 0) return ok();
  if (!q || !kcache || !vcache || !lens || !out)
    return fail(GQA_E_NULL, "q, kcache, vcache, lens and out are required");
  if (!aligned16(q) || !aligned16(kcache) || !aligned16(vcache) || !aligned16(out))
    return fail(GQA_E_VALUE, "q, kcache, vcache and out must be 16-byte aligned");
  gqa::AttnArgs a = base_args(cfg);
  const int64_t D = cfg->head_dim;
  a.q = q;
  a.k = kcache;
  a.v = vcache;
  a.out = out;
  a.q_h = D;
  a.q_i = 0;
  a.q_b = (int64_t)a.Hq * D;
  a.o_h = D;
  a.o_i = 0;
  a.o_b = a.q_b;
  a.k_j = D;
  a.k_h = (int64_t)Smax * D;
  a.k_b = (int64_t)a.Hkv * a.k_h;
  a.qpos = nullptr;
  a.kpos = nullptr;
  a.lens = lens;
  a.B = B;
  a.L = 1;
  a.S = Smax;
  a.n_cached = Smax;  // every cache row is used as stored
  a.window = window;
  if (decode_uses_mfma(cfg)) {
    const size_t need =
        gqa::decode_mfma_workspace_bytes(B, a.Hkv, a.G, cfg->head_dim, Smax);
    if (noalloc) {
      if (need > GQA_DECODE_NOALLOC_MAX_BYTES)
        return fail(GQA_E_WORKSPACE, "decode of B=%d sequences with Smax=%d needs %zu bytes of "
                    "scratch, more than the %zu of the no-allocation entry point; call "
                    "gqa_attn_decode with a workspace", B, Smax, need,
                    (size_t)GQA_DECODE_NOALLOC_MAX_BYTES);
      hipError_t e = gqa::decode_scratch(&workspace);
      if (e != hipSuccess) return hip_status(e, "decode scratch address");
      workspace_bytes = GQA_DECODE_NOALLOC_MAX_BYTES;
    }
    if (!workspace || workspace_bytes < need)
      return fail(GQA_E_WORKSPACE, "decode needs a workspace of %zu bytes, got %zu%s", need,
                  workspace_bytes, workspace ? "" : " (null)");
    if (((uintptr_t)workspace & 255u) != 0)
      return fail(GQA_E_WORKSPACE, "workspace must be 256-byte aligned");
    return hip_status(gqa::launch_decode_mfma(a, workspace, stream, nullptr, decode_split_mode(cfg)),
                      "decode (mfma) launch");
  }
  return hip_status(gqa::launch_attn_generic(a, cfg->dtype == GQA_BF16, stream),
                    "decode (generic) launch");
}

gqa_status gqa_attn_decode(const gqa_attn_cfg* cfg, const void* q, const void* kcache,
                           const void* vcache, const int32_t* lens, int32_t B, int32_t Smax,
                           int32_t window, void* out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  return decode_impl(cfg, q, kcache, vcache, lens, B, Smax, window, out, workspace,
                     workspace_bytes, stream, false);
}

gqa_status gqa_attn_decode_noalloc(const gqa_attn_cfg* cfg, const void* q, const void* kcache,
                                   const void* vcache, const int32_t* lens, int32_t B,
                                   int32_t Smax, int32_t window, void* out, hipStream_t stream) {
  return decode_impl(cfg, q, kcache, vcache, lens, B, Smax, window, out, nullptr, 0, stream, true);
}

static gqa_status check_paged(const gqa_attn_cfg* cfg, const gqa_paged_kv* kv, gqa::PagedKV* out) {
  if (!kv) return fail(GQA_E_NULL, "paged kv pointer is null");
  if (!kv->k_pool || !kv->v_pool || !kv->block_table)
    return fail(GQA_E_NULL, "k_pool, v_pool and block_table are required");
  if (!aligned16(kv->k_pool) || !aligned16(kv->v_pool))
    return fail(GQA_E_VALUE, "k_pool and v_pool must be 16-byte aligned");
  const int bs = kv->block_size;
  if (bs < 16 || bs > 1024 || (bs & (bs - 1)))
    return fail(GQA_E_VALUE, "block_size must be a power of two in [16, 1024], got %d", bs);
  if (kv->max_blocks < 1 || kv->num_blocks < 1)
    return fail(GQA_E_SHAPE, "max_blocks and num_blocks must be >= 1, got %d, %d", kv->max_blocks,
                kv->num_blocks);
  if ((int64_t)kv->max_blocks * bs * cfg->head_dim * 2 > INT32_MAX)
    return fail(GQA_E_SHAPE, "max_blocks * block_size is too large (%d * %d)", kv->max_blocks, bs);
  if (kv->reserved != 0) return fail(GQA_E_VALUE, "paged kv reserved field must be 0");
  if (cfg->dtype != GQA_BF16 || cfg->head_dim != 128)
    return fail(GQA_E_UNSUPPORTED, "the paged pool takes bf16 with head_dim 128");
  out->table = kv->block_table;
  out->max_blocks = kv->max_blocks;
  int l2 = 0;
  while ((1 << l2) < bs) ++l2;
  out->log2bs = l2;
  out->num_blocks = kv->num_blocks;
  return ok();
}

gqa_status gqa_paged_append(const gqa_attn_cfg* cfg, const gqa_paged_kv* kv, const void* k_new,
                            const void* v_new, const int32_t* key_positions,
                            int64_t kpos_batch_stride, const int32_t* start, int32_t B, int32_t L,
                            hipStream_t stream) {
  gqa_status st = check_cfg(cfg);
  if (st != GQA_OK) return st;
  gqa::PagedKV pk;
  st = check_paged(cfg, kv, &pk);
  if (st != GQA_OK) return st;
  if (B < 0 || L < 0) return fail(GQA_E_SHAPE, "B and L must be >= 0, got %d, %d", B, L);
  if (B > 65535) return fail(GQA_E_SHAPE, "B must be <= 65535, got %d", B);
  if ((int64_t)L * cfg->num_kv_heads > INT32_MAX / 8)
    return fail(GQA_E_SHAPE, "L * num_kv_heads is too large");
  if (kpos_batch_stride < 0) return fail(GQA_E_SHAPE, "kpos_batch_stride must be >= 0");
  gqa::AttnArgs a = base_args(cfg);
  if (!gqa::prep_keys_supported(a))
    return fail(GQA_E_UNSUPPORTED, "paged append covers the rotary widths of gqa_prep_keys");
  if (B == 0 || L == 0) return ok();
  if (!k_new || !v_new || !start || (cfg->rotary_dim > 0 && !key_positions))
    return fail(GQA_E_NULL, "k_new, v_new, start and (with rotation) key_positions are required");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(GQA_E_VALUE, "k_new and v_new must be 16-byte aligned");
  const int64_t D = cfg->head_dim;
  a.k = k_new;
  a.v = v_new;
  a.k_h = D;
  a.k_j = (int64_t)a.Hkv * D;
  a.k_b = (int64_t)L * a.k_j;
  a.kpos = key_positions;
  a.kpos_b = kpos_batch_stride;
  a.B = B;
  a.L = L;
  a.S = L;
  a.n_cached = 0;
  return hip_status(gqa::launch_paged_append(a, pk, kv->k_pool, kv->v_pool, start, stream),
                    "paged append launch");
}

size_t gqa_paged_decode_workspace_bytes(const gqa_attn_cfg* cfg, const gqa_paged_kv* kv,
                                        int32_t B) {
  if (check_cfg(cfg) != GQA_OK) return 0;
  gqa::PagedKV pk;
  if (check_paged(cfg, kv, &pk) != GQA_OK) return 0;
  if (B < 0) {
    fail(GQA_E_SHAPE, "B must be >= 0, got %d", B);
    return 0;
  }
  if (cfg->num_q_heads / cfg->num_kv_heads > 16) {
    fail(GQA_E_UNSUPPORTED, "paged decode takes at most 16 query heads per KV head");
    return 0;
  }
  return gqa::decode_mfma_workspace_bytes(B, cfg->num_kv_heads,
                                          cfg->num_q_heads / cfg->num_kv_heads, cfg->head_dim,
                                          kv->max_blocks * kv->block_size);
}

gqa_status gqa_attn_decode_paged(const gqa_attn_cfg* cfg, const void* q, const gqa_paged_kv* kv,
                                 const int32_t* lens, int32_t B, int32_t window, void* out,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  gqa_status st = check_cfg(cfg);
  if (st != GQA_OK) return st;
  gqa::PagedKV pk;
  st = check_paged(cfg, kv, &pk);
  if (st != GQA_OK) return st;
  if (B < 0) return fail(GQA_E_SHAPE, "B must be >= 0, got %d", B);
  if (B > 65535) return fail(GQA_E_SHAPE, "B must be <= 65535, got %d", B);
  if (window < 0) return fail(GQA_E_SHAPE, "window must be >= 0, got %d", window);
  gqa::AttnArgs a = base_args(cfg);
  const int Smax = kv->max_blocks * kv->block_size;
  a.S = Smax;
  if (!gqa::decode_mfma_supported(a))
    return fail(GQA_E_UNSUPPORTED, "paged decode takes at most 16 query heads per KV head");
  if (B == 0) return ok();
  if (!q || !lens || !out) return fail(GQA_E_NULL, "q, lens and out are required");
  if (!aligned16(q) || !aligned16(out)) return fail(GQA_E_VALUE, "q and out must be 16-byte aligned");
  const size_t need = gqa::decode_mfma_workspace_bytes(B, a.Hkv, a.G, cfg->head_dim, Smax);
  if (!workspace || workspace_bytes < need)
    return fail(GQA_E_WORKSPACE, "paged decode needs a workspace of %zu bytes, got %zu%s", need,
                workspace_bytes, workspace ? "" : " (null)");
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(GQA_E_WORKSPACE, "workspace must be 256-byte aligned");
  const int64_t D = cfg->head_dim;
  a.q = q;
  a.k = kv->k_pool;
  a.v = kv->v_pool;
  a.out = out;
  a.q_h = D;
  a.q_i = 0;
  a.q_b = (int64_t)a.Hq * D;
  a.o_h = D;
  a.o_i = 0;
  a.o_b = a.q_b;
  a.k_j = D;
  a.k_h = 0;
  a.k_b = 0;
  a.qpos = nullptr;
  a.kpos = nullptr;
  a.lens = lens;
  a.B = B;
  a.L = 1;
  a.n_cached = Smax;
  a.window = window;
  return hip_status(gqa::launch_decode_mfma(a, workspace, stream, &pk, decode_split_mode(cfg)),
                    "paged decode launch");
}

size_t gqa_mla_decode_workspace_bytes(int32_t B, int32_t H, int32_t Smax) {
  if (B < 0 || H < 16 || H % 16 || H > 65535 || Smax < 1) {
    fail(GQA_E_SHAPE, "need B >= 0, H a multiple of 16 in [16, 65535] and Smax >= 1, got %d, %d, %d",
         B, H, Smax);
    return 0;
  }
  ok();
  return gqa::mla_decode_workspace_bytes(B, H, Smax);
}

gqa_status gqa_mla_decode(const void* q, const void* cache, const int32_t* lens, int32_t B,
                          int32_t H, int32_t Smax, double scale, void* out, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  if (B < 0 || B > 65535) return fail(GQA_E_SHAPE, "B must be in [0, 65535], got %d", B);
  if (H < 16 || H % 16 || H > 65535)
    return fail(GQA_E_SHAPE, "H must be a multiple of 16 in [16, 65535], got %d", H);
  if (Smax < 1) return fail(GQA_E_SHAPE, "Smax must be >= 1, got %d", Smax);
  if ((int64_t)Smax * 576 * 2 > ((int64_t)1 << 40))
    return fail(GQA_E_SHAPE, "Smax is too large (%d)", Smax);
  if ((int64_t)B * ((Smax + 31) / 32) >= ((int64_t)1 << 31))
    return fail(GQA_E_SHAPE, "B * Smax is too large (%d x %d): the batch's 32-key blocks are "
                "counted in 32 bits", B, Smax);
  if (!(std::isfinite(scale) && scale > 0.0))
    return fail(GQA_E_VALUE, "scale must be finite and > 0, got %g", scale);
  if (B == 0) return ok();
  if (!q || !cache || !lens || !out) return fail(GQA_E_NULL, "q, cache, lens and out are required");
  if (!aligned16(q) || !aligned16(cache) || !aligned16(out))
    return fail(GQA_E_VALUE, "q, cache and out must be 16-byte aligned");
  const size_t need = gqa::mla_decode_workspace_bytes(B, H, Smax);
  if (!workspace || workspace_bytes < need)
    return fail(GQA_E_WORKSPACE, "latent-attention decode needs a workspace of %zu bytes, got %zu%s",
                need, workspace_bytes, workspace ? "" : " (null)");
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(GQA_E_WORKSPACE, "workspace must be 256-byte aligned");
  return hip_status(gqa::launch_mla_decode(q, cache, lens, B, H, Smax, (float)scale, out,
                                           workspace, stream),
                    "latent-attention decode launch");
}

}  // extern "C"
