// Host-side launchers of the HIP kernels (internal to libgqa_rope; the public ABI is gqa_rope.h).
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace gqa {

constexpr int kMaxPairs = 256;  // rotary_dim <= 512

// cos/sin tables [table_len, half] from host-computed frequencies (double), both scaled by the
// attention factor.
hipError_t launch_rope_tables(const double* inv_freq, double attention_factor, int half,
                              int table_len, float* cos_out, float* sin_out, hipStream_t stream);

// Any head_dim <= 256, any grouping, fp32 or bf16: one wave per (query row, head).
// Serves fp32 problems and shapes the MFMA kernels do not cover.
hipError_t launch_attn_generic(const AttnArgs& a, bool bf16, hipStream_t stream);

// bf16 MFMA prefill for head_dim 128.  Returns hipErrorNotSupported when the shape is outside
// what the kernel covers (the caller then uses the generic kernel).
bool prefill_mfma_supported(const AttnArgs& a);
hipError_t launch_prefill_mfma(const AttnArgs& a, hipStream_t stream);

// bf16 MFMA prefill over prepared keys (K/V streamed HBM -> LDS): an optional key-preparation
// pass into `workspace`, then the attention kernel.
bool prefill_needs_kprep(const AttnArgs& a);
bool prefill_stream_supported(const AttnArgs& a);
size_t prefill_stream_workspace_bytes(const AttnArgs& a);
size_t prefill_stream_required_bytes(const AttnArgs& a);
// Which streaming attention kernel runs: chosen from the mean key band per workgroup, or forced.
enum class StreamKernel { kAuto = 0, kLong = 1, kShort = 2 };
// workspace: the prepared keys (prefill_stream_required_bytes; required when keys need
// preparing), then room for split partials (the rest of prefill_stream_workspace_bytes; used when
// present).
hipError_t launch_prefill_stream(const AttnArgs& a, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream, StreamKernel which = StreamKernel::kAuto);
// True when launch_prefill_stream runs the four-wavefront kernel for this call.
bool prefill_stream_short(const AttnArgs& a, StreamKernel which);
// The key-preparation pass on its own: rows [n_cached, S) of a.k, normed and rotated, written to
// k_out with k's layout [B, S, Hkv, D].
bool prep_keys_supported(const AttnArgs& a);
hipError_t launch_prep_keys(const AttnArgs& a, void* k_out, hipStream_t stream);

// Paged KV pool: pools [num_blocks, Hkv, 2^log2bs, D]; slot j of sequence b is row j % bs of
// block table[b * max_blocks + j / bs] (entries are clamped into [0, num_blocks)).
struct PagedKV {
  const int32_t* table;
  int32_t max_blocks, log2bs, num_blocks;
};

// bf16 split-KV decode for head_dim 128 (query preparation, split kernel, combine kernel); the
// workspace holds the split partials and the prepared queries.  With `paged`, a.k and a.v are
// the pools and a.S = max_blocks * block size.
// Split size of the decode walks: chosen per launch from the batch (kAuto), or fixed at 1024
// keys (kShort) or 2048 keys for walks longer than 1024 (kLong).
enum class SplitMode { kAuto = 0, kShort = 1, kLong = 2 };
bool decode_mfma_supported(const AttnArgs& a);
size_t decode_mfma_workspace_bytes(int B, int Hkv, int G, int D, int Smax);
hipError_t launch_decode_mfma(const AttnArgs& a, void* workspace, hipStream_t stream,
                              const PagedKV* paged = nullptr, SplitMode mode = SplitMode::kAuto);

// Decode scratch that needs no allocation: the address of this GPU's fixed array of
// kDecodeScratchBytes (taken once per device, with the device current).  Calls on one GPU share it.
constexpr size_t kDecodeScratchBytes = (size_t)64 << 20;
hipError_t decode_scratch(void** ptr);

// cache.update into a paged pool: rows i < a.L of a.k (normed and rotated at a.kpos, as the key
// preparation does) and of a.v (copied) go to slots start[b] + i.
hipError_t launch_paged_append(const AttnArgs& a, const PagedKV& kv, void* k_pool, void* v_pool,
                               const int32_t* start, hipStream_t stream);
int decode_split_keys();

// Absorbed multi-head latent attention decode core (bf16): q [B, H, 576], cache [B, Smax, 576],
// out [B, H, 512]; H a multiple of 16.  The workspace holds the split partials.
size_t mla_decode_workspace_bytes(int B, int H, int Smax);
hipError_t launch_mla_decode(const void* q, const void* cache, const int32_t* lens, int B, int H,
                             int Smax, float scale, void* out, void* workspace,
                             hipStream_t stream);

}  // namespace gqa
