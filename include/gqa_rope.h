/*
 * gqa_rope.h -- rotary grouped-query causal attention on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libgqa_rope.so.  Every pointer named "device" is HIP device memory that the caller
 * allocated and owns; the library keeps no state between calls and never allocates, frees or
 * synchronises in these calls.  Work is enqueued on the caller's stream and runs asynchronously.
 *
 * The operations restate three web pages (cited by title and section):
 *   [Models] "42. More models: a registry, scaled RoPE, sliding windows and latent attention"
 *   [Ster]   "Model resolution", section "Overview"
 *   [Guide]  "MoE, optimisers, decoding -- every line, every shape."
 *
 * Errors: every call validates its host-side arguments (null pointers, shapes, dtype, rotary
 * width parity, head grouping, rope kind, workspace size) before anything is launched and returns
 * a gqa_status; gqa_last_error() then names the offending argument (thread-local string).  A HIP
 * launch failure returns GQA_E_HIP with HIP's message.  Preconditions on device data are not
 * checked (positions within the table, key positions nondecreasing, 1 <= lens <= Smax): device
 * indices are clamped into their buffers so a violation yields wrong numbers, never an
 * out-of-bounds access.
 */
#ifndef GQA_ROPE_H
#define GQA_ROPE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gqa_status {
  GQA_OK = 0,
  GQA_E_NULL = 1,        /* a required pointer is null */
  GQA_E_SHAPE = 2,       /* a size is out of range or sizes disagree */
  GQA_E_DTYPE = 3,       /* unknown dtype */
  GQA_E_UNSUPPORTED = 4, /* valid request this build does not implement (e.g. head_dim > 256) */
  GQA_E_WORKSPACE = 5,   /* workspace missing or smaller than gqa_decode_workspace_bytes() */
  GQA_E_HIP = 6,         /* a HIP call failed; message from hipGetErrorString */
  GQA_E_VALUE = 7        /* a scalar parameter is out of range (theta, factor, eps, ...) */
} gqa_status;

typedef enum gqa_dtype { GQA_F32 = 0, GQA_BF16 = 1 } gqa_dtype;

/* [Models] "Scaled RoPE": the frequency schedules of rope_scaling (yarn included), and LongRoPE's
 * per-pair factor tables ([Ster] "Overview"). */
typedef enum gqa_rope_kind {
  GQA_ROPE_DEFAULT = 0,
  GQA_ROPE_LINEAR = 1,
  GQA_ROPE_LLAMA3 = 2,
  GQA_ROPE_YARN = 3,
  GQA_ROPE_LONGROPE = 4
} gqa_rope_kind;

/* Pairing of rotated features: half-split pairs (i, i + R/2) ([Guide] section 4 "Rotary");
 * interleaved pairs (2i, 2i + 1) ([Models] "Serving it: absorbing the up-projections"). */
typedef enum gqa_rot_style { GQA_ROT_HALF = 0, GQA_ROT_INTERLEAVED = 1 } gqa_rot_style;

/* Rotary frequency schedule ([Models] "Scaled RoPE", rope_inv_freq).  A zero-initialised struct
 * with rotary_dim, kind and theta set selects the pages' defaults for every other field.
 * rotary_dim R: number of rotated features, even, 0 <= R <= 512; R = head_dim *
 * partial_rotary_factor ([Ster] "Overview": only that share of each head rotates, and the
 * frequencies run over that share).  theta > 0.  factor > 0 (linear, llama3, yarn; yarn callers
 * whose config omits it pass max_positions / original_max_pos, as the page does).  llama3 also
 * needs 0 < low_freq_factor < high_freq_factor; llama3, yarn and longrope need
 * original_max_pos > 0.
 *   yarn: pairs turning more than beta_fast times over original_max_pos keep their frequency,
 *     pairs turning fewer than beta_slow times are divided by factor, a linear ramp over the pair
 *     index in between, its ends rounded outwards unless yarn_no_truncate.  Attention factor:
 *     attention_factor when > 0, else mscale(factor, mscale) / mscale(factor, mscale_all_dim)
 *     when both are > 0, else mscale(factor), with mscale(s, m) = 0.1 m ln s + 1 (1 for s <= 1).
 *   longrope: frequency i divided by short_factor[i] while seq_len <= original_max_pos, by
 *     long_factor[i] once seq_len goes past ([Ster] "Overview"); both tables host memory, R/2
 *     positive doubles, read during the call only.  Attention factor: attention_factor when > 0,
 *     else 1 (the pages give the factor no formula). */
typedef struct gqa_rope_params {
  int32_t rotary_dim;
  int32_t kind;               /* gqa_rope_kind */
  double theta;
  double factor;
  double low_freq_factor;
  double high_freq_factor;
  double original_max_pos;    /* original_max_position_embeddings */
  double beta_fast;           /* yarn: 0 selects 32 */
  double beta_slow;           /* yarn: 0 selects 1; beta_fast > beta_slow */
  int32_t yarn_no_truncate;   /* yarn: nonzero keeps the ramp ends unrounded (truncate: false) */
  int32_t reserved;           /* must be 0 */
  double mscale;              /* yarn: 0 = absent */
  double mscale_all_dim;      /* yarn: 0 = absent */
  double attention_factor;    /* yarn, longrope: > 0 given; 0 = derived as above */
  const double* short_factor; /* longrope: host [R/2] */
  const double* long_factor;  /* longrope: host [R/2] */
  int64_t seq_len;            /* longrope: sequence length that selects the table */
} gqa_rope_params;

/* Attention configuration shared by prefill and decode. */
typedef struct gqa_attn_cfg {
  int32_t dtype;              /* gqa_dtype of q, k, v, out and the norm gains */
  int32_t head_dim;           /* D: 1..256, multiple of 8 */
  int32_t num_q_heads;        /* Hq */
  int32_t num_kv_heads;       /* Hkv; Hq % Hkv == 0.  Query head h reads KV head h / (Hq/Hkv) */
  int32_t rotary_dim;         /* R, must equal the R the tables were built with; 0 = no rotation */
  int32_t rot_style;          /* gqa_rot_style */
  const float* cos_table;     /* device [table_len, R/2] fp32 from gqa_rope_tables (may be null if R == 0) */
  const float* sin_table;     /* device [table_len, R/2] */
  int32_t table_len;          /* rows of the tables: valid positions are 0 .. table_len-1 */
  int32_t qk_norm;            /* 1: per-head RMSNorm of q and new k before rotation ([Models] "What differs") */
  double eps;                 /* RMSNorm epsilon ([Guide] section 3.2), >= 0 */
  const void* q_norm_w;       /* device [D] gain in dtype (required when qk_norm) */
  const void* k_norm_w;       /* device [D] gain in dtype (required when qk_norm) */
  double scale;               /* score scale; 0 selects 1/sqrt(head_dim) ([Guide] section 3.4) */
  double softcap;             /* > 0: scores become softcap * tanh(score / softcap); 0: off */
  /* Learned attention sinks ([Ster] gpt_oss paragraph): device [num_q_heads] fp32, one logit per
   * query head that joins every softmax of that head with no value, so its share of the weight is
   * dropped.  The logit is in the units of the scaled scores and is not soft-capped.  Null: no
   * sinks.  Read-only during the call; 4-byte aligned. */
  const float* sinks;
  /* Chunked attention ([Ster] llama4_text and Rnj-1.5 paragraphs): positions fall in chunks of
   * chunk_size (chunk c = positions c*chunk_size .. (c+1)*chunk_size - 1, negative positions
   * included); a query sees the keys of its own chunk and of the chunk_lookback chunks before it
   * (Llama 4: 0, Rnj-1.5: 1), still causally and still inside the window when one is given.
   * chunk_size 0: no chunking.  Both >= 0. */
  int32_t chunk_size;
  int32_t chunk_lookback;
  /* Kernel selection for this call (gqa_kernel_select); production callers leave it 0.  Every
   * choice computes the same result up to rounding order. */
  int32_t kernel;
  int32_t reserved;           /* must be 0 */
} gqa_attn_cfg;

/* Values of gqa_attn_cfg.kernel.  The choice is per call: the library holds no selection state.
 *   GQA_KERNEL_AUTO          bf16 problems run on the MFMA kernels wherever their shape is
 *                            covered, everything else on the generic kernel
 *   GQA_KERNEL_GENERIC       every problem on the generic kernel (one wavefront per query row and
 *                            head, fp32 arithmetic): a second implementation to compare against
 *   GQA_KERNEL_DECODE_SHORT  decode on the MFMA kernels with 1024-key splits for every walk
 *   GQA_KERNEL_DECODE_LONG   decode on the MFMA kernels with 2048-key splits for every walk
 *                            longer than 1024 keys (AUTO picks between the two by the batch's
 *                            size); for prefill calls the two act as AUTO
 *   GQA_KERNEL_PREFILL_LONG  bf16 prefill with a workspace on the eight-wavefront streaming
 *                            kernel (one workgroup per CU, deep tile pipeline)
 *   GQA_KERNEL_PREFILL_SHORT bf16 prefill with a workspace on the four-wavefront streaming kernel
 *                            (two workgroups per CU); AUTO picks between the two by the mean
 *                            number of keys a workgroup visits (below 768: short); without a
 *                            workspace, and for decode calls, the two act as AUTO */
typedef enum gqa_kernel_select {
  GQA_KERNEL_AUTO = 0,
  GQA_KERNEL_GENERIC = 1,
  GQA_KERNEL_DECODE_SHORT = 2,
  GQA_KERNEL_DECODE_LONG = 3,
  GQA_KERNEL_PREFILL_LONG = 4,
  GQA_KERNEL_PREFILL_SHORT = 5
} gqa_kernel_select;

/* Build cos/sin tables for positions 0 .. table_len-1 ([Models] "Scaled RoPE", rope_tables):
 * cos_out[p*(R/2) + i] = a * cos(p * inv_freq[i]), sin_out likewise, with a the attention factor
 * (1 except for yarn and longrope).  inv_freq is computed on the host in double precision and the
 * angles, their sine/cosine and the product with a on the device in double precision, then
 * stored as fp32.  cos_out, sin_out: device, table_len * R/2 floats each,
 * caller-owned.  table_len >= 1.  R == 0 is a valid no-op. */
gqa_status gqa_rope_tables(const gqa_rope_params* rope, int32_t table_len, float* cos_out,
                           float* sin_out, hipStream_t stream);

/* Host-side copy of the frequencies the tables use (R/2 doubles into inv_freq_out, host memory).
 * Lets a caller inspect the schedule without a GPU. */
gqa_status gqa_rope_inv_freq(const gqa_rope_params* rope, double* inv_freq_out);

/* The attention factor the tables are multiplied by ([Models] "Scaled RoPE"), into *out (host). */
gqa_status gqa_rope_attention_factor(const gqa_rope_params* rope, double* out);

/* Softmax scale for a query/key width qk_dim > 0 ([Models] "Multi-head latent attention": YaRN's
 * temperature applied to the scale): qk_dim^-0.5, times m^2 with m = 0.1 * mscale_all_dim *
 * ln(factor) + 1 when the schedule is yarn with mscale_all_dim > 0 and factor > 1.  Into *out
 * (host); pass it as gqa_attn_cfg.scale. */
gqa_status gqa_rope_softmax_scale(const gqa_rope_params* rope, int32_t qk_dim, double* out);

/* Prepare new keys for a cache: for every row j in [n_cached, S) of k [B, S, Hkv, D] and every KV
 * head, RMS-norm the row (when cfg->qk_norm, gain k_norm_w) and rotate its first rotary_dim
 * features at key_positions[b, j], then store it (dtype of cfg) at the same (b, j, g) of k_out
 * [B, S, Hkv, D] ([Models] "What differs between model families": keys are normed and rotated,
 * then appended to the cache by cache.update).  Rows j < n_cached of k_out are not touched.  k_out
 * may be k itself (in place).  A following gqa_attn_prefill over k_out with n_cached = S then uses
 * every key as stored.  bf16 with head_dim 128 and the rotary widths the MFMA kernels accept
 * (any multiple of 8 interleaved, 16/32/64/128 half-split); otherwise GQA_E_UNSUPPORTED. */
gqa_status gqa_prep_keys(const gqa_attn_cfg* cfg, const void* k, const int32_t* key_positions,
                         int64_t kpos_batch_stride, int32_t B, int32_t S, int32_t n_cached,
                         void* k_out, hipStream_t stream);

/* Bytes of device workspace for gqa_attn_prefill's streaming kernels (0 where they do not apply:
 * fp32, the generic kernel, shapes the MFMA kernels do not cover).  It holds (1) the new keys,
 * normed and rotated once instead of in every key tile -- needed whenever some key must be
 * prepared (a norm or a rotation, and n_cached < S) -- and (2) about 35 MB into which, when the
 * query blocks leave a last, partial round of the GPU, those blocks' key walks are split over
 * two workgroups each and their partial results merged.  Returns 0 and sets the error on
 * invalid arguments. */
size_t gqa_prefill_workspace_bytes(const gqa_attn_cfg* cfg, int32_t B, int32_t S, int32_t n_cached);

/* Which kernel a gqa_attn_prefill call with these sizes runs (host-only, no device work), for
 * tools that label measurements: with_workspace != 0 means a workspace of at least
 * gqa_prefill_workspace_bytes() bytes is passed.  *which (host int32) receives a
 * gqa_prefill_kernel_id.  Errors as gqa_attn_prefill's argument checks. */
typedef enum gqa_prefill_kernel_id {
  GQA_PREFILL_GENERIC = 0,       /* one wavefront per query row and head, fp32 arithmetic */
  GQA_PREFILL_FUSED = 1,         /* MFMA kernel preparing new keys on the fly (no workspace) */
  GQA_PREFILL_STREAM_LONG = 2,   /* key-preparation pass + eight-wavefront streaming kernel */
  GQA_PREFILL_STREAM_SHORT = 3   /* key-preparation pass + four-wavefront streaming kernel */
} gqa_prefill_kernel_id;
gqa_status gqa_prefill_kernel(const gqa_attn_cfg* cfg, int32_t B, int32_t L, int32_t S,
                              int32_t n_cached, int32_t window, int32_t with_workspace,
                              int32_t* which);

/* Causal prefill ([Models] "What differs between model families", DecoderAttention.forward;
 * [Guide] section 3.4 "Attention").
 *   q   device [B, L, Hq, D]  new queries (contiguous)
 *   k,v device [B, S, Hkv, D] keys/values; rows j < n_cached are cache rows used as stored
 *       (already normed and rotated); rows j >= n_cached are new and get the k-norm and the
 *       rotation at key_positions[j]; values are never rotated
 *   positions      device int32 [B, L] (pos_batch_stride = L) or [L] shared (stride 0)
 *   key_positions  device int32 [B, S] or [S] shared; must be nondecreasing in j
 *   window         0 = full causal; w > 0: a query at position p sees keys at positions
 *                  p-w+1 .. p ([Models] "Sliding windows": keys more than w-1 back are masked)
 *   out  device [B, L, Hq, D] (contiguous, caller-owned), never aliasing the inputs.
 *   workspace  optional device scratch, 256-byte aligned, caller-owned, contents ignored.  With
 *              gqa_prefill_workspace_bytes() bytes the streaming kernels run: the new keys are
 *              normed and rotated once into it (one pass) and, when the query blocks leave a
 *              last, partial round of the GPU, those blocks' key walks are split in two and
 *              merged through it.  A smaller workspace that still holds the prepared keys runs
 *              them without the split (GQA_E_WORKSPACE when it does not).  Null: the streaming
 *              kernels when no key needs preparing, else the fused kernel, which normalises and
 *              rotates new keys on the fly.  All give the same result up to rounding order.
 *              Calls sharing a workspace must be ordered on one stream.
 * Result per (b, i, h): softmax over allowed keys of scale*<q', k'> (soft-capped if set), times
 * v; a row with no allowed key is 0.  B, L, S >= 0 (an empty problem is a no-op); n_cached in
 * [0, S]. */
gqa_status gqa_attn_prefill(const gqa_attn_cfg* cfg, const void* q, const void* k, const void* v,
                            const int32_t* positions, int64_t pos_batch_stride,
                            const int32_t* key_positions, int64_t kpos_batch_stride, int32_t B,
                            int32_t L, int32_t S, int32_t n_cached, int32_t window, void* out,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace gqa_attn_decode needs for B sequences of capacity Smax (0 if the
 * chosen kernel needs none).  Returns 0 and sets the error on invalid arguments. */
size_t gqa_decode_workspace_bytes(const gqa_attn_cfg* cfg, int32_t B, int32_t Smax);

/* Single-token decode against a KV cache ([Guide] section 3.3 "KVCache", section 3.7).
 *   q          device [B, Hq, D], the new token's query (normed and rotated here, at lens[b]-1)
 *   kcache     device [B, Hkv, Smax, D]: slot j of sequence b holds the key at position j,
 *              already normed and rotated; slot lens[b]-1 holds the new token's key
 *   vcache     device [B, Hkv, Smax, D]
 *   lens       device int32 [B], 1 <= lens[b] <= Smax
 *   window     0 = every cached key; w > 0: only the last w keys
 *   out        device [B, Hq, D]
 *   workspace  device, >= gqa_decode_workspace_bytes(cfg, B, Smax) bytes (split partials),
 *              caller-owned; contents on entry are ignored.
 * Two calls that share a workspace must be ordered on one stream. */
gqa_status gqa_attn_decode(const gqa_attn_cfg* cfg, const void* q, const void* kcache,
                           const void* vcache, const int32_t* lens, int32_t B, int32_t Smax,
                           int32_t window, void* out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* gqa_attn_decode for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments (less the workspace),
 * layouts, errors and result as gqa_attn_decode; the split partials live in a fixed array of
 * GQA_DECODE_NOALLOC_MAX_BYTES inside the library instead, one per GPU, which that GPU holds from
 * the first call (or library load) until the process ends.  The call allocates nothing.  Sizes
 * whose gqa_decode_workspace_bytes(cfg, B, Smax) exceed the limit return GQA_E_WORKSPACE (the
 * Llama-3.1-style batch of 64 sequences of up to 32768 keys, Hkv 8, G 4 needs ~34 MiB).  Every
 * call on one GPU shares that GPU's array and leaves its last contents there (nothing in it has
 * to start at zero): calls that overlap on one GPU -- unordered streams, or several host threads
 * -- race and give wrong results, so order them on one stream. */
#define GQA_DECODE_NOALLOC_MAX_BYTES ((size_t)64 << 20)
gqa_status gqa_attn_decode_noalloc(const gqa_attn_cfg* cfg, const void* q, const void* kcache,
                                   const void* vcache, const int32_t* lens, int32_t B,
                                   int32_t Smax, int32_t window, void* out, hipStream_t stream);

/* Paged KV pool (the block manager's layout behind cache.update: [Models] "What differs" (the
 * cache.update call), "Sliding windows" (blocks that leave every window can be recycled) and the
 * multi-head latent attention section's paged pool; [Guide] section 3.3 for what the cache holds).
 *   k_pool, v_pool  device [num_blocks, Hkv, block_size, D] in cfg.dtype, caller-owned
 *   block_table     device int32 [B, max_blocks]: slot j of sequence b (the key at position j) is
 *                   row j % block_size of physical block block_table[b * max_blocks + j /
 *                   block_size]
 *   block_size      a power of two in [16, 1024]
 *   num_blocks      blocks in each pool; table entries are clamped into [0, num_blocks), so a bad
 *                   entry reads or writes a wrong block, never outside the pools
 * Only the entries of blocks that hold a visible slot are read: with a window (or chunks) the
 * entries of blocks wholly before it may be stale or reused for other sequences (recycling). */
typedef struct gqa_paged_kv {
  void* k_pool;
  void* v_pool;
  const int32_t* block_table;
  int32_t max_blocks;
  int32_t block_size;
  int32_t num_blocks;
  int32_t reserved;  /* must be 0 */
} gqa_paged_kv;

/* cache.update with the key preparation fused in ([Models] "What differs": k-norm, rotation,
 * then cache.update; [Guide] section 3.3 update): rows k_new, v_new device [B, L, Hkv, D]
 * (contiguous) go to slots start[b] .. start[b] + L - 1 of each sequence; each key row is
 * RMS-normed with cfg.k_norm_w when cfg.qk_norm, then rotated at key_positions[b *
 * kpos_batch_stride + i]; value rows are copied.  start: device int32 [B] (the sequences' lengths
 * before the append); start[b] + L <= max_blocks * block_size is the caller's to keep (slots past
 * it are clamped into the table).  bf16, head_dim 128 and the rotary widths of gqa_prep_keys. */
gqa_status gqa_paged_append(const gqa_attn_cfg* cfg, const gqa_paged_kv* kv, const void* k_new,
                            const void* v_new, const int32_t* key_positions,
                            int64_t kpos_batch_stride, const int32_t* start, int32_t B, int32_t L,
                            hipStream_t stream);

/* Bytes of device workspace gqa_attn_decode_paged needs (0 on invalid arguments). */
size_t gqa_paged_decode_workspace_bytes(const gqa_attn_cfg* cfg, const gqa_paged_kv* kv,
                                        int32_t B);

/* gqa_attn_decode over a paged pool: sequence b's keys are its slots 0 .. lens[b]-1, the query
 * sits at position lens[b]-1 and is normed and rotated there; 1 <= lens[b] <= max_blocks *
 * block_size.  q, out device [B, Hq, D].  bf16, head_dim 128, Hq/Hkv <= 16; workspace as for
 * gqa_attn_decode.  Two calls that share a workspace must be ordered on one stream. */
gqa_status gqa_attn_decode_paged(const gqa_attn_cfg* cfg, const void* q, const gqa_paged_kv* kv,
                                 const int32_t* lens, int32_t B, int32_t window, void* out,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Absorbed multi-head latent attention decode core ([Models] "Multi-head latent attention",
 * paged_forward; DeepSeek-V2/V3 and Kimi K2 widths): multi-query attention with one key/value head
 * 576 wide (kv_lora_rank 512 + qk_rope_head_dim 64) whose values are the first 512 features of
 * the same rows.
 *   q      device bf16 [B, H, 576]: per head, the absorbed query W_uk^T q_nope (512) followed by
 *          the rotated q_rope (64), as the page builds it before its backend call
 *   cache  device bf16 [B, Smax, 576]: slot j of sequence b holds [c, k_rope] of position j
 *   lens   device int32 [B], 0 <= lens[b] <= Smax; the query sees slots 0 .. lens[b]-1 (a
 *          sequence with none gets a zero output)
 *   H      query heads, a multiple of 16 in [16, 65535]
 *   scale  softmax scale (the caller's qk_head_dim^-0.5, times YaRN's m^2 where it applies), > 0
 *   out    device bf16 [B, H, 512], before W_uv
 *   workspace  device, >= gqa_mla_decode_workspace_bytes(B, H, Smax) bytes, 256-byte aligned:
 *              partial results of the (256 + B) pieces the batch is cut into (its blocks of 32
 *              keys are dealt out in 256 equal shares; a share may hold pieces of several
 *              sequences), (256 + B) * H * (512 + 2) floats (each part 256-byte aligned),
 *              then one int32 flag per (group of 128 heads, share, quarter of the group)
 *              marking a share whose weights could pass 2^64 against its first block's
 *              maximum, which a second kernel then computes again with rescaling.
 * Errors: GQA_E_SHAPE also when B * ceil(Smax / 32) >= 2^31.
 * Two calls that share a workspace must be ordered on one stream. */
size_t gqa_mla_decode_workspace_bytes(int32_t B, int32_t H, int32_t Smax);
gqa_status gqa_mla_decode(const void* q, const void* cache, const int32_t* lens, int32_t B,
                          int32_t H, int32_t Smax, double scale, void* out, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* Message for the last non-OK status returned on this thread ("" if none).  The error style
 * follows the pages: a rope type outside the known set is rejected by name ([Models] "Scaled
 * RoPE", rope_inv_freq); each refusal message names what failed ([Ster] "Refusals"); and a
 * request this build cannot serve is refused before any work, never served by a fallback ([Ster]
 * "Device choice").  Messages here name the offending argument and its accepted range. */
const char* gqa_last_error(void);

/* Library version string. */
const char* gqa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GQA_ROPE_H */
