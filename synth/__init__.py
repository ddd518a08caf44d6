"""Seeded synthetic workloads for rotary grouped-query attention.

The one module that both the HIP path's tests/bench and the oracle consume.  It holds only
random draws, shapes, position arrays and changes of representation (rounding a float32 draw to
the run dtype, bf16 bit patterns); none of the method's arithmetic lives here.

Recipe (every draw from numpy's PCG64 ``default_rng``; seed = workload number unless a test says
otherwise): q, k, v ~ N(0, 1) drawn in float32 in that order, then rounded to the run dtype with
round-to-nearest-even; per-head norm gains 1 + N(0, 0.02) drawn after v; decode lengths uniform
on [lo, hi] drawn first, then q, then each sequence's cache from its own stream
``default_rng([seed, 1000 + b])`` (K then V, [Hkv, len, D]) so a sequence can be regenerated alone.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "prefill" | "decode"
    dtype: str                # "f32" | "bf16"
    B: int
    L: int                    # new query tokens per sequence (1 for decode)
    S: int                    # keys per sequence (prefill); Smax for decode
    Hq: int
    Hkv: int
    D: int
    rotary_dim: int
    style: str = "half"       # "half" | "interleaved"
    theta: float = 1e4
    rope_kind: str = "default"
    factor: float = 1.0
    low_freq_factor: float = 1.0
    high_freq_factor: float = 4.0
    original_max_pos: float = 8192.0
    window: int = 0
    qk_norm: bool = False
    eps: float = 1e-6
    softcap: float = 0.0
    n_cached: int = 0         # prefill: keys [0, n_cached) are cache rows used as stored
    lens_lo: int = 0          # decode: cache lengths uniform on [lens_lo, lens_hi]
    lens_hi: int = 0
    seed: int = 0
    chunk: int = 0            # chunked attention: chunk length in positions (0 = off)
    chunk_lookback: int = 0   # chunks before the query's own that stay visible
    sinks: bool = False       # one learned sink logit per query head (drawn by draw_sinks)

    @property
    def G(self):
        return self.Hq // self.Hkv

    def with_(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    # 1. tiny causal prefill, fp32
    "tiny_causal_f32": Workload("tiny_causal_f32", "prefill", "f32", B=1, L=16, S=16, Hq=4,
                                Hkv=2, D=32, rotary_dim=32, theta=1e4, seed=1),
    # 2. Qwen3-style prefill: per-head q/k RMSNorm, full causal
    "qwen3_prefill_bf16": Workload("qwen3_prefill_bf16", "prefill", "bf16", B=4, L=2048, S=2048,
                                   Hq=32, Hkv=8, D=128, rotary_dim=128, theta=1e6, qk_norm=True,
                                   eps=1e-6, seed=2),
    # 3. Mistral-style sliding-window prefill
    "mistral_swa_prefill_bf16": Workload("mistral_swa_prefill_bf16", "prefill", "bf16", B=2,
                                         L=8192, S=8192, Hq=32, Hkv=8, D=128, rotary_dim=128,
                                         theta=1e6, window=4096, seed=3),
    # 4. Llama-3.1-style decode, llama3 rope scaling
    "llama31_decode_bf16": Workload("llama31_decode_bf16", "decode", "bf16", B=64, L=1, S=32768,
                                    Hq=32, Hkv=8, D=128, rotary_dim=128, theta=5e5,
                                    rope_kind="llama3", factor=8.0, low_freq_factor=1.0,
                                    high_freq_factor=4.0, original_max_pos=8192.0,
                                    lens_lo=1024, lens_hi=32768, seed=4),
    # 5. mixed chunked prefill: 512 new tokens after 3584 cached, partial interleaved rotation,
    #    soft-cap 50; the two layer kinds (window 4096 / full) share one draw
    "chunked_prefill_bf16_w4096": Workload("chunked_prefill_bf16_w4096", "prefill", "bf16", B=8,
                                           L=512, S=4096, Hq=24, Hkv=8, D=128, rotary_dim=64,
                                           style="interleaved", theta=1e4, window=4096,
                                           softcap=50.0, n_cached=3584, seed=5),
    "chunked_prefill_bf16_full": Workload("chunked_prefill_bf16_full", "prefill", "bf16", B=8,
                                          L=512, S=4096, Hq=24, Hkv=8, D=128, rotary_dim=64,
                                          style="interleaved", theta=1e4, window=0, softcap=50.0,
                                          n_cached=3584, seed=5),
    # Widened rows, measured beside the five above.  Learned sinks with a 128-key sliding window
    # (the gpt-oss layer kind; its head_dim of 64 is replaced by 128, the width the MFMA kernels
    # take), and Llama 4's chunked attention (chunks of 8192 positions, each query in its own).
    "sinks_swa128_prefill_bf16": Workload("sinks_swa128_prefill_bf16", "prefill", "bf16", B=4,
                                          L=4096, S=4096, Hq=64, Hkv=8, D=128, rotary_dim=128,
                                          theta=1.5e5, window=128, sinks=True, seed=6),
    "llama4_chunked_prefill_bf16": Workload("llama4_chunked_prefill_bf16", "prefill", "bf16",
                                            B=1, L=16384, S=16384, Hq=40, Hkv=8, D=128,
                                            rotary_dim=128, theta=5e5, chunk=8192, seed=7),
    # Absorbed latent-attention decode (DeepSeek-V3 widths): 128 query heads against one KV head
    # of 576 features (512 latent + 64 rotary); D here is the row width
    "deepseek_mla_decode_bf16": Workload("deepseek_mla_decode_bf16", "decode", "bf16", B=64, L=1,
                                         S=32768, Hq=128, Hkv=1, D=576, rotary_dim=64,
                                         lens_lo=1024, lens_hi=32768, seed=9),
    "sinks_chunk_decode_bf16": Workload("sinks_chunk_decode_bf16", "decode", "bf16", B=64, L=1,
                                        S=32768, Hq=32, Hkv=8, D=128, rotary_dim=128, theta=5e5,
                                        chunk=8192, sinks=True, lens_lo=1024, lens_hi=32768,
                                        seed=8),
}


# ---------------------------------------------------------------------------------------------
# Representation
# ---------------------------------------------------------------------------------------------
def bf16_bits(x):
    """float32 array -> uint16 bf16 bit patterns, round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to(x, dtype):
    """The value the device receives for a float32 draw."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_to_f32(bf16_bits(x))
    raise ValueError(dtype)


def device_bits(x, dtype):
    """Array to upload: float32 as is, bf16 as uint16 bit patterns."""
    return np.ascontiguousarray(x, np.float32) if dtype == "f32" else bf16_bits(x)


# ---------------------------------------------------------------------------------------------
# Draws
# ---------------------------------------------------------------------------------------------
def prefill_inputs(wl: Workload, seed=None, q_scale=1.0, k_scale=1.0, offset=0.0, B=None, L=None,
                   S=None):
    """Seeded prefill inputs (already rounded to the run dtype, held as float32).

    q_scale/k_scale/offset build stress inputs (peaky logits, non-unit RMS)."""
    seed = wl.seed if seed is None else seed
    B = wl.B if B is None else B
    L = wl.L if L is None else L
    S = wl.S if S is None else S
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, L, wl.Hq, wl.D), dtype=np.float32)
    k = rng.standard_normal((B, S, wl.Hkv, wl.D), dtype=np.float32)
    v = rng.standard_normal((B, S, wl.Hkv, wl.D), dtype=np.float32)
    if q_scale != 1.0 or offset:
        q = q * np.float32(q_scale) + np.float32(offset)
    if k_scale != 1.0 or offset:
        k = k * np.float32(k_scale) + np.float32(offset)
    out = dict(q=round_to(q, wl.dtype), k=round_to(k, wl.dtype), v=round_to(v, wl.dtype))
    if wl.qk_norm:
        out["q_norm_w"] = round_to(1.0 + 0.02 * rng.standard_normal(wl.D, dtype=np.float32), wl.dtype)
        out["k_norm_w"] = round_to(1.0 + 0.02 * rng.standard_normal(wl.D, dtype=np.float32), wl.dtype)
    out["key_positions"] = np.broadcast_to(np.arange(S, dtype=np.int32), (B, S)).copy()
    # new queries are the last L of the S keys (chunked prefill), else positions 0..L-1
    start = S - L if wl.n_cached else 0
    out["positions"] = np.broadcast_to(np.arange(start, start + L, dtype=np.int32), (B, L)).copy()
    return out


def decode_lens_q(wl: Workload, seed=None):
    """(lens [B] int32, q [B, Hq, D] float32 rounded) for a decode workload."""
    seed = wl.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    lens = rng.integers(wl.lens_lo, wl.lens_hi + 1, size=wl.B).astype(np.int32)
    q = round_to(rng.standard_normal((wl.B, wl.Hq, wl.D), dtype=np.float32), wl.dtype)
    qn = None
    if wl.qk_norm:
        qn = round_to(1.0 + 0.02 * rng.standard_normal(wl.D, dtype=np.float32), wl.dtype)
    return lens, q, qn


def decode_cache_seq(wl: Workload, b, n, seed=None):
    """Cache rows of sequence b: (k, v) each [Hkv, n, D] float32 rounded to the run dtype."""
    seed = wl.seed if seed is None else seed
    rng = np.random.default_rng([seed, 1000 + b])
    k = rng.standard_normal((wl.Hkv, n, wl.D), dtype=np.float32)
    v = rng.standard_normal((wl.Hkv, n, wl.D), dtype=np.float32)
    return round_to(k, wl.dtype), round_to(v, wl.dtype)


def draw_sinks(wl: Workload, seed=None):
    """Sink logits [Hq] float32 (None unless wl.sinks): N(0, 3^2) from their own seeded stream,
    with head 0 at +8 (the sink takes most of the weight) and the last head at -30 (none)."""
    if not wl.sinks:
        return None
    seed = wl.seed if seed is None else seed
    rng = np.random.default_rng([seed, 77])
    s = (3.0 * rng.standard_normal(wl.Hq)).astype(np.float32)
    s[0] = 8.0
    if wl.Hq > 1:
        s[-1] = -30.0
    return s


def paged_pool_inputs(B, Hkv, D, block_size, max_blocks, dtype="bf16", spare=4, seed=0):
    """A paged KV pool with room for every sequence's max_blocks blocks plus `spare` blocks:
    k_pool, v_pool [B * max_blocks + spare, Hkv, block_size, D] of N(0, 1) draws rounded to the
    run dtype, and a block table [B, max_blocks] that is a seeded random permutation of the first
    B * max_blocks of all blocks (the remaining spares stay unreferenced)."""
    rng = np.random.default_rng([seed, 424242])
    nb = B * max_blocks + spare
    kp = round_to(rng.standard_normal((nb, Hkv, block_size, D), dtype=np.float32), dtype)
    vp = round_to(rng.standard_normal((nb, Hkv, block_size, D), dtype=np.float32), dtype)
    table = rng.permutation(nb)[: B * max_blocks].reshape(B, max_blocks).astype(np.int32)
    return kp, vp, table


def rope_params(wl: Workload):
    """Keyword arguments describing the rotation (plain data)."""
    return dict(rotary_dim=wl.rotary_dim, theta=wl.theta, kind=wl.rope_kind, factor=wl.factor,
                low_freq_factor=wl.low_freq_factor, high_freq_factor=wl.high_freq_factor,
                original_max_position_embeddings=wl.original_max_pos)


# ---------------------------------------------------------------------------------------------
# Device-side draws (large workloads): torch's seeded generator on the GPU.  Tests and the bench
# read back the sampled slices they hand to the oracle.
# ---------------------------------------------------------------------------------------------
def device_normal(shape, seed, dtype, device="cuda"):
    """N(0, 1) draw of `shape` on the device from torch's generator seeded with `seed`, rounded to
    the run dtype ("bf16" or "f32")."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def decode_device_inputs(wl: Workload, seed=None, device="cuda"):
    """Decode workload on the device: lens (numpy stream of `seed`), q and the full caches
    [B, Hkv, Smax, D] drawn sequence by sequence from one seeded device generator."""
    import torch
    seed = wl.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    lens = rng.integers(wl.lens_lo, wl.lens_hi + 1, size=wl.B).astype(np.int32)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 7919 + 17)
    q = torch.randn((wl.B, wl.Hq, wl.D), generator=gen, device=device).to(dt)
    k = torch.empty((wl.B, wl.Hkv, wl.S, wl.D), dtype=dt, device=device)
    v = torch.empty_like(k)
    for b in range(wl.B):
        k[b] = torch.randn((wl.Hkv, wl.S, wl.D), generator=gen, device=device).to(dt)
        v[b] = torch.randn((wl.Hkv, wl.S, wl.D), generator=gen, device=device).to(dt)
    out = dict(lens=torch.from_numpy(lens).to(device), q=q, k=k, v=v)
    if wl.qk_norm:
        out["qw"] = (1.0 + 0.02 * torch.randn((wl.D,), generator=gen, device=device)).to(dt)
        out["kw"] = (1.0 + 0.02 * torch.randn((wl.D,), generator=gen, device=device)).to(dt)
    return out
