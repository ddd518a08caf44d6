"""Oracle: a plain, slow float64 CPU definition of rotary grouped-query causal attention.

TEST INFRASTRUCTURE, NOT THE PRODUCT.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The HIP library under
``gqa_scaled_rope_amd/`` never imports, links or calls it, and this module imports nothing from
there: the two sides share no code.  Inputs reach both sides from ``synth/`` (seeded draws only).

Every function restates a definition from one of three web pages (cited by title and section):

  [Models] "42. More models: a registry, scaled RoPE, sliding windows and latent attention"
           (a chapter of a from-scratch LLM inference-engine tutorial)
  [Ster]   "Model resolution" (documentation of the Ster runtime), section "Overview"
  [Guide]  "MoE, optimisers, decoding -- every line, every shape." (a study guide)

Where the pages leave a step open, the reading taken is stated at the function that takes it.
All arithmetic is numpy float64 on the exact values the GPU receives (inputs already rounded to the
run dtype), with library matmul / exp / tanh / sin / cos as the only primitives.

Pins (tests/test_oracle_pins.py, all CPU): the page's worked RoPE wavelength; position-squeezing
of linear scaling; llama3 per-band behaviour; YaRN's rotation-count split, ramp monotonicity,
reduction to plain RoPE at factor 1 and its sharpening values; LongRoPE's reduction to plain and
linear RoPE and its short/long switch; the attention factor on the table norm; complex-multiplication form of the rotation; the
half-split pairing of the study guide; deinterleave equivalence; norm preservation; relative
position; RMS of the normed vector; soft-cap limits; integer mask probes (windows, chunks with
and without lookback, floor chunks of negative positions); the sink's closed forms (one key: a
logistic weight; constant values: the share the keys keep) and torch's SDPA with the sink as one
more key; chunks without lookback restarting the sequence; paged rows equal the contiguous
cache under identity and permuted block tables, paged update writes exactly the next slots, and
decode over a pool filled by append_rows equals the last prefill row; the latent-attention core
equals decompressed attention (the absorption identity) and one-head attention by brute force;
window and GQA equivalences; decode == last prefill row; chunked prefill == tail of full prefill; brute-force
scalar loops; and torch's CPU scaled_dot_product_attention in float64.  No function here is
"parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

ROPE_KINDS = ("default", "linear", "llama3", "yarn", "longrope")
ROT_STYLES = ("half", "interleaved")


# ----------------------------------------------------------------------------------------------
# Rotary frequencies and angles
# ----------------------------------------------------------------------------------------------
def rope_inv_freq(rotary_dim, theta, kind="default", factor=1.0, low_freq_factor=1.0,
                  high_freq_factor=4.0, original_max_position_embeddings=8192.0, *,
                  beta_fast=None, beta_slow=None, truncate=True, short_factor=None,
                  long_factor=None, seq_len=None):
    """Rotation frequency of each of the rotary_dim/2 feature pairs.

    [Models] "Scaled RoPE": pair i turns by p * theta^(-2i/d) at position p; d here is the
    rotated width (reading for partial rotation: [Ster] "Overview" rotates only the
    partial_rotary_factor share of each head, so the frequencies run over that share).
      default: theta^(-2i/d)
      linear:  every frequency divided by the extension factor (position p looks like p/factor)
      llama3:  pairs with wavelength shorter than original/high_freq_factor are kept, pairs longer
               than original/low_freq_factor are divided by factor, and in between the two are
               blended linearly with weight s = (original/wavelength - low)/(high - low) on the
               kept value.
      yarn:    the same split chosen by counting rotations over the original context: pairs
               that turn more than beta_fast (default 32) times keep their frequency, pairs that
               turn fewer than beta_slow (default 1) times are divided by factor, with a linear
               ramp over the pair index between the two (ends rounded outwards unless
               truncate is false).  The pair index that turns r times over the original context
               solves original * theta^(-2x/d) = 2*pi*r for x.
      longrope ([Ster] "Overview", [Ster] phimoe paragraph): per-pair factors, the short table
               while the sequence is within original_max_position_embeddings and the long one
               once it goes past; frequency i is divided by the table's entry i.  Reading: the
               sequence length that decides is seq_len (positions 0 .. seq_len-1).
    The attention factor that multiplies cos and sin is rope_attention_factor(); it is 1 for the
    first three kinds.
    """
    if rotary_dim < 0 or rotary_dim % 2:
        raise ValueError(f"rotary_dim must be even and >= 0, got {rotary_dim}")
    if kind not in ROPE_KINDS:
        raise ValueError(f"unknown rope scaling kind {kind!r}; known kinds: {', '.join(ROPE_KINDS)}")
    half = rotary_dim // 2
    out = np.empty(half, dtype=np.float64)
    if kind == "yarn":
        # Rotation counts: pair i makes turns[i] = original * theta^(-2i/d) / (2 pi) full turns
        # over the original context, fewer the higher i.  The ramp's index range is 0 .. d-1.
        fast = float(beta_fast) if beta_fast else 32.0
        slow = float(beta_slow) if beta_slow else 1.0
        old = float(original_max_position_embeddings)
        idx = np.arange(rotary_dim, dtype=np.float64)
        turns = old * float(theta) ** (-2.0 * idx / rotary_dim) / (2.0 * math.pi)
        if truncate:
            # whole-index ends: the last index that still turns `fast` times, the first that
            # turns no more than `slow` times
            start = max(int(np.count_nonzero(turns >= fast)) - 1, 0)
            stop = min(int(np.count_nonzero(turns > slow)), rotary_dim - 1)
        else:
            # fractional ends: the index at which the turn count equals fast (resp. slow)
            turns0 = old / (2.0 * math.pi)
            start = max(0.5 * rotary_dim * math.log(turns0 / fast) / math.log(theta), 0.0)
            stop = min(0.5 * rotary_dim * math.log(turns0 / slow) / math.log(theta),
                       rotary_dim - 1.0)
        for i in range(half):
            base = float(theta) ** (-2.0 * i / rotary_dim)
            if stop > start:    # share of the frequency that is divided by the factor
                share = min(max((i - start) / (stop - start), 0.0), 1.0)
            else:               # the two ends meet: a step after the first one
                share = 1.0 if i > start else 0.0
            out[i] = base * (1.0 - share) + base / factor * share
        return out
    if kind == "longrope":
        old = float(original_max_position_embeddings)
        table = long_factor if (seq_len is not None and seq_len > old) else short_factor
        table = np.asarray(table, np.float64)
        if table.shape != (half,):
            raise ValueError(f"longrope factor tables must have {half} entries")
        for i in range(half):
            out[i] = float(theta) ** (-2.0 * i / rotary_dim) / table[i]
        return out
    for i in range(half):
        base = float(theta) ** (-2.0 * i / rotary_dim)
        if kind == "default":
            f = base
        elif kind == "linear":
            f = base / factor
        else:
            old, low, high = (float(original_max_position_embeddings), float(low_freq_factor),
                              float(high_freq_factor))
            wavelength = 2.0 * math.pi / base
            if wavelength < old / high:          # fast pair: kept
                f = base
            elif wavelength > old / low:         # slow pair: interpolated
                f = base / factor
            else:                                # between: linear blend
                s = (old / wavelength - low) / (high - low)
                f = (1.0 - s) * base / factor + s * base
        out[i] = f
    return out


def _mscale(scale, m=1.0):
    # [Models] "Scaled RoPE": the sharpening 0.1 * m * ln(s) + 1, and 1 for s <= 1
    return 1.0 if scale <= 1 else 0.1 * m * math.log(scale) + 1.0


def rope_attention_factor(kind="default", factor=1.0, *, mscale=None, mscale_all_dim=None,
                          attention_factor=None):
    """Factor multiplying cos and sin ([Models] "Scaled RoPE", rope_inv_freq and rope_tables).

    yarn: the given attention_factor, else mscale(factor, mscale) / mscale(factor, mscale_all_dim)
    when both are given and nonzero, else mscale(factor) = 0.1 ln(factor) + 1 (1 for factor <= 1).
    longrope: [Ster] scales both tables by "the attention factor" without a formula; reading: the
    given attention_factor, 1 when absent.  Other kinds: 1."""
    if kind == "yarn":
        if attention_factor is not None:
            return float(attention_factor)
        if mscale and mscale_all_dim:
            return _mscale(factor, mscale) / _mscale(factor, mscale_all_dim)
        return _mscale(factor)
    if kind == "longrope":
        return 1.0 if attention_factor is None else float(attention_factor)
    return 1.0


def yarn_softmax_scale(qk_dim, factor, mscale_all_dim=None):
    """Softmax scale with YaRN's temperature ([Models] "Multi-head latent attention": DeepSeek
    applies it to the scale): qk_dim^-0.5 times m^2, m = 0.1 * mscale_all_dim * ln(factor) + 1
    when mscale_all_dim is given and factor > 1, else m = 1."""
    sc = float(qk_dim) ** -0.5
    if mscale_all_dim:
        m = 0.1 * mscale_all_dim * math.log(factor) + 1.0 if factor > 1 else 1.0
        sc *= m * m
    return sc


def rope_angles(positions, inv_freq):
    """Angle of pair i at position p: p * inv_freq[i] ([Models] "Scaled RoPE", rope_tables;
    [Guide] §4 Rotary).  Returns positions.shape + (len(inv_freq),)."""
    return np.asarray(positions, dtype=np.float64)[..., None] * np.asarray(inv_freq, np.float64)


# ----------------------------------------------------------------------------------------------
# Per-row operations on head vectors
# ----------------------------------------------------------------------------------------------
def rms_norm(x, weight, eps):
    """[Guide] §3.2 RMSNorm: x / sqrt(mean(x^2) + eps), times the gain, over the last axis.

    Reading: the page rounds to the input dtype before the gain; the oracle keeps everything
    in float64 (exact definition), and the rounding difference is far inside the tolerance."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(weight, dtype=np.float64)


def rotate(x, positions, inv_freq, style="half", attention_factor=1.0):
    """Rotate the first R = 2*len(inv_freq) features of each row of x by its position.

    half:        pair (i, i + R/2)      ([Guide] §4 Rotary: feature i with feature i + hd/2)
    interleaved: pair (2i, 2i + 1)      ([Models] "Serving it": adjacent pairs; [Ster] "Overview")
    Each pair (a, b) at angle t becomes (a cos t - b sin t, a sin t + b cos t), with cos and sin
    multiplied by the attention factor ([Models] "Scaled RoPE", rope_tables).  Features at
    index >= R pass through unchanged ([Ster] "Overview": only that share rotates).
    positions must broadcast to x.shape[:-1]."""
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    half = len(inv_freq)
    if half == 0:
        return out
    R = 2 * half
    if R > x.shape[-1]:
        raise ValueError("rotary width exceeds head_dim")
    ang = rope_angles(np.broadcast_to(positions, x.shape[:-1]), inv_freq)
    c, s = attention_factor * np.cos(ang), attention_factor * np.sin(ang)
    if style == "half":
        a, b = x[..., :half], x[..., half:R]
        out[..., :half] = a * c - b * s
        out[..., half:R] = a * s + b * c
    elif style == "interleaved":
        a, b = x[..., 0:R:2], x[..., 1:R:2]
        out[..., 0:R:2] = a * c - b * s
        out[..., 1:R:2] = a * s + b * c
    else:
        raise ValueError(f"unknown rotation style {style!r}")
    return out


# ----------------------------------------------------------------------------------------------
# Mask and softmax core
# ----------------------------------------------------------------------------------------------
def allowed_mask(query_positions, key_positions, window, chunk=0, chunk_lookback=0):
    """May query at position qp attend key at position kp?

    Causal by positions, not indices ([Models] "What differs": causal_attention takes positions
    and key_positions).  Sliding window ([Models] "Sliding windows"): keys more than w - 1
    positions back are masked, so a query sees at most w keys including itself; w = 0 means
    no window.  Chunked attention ([Ster] llama4_text and Rnj-1.5 paragraphs): positions fall in
    chunks of `chunk` (chunk c holds c*chunk .. (c+1)*chunk - 1); a query sees the keys of its own
    chunk (llama4) and of the chunk_lookback chunks before it (Rnj-1.5: one); chunk = 0 means no
    chunking.  Reading: when both are set the key must pass both tests.
    Returns a [len(qp), len(kp)] bool array."""
    qp = np.asarray(query_positions, dtype=np.int64)[:, None]
    kp = np.asarray(key_positions, dtype=np.int64)[None, :]
    ok = kp <= qp
    if window > 0:
        ok &= (qp - kp) <= (window - 1)
    if chunk > 0:
        ok &= (kp // chunk) >= (qp // chunk) - chunk_lookback     # floor division
    return ok


def softmax_attention(q, k, v, allowed, scale, softcap=0.0, sink=None):
    """Masked softmax attention of one head: out_i = sum_j p_ij v_j with
    p_i = softmax over allowed j of s_ij, s_ij = scale * <q_i, k_j> ([Guide] §3.4 Attention).

    Soft-cap (reading; the pages name it without a formula, [Ster] "Overview"): s <- cap *
    tanh(s / cap) after scaling and before masking; cap = 0 means off.
    Learned sink ([Ster] gpt_oss paragraph): one more logit `sink` joins every row's softmax and
    its share is dropped: p_ij = exp(s_ij) / (sum_allowed exp(s_ij') + exp(sink)).  Reading: the
    sink is a logit in the units of the scaled scores, not scaled and not soft-capped.
    Max subtraction as in [Guide] §2.3.  A row with no allowed key has output 0 (reading:
    [Guide] §3.7 notes that such a row would otherwise be NaN; with a sink the sink takes the
    whole share, which gives the same 0)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    s = scale * (q @ k.T)
    if softcap > 0.0:
        s = softcap * np.tanh(s / softcap)
    out = np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    any_allowed = allowed.any(axis=1)
    if not any_allowed.any():
        return out
    s_masked = np.where(allowed, s, -np.inf)
    m = np.max(s_masked[any_allowed], axis=1, keepdims=True)
    if sink is not None:
        m = np.maximum(m, float(sink))
    p = np.where(allowed[any_allowed], np.exp(s[any_allowed] - m), 0.0)
    den = p.sum(axis=1, keepdims=True)
    if sink is not None:
        den = den + np.exp(float(sink) - m)
    out[any_allowed] = (p @ v) / den
    return out


# ----------------------------------------------------------------------------------------------
# The two entry points
# ----------------------------------------------------------------------------------------------
def _scale(head_dim, scale):
    # [Guide] §3.4: scores divided by sqrt(head_dim); [Ster] "Overview" lets a family replace it.
    return 1.0 / math.sqrt(head_dim) if not scale else float(scale)


def attn_prefill(q, k, v, positions, key_positions, *, inv_freq, style="half", n_cached=0,
                 window=0, q_norm_w=None, k_norm_w=None, eps=1e-6, scale=0.0, softcap=0.0,
                 query_rows=None, heads=None, batches=None, attention_factor=1.0, sinks=None,
                 chunk=0, chunk_lookback=0):
    """Causal prefill of one layer: [Models] "What differs" (DecoderAttention.forward).

    q [B, L, Hq, D], k and v [B, S, Hkv, D], positions [B, L], key_positions [B, S].
    Steps, in the page's order: per-head RMSNorm of q and of the new keys (when weights are
    given), then rotation of q at positions and of new keys at key_positions; keys j < n_cached
    come from the cache and are used as stored (already normed and rotated), values are never
    rotated.  Query head h reads KV head h // (Hq/Hkv) (reading: consecutive query heads share a
    KV head, i.e. K/V repeated with repeat_interleave, [Guide] §1.6).  Then masked softmax
    attention per head.  Returns out [B', L', Hq', D] for the selected batches, rows and heads.
    sinks: None or one logit per query head [Hq]; chunk, chunk_lookback: see allowed_mask.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, L, Hq, D = q.shape
    S, Hkv = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    positions = np.broadcast_to(np.asarray(positions, np.int64), (B, L))
    key_positions = np.broadcast_to(np.asarray(key_positions, np.int64), (B, S))
    batches = range(B) if batches is None else batches
    rows = np.arange(L) if query_rows is None else np.asarray(query_rows)
    heads = range(Hq) if heads is None else heads
    sc = _scale(D, scale)
    out = np.zeros((len(batches), len(rows), len(heads), D), dtype=np.float64)
    for bi, b in enumerate(batches):
        qb = q[b, rows]                                   # [L', Hq, D]
        kb = k[b].copy()                                  # [S, Hkv, D]
        if q_norm_w is not None:
            qb = rms_norm(qb, q_norm_w, eps)
        qb = rotate(qb, positions[b, rows][:, None], inv_freq, style, attention_factor)
        new = slice(n_cached, S)
        kn = kb[new]
        if k_norm_w is not None:
            kn = rms_norm(kn, k_norm_w, eps)
        kb[new] = rotate(kn, key_positions[b, new][:, None], inv_freq, style, attention_factor)
        allowed = allowed_mask(positions[b, rows], key_positions[b], window, chunk, chunk_lookback)
        for hi, h in enumerate(heads):
            g = h // G
            out[bi, :, hi] = softmax_attention(qb[:, h], kb[:, g], v[b, :, g], allowed, sc, softcap,
                                               None if sinks is None else sinks[h])
    return out


def attn_decode_one(q, k, v, n, *, inv_freq, style="half", window=0, q_norm_w=None, eps=1e-6,
                    scale=0.0, softcap=0.0, heads=None, attention_factor=1.0, sinks=None,
                    chunk=0, chunk_lookback=0):
    """Single-token decode of one sequence against its cache ([Guide] §3.3 KVCache, §3.7).

    q [Hq, D]; k, v [Hkv, >= n, D] hold the sequence's cache rows, slot j at position j, already
    normed and rotated (the new token's row is in slot n - 1: [Models] "What differs" rotates
    then appends).  The query sits at position n - 1: q is normed (when weighted) and rotated
    there; every cached key is in its past, so only the window can mask.  Returns [Hq', D]."""
    q = np.asarray(q, np.float64)
    Hq, D = q.shape
    Hkv = k.shape[0]
    G = Hq // Hkv
    heads = range(Hq) if heads is None else heads
    pos = n - 1
    qq = q if q_norm_w is None else rms_norm(q, q_norm_w, eps)
    qq = rotate(qq, np.full(Hq, pos), inv_freq, style, attention_factor)
    allowed = allowed_mask([pos], np.arange(n), window, chunk, chunk_lookback)
    sc = _scale(D, scale)
    out = np.zeros((len(heads), D), dtype=np.float64)
    for hi, h in enumerate(heads):
        g = h // G
        kk = np.asarray(k[g, :n], np.float64)
        vv = np.asarray(v[g, :n], np.float64)
        out[hi] = softmax_attention(qq[h:h + 1], kk, vv, allowed, sc, softcap,
                                    None if sinks is None else sinks[h])[0]
    return out


def attn_decode(q, kcache, vcache, lens, **kw):
    """attn_decode_one over a batch: q [B, Hq, D], caches [B, Hkv, Smax, D], lens [B]."""
    return np.stack([attn_decode_one(q[b], kcache[b], vcache[b], int(lens[b]), **kw)
                     for b in range(len(lens))])


# ----------------------------------------------------------------------------------------------
# Paged KV cache (reading of the pages' block manager, [Models] "Sliding windows" and the MLA
# section's paged pool; [Guide] §3.3 KVCache for what update computes)
# ----------------------------------------------------------------------------------------------
# Reading: a pool holds num_blocks blocks of block_size token slots for every KV head, laid out
# [num_blocks, Hkv, block_size, D]; sequence b's logical slot j (position j) lives in physical
# block table[b, j // block_size], slot j % block_size.  cache.update writes the step's rows at
# the sequence's next slots; attention then reads slots 0 .. len-1 in order.
def paged_rows(pool, table, b, n, block_size):
    """Logical rows 0 .. n-1 of sequence b: [Hkv, n, D] gathered slot by slot."""
    pool = np.asarray(pool)
    Hkv, D = pool.shape[1], pool.shape[3]
    out = np.empty((Hkv, n, D), dtype=np.float64)
    for j in range(n):
        blk = int(table[b][j // block_size])
        out[:, j] = pool[blk, :, j % block_size]
    return out


def paged_update(pool, table, start, rows, block_size):
    """cache.update on a paged pool: rows [B, L, Hkv, D] go to logical slots start[b] .. start[b] +
    L - 1 of each sequence; returns the new pool (a copy)."""
    pool = np.array(pool, copy=True)
    B, L = rows.shape[0], rows.shape[1]
    for b in range(B):
        for i in range(L):
            j = int(start[b]) + i
            pool[int(table[b][j // block_size]), :, j % block_size] = rows[b, i]
    return pool


def append_rows(k_new, key_positions, *, inv_freq, style="half", k_norm_w=None, eps=1e-6,
                attention_factor=1.0):
    """The rows cache.update receives for new keys ([Models] "What differs": k-norm when
    weighted, then rotation at the keys' positions; values are stored as they are)."""
    k = np.asarray(k_new, np.float64)
    if k_norm_w is not None:
        k = rms_norm(k, k_norm_w, eps)
    return rotate(k, np.asarray(key_positions)[..., None], inv_freq, style, attention_factor)


def attn_decode_paged(q, k_pool, v_pool, table, lens, block_size, **kw):
    """attn_decode over a paged pool: each sequence's cache rows gathered through its table."""
    outs = []
    for b in range(len(lens)):
        n = int(lens[b])
        kk = paged_rows(k_pool, table, b, n, block_size)
        vv = paged_rows(v_pool, table, b, n, block_size)
        outs.append(attn_decode_one(q[b], kk, vv, n, **kw))
    return np.stack(outs)


# ----------------------------------------------------------------------------------------------
# Multi-head latent attention, absorbed decode core ([Models] "Multi-head latent attention",
# paged_forward)
# ----------------------------------------------------------------------------------------------
MLA_LATENT = 512   # kv_lora_rank of DeepSeek-V2/V3 and Kimi K2
MLA_ROPE = 64      # qk_rope_head_dim


def mla_decode_one(q, rows, n, scale):
    """One sequence: q [H, 576] (the absorbed query W_uk^T q_nope followed by the rotated q_rope),
    rows [>= n, 576] (the cached [c, k_rope] rows, slot j at position j).  Multi-query attention
    with one KV head of width 576 whose values are the first 512 features of the same rows:
    out [H, 512] = softmax(scale * q rows^T) rows[:, :512].  The query sits at position n - 1 and
    sees every cached row."""
    q = np.asarray(q, np.float64)
    rows = np.asarray(rows[:n], np.float64)
    allowed = np.ones((q.shape[0], n), bool)
    return softmax_attention(q, rows, rows[:, :MLA_LATENT], allowed, float(scale))


def mla_decode(q, cache, lens, scale):
    """mla_decode_one over a batch: q [B, H, 576], cache [B, Smax, 576], lens [B]."""
    return np.stack([mla_decode_one(q[b], cache[b], int(lens[b]), scale)
                     for b in range(len(lens))])
