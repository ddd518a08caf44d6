"""Pins of the float64 oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: a number the pages print (tests/golden/), a
closed form or invariant the pages state, a textbook/library routine (complex multiplication,
torch's CPU scaled_dot_product_attention in float64), or brute force on tiny inputs.  Together
they are chosen so that a dropped term, a wrong sign, a wrong pairing, a wrong head map, an
off-by-one window or a wrong scale in the oracle fails at least one of them.
"""
import math

import numpy as np
import pytest

import oracle
from synth import WORKLOADS, prefill_inputs

rng = np.random.default_rng(12345)


# ----------------------------------------------------------------------------------------------
# Frequencies
# ----------------------------------------------------------------------------------------------
def test_last_pair_wavelength_matches_page(golden):
    g = golden("rope_worked_values.json")["last_pair_wavelength"]
    f = oracle.rope_inv_freq(g["head_dim"], g["theta"])
    wavelength = 2 * math.pi / f[-1]
    # "about 2.6 million": two significant digits
    assert round(wavelength, -5) == g["approx_positions"]


def test_first_pair_period_matches_page(golden):
    g = golden("rope_worked_values.json")["first_pair_period"]
    for d, theta in ((128, 5e5), (64, 1e4), (32, 1e6)):
        f = oracle.rope_inv_freq(d, theta)
        assert 2 * math.pi / f[0] == pytest.approx(g["period_positions"], rel=0, abs=1e-12)


def test_guide_frequencies(golden):
    g = golden("rope_worked_values.json")["guide_pairing"]
    d, base = g["head_dim"], g["base"]
    f = oracle.rope_inv_freq(d, base)
    assert len(f) == d // 2 == g["partner_offset"]
    # theta_i = base^(-2i/d): successive pairs slow down by the constant ratio base^(-2/d)
    ratios = f[1:] / f[:-1]
    assert np.allclose(ratios, base ** (-2.0 / d), rtol=1e-13)
    assert f[0] == 1.0


def test_linear_squeezes_positions():
    # [Models] Scaled RoPE: under linear scaling position p looks like p / factor
    d, theta, s = 64, 1e4, 4.0
    x = rng.standard_normal((7, d))
    p = rng.uniform(0, 5000, size=7)
    a = oracle.rotate(x, p[:, None][:, 0], oracle.rope_inv_freq(d, theta, "linear", factor=s))
    b = oracle.rotate(x, (p / s), oracle.rope_inv_freq(d, theta))
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-9)


def test_scalings_reduce_to_default_at_factor_one():
    for d, theta in ((128, 5e5), (64, 1e4)):
        base = oracle.rope_inv_freq(d, theta)
        lin = oracle.rope_inv_freq(d, theta, "linear", factor=1.0)
        l3 = oracle.rope_inv_freq(d, theta, "llama3", factor=1.0, low_freq_factor=1.0,
                                  high_freq_factor=4.0, original_max_position_embeddings=8192)
        np.testing.assert_allclose(lin, base, rtol=1e-15)
        np.testing.assert_allclose(l3, base, rtol=1e-14)


def _llama3(d=128, theta=5e5, factor=8.0, low=1.0, high=4.0, old=8192.0):
    return oracle.rope_inv_freq(d, theta, "llama3", factor=factor, low_freq_factor=low,
                                high_freq_factor=high, original_max_position_embeddings=old)


def test_llama3_bands_follow_page_prose():
    # [Models] Scaled RoPE: keep pairs with wavelength < old/high, divide pairs with wavelength
    # > old/low by the factor, blend in between.  The llama3 workload: factor 8, low 1, high 4,
    # original context 8192, so the bands are split at wavelengths 2048 and 8192.
    base = oracle.rope_inv_freq(128, 5e5)
    f = _llama3()
    wl = 2 * math.pi / base
    kept, divided = wl < 2048, wl > 8192
    mid = ~kept & ~divided
    np.testing.assert_array_equal(f[kept], base[kept])
    np.testing.assert_allclose(f[divided], base[divided] / 8, rtol=1e-15)
    assert np.all(f[mid] < base[mid]) and np.all(f[mid] > base[mid] / 8)
    # the per-pair divisor form (GGUF rope_freqs, [Models] "The registry") lies in [1, factor]
    div = base / f
    assert np.all(div >= 1 - 1e-15) and np.all(div <= 8 + 1e-12)
    # divisors never decrease from fast pairs to slow pairs
    assert np.all(np.diff(div) >= -1e-12)
    assert (kept.sum(), mid.sum(), divided.sum()) == (29, 6, 29)


def test_llama3_is_continuous_at_band_edges():
    # Move theta so that a pair sits exactly on each band edge and just beside it.
    d, factor, low, high, old = 8, 8.0, 1.0, 4.0, 8192.0
    for edge in (old / high, old / low):
        # choose theta so that pair 1 has wavelength `edge`: 2*pi*theta^(2/d) = edge
        theta = (edge / (2 * math.pi)) ** (d / 2)
        for eps in (-1e-9, 0.0, 1e-9):
            f = _llama3(d, theta * (1 + eps), factor, low, high, old)
            f0 = _llama3(d, theta, factor, low, high, old)
            assert f[1] == pytest.approx(f0[1], rel=1e-7)


def _rotations_over(old, inv_freq):
    # full turns a pair makes over the original context: old * frequency / (2 pi)
    return old * np.asarray(inv_freq) / (2 * math.pi)


@pytest.mark.parametrize("d,theta,old,factor", [(128, 1e4, 4096, 4.0), (128, 1e6, 32768, 4.0),
                                                (64, 5e5, 8192, 16.0)])
def test_yarn_split_follows_rotation_counts(d, theta, old, factor):
    # [Models] Scaled RoPE: YaRN keeps pairs that turn more than beta_fast (32) times over the
    # original context, interpolates pairs that turn fewer than beta_slow (1) times, and ramps
    # linearly in between.  The turn counts here come from the plain frequencies, not from the
    # oracle's ramp; rounding the ramp ends outwards keeps these two sets exact.
    base = oracle.rope_inv_freq(d, theta)
    f = oracle.rope_inv_freq(d, theta, "yarn", factor, original_max_position_embeddings=old)
    turns = _rotations_over(old, base)
    fast, slow = turns >= 32, turns <= 1
    assert fast.any() and slow.any()
    np.testing.assert_array_equal(f[fast], base[fast])
    np.testing.assert_allclose(f[slow], base[slow] / factor, rtol=1e-15)
    ratio = f / base
    assert np.all(ratio <= 1 + 1e-15) and np.all(ratio >= 1 / factor - 1e-15)
    assert np.all(np.diff(ratio) <= 1e-15)                 # never rises from fast to slow pairs
    mid = ~fast & ~slow
    assert np.all(ratio[mid][1:-1] < 1) and np.all(ratio[mid][1:-1] > 1 / factor)
    # other beta thresholds move the split accordingly
    f2 = oracle.rope_inv_freq(d, theta, "yarn", factor, original_max_position_embeddings=old,
                              beta_fast=8, beta_slow=2)
    np.testing.assert_array_equal(f2[turns >= 8], base[turns >= 8])
    np.testing.assert_allclose(f2[turns <= 2], base[turns <= 2] / factor, rtol=1e-15)


def test_yarn_truncate_only_widens_the_ramp_ends():
    # truncate=False keeps the continuous ramp ends; the rounded ends can only widen the kept and
    # the interpolated sets, so each frequency moves toward the nearer end
    base = oracle.rope_inv_freq(128, 1e4)
    t = oracle.rope_inv_freq(128, 1e4, "yarn", 4.0, original_max_position_embeddings=4096)
    c = oracle.rope_inv_freq(128, 1e4, "yarn", 4.0, original_max_position_embeddings=4096,
                             truncate=False)
    turns = _rotations_over(4096, base)
    np.testing.assert_array_equal(c[turns >= 32], base[turns >= 32])
    np.testing.assert_allclose(c[turns <= 1], base[turns <= 1] / 4, rtol=1e-15)
    assert not np.array_equal(t, c)


def test_yarn_and_longrope_reduce_to_plain_rope():
    base = oracle.rope_inv_freq(128, 1e6)
    np.testing.assert_allclose(
        oracle.rope_inv_freq(128, 1e6, "yarn", 1.0, original_max_position_embeddings=8192), base,
        rtol=1e-15)
    assert oracle.rope_attention_factor("yarn", 1.0) == 1.0
    ones = np.ones(64)
    np.testing.assert_allclose(
        oracle.rope_inv_freq(128, 1e6, "longrope", original_max_position_embeddings=4096,
                             short_factor=ones, long_factor=ones * 3, seq_len=100), base, rtol=0)
    # all long factors equal to s: linear scaling by s once the sequence passes the original
    np.testing.assert_allclose(
        oracle.rope_inv_freq(128, 1e6, "longrope", original_max_position_embeddings=4096,
                             short_factor=ones, long_factor=ones * 3, seq_len=4097),
        oracle.rope_inv_freq(128, 1e6, "linear", 3.0), rtol=1e-15)


def test_longrope_switches_past_the_original_context():
    # [Ster] Overview: short factors while the sequence is within original_max_position_embeddings,
    # long ones once it goes past
    short, long_ = np.linspace(1, 2, 32), np.linspace(1, 8, 32)
    kw = dict(original_max_position_embeddings=4096, short_factor=short, long_factor=long_)
    base = oracle.rope_inv_freq(64, 1e4)
    np.testing.assert_allclose(oracle.rope_inv_freq(64, 1e4, "longrope", seq_len=4096, **kw),
                               base / short, rtol=1e-15)
    np.testing.assert_allclose(oracle.rope_inv_freq(64, 1e4, "longrope", seq_len=4097, **kw),
                               base / long_, rtol=1e-15)


def test_yarn_sharpening_values():
    # [Models] Scaled RoPE: cos and sin multiplied by 0.1 ln s + 1; with both mscale and
    # mscale_all_dim given (DeepSeek) the factor is their ratio, which is 1 when they are equal;
    # a stated attention_factor is used as is.  Checked at s = e^5 (0.1 * 5 + 1 = 1.5).
    assert oracle.rope_attention_factor("yarn", math.exp(5.0)) == pytest.approx(1.5, rel=1e-15)
    assert oracle.rope_attention_factor("yarn", 40.0, mscale=1.0, mscale_all_dim=1.0) == 1.0
    assert oracle.rope_attention_factor("yarn", 40.0, mscale=0.707, mscale_all_dim=0.707) == 1.0
    assert oracle.rope_attention_factor("yarn", 40.0, attention_factor=1.25) == 1.25
    assert oracle.rope_attention_factor("longrope", 8.0) == 1.0
    assert oracle.rope_attention_factor("llama3", 8.0) == 1.0
    # temperature on the softmax scale ([Models] MLA): 1/sqrt(qk) times m^2 with
    # m = 0.1 * mscale_all_dim * ln(factor) + 1; at factor e^10 and mscale_all_dim 1, m = 2
    assert oracle.yarn_softmax_scale(192, math.exp(10.0), 1.0) == pytest.approx(4 / math.sqrt(192),
                                                                              rel=1e-14)
    assert oracle.yarn_softmax_scale(192, 1.0, 1.0) == 192 ** -0.5
    assert oracle.yarn_softmax_scale(128, 40.0) == 128 ** -0.5


@pytest.mark.parametrize("style", ["half", "interleaved"])
def test_attention_factor_scales_rotated_norm(style):
    # cos and sin both multiplied by a: each rotated pair's length is multiplied by a, the
    # features past the rotary width are untouched
    x = rng.standard_normal((5, 3, 96))
    f = oracle.rope_inv_freq(64, 1e4, "yarn", 8.0, original_max_position_embeddings=2048)
    a = oracle.rope_attention_factor("yarn", 8.0)
    y = oracle.rotate(x, np.arange(5)[:, None] * 997, f, style, attention_factor=a)
    np.testing.assert_allclose(np.linalg.norm(y[..., :64], axis=-1),
                               a * np.linalg.norm(x[..., :64], axis=-1), rtol=1e-12)
    np.testing.assert_array_equal(y[..., 64:], x[..., 64:])


def test_unknown_rope_kind_raises():
    with pytest.raises(ValueError):
        oracle.rope_inv_freq(64, 1e4, "dynamic")
    with pytest.raises(ValueError):
        oracle.rope_inv_freq(64, 1e4, "longrope", short_factor=np.ones(3), seq_len=1)
    with pytest.raises(ValueError):
        oracle.rope_inv_freq(63, 1e4)


# ----------------------------------------------------------------------------------------------
# Rotation
# ----------------------------------------------------------------------------------------------
def test_half_split_rotation_is_complex_multiplication():
    d, R = 64, 64
    f = oracle.rope_inv_freq(R, 1e4)
    x = rng.standard_normal((5, d))
    p = np.array([0, 1, 17, 999, 4095])
    y = oracle.rotate(x, p, f, "half")
    z = (x[:, :R // 2] + 1j * x[:, R // 2:R]) * np.exp(1j * np.outer(p, f))
    np.testing.assert_allclose(y[:, :R // 2], z.real, atol=1e-12)
    np.testing.assert_allclose(y[:, R // 2:R], z.imag, atol=1e-12)


def test_guide_pairing_one_hot(golden):
    g = golden("rope_worked_values.json")["guide_pairing"]
    d, off, base = g["head_dim"], g["partner_offset"], g["base"]
    f = oracle.rope_inv_freq(d, base)
    m = 37
    for i in (0, 5, 31):
        e = np.zeros(d)
        e[i] = 1.0
        y = oracle.rotate(e[None], np.array([m]), f, "half")[0]
        nz = set(np.flatnonzero(np.abs(y) > 1e-15))
        assert nz <= {i, i + off}
        ang = m * base ** (-2.0 * i / d)
        assert y[i] == pytest.approx(math.cos(ang), abs=1e-12)
        assert y[i + off] == pytest.approx(math.sin(ang), abs=1e-12)


def _deinterleave(R, D):
    # [Models] "Serving it": adjacent pairs (0,1),(2,3),... reordered to split-half pairing
    return np.concatenate([np.arange(0, R, 2), np.arange(1, R, 2), np.arange(R, D)])


@pytest.mark.parametrize("R,D", [(64, 64), (64, 128), (32, 128)])
def test_interleaved_equals_half_after_deinterleave(R, D):
    f = oracle.rope_inv_freq(R, 1e4)
    x = rng.standard_normal((6, D))
    p = rng.integers(0, 10000, size=6)
    P = _deinterleave(R, D)
    a = oracle.rotate(x, p, f, "interleaved")[:, P]
    b = oracle.rotate(x[:, P], p, f, "half")
    np.testing.assert_allclose(a, b, atol=1e-12)


@pytest.mark.parametrize("style", ["half", "interleaved"])
def test_rotation_preserves_norm_and_tail(style):
    D, R = 128, 64
    f = oracle.rope_inv_freq(R, 1e4)
    x = rng.standard_normal((9, D))
    p = rng.integers(0, 50000, size=9)
    y = oracle.rotate(x, p, f, style)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    np.testing.assert_array_equal(y[:, R:], x[:, R:])


def test_zero_rotary_dim_is_identity():
    x = rng.standard_normal((3, 16))
    np.testing.assert_array_equal(oracle.rotate(x, np.array([1, 2, 3]), np.zeros(0)), x)


@pytest.mark.parametrize("style", ["half", "interleaved"])
def test_scores_depend_only_on_position_difference(style):
    D = 64
    f = oracle.rope_inv_freq(D, 1e4)
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    ref = oracle.rotate(q[None], np.array([50]), f, style)[0] @ oracle.rotate(k[None], np.array([20]), f, style)[0]
    for shift in (1, 123, 7777):
        s = (oracle.rotate(q[None], np.array([50 + shift]), f, style)[0]
             @ oracle.rotate(k[None], np.array([20 + shift]), f, style)[0])
        assert s == pytest.approx(ref, abs=1e-10)


# ----------------------------------------------------------------------------------------------
# Norm, scale, soft-cap
# ----------------------------------------------------------------------------------------------
def test_rms_norm_unit_rms_and_scale_invariance():
    x = rng.standard_normal((4, 128)) * 3.7 + 0.5
    y = oracle.rms_norm(x, np.ones(128), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-14)
    np.testing.assert_allclose(oracle.rms_norm(5.0 * x, np.ones(128), 0.0), y, rtol=1e-13)
    w = rng.uniform(0.5, 1.5, 128)
    np.testing.assert_allclose(oracle.rms_norm(x, w, 0.0), y * w, rtol=1e-14)
    # eps enters under the square root: x == 0 stays 0, tiny rows are damped
    np.testing.assert_array_equal(oracle.rms_norm(np.zeros((1, 8)), np.ones(8), 1e-6), 0.0)


def test_scale_gives_unit_score_variance(golden):
    g = golden("score_variance.json")
    d = g["head_dim"]
    r = np.random.default_rng(7)
    q = r.standard_normal((20000, d))
    k = r.standard_normal((20000, d))
    raw = np.einsum("nd,nd->n", q, k)
    assert raw.var() == pytest.approx(g["unscaled_variance"], rel=0.05)
    # the oracle's default scale applied through the full path: one key, v = score probe
    allowed = np.ones((1, 1), bool)
    s = np.array([oracle.softmax_attention(q[i:i + 1], k[i:i + 1], np.array([[1.0]]), allowed, 0)[0, 0]
                  for i in range(3)])
    assert np.all(s == 1.0)  # single key: weight 1 whatever the scale
    from oracle.gqa_oracle import _scale
    assert (raw * _scale(d, 0.0)).var() == pytest.approx(g["scaled_variance"], rel=0.05)


def test_softcap_limits():
    q = rng.standard_normal((3, 16)) * 6
    k = rng.standard_normal((10, 16)) * 6
    v = rng.standard_normal((10, 4))
    allowed = np.ones((3, 10), bool)
    a = oracle.softmax_attention(q, k, v, allowed, 0.25, 0.0)
    b = oracle.softmax_attention(q, k, v, allowed, 0.25, 1e9)
    np.testing.assert_allclose(a, b, atol=1e-12)
    # capped scores stay inside (-cap, cap): with cap 1 the weights' ratio is at most e^2
    c = oracle.softmax_attention(q, k, np.eye(10), allowed, 0.25, 1.0)
    assert np.all(c.max(axis=1) / c.min(axis=1) <= math.exp(2.0) + 1e-9)


def test_softmax_core_brute_force():
    # scalar loops with math.exp / math.tanh against the vectorised core
    q = rng.standard_normal((5, 8))
    k = rng.standard_normal((7, 8))
    v = rng.standard_normal((7, 3))
    allowed = rng.random((5, 7)) < 0.6
    allowed[0] = False
    for cap in (0.0, 2.0):
        got = oracle.softmax_attention(q, k, v, allowed, 0.3, cap)
        for i in range(5):
            sc = []
            for j in range(7):
                if allowed[i, j]:
                    s = 0.3 * sum(q[i, t] * k[j, t] for t in range(8))
                    if cap:
                        s = cap * math.tanh(s / cap)
                    sc.append((s, j))
            if not sc:
                assert np.all(got[i] == 0)
                continue
            m = max(s for s, _ in sc)
            w = [(math.exp(s - m), j) for s, j in sc]
            tot = sum(e for e, _ in w)
            for c in range(3):
                assert got[i, c] == pytest.approx(sum(e * v[j, c] for e, j in w) / tot, abs=1e-12)


# ----------------------------------------------------------------------------------------------
# Mask and positions (integer exact)
# ----------------------------------------------------------------------------------------------
@pytest.mark.parametrize("window", [0, 1, 2, 5, 16, 17, 100])
def test_mask_probe_counts_allowed_keys(window):
    # q = 0 gives a uniform softmax over the allowed keys; v = [1, kp, kp^2] then reports the
    # count-normalised first and second moments, which fix the allowed set when it is an
    # interval.  [Models] "Sliding windows": keys more than w - 1 positions back are masked.
    S, L = 40, 40
    kp = np.arange(S)
    qp = np.arange(L)
    v = np.stack([np.ones(S), kp, kp.astype(float) ** 2], axis=1)
    out = oracle.softmax_attention(np.zeros((L, 4)), np.ones((S, 4)), v,
                                   oracle.allowed_mask(qp, kp, window), 1.0)
    for i in range(L):
        lo = 0 if window == 0 else max(0, i - window + 1)
        keys = np.arange(lo, i + 1)                          # integer definition
        assert out[i, 0] == pytest.approx(1.0)
        assert out[i, 1] == pytest.approx(keys.mean(), abs=1e-9)
        assert out[i, 2] == pytest.approx((keys.astype(float) ** 2).mean(), abs=1e-7)


def test_mask_by_positions_not_indices():
    # causal_attention masks by positions: a query at position 10 sees keys at positions <= 10
    m = oracle.allowed_mask([10], [3, 8, 10, 11, 40], 0)
    np.testing.assert_array_equal(m[0], [True, True, True, False, False])
    m = oracle.allowed_mask([10], [3, 8, 10, 11, 40], 3)
    np.testing.assert_array_equal(m[0], [False, True, True, False, False])


def test_fully_masked_row_is_zero():
    out = oracle.softmax_attention(np.ones((2, 4)), np.ones((3, 4)), np.ones((3, 2)),
                                   np.array([[False] * 3, [True] * 3]), 1.0)
    np.testing.assert_array_equal(out[0], 0.0)
    np.testing.assert_allclose(out[1], 1.0)


@pytest.mark.parametrize("chunk,lookback", [(1, 0), (4, 0), (7, 0), (8, 1), (5, 1), (6, 2),
                                            (64, 0)])
def test_chunk_mask_probe_counts_allowed_keys(chunk, lookback):
    # [Ster] llama4_text: a query sees only the keys of its own chunk of attention_chunk_size
    # positions; Rnj-1.5: also the chunk before it.  Integer definition: the query's chunk starts
    # at i - i mod chunk, and `lookback` whole chunks before that are visible too.
    S = L = 40
    kp = np.arange(S)
    v = np.stack([np.ones(S), kp, kp.astype(float) ** 2], axis=1)
    out = oracle.softmax_attention(np.zeros((L, 4)), np.ones((S, 4)), v,
                                   oracle.allowed_mask(np.arange(L), kp, 0, chunk, lookback), 1.0)
    for i in range(L):
        start = i - i % chunk
        keys = np.arange(max(0, start - lookback * chunk), i + 1)
        assert out[i, 0] == pytest.approx(1.0)
        assert out[i, 1] == pytest.approx(keys.mean(), abs=1e-9)
        assert out[i, 2] == pytest.approx((keys.astype(float) ** 2).mean(), abs=1e-7)


def test_chunk_mask_with_window_and_negative_positions():
    # both tests apply; chunks tile negative positions too (chunk c = [c*C, (c+1)*C))
    m = oracle.allowed_mask([9], np.arange(0, 12), 3, 4, 1)
    np.testing.assert_array_equal(np.flatnonzero(m[0]), [7, 8, 9])
    m = oracle.allowed_mask([-3], np.arange(-12, 0), 0, 4, 0)
    np.testing.assert_array_equal(np.flatnonzero(m[0]) - 12, [-4, -3])


def test_sink_closed_forms():
    # [Ster] gpt_oss: one extra logit per head joins the softmax and its share is dropped.
    # One allowed key with score s: weight e^s / (e^s + e^sink) = 1 / (1 + e^(sink - s)).
    q = np.array([[0.5, -1.0, 2.0]])
    k = np.array([[1.0, 0.25, 0.75]])
    v = np.array([[3.0, -2.0]])
    s0 = 0.4 * (0.5 - 0.25 + 1.5)
    for sink in (-3.0, 0.0, 1.7, 40.0):
        got = oracle.softmax_attention(q, k, v, np.array([[True]]), 0.4, sink=sink)
        w = 1.0 / (1.0 + math.exp(sink - s0))
        np.testing.assert_allclose(got[0], w * v[0], rtol=1e-13)
    # constant values: the output is the share the keys keep, Z / (Z + e^sink)
    qq = rng.standard_normal((3, 6))
    kk = rng.standard_normal((9, 6))
    allowed = np.tril(np.ones((3, 9), bool), 6)
    got = oracle.softmax_attention(qq, kk, np.ones((9, 1)), allowed, 0.5, sink=0.3)
    for i in range(3):
        z = sum(math.exp(0.5 * float(qq[i] @ kk[j])) for j in range(9) if allowed[i, j])
        assert got[i, 0] == pytest.approx(z / (z + math.exp(0.3)), rel=1e-13)
    # a sink at -inf is no sink; a row with no allowed key stays 0
    vv = rng.standard_normal((9, 2))
    np.testing.assert_array_equal(oracle.softmax_attention(qq, kk, vv, allowed, 0.5, sink=-np.inf),
                                  oracle.softmax_attention(qq, kk, vv, allowed, 0.5))
    z = oracle.softmax_attention(qq, kk, np.ones((9, 2)), np.zeros((3, 9), bool), 0.5, sink=2.0)
    np.testing.assert_array_equal(z, 0.0)


@pytest.mark.parametrize("cap", [0.0, 2.0])
def test_sink_against_torch_sdpa_virtual_key(cap):
    # the sink as one more key: give q an extra feature 1 and that key the feature sink/scale with
    # value 0, every real key feature 0; torch's float64 SDPA then sees exactly the sink logit.
    # (Soft-cap changes the real scores only; with a cap the check runs on the capped scores.)
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    L, S, D, scale = 6, 11, 8, 0.37
    q = rng.standard_normal((L, D))
    k = rng.standard_normal((S, D))
    v = rng.standard_normal((S, 3))
    allowed = oracle.allowed_mask(np.arange(5, 5 + L), np.arange(S), 4)
    sink = 0.8
    got = oracle.softmax_attention(q, k, v, allowed, scale, cap, sink=sink)
    if cap:
        s = cap * np.tanh(scale * (q @ k.T) / cap)          # capped scores, then as logits
        qx = np.concatenate([s, np.ones((L, 1))], axis=1)
        kx = np.concatenate([np.eye(S), np.zeros((S, 1))], axis=1)
        vk = np.concatenate([np.zeros((1, S)), [[sink]]], axis=1)
        kx = np.concatenate([kx, vk], axis=0)
        sc = 1.0
    else:
        qx = np.concatenate([q, np.ones((L, 1))], axis=1)
        kx = np.concatenate([np.concatenate([k, np.zeros((S, 1))], axis=1),
                             np.concatenate([np.zeros((1, D)), [[sink / scale]]], axis=1)])
        sc = scale
    vx = np.concatenate([v, np.zeros((1, 3))])
    mask = np.concatenate([allowed, np.ones((L, 1), bool)], axis=1)
    ref = F.scaled_dot_product_attention(torch.from_numpy(qx)[None], torch.from_numpy(kx)[None],
                                         torch.from_numpy(vx)[None],
                                         attn_mask=torch.from_numpy(mask)[None], scale=sc)
    np.testing.assert_allclose(got, ref[0].numpy(), atol=1e-13)


# ----------------------------------------------------------------------------------------------
# Whole-path equivalences and library cross-checks
# ----------------------------------------------------------------------------------------------
def _small(wl_name="qwen3_prefill_bf16", **kw):
    wl = WORKLOADS[wl_name].with_(**kw)
    return wl


def _prefill(wl, x, **extra):
    kw = dict(inv_freq=oracle.rope_inv_freq(wl.rotary_dim, wl.theta, wl.rope_kind, wl.factor,
                                            wl.low_freq_factor, wl.high_freq_factor,
                                            wl.original_max_pos),
              style=wl.style, n_cached=wl.n_cached, window=wl.window, eps=wl.eps,
              softcap=wl.softcap, q_norm_w=x.get("q_norm_w"), k_norm_w=x.get("k_norm_w"))
    kw.update(extra)
    return oracle.attn_prefill(x["q"], x["k"], x["v"], x["positions"], x["key_positions"], **kw)


def test_window_zero_equals_window_beyond_sequence():
    wl = _small(B=1, L=48, S=48, Hq=4, Hkv=2, D=16, rotary_dim=16)
    x = prefill_inputs(wl, seed=11)
    a = _prefill(wl.with_(window=0), x)
    b = _prefill(wl.with_(window=48), x)
    c = _prefill(wl.with_(window=10**6), x)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a, c)
    d = _prefill(wl.with_(window=47), x)
    assert np.abs(d - a).max() > 1e-6          # one key fewer for the last query


def test_gqa_equals_mha_with_repeated_kv():
    wl = _small(B=2, L=20, S=20, Hq=6, Hkv=2, D=16, rotary_dim=8, window=7)
    x = prefill_inputs(wl, seed=12)
    a = _prefill(wl, x)
    G = wl.Hq // wl.Hkv
    xm = dict(x)
    xm["k"] = np.repeat(x["k"], G, axis=2)       # repeat_interleave on the head axis
    xm["v"] = np.repeat(x["v"], G, axis=2)
    b = _prefill(wl.with_(Hkv=wl.Hq), xm)
    np.testing.assert_allclose(a, b, atol=1e-13)


@pytest.mark.parametrize("window", [0, 5])
def test_against_torch_sdpa_float64(window):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    wl = _small(B=2, L=24, S=24, Hq=8, Hkv=2, D=16, rotary_dim=0, qk_norm=False, window=window)
    x = prefill_inputs(wl, seed=13, q_scale=2.0)
    got = _prefill(wl, x)                                         # [B, L, Hq, D]
    q = torch.from_numpy(x["q"].astype(np.float64)).permute(0, 2, 1, 3)
    k = torch.from_numpy(x["k"].astype(np.float64)).permute(0, 2, 1, 3)
    v = torch.from_numpy(x["v"].astype(np.float64)).permute(0, 2, 1, 3)
    i = torch.arange(24)
    mask = (i[None, :] <= i[:, None])
    if window:
        mask &= (i[:, None] - i[None, :]) <= window - 1
    ref = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, enable_gqa=True)
    np.testing.assert_allclose(got, ref.permute(0, 2, 1, 3).numpy(), atol=1e-12)


def test_decode_equals_last_prefill_row():
    # [Guide] section 9.3: cached decoding equals recomputing the whole sequence
    wl = _small("llama31_decode_bf16", B=1, L=30, S=30, Hq=8, Hkv=2, D=32, rotary_dim=32,
                qk_norm=True, window=9)
    x = prefill_inputs(wl.with_(kind="prefill"), seed=14)
    inv = oracle.rope_inv_freq(32, 5e5, "llama3", 8.0, 1.0, 4.0, 8192.0)
    full = _prefill(wl, x, inv_freq=inv)[0, -1]                  # [Hq, D]
    # the cache holds normed, rotated keys at their positions
    kc = oracle.rotate(oracle.rms_norm(x["k"][0], x["k_norm_w"], wl.eps),
                       np.arange(30)[:, None], inv, "half")
    kc = kc.transpose(1, 0, 2)                                     # [Hkv, S, D]
    vc = x["v"][0].transpose(1, 0, 2)
    dec = oracle.attn_decode_one(x["q"][0, -1], kc, vc, 30, inv_freq=inv, window=9,
                                 q_norm_w=x["q_norm_w"], eps=wl.eps)
    np.testing.assert_allclose(dec, full, atol=1e-13)


def test_chunked_prefill_equals_tail_of_full_prefill():
    wl = _small("chunked_prefill_bf16_w4096", B=1, L=40, S=40, n_cached=0, Hq=6, Hkv=2, D=32,
                rotary_dim=16, window=13, softcap=3.0, qk_norm=True)
    x = prefill_inputs(wl, seed=15)
    inv = oracle.rope_inv_freq(16, 1e4)
    full = _prefill(wl, x, inv_freq=inv)
    nc = 28
    kc = x["k"].astype(np.float64)
    kc[:, :nc] = oracle.rotate(oracle.rms_norm(x["k"][:, :nc], x["k_norm_w"], wl.eps),
                               x["key_positions"][:, :nc, None], inv, "interleaved")
    xc = dict(x, k=kc, q=x["q"][:, nc:], positions=x["positions"][:, nc:])
    tail = _prefill(wl.with_(n_cached=nc), xc, inv_freq=inv)
    np.testing.assert_allclose(tail, full[:, nc:], atol=1e-13)


def test_selected_rows_and_heads_match_full():
    wl = _small(B=2, L=33, S=33, Hq=4, Hkv=2, D=16, rotary_dim=16)
    x = prefill_inputs(wl, seed=16)
    full = _prefill(wl, x)
    part = _prefill(wl, x, query_rows=[0, 7, 32], heads=[3, 1], batches=[1])
    np.testing.assert_array_equal(part[0], full[1][[0, 7, 32]][:, [3, 1]])


def test_chunks_without_lookback_restart_the_sequence():
    # [Ster] llama4_text: each query sees only its own chunk, so attending the whole sequence
    # equals attending each chunk on its own (positions kept, rotation included)
    wl = _small(B=1, L=30, S=30, Hq=4, Hkv=2, D=16, rotary_dim=16, qk_norm=True)
    x = prefill_inputs(wl, seed=15)
    C = 8
    whole = _prefill(wl, x, chunk=C)
    for c0 in range(0, 30, C):
        part = {k: (v[:, c0:c0 + C] if k in ("q", "k", "v", "positions", "key_positions") else v)
                for k, v in x.items()}
        alone = _prefill(wl.with_(L=len(range(c0, min(30, c0 + C)))), part)
        np.testing.assert_allclose(whole[:, c0:c0 + C], alone, atol=1e-13)


def test_decode_equals_last_prefill_row_with_sinks_and_chunks():
    wl = _small("llama31_decode_bf16", B=1, L=37, S=37, Hq=8, Hkv=2, D=32, rotary_dim=32)
    x = prefill_inputs(wl.with_(kind="prefill"), seed=16)
    inv = oracle.rope_inv_freq(32, 5e5, "llama3", 8.0, 1.0, 4.0, 8192.0)
    sinks = rng.standard_normal(8) * 2.0
    for chunk, lookback in ((8, 1), (16, 0), (0, 0)):
        full = _prefill(wl, x, inv_freq=inv, sinks=sinks, chunk=chunk,
                        chunk_lookback=lookback)[0, -1]
        kc = oracle.rotate(x["k"][0], np.arange(37)[:, None], inv, "half").transpose(1, 0, 2)
        vc = x["v"][0].transpose(1, 0, 2)
        dec = oracle.attn_decode_one(x["q"][0, -1], kc, vc, 37, inv_freq=inv, sinks=sinks,
                                     chunk=chunk, chunk_lookback=lookback)
        np.testing.assert_allclose(dec, full, atol=1e-13)


# ----------------------------------------------------------------------------------------------
# Paged cache
# ----------------------------------------------------------------------------------------------
def _contiguous_to_pool(cache, block_size, perm):
    """A [B, Hkv, Smax, D] cache cut into blocks; logical block i of sequence b goes to physical
    block perm[b * nbps + i]."""
    B, Hkv, Smax, D = cache.shape
    nbps = Smax // block_size
    pool = np.full((B * nbps, Hkv, block_size, D), np.nan)
    table = np.zeros((B, nbps), np.int32)
    for b in range(B):
        for i in range(nbps):
            phys = perm[b * nbps + i]
            pool[phys] = cache[b, :, i * block_size:(i + 1) * block_size]
            table[b, i] = phys
    return pool, table


@pytest.mark.parametrize("block_size", [1, 4, 16])
def test_paged_rows_read_the_contiguous_cache(block_size):
    # [Guide] §3.3: the cache holds slot j of sequence b at position j; a paged pool holds the same
    # rows behind a block table, whatever the physical order
    B, Hkv, Smax, D = 3, 2, 32, 8
    cache = rng.standard_normal((B, Hkv, Smax, D))
    for perm in (np.arange(B * Smax // block_size),
                 rng.permutation(B * Smax // block_size)):
        pool, table = _contiguous_to_pool(cache, block_size, perm)
        for b, n in ((0, 1), (1, 17), (2, 32)):
            np.testing.assert_array_equal(oracle.paged_rows(pool, table, b, n, block_size),
                                          cache[b, :, :n])


def test_paged_update_appends_and_leaves_other_slots():
    # [Guide] §3.3 update: the L new rows land at slots len .. len+L-1, everything else is kept
    B, Hkv, D, bs = 2, 2, 4, 4
    pool = rng.standard_normal((10, Hkv, bs, D))
    table = np.array([[7, 2, 5], [0, 9, 3]], np.int32)
    start = np.array([3, 6])
    rows = rng.standard_normal((B, 5, Hkv, D))
    new = oracle.paged_update(pool, table, start, rows, bs)
    for b in range(B):
        got = oracle.paged_rows(new, table, b, int(start[b]) + 5, bs)
        np.testing.assert_array_equal(got[:, :start[b]],
                                      oracle.paged_rows(pool, table, b, int(start[b]), bs))
        np.testing.assert_array_equal(got[:, start[b]:], rows[b].transpose(1, 0, 2))
    touched = {(int(table[b][(int(start[b]) + i) // bs]), (int(start[b]) + i) % bs)
               for b in range(B) for i in range(5)}
    for blk in range(10):
        for s in range(bs):
            if (blk, s) not in touched:
                np.testing.assert_array_equal(new[blk, :, s], pool[blk, :, s])


def test_paged_decode_after_append_equals_last_prefill_row():
    # the whole step: new keys normed and rotated by append_rows, written through a permuted
    # table, then decode over the pool == the last row of prefill over the same sequence
    wl = _small("llama31_decode_bf16", B=2, L=37, S=37, Hq=8, Hkv=2, D=32, rotary_dim=32,
                qk_norm=True, window=20)
    x = prefill_inputs(wl.with_(kind="prefill"), seed=17)
    inv = oracle.rope_inv_freq(32, 5e5, "llama3", 8.0, 1.0, 4.0, 8192.0)
    bs, nbps = 4, 10
    perm = rng.permutation(2 * nbps)
    table = perm.reshape(2, nbps).astype(np.int32)
    kpool = np.zeros((2 * nbps, 2, bs, 32))
    vpool = np.zeros_like(kpool)
    krows = oracle.append_rows(x["k"], x["key_positions"], inv_freq=inv, k_norm_w=x["k_norm_w"],
                               eps=wl.eps)
    start = np.zeros(2, np.int64)
    kpool = oracle.paged_update(kpool, table, start, krows, bs)
    vpool = oracle.paged_update(vpool, table, start, x["v"], bs)
    sinks = np.array([0.5, -1.0, 2.0, 0.0, 1.0, -3.0, 0.25, 4.0])
    dec = oracle.attn_decode_paged(x["q"][:, -1], kpool, vpool, table, np.full(2, 37), bs,
                                   inv_freq=inv, window=20, q_norm_w=x["q_norm_w"], eps=wl.eps,
                                   sinks=sinks)
    full = _prefill(wl, x, inv_freq=inv, sinks=sinks)[:, -1]
    np.testing.assert_allclose(dec, full, atol=1e-13)


# ----------------------------------------------------------------------------------------------
# Multi-head latent attention: the absorbed core
# ----------------------------------------------------------------------------------------------
def test_mla_absorbed_core_equals_decompressed_attention():
    # [Models] "Multi-head latent attention": q_nope . (W_uk c) + q_rope . k_rope =
    # (W_uk^T q_nope) . c + q_rope . k_rope, and W_uv is applied after attention; so the absorbed
    # core over the cached [c, k_rope] rows equals ordinary attention with decompressed keys and
    # values.  Small sizes stand in for 128 heads x (128 nope + 64 rope), 512 latents.
    H, n, dn, dr, dv, r = 4, 23, 16, 8, 12, oracle.MLA_LATENT
    W_uk = rng.standard_normal((H, dn, r)) / np.sqrt(r)
    W_uv = rng.standard_normal((H, dv, r)) / np.sqrt(r)
    c = rng.standard_normal((n, r))
    k_rope = rng.standard_normal((n, oracle.MLA_ROPE))
    q_nope = rng.standard_normal((H, dn))
    q_rope = rng.standard_normal((H, oracle.MLA_ROPE))
    scale = (dn + dr) ** -0.5
    # decompressed: per head, keys [W_uk c, k_rope], values W_uv c
    full = np.stack([oracle.softmax_attention(
        np.concatenate([q_nope[h], q_rope[h]])[None],
        np.concatenate([c @ W_uk[h].T, k_rope], axis=1), c @ W_uv[h].T,
        np.ones((1, n), bool), scale)[0] for h in range(H)])
    # absorbed: one 576-wide head
    q_lat = np.einsum("hd,hdr->hr", q_nope, W_uk)
    q = np.concatenate([q_lat, q_rope], axis=1)
    rows = np.concatenate([c, k_rope], axis=1)
    lat = oracle.mla_decode_one(q, rows, n, scale)                 # [H, 512]
    absorbed = np.einsum("hr,hvr->hv", lat, W_uv)
    np.testing.assert_allclose(absorbed, full, atol=1e-12)


def test_mla_core_is_one_head_attention_with_values_in_the_rows():
    # the core equals attention with a single KV head whose values are the rows' first 512
    # features, the same for every query head (brute force per head with math.exp)
    H, n = 3, 9
    q = rng.standard_normal((H, 576))
    rows = rng.standard_normal((n + 4, 576))
    got = oracle.mla_decode_one(q, rows, n, 0.05)
    for h in range(H):
        s = [0.05 * float(q[h] @ rows[j]) for j in range(n)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        ref = sum(w[j] * rows[j, :512] for j in range(n)) / sum(w)
        np.testing.assert_allclose(got[h], ref, rtol=1e-12)
