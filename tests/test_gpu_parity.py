"""GPU parity of the HIP path (through the C ABI) against the float64 oracle.

Tolerances (from the arithmetic): fp32 |err| <= 1e-4; bf16 |err| <= 2e-2 + 2e-2 |ref| elementwise
and, tighter, ||err|| / ||ref|| <= 1e-2 per (sequence, head); masks and positions bit-exact
(probe: with q = 0 every allowed key gets weight 1/n and every masked key exactly 0, so one-hot
values reveal the allowed set exactly).
"""
import zlib

import numpy as np
import pytest

import oracle
from synth import (WORKLOADS, decode_cache_seq, decode_device_inputs, decode_lens_q, draw_sinks,
                   prefill_inputs)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
g = pytest.importorskip("gqa_scaled_rope_amd")

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def say(*a):
    print(*a, flush=True)


def dev(a, dt=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt)


def tdt(wl):
    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def inv_freq(wl):
    return oracle.rope_inv_freq(wl.rotary_dim, wl.theta, wl.rope_kind, wl.factor,
                                wl.low_freq_factor, wl.high_freq_factor, wl.original_max_pos)


def spec(wl):
    return g.RopeSpec(wl.rotary_dim, wl.rope_kind, wl.theta, wl.factor, wl.low_freq_factor,
                      wl.high_freq_factor, wl.original_max_pos)


# The kernel path a test runs, carried into every config the helpers build (cfg.kernel is a
# per-call field; the library holds no selection state).
PATH = {"path": "stream", "kernel": "auto"}


def cfg_of(*args, **kw):
    """AttnConfig with the current test's kernel choice."""
    kw.setdefault("kernel", PATH["kernel"])
    return g.AttnConfig(*args, **kw)


@pytest.fixture(params=["stream", "stream_short", "fused", "generic"])
def policy(request):
    """Kernel path: stream (key-prep pass + the eight-wavefront streaming MFMA kernel),
    stream_short (key-prep pass + the four-wavefront one), fused (MFMA kernel that preps keys on
    the fly, no workspace), generic (one wave per row, fp32 math)."""
    PATH["kernel"] = {"stream": "prefill_long", "stream_short": "prefill_short",
                      "fused": "auto", "generic": "generic"}[request.param]
    PATH["path"] = request.param
    yield request.param
    PATH["kernel"] = "auto"
    PATH["path"] = "stream"


@pytest.fixture(params=["mfma", "mfma_long", "generic"])
def dpolicy(request):
    """Decode kernel path: the MFMA split-KV kernels (split size chosen from the batch, or 2048
    keys forced), or generic (one wave per row, fp32 math)."""
    PATH["kernel"] = {"mfma": "auto", "mfma_long": "decode_long", "generic": "generic"}[
        request.param]
    yield request.param
    PATH["kernel"] = "auto"


def mask_kw(wl):
    """Sinks and chunking of a workload, as oracle keyword arguments."""
    return dict(sinks=draw_sinks(wl), chunk=wl.chunk, chunk_lookback=wl.chunk_lookback)


def cfg_extra(wl):
    """Sinks and chunking of a workload, as AttnConfig fields."""
    sk = draw_sinks(wl)
    return dict(sinks=None if sk is None else dev(sk, torch.float32), chunk_size=wl.chunk,
                chunk_lookback=wl.chunk_lookback)


def gpu_prefill(wl, x, table_len=None, shared_pos=False):
    dt = tdt(wl)
    tl = table_len or int(max(x["positions"].max(), x["key_positions"].max())) + 1
    cos, sin = g.rope_tables(spec(wl), tl) if wl.rotary_dim else (None, None)
    cfg = cfg_of(wl.dtype, wl.D, wl.Hq, wl.Hkv, wl.rotary_dim, wl.style, cos, sin,
                       wl.qk_norm, wl.eps,
                       dev(x["q_norm_w"], dt) if wl.qk_norm else None,
                       dev(x["k_norm_w"], dt) if wl.qk_norm else None, 0.0, wl.softcap,
                       **cfg_extra(wl))
    pos = x["positions"][0] if shared_pos else x["positions"]
    kpos = x["key_positions"][0] if shared_pos else x["key_positions"]
    ws = None if PATH["path"] == "fused" else "auto"
    out = g.attn_prefill(cfg, dev(x["q"], dt), dev(x["k"], dt), dev(x["v"], dt),
                         dev(pos, torch.int32), dev(kpos, torch.int32), wl.n_cached, wl.window,
                         workspace=ws)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def ref_prefill(wl, x, **kw):
    return oracle.attn_prefill(x["q"], x["k"], x["v"], x["positions"], x["key_positions"],
                               inv_freq=inv_freq(wl), style=wl.style, n_cached=wl.n_cached,
                               window=wl.window, q_norm_w=x.get("q_norm_w"),
                               k_norm_w=x.get("k_norm_w"), eps=wl.eps, softcap=wl.softcap,
                               **{**mask_kw(wl), **kw})


def check(got, ref, dtype="bf16", head_axis=2):
    err = np.abs(got - ref)
    if dtype == "f32":
        assert err.max() <= 1e-4, f"fp32 max err {err.max()}"
        return
    bad = err > 2e-2 + 2e-2 * np.abs(ref)
    assert not bad.any(), f"{bad.sum()} elements out of tolerance, max err {err.max()} at {np.argwhere(bad)[:3]}"
    # relative norm per (sequence, head): all axes but batch and head reduced
    axes = tuple(i for i in range(ref.ndim) if i not in (0, head_axis))
    num = np.sqrt((err ** 2).sum(axis=axes))
    den = np.sqrt((ref ** 2).sum(axis=axes)) + 1e-30
    rel = num / den
    assert rel.max() <= 1e-2, f"relative norm error {rel.max()}"


# ----------------------------------------------------------------------------------------------
def test_rope_tables_match_oracle():
    for wl in (WORKLOADS["qwen3_prefill_bf16"], WORKLOADS["llama31_decode_bf16"],
               WORKLOADS["chunked_prefill_bf16_full"],
               WORKLOADS["tiny_causal_f32"].with_(rope_kind="linear", factor=4.0)):
        say("tables", wl.name)
        n = wl.S
        cos, sin = g.rope_tables(spec(wl), n)
        torch.cuda.synchronize()
        ang = oracle.rope_angles(np.arange(n), inv_freq(wl))
        np.testing.assert_allclose(cos.cpu().numpy(), np.cos(ang), rtol=0, atol=2e-7)
        np.testing.assert_allclose(sin.cpu().numpy(), np.sin(ang), rtol=0, atol=2e-7)


def test_tiny_causal_f32():
    wl = WORKLOADS["tiny_causal_f32"]
    x = prefill_inputs(wl)
    check(gpu_prefill(wl, x), ref_prefill(wl, x), "f32")


BASE = WORKLOADS["qwen3_prefill_bf16"].with_(B=2, L=300, S=300, Hq=8, Hkv=2)
VARIANTS = {
    "qknorm_half128": BASE,
    "window77": BASE.with_(qk_norm=False, window=77),
    "window1": BASE.with_(qk_norm=False, window=1),
    "interleaved64_cap_chunk": BASE.with_(Hq=6, Hkv=2, rotary_dim=64, style="interleaved",
                                         softcap=50.0, qk_norm=False, n_cached=180, theta=1e4),
    "interleaved64_window_chunk": BASE.with_(Hq=6, Hkv=2, rotary_dim=64, style="interleaved",
                                            softcap=50.0, qk_norm=False, n_cached=180,
                                            window=100, theta=1e4),
    "half64_partial": BASE.with_(rotary_dim=64),
    "half32_partial": BASE.with_(rotary_dim=32, qk_norm=False),
    "half16_partial": BASE.with_(rotary_dim=16, qk_norm=False),
    "norope": BASE.with_(rotary_dim=0),
    "mha_G1": BASE.with_(Hq=4, Hkv=4),
    "G8": BASE.with_(Hq=16, Hkv=2, L=100, S=100),
    "llama3_long_positions": BASE.with_(rope_kind="llama3", theta=5e5, factor=8.0, qk_norm=False),
    "ragged_L257": BASE.with_(L=257, S=257),
    "single_token": BASE.with_(L=1, S=1),
    "chunk_L1": BASE.with_(L=1, S=300, n_cached=299, qk_norm=False),
    # learned sinks ([Ster] gpt_oss) and chunked attention ([Ster] llama4_text, Rnj-1.5)
    "sinks": BASE.with_(sinks=True),
    "sinks_interleaved_cap_cached": BASE.with_(Hq=6, Hkv=2, rotary_dim=64, style="interleaved",
                                               softcap=50.0, qk_norm=False, n_cached=180,
                                               theta=1e4, sinks=True),
    "chunk64_llama4": BASE.with_(chunk=64),
    "chunk50_lookback1_sinks": BASE.with_(qk_norm=False, chunk=50, chunk_lookback=1, sinks=True),
    "chunk8_lookback2_window20": BASE.with_(qk_norm=False, chunk=8, chunk_lookback=2, window=20),
}


@pytest.mark.parametrize("name", list(VARIANTS))
def test_prefill_variants(name, policy):
    wl = VARIANTS[name]
    say("prefill variant", name, "policy", policy)
    x = prefill_inputs(wl, seed=zlib.crc32(name.encode()) % 1000)
    check(gpu_prefill(wl, x), ref_prefill(wl, x))


# room the workspace keeps for the split key walks of a last, partial round of query blocks:
# 128 query blocks x 2 halves x 66 values x 512 threads x 4 bytes
SPLIT_BYTES = 128 * 2 * 66 * 512 * 4


@pytest.mark.parametrize("name", ["qknorm_half128", "sinks_interleaved_cap_cached",
                                  "chunk50_lookback1_sinks"])
def test_split_walk_matches_whole_walk(name):
    # 20-30 query blocks on a 256-CU GPU: with the full workspace every block's key walk is split
    # over two workgroups and merged; with only the prepared keys' room (or none) each block is
    # walked whole.  Both must match the oracle and each other up to rounding.
    wl = VARIANTS[name]
    say("split against whole walks", name)
    x = prefill_inputs(wl, seed=zlib.crc32(name.encode()) % 1000)
    PATH["kernel"] = "prefill_long"
    try:
        split = gpu_prefill(wl, x)
        dt = tdt(wl)
        tl = int(max(x["positions"].max(), x["key_positions"].max())) + 1
        cos, sin = g.rope_tables(spec(wl), tl) if wl.rotary_dim else (None, None)
        cfg = cfg_of(wl.dtype, wl.D, wl.Hq, wl.Hkv, wl.rotary_dim, wl.style, cos, sin,
                     wl.qk_norm, wl.eps,
                     dev(x["q_norm_w"], dt) if wl.qk_norm else None,
                     dev(x["k_norm_w"], dt) if wl.qk_norm else None, 0.0, wl.softcap,
                     **cfg_extra(wl))
        need = g.prefill_workspace_bytes(cfg, wl.B, wl.S, wl.n_cached) - SPLIT_BYTES
        ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need > 0 else None
        whole = g.attn_prefill(cfg, dev(x["q"], dt), dev(x["k"], dt), dev(x["v"], dt),
                               dev(x["positions"], torch.int32),
                               dev(x["key_positions"], torch.int32), wl.n_cached, wl.window,
                               workspace=ws)
        torch.cuda.synchronize()
        whole = whole.float().cpu().numpy()
    finally:
        PATH["kernel"] = "auto"
    ref = ref_prefill(wl, x)
    check(split, ref)
    check(whole, ref)
    assert np.abs(split - whole).max() <= 1e-2


@pytest.mark.parametrize("name,kw", [
    ("peaky_q4_offset_norm", dict(q_scale=4.0, offset=0.3)),
    ("peaky_k4", dict(k_scale=4.0)),
])
def test_prefill_stress_norm(name, kw, policy):
    # non-unit RMS inputs: skipping the norm would fail; peaky logits
    wl = BASE
    say("stress", name, "policy", policy)
    x = prefill_inputs(wl, seed=7, **kw)
    check(gpu_prefill(wl, x), ref_prefill(wl, x))


@pytest.mark.parametrize("cap", [1.0, 5.0])
def test_prefill_stress_softcap(cap, policy):
    # with q x 8 the cap changes the logits by O(1): a missing or misplaced cap fails
    wl = BASE.with_(qk_norm=False, softcap=cap, rotary_dim=64, style="interleaved")
    x = prefill_inputs(wl, seed=8, q_scale=8.0)
    got, ref = gpu_prefill(wl, x), ref_prefill(wl, x)
    check(got, ref)
    ref_nocap = ref_prefill(wl.with_(softcap=0.0), x)
    assert np.abs(ref_nocap - ref).max() > 0.1  # the stress input really exercises the cap


def test_prefill_per_sequence_positions(policy):
    # each sequence has its own position offsets (batch stride L / S), chunked queries
    wl = BASE.with_(qk_norm=False, window=50, n_cached=200, L=100, S=300)
    x = prefill_inputs(wl, seed=9)
    for b in range(wl.B):
        x["key_positions"][b] += 37 * b
        x["positions"][b] += 37 * b
    check(gpu_prefill(wl, x), ref_prefill(wl, x))


@pytest.mark.parametrize("window,chunk,n_cached", [(0, 0, 0), (37, 0, 0), (100, 0, 150),
                                                  (0, 48, 0), (0, 40, 120)])
def test_prefill_gapped_key_positions(window, chunk, n_cached, policy):
    # nondecreasing key positions with gaps and repeats (the queries sit at the new keys'
    # positions): the band edges cannot be inferred from the first key's position, so the kernel
    # has to search for them
    wl = BASE.with_(qk_norm=False, window=window, chunk=chunk, n_cached=n_cached,
                    L=300 - n_cached, S=300)
    say("gapped key positions", window, chunk, n_cached, "policy", policy)
    x = prefill_inputs(wl, seed=13)
    rng = np.random.default_rng(13)
    for b in range(wl.B):
        kp = (np.cumsum(rng.integers(0, 4, wl.S)) + 5 * b).astype(np.int32)
        x["key_positions"][b] = kp
        x["positions"][b] = kp[n_cached:]
    assert (np.diff(x["key_positions"], axis=1) == 0).any()
    check(gpu_prefill(wl, x), ref_prefill(wl, x))


def test_prefill_shared_positions_stride0():
    wl = BASE.with_(qk_norm=False, window=64)
    x = prefill_inputs(wl, seed=10)
    check(gpu_prefill(wl, x, shared_pos=True), ref_prefill(wl, x))


def test_prefill_no_keys_rows_are_zero():
    # queries whose positions precede every key position see nothing -> exact zeros
    wl = BASE.with_(qk_norm=False, L=64, S=64)
    x = prefill_inputs(wl, seed=11)
    x["key_positions"] += 1000
    got = gpu_prefill(wl, x, table_len=2000)
    ref = ref_prefill(wl, x)
    assert np.all(ref == 0) and np.all(got == 0)


@pytest.mark.parametrize("window,n_cached,shift,chunk,lookback", [
    (0, 0, 0, 0, 0), (1, 0, 0, 0, 0), (5, 0, 0, 0, 0), (64, 0, 3, 0, 0), (100, 120, 0, 0, 0),
    (0, 200, 5, 0, 0), (129, 0, 0, 0, 0),
    # chunked attention: own chunk (Llama 4), one chunk of lookback (Rnj-1.5), tile-aligned and
    # not, with a window, chunk 1, and positions below zero (floor chunks)
    (0, 0, 0, 64, 0), (0, 0, 0, 50, 1), (0, 120, 7, 33, 2), (40, 0, 0, 32, 1), (0, 0, 0, 1, 0),
    (0, 0, -150, 48, 0), (0, 0, -301, 7, 1), (0, 0, 0, 1 << 30, 0),
])
def test_mask_probe_bitexact(window, n_cached, shift, chunk, lookback, policy):
    wl = BASE.with_(qk_norm=False, rotary_dim=0, window=window, n_cached=n_cached, L=300 - n_cached,
                    S=300, chunk=chunk, chunk_lookback=lookback)
    say("mask probe", window, n_cached, shift, chunk, lookback, "policy", policy)
    x = prefill_inputs(wl, seed=12)
    x["q"][:] = 0.0
    for b in range(wl.B):
        x["key_positions"][b] += shift * b
        x["positions"][b] += shift * b
    allowed = [oracle.allowed_mask(x["positions"][b], x["key_positions"][b], window, wl.chunk,
                                   wl.chunk_lookback) for b in range(wl.B)]
    for blk in range(0, wl.S, wl.D):
        v = np.zeros_like(x["v"])
        n = min(wl.D, wl.S - blk)
        for d in range(n):
            v[:, blk + d, :, d] = 1.0
        xx = dict(x, v=v)
        got = gpu_prefill(wl, xx)                          # [B, L, Hq, D]
        for b in range(wl.B):
            nz = got[b] != 0                               # [L, Hq, D]
            want = allowed[b][:, blk:blk + n]              # [L, n]
            for h in range(wl.Hq):
                np.testing.assert_array_equal(nz[:, h, :n], want)
            assert not nz[:, :, n:].any()


# ----------------------------------------------------------------------------------------------
def gpu_decode(wl, q, kc, vc, lens, qw=None):
    dt = tdt(wl)
    cos, sin = g.rope_tables(spec(wl), kc.shape[2]) if wl.rotary_dim else (None, None)
    cfg = cfg_of(wl.dtype, wl.D, wl.Hq, wl.Hkv, wl.rotary_dim, wl.style, cos, sin,
                       wl.qk_norm, wl.eps, dev(qw, dt) if wl.qk_norm else None,
                       dev(qw, dt) if wl.qk_norm else None, 0.0, wl.softcap, **cfg_extra(wl))
    out = g.attn_decode(cfg, dev(q, dt), dev(kc, dt), dev(vc, dt), dev(lens, torch.int32),
                        wl.window)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


DEC = WORKLOADS["llama31_decode_bf16"].with_(B=5, S=2600, lens_lo=1, lens_hi=2600)
DEC_VARIANTS = {
    "llama3": DEC,
    "window100": DEC.with_(window=100),
    "window_big": DEC.with_(window=1500),
    "qknorm_interleaved64_cap": DEC.with_(qk_norm=True, rotary_dim=64, style="interleaved",
                                          softcap=5.0, rope_kind="default", theta=1e4),
    "G3": DEC.with_(Hq=24, Hkv=8),
    "G16": DEC.with_(Hq=32, Hkv=2),
    "half32": DEC.with_(rotary_dim=32),
    "sinks": DEC.with_(sinks=True),
    "chunk1000_lookback1": DEC.with_(chunk=1000, chunk_lookback=1),
    "chunk2048_window1500_sinks": DEC.with_(chunk=2048, window=1500, sinks=True),
    "chunk256_G16_sinks": DEC.with_(Hq=32, Hkv=2, chunk=256, sinks=True),
}


@pytest.mark.parametrize("name", list(DEC_VARIANTS))
def test_decode_variants(name, dpolicy):
    policy = dpolicy
    wl = DEC_VARIANTS[name]
    say("decode variant", name, "policy", policy)
    lens, q, qw = decode_lens_q(wl, seed=21)
    lens[0], lens[1] = 1, wl.S                # edge lengths: one key, full capacity
    kc = np.full((wl.B, wl.Hkv, wl.S, wl.D), np.nan, np.float32)  # unread slots are NaN
    vc = np.full_like(kc, np.nan)
    for b in range(wl.B):
        kk, vv = decode_cache_seq(wl, b, int(lens[b]), seed=21)
        kc[b, :, :lens[b]] = kk
        vc[b, :, :lens[b]] = vv
    got = gpu_decode(wl, q, kc, vc, lens, qw)
    ref = oracle.attn_decode(q, np.nan_to_num(kc), np.nan_to_num(vc), lens, inv_freq=inv_freq(wl),
                             style=wl.style, window=wl.window, q_norm_w=qw, eps=wl.eps,
                             softcap=wl.softcap, **mask_kw(wl))
    check(got, ref, head_axis=1)


def test_decode_equals_last_prefill_row():
    # decode against a cache filled with normed, rotated keys == last row of prefill
    wl = BASE.with_(B=2, L=333, S=333, window=0)
    x = prefill_inputs(wl, seed=31)
    full = gpu_prefill(wl, x)[:, -1]                                   # [B, Hq, D]
    inv = inv_freq(wl)
    kc = oracle.rotate(oracle.rms_norm(x["k"], x["k_norm_w"], wl.eps),
                       x["key_positions"][:, :, None], inv, wl.style)
    kc = kc.transpose(0, 2, 1, 3).astype(np.float32)
    vc = x["v"].transpose(0, 2, 1, 3)
    lens = np.full(wl.B, wl.S, np.int32)
    dwl = wl.with_(qk_norm=True)
    dt = torch.bfloat16
    cos, sin = g.rope_tables(spec(wl), wl.S)
    cfg = cfg_of("bf16", wl.D, wl.Hq, wl.Hkv, wl.rotary_dim, wl.style, cos, sin, True,
                       wl.eps, dev(x["q_norm_w"]), dev(x["k_norm_w"]))
    dec = g.attn_decode(cfg, dev(x["q"][:, -1]), dev(kc), dev(vc), dev(lens, torch.int32), 0)
    torch.cuda.synchronize()
    del dwl
    ref = ref_prefill(wl, x, query_rows=[wl.L - 1])[:, 0]
    check(dec.float().cpu().numpy(), ref, head_axis=1)
    check(full, ref, head_axis=1)


# ----------------------------------------------------------------------------------------------
# Full-size workloads, sampled outputs, in the launch configuration the bench times
# ----------------------------------------------------------------------------------------------
@pytest.mark.parametrize("name,batches,rows", [
    ("qwen3_prefill_bf16", [0, 3], [0, 1, 63, 64, 65, 1000, 2046, 2047]),
    ("mistral_swa_prefill_bf16", [1], [0, 4094, 4095, 4096, 4097, 6000, 8191]),
    ("chunked_prefill_bf16_w4096", [0, 7], [0, 1, 255, 256, 511]),
    ("chunked_prefill_bf16_full", [5], [0, 300, 511]),
    ("sinks_swa128_prefill_bf16", [0, 3], [0, 127, 128, 129, 2000, 4095]),
    ("llama4_chunked_prefill_bf16", [0], [0, 8191, 8192, 8193, 16383]),
])
@pytest.mark.parametrize("path", ["stream", "fused"])
def test_full_size_prefill_sampled(name, batches, rows, path):
    PATH["path"] = path
    wl = WORKLOADS[name]
    say("full size", name, path)
    x = prefill_inputs(wl)
    got = gpu_prefill(wl, x, shared_pos=True)
    ref = ref_prefill(wl, x, query_rows=rows, batches=batches)
    PATH["path"] = "stream"
    check(got[batches][:, rows], ref)
    assert np.isfinite(got).all()


def test_chunked_window4096_equals_full_bitwise():
    # max distance in the chunk is 4095 = w - 1, so the two layer kinds see the same keys
    a = WORKLOADS["chunked_prefill_bf16_w4096"]
    b = WORKLOADS["chunked_prefill_bf16_full"]
    x = prefill_inputs(a)
    np.testing.assert_array_equal(gpu_prefill(a, x, shared_pos=True),
                                  gpu_prefill(b, x, shared_pos=True))


@pytest.mark.parametrize("name", ["llama31_decode_bf16", "sinks_chunk_decode_bf16"])
def test_full_size_decode_sampled(name):
    wl = WORKLOADS[name]
    say("full size decode", wl.name)
    x = decode_device_inputs(wl)
    cos, sin = g.rope_tables(spec(wl), wl.S)
    cfg = cfg_of("bf16", wl.D, wl.Hq, wl.Hkv, wl.rotary_dim, wl.style, cos, sin,
                       **cfg_extra(wl))
    out = g.attn_decode(cfg, x["q"], x["k"], x["v"], x["lens"], wl.window)
    torch.cuda.synchronize()
    lens = x["lens"].cpu().numpy()
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    inv = inv_freq(wl)
    for b in sorted({int(np.argmin(lens)), int(np.argmax(lens)), 0, 17, 63}):
        n = int(lens[b])
        ref = oracle.attn_decode_one(x["q"][b].float().cpu().numpy(),
                                     x["k"][b, :, :n].float().cpu().numpy(),
                                     x["v"][b, :, :n].float().cpu().numpy(), n, inv_freq=inv,
                                     window=wl.window, **mask_kw(wl))
        check(got[b][None], ref[None], head_axis=1)


def test_decode_several_split_launches():
    # more than 2048 sequences: the split kernel runs in two launches sharing one combine.  With
    # 2100 sequences of 1025-2100 keys the first launch (2048 sequences) holds enough work for the
    # 2048-key splits and the second (52) does not, so the two launches choose differently and the
    # combine must take each sequence's choice from its own launch.
    wl = WORKLOADS["llama31_decode_bf16"].with_(B=2100, S=2100, Hq=8, Hkv=2, lens_lo=1025,
                                                 lens_hi=2100, seed=61)
    say("decode, two split launches", wl.B, wl.S)
    x = decode_device_inputs(wl)
    cos, sin = g.rope_tables(spec(wl), wl.S)
    cfg = cfg_of("bf16", wl.D, wl.Hq, wl.Hkv, wl.rotary_dim, wl.style, cos, sin)
    out = g.attn_decode(cfg, x["q"], x["k"], x["v"], x["lens"], 0)
    torch.cuda.synchronize()
    lens = x["lens"].cpu().numpy()
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    inv = inv_freq(wl)
    for b in sorted({0, 1, 1000, 2046, 2047, 2048, 2049, 2099, int(np.argmin(lens[2048:])) + 2048,
                     int(np.argmax(lens[2048:])) + 2048, int(np.argmax(lens[:2048]))}):
        n = int(lens[b])
        ref = oracle.attn_decode_one(x["q"][b].float().cpu().numpy(),
                                     x["k"][b, :, :n].float().cpu().numpy(),
                                     x["v"][b, :, :n].float().cpu().numpy(), n, inv_freq=inv)
        check(got[b][None], ref[None], head_axis=1)
    # every split size gives the same result up to rounding
    for k in ("decode_short", "decode_long"):
        cfg_k = cfg_of("bf16", wl.D, wl.Hq, wl.Hkv, wl.rotary_dim, wl.style, cos, sin, kernel=k)
        other = g.attn_decode(cfg_k, x["q"], x["k"], x["v"], x["lens"], 0)
        torch.cuda.synchronize()
        diff = np.abs(other.float().cpu().numpy() - got)
        assert diff.max() <= 2e-2, (k, diff.max())


@pytest.mark.parametrize("path", ["stream", "fused"])
def test_full_size_window_edge_probe_bitexact(path):
    # [Models] "Sliding windows": a query at position p sees keys p-4095 .. p at window 4096.  At
    # the Mistral-style size one key more or less moves an output by ~1/4096, below the bf16
    # tolerance, so the edges are probed exactly: q = 0 gives every allowed key weight exactly 1/n,
    # and one-hot values over a key block make output column d nonzero iff key blk+d is allowed.
    wl = WORKLOADS["mistral_swa_prefill_bf16"]
    say("full-size window edge probe", path)
    B, L, Hq, Hkv, D = wl.B, wl.L, wl.Hq, wl.Hkv, wl.D
    from synth import device_normal
    q = torch.zeros((B, L, Hq, D), dtype=torch.bfloat16, device="cuda")
    k = device_normal((B, L, Hkv, D), 3 * 10 + 2, "bf16")
    pos = torch.arange(L, dtype=torch.int32, device="cuda")
    cos, sin = g.rope_tables(spec(wl), L)
    cfg = cfg_of("bf16", D, Hq, Hkv, wl.rotary_dim, wl.style, cos, sin)
    rows = [0, 1, 4094, 4095, 4096, 4097, 4160, 6000, 8191]
    for blk in (0, 4032, 8064):
        v = torch.zeros((B, L, Hkv, D), dtype=torch.bfloat16, device="cuda")
        idx = torch.arange(D, device="cuda")
        v[:, blk + idx, :, idx] = 1.0
        out = g.attn_prefill(cfg, q, k, v, pos, pos, 0, wl.window,
                             workspace=None if path == "fused" else "auto")
        torch.cuda.synchronize()
        got = out[:, rows].float().cpu().numpy()            # [B, rows, Hq, D]
        for ri, i in enumerate(rows):
            kp = blk + np.arange(D)
            allowed = (kp <= i) & (i - kp <= wl.window - 1)
            n = min(i, wl.window - 1) + 1                   # keys the row sees in all
            for b in range(B):
                nz = got[b, ri] != 0                        # [Hq, D]
                assert (nz == allowed[None, :]).all(), (blk, i, b)
                if allowed.any():
                    vals = got[b, ri][:, allowed]
                    np.testing.assert_allclose(vals, 1.0 / n, rtol=2 ** -8)


@pytest.mark.parametrize("name", ["qknorm_half128", "interleaved64_cap_chunk", "half32_partial",
                                  "norope"])
def test_prep_keys_then_cached_prefill(name):
    # append step + attention over the cache with every key used as stored == one prefill call
    wl = VARIANTS[name]
    if wl.rotary_dim == 0 and not wl.qk_norm:
        wl = wl.with_(qk_norm=True)
    x = prefill_inputs(wl, seed=41)
    dt = torch.bfloat16
    tl = int(x["key_positions"].max()) + 1
    cos, sin = g.rope_tables(spec(wl), tl) if wl.rotary_dim else (None, None)
    cfg = cfg_of("bf16", wl.D, wl.Hq, wl.Hkv, wl.rotary_dim, wl.style, cos, sin, wl.qk_norm,
                       wl.eps, dev(x["q_norm_w"]) if wl.qk_norm else None,
                       dev(x["k_norm_w"]) if wl.qk_norm else None, 0.0, wl.softcap)
    k = dev(x["k"])
    kpos = dev(x["key_positions"], torch.int32)
    kc = g.prep_keys(cfg, k, kpos, wl.n_cached, k_out=k.clone())
    # in place gives the same rows
    k2 = k.clone()
    g.prep_keys(cfg, k2, kpos, wl.n_cached, k_out=k2)
    torch.cuda.synchronize()
    assert torch.equal(kc, k2)
    # cached rows untouched; new rows equal the oracle's norm + rotation up to bf16 rounding
    assert torch.equal(kc[:, :wl.n_cached], k[:, :wl.n_cached])
    kn = x["k"][:, wl.n_cached:].astype(np.float64)
    if wl.qk_norm:
        kn = oracle.rms_norm(kn, x["k_norm_w"], wl.eps)
    kn = oracle.rotate(kn, x["key_positions"][:, wl.n_cached:, None], inv_freq(wl), wl.style)
    got = kc[:, wl.n_cached:].float().cpu().numpy()
    np.testing.assert_allclose(got, kn, rtol=2 ** -8, atol=1e-6)
    out = g.attn_prefill(cfg, dev(x["q"]), kc, dev(x["v"]), dev(x["positions"], torch.int32), kpos,
                         wl.S, wl.window)
    torch.cuda.synchronize()
    check(out.float().cpu().numpy(), ref_prefill(wl, x))


def test_all_scores_far_below_zero(policy):
    # every score about -147 in log2 units: exp2 of the unshifted scores underflows, so the
    # kernels must take the running max from the first scores they see
    wl = BASE.with_(qk_norm=False, rotary_dim=0, L=130, S=130)
    x = prefill_inputs(wl, seed=51)
    r = np.random.default_rng(51)
    u = np.ones(wl.D, np.float32)
    x["q"] = (3.0 * u + 0.3 * r.standard_normal(x["q"].shape)).astype(np.float32)
    x["k"] = (-3.0 * u + 0.3 * r.standard_normal(x["k"].shape)).astype(np.float32)
    from synth import round_to
    x["q"], x["k"] = round_to(x["q"], "bf16"), round_to(x["k"], "bf16")
    ref = ref_prefill(wl, x)
    assert np.abs(ref).max() > 0.05      # a real (non-degenerate) softmax
    check(gpu_prefill(wl, x), ref)


# ----------------------------------------------------------------------------------------------
# YaRN and LongRoPE: the tables carry the attention factor, YaRN's temperature enters through the
# softmax scale.  Original contexts are short so that the test positions go well past them and the
# kept, ramped and divided pairs all occur.
_LR_SHORT = [1.0 + 0.02 * i for i in range(64)]
_LR_LONG = [1.0 + 0.25 * i for i in range(64)]
SCHED = {
    "yarn_mscale": dict(kind="yarn", theta=1e4, factor=8.0, original_max_pos=128.0, mscale=1.0,
                        mscale_all_dim=0.707),
    "yarn_default": dict(kind="yarn", theta=1e6, factor=16.0, original_max_pos=64.0),
    "yarn_betas_untruncated": dict(kind="yarn", theta=1e4, factor=4.0, original_max_pos=200.0,
                                   beta_fast=8.0, beta_slow=2.0, truncate=False),
    "longrope_long": dict(kind="longrope", theta=1e4, original_max_pos=128.0,
                          attention_factor=1.19),
    "longrope_short": dict(kind="longrope", theta=1e4, original_max_pos=4096.0),
}


def sched_spec(name, R, seq_len):
    kw = dict(SCHED[name])
    if kw["kind"] == "longrope":
        kw.update(short_factor=_LR_SHORT[: R // 2], long_factor=_LR_LONG[: R // 2],
                  seq_len=seq_len)
    return g.RopeSpec(R, **kw)


def sched_oracle(name, R, seq_len, qk_dim):
    """(inv_freq, attention_factor, softmax scale) from the oracle."""
    kw = dict(SCHED[name])
    kind, theta = kw.pop("kind"), kw.pop("theta")
    old = kw.pop("original_max_pos")
    factor = kw.pop("factor", 1.0)
    af_kw = {k: kw.pop(k) for k in ("mscale", "mscale_all_dim", "attention_factor") if k in kw}
    if kind == "longrope":
        kw.update(short_factor=_LR_SHORT[: R // 2], long_factor=_LR_LONG[: R // 2],
                  seq_len=seq_len)
    inv = oracle.rope_inv_freq(R, theta, kind, factor, original_max_position_embeddings=old, **kw)
    af = oracle.rope_attention_factor(kind, factor, **af_kw)
    sc = (oracle.yarn_softmax_scale(qk_dim, factor, af_kw.get("mscale_all_dim"))
          if kind == "yarn" else qk_dim ** -0.5)
    return inv, af, sc


@pytest.mark.parametrize("name", list(SCHED))
def test_schedule_tables_match_oracle(name):
    say("tables", name)
    R, n = 128, 3000
    cos, sin = g.rope_tables(sched_spec(name, R, n), n)
    torch.cuda.synchronize()
    inv, af, _ = sched_oracle(name, R, n, 128)
    assert (af != 1.0) == (name in ("yarn_mscale", "yarn_default", "yarn_betas_untruncated",
                                    "longrope_long"))
    ang = oracle.rope_angles(np.arange(n), inv)
    np.testing.assert_allclose(cos.cpu().numpy(), af * np.cos(ang), rtol=0, atol=3e-7)
    np.testing.assert_allclose(sin.cpu().numpy(), af * np.sin(ang), rtol=0, atol=3e-7)


@pytest.mark.parametrize("name,wkw", [
    ("yarn_mscale", dict(qk_norm=True)),
    ("yarn_default", dict(rotary_dim=64, style="interleaved", softcap=30.0, n_cached=150)),
    ("yarn_betas_untruncated", dict(window=90)),
    ("longrope_long", dict(rotary_dim=64)),
    ("longrope_short", dict(qk_norm=True)),
])
def test_prefill_rope_schedules(name, wkw, policy):
    wl = BASE.with_(**{**dict(qk_norm=False), **wkw})
    say("prefill schedule", name, wkw, "policy", policy)
    x = prefill_inputs(wl, seed=zlib.crc32(name.encode()) % 1000)
    spec_ = sched_spec(name, wl.rotary_dim, wl.S)
    cos, sin = g.rope_tables(spec_, wl.S)
    scale = g.rope_softmax_scale(spec_, wl.D)
    cfg = cfg_of("bf16", wl.D, wl.Hq, wl.Hkv, wl.rotary_dim, wl.style, cos, sin, wl.qk_norm,
                       wl.eps, dev(x["q_norm_w"]) if wl.qk_norm else None,
                       dev(x["k_norm_w"]) if wl.qk_norm else None, scale, wl.softcap)
    out = g.attn_prefill(cfg, dev(x["q"]), dev(x["k"]), dev(x["v"]),
                         dev(x["positions"], torch.int32), dev(x["key_positions"], torch.int32),
                         wl.n_cached, wl.window,
                         workspace=None if policy == "fused" else "auto")
    torch.cuda.synchronize()
    inv, af, sc = sched_oracle(name, wl.rotary_dim, wl.S, wl.D)
    assert scale == pytest.approx(sc, rel=1e-12)
    ref = oracle.attn_prefill(x["q"], x["k"], x["v"], x["positions"], x["key_positions"],
                              inv_freq=inv, style=wl.style, n_cached=wl.n_cached,
                              window=wl.window, q_norm_w=x.get("q_norm_w"),
                              k_norm_w=x.get("k_norm_w"), eps=wl.eps, softcap=wl.softcap,
                              attention_factor=af, scale=sc)
    if name == "yarn_mscale":
        # the schedule changes the result: plain RoPE at the default scale is far off
        plain = ref_prefill(wl, x)
        assert np.abs(plain - ref).max() > 0.1
    check(out.float().cpu().numpy(), ref)


@pytest.mark.parametrize("name", ["yarn_mscale", "longrope_long"])
def test_decode_rope_schedules(name, dpolicy):
    policy = dpolicy
    wl = DEC.with_(rope_kind="default", theta=1e4, qk_norm=True)
    say("decode schedule", name, "policy", policy)
    lens, q, qw = decode_lens_q(wl, seed=23)
    lens[0], lens[1] = 1, wl.S
    kc = np.zeros((wl.B, wl.Hkv, wl.S, wl.D), np.float32)
    vc = np.zeros_like(kc)
    for b in range(wl.B):
        kk, vv = decode_cache_seq(wl, b, int(lens[b]), seed=23)
        kc[b, :, :lens[b]] = kk
        vc[b, :, :lens[b]] = vv
    spec_ = sched_spec(name, wl.rotary_dim, wl.S)
    cos, sin = g.rope_tables(spec_, wl.S)
    scale = g.rope_softmax_scale(spec_, wl.D)
    cfg = cfg_of("bf16", wl.D, wl.Hq, wl.Hkv, wl.rotary_dim, wl.style, cos, sin, True,
                       wl.eps, dev(qw), dev(qw), scale, wl.softcap)
    out = g.attn_decode(cfg, dev(q), dev(kc), dev(vc), dev(lens, torch.int32), wl.window)
    torch.cuda.synchronize()
    inv, af, sc = sched_oracle(name, wl.rotary_dim, wl.S, wl.D)
    ref = oracle.attn_decode(q, kc, vc, lens, inv_freq=inv, style=wl.style, window=wl.window,
                             q_norm_w=qw, eps=wl.eps, softcap=wl.softcap, attention_factor=af,
                             scale=sc)
    check(out.float().cpu().numpy(), ref, head_axis=1)


# ----------------------------------------------------------------------------------------------
# Paged KV pool: the fused append (cache.update) and decode through block tables
# ----------------------------------------------------------------------------------------------
from synth import paged_pool_inputs, round_to  # noqa: E402


def _paged_kv(kp, vp, table):
    return g.PagedKV(dev(kp), dev(vp), dev(table, torch.int32))


@pytest.mark.parametrize("bs,L,R,style,norm", [
    (16, 1, 128, "half", True), (64, 37, 64, "interleaved", False), (32, 50, 128, "half", False),
    (16, 20, 0, "half", True), (128, 3, 32, "half", True),
])
def test_paged_append_matches_oracle(bs, L, R, style, norm):
    B, Hkv, D = 3, 2, 128
    start = np.array([0, 5, 77], np.int32)
    max_blocks = (int(start.max()) + L + bs - 1) // bs + 1
    say("paged append", bs, L, R, style, norm)
    kp, vp, table = paged_pool_inputs(B, Hkv, D, bs, max_blocks, seed=bs + L)
    r = np.random.default_rng(bs * 7 + L)
    k_new = round_to(r.standard_normal((B, L, Hkv, D)).astype(np.float32), "bf16")
    v_new = round_to(r.standard_normal((B, L, Hkv, D)).astype(np.float32), "bf16")
    kw = round_to((1.0 + 0.02 * r.standard_normal(D)).astype(np.float32), "bf16")
    kpos = (start[:, None] + np.arange(L)[None, :]).astype(np.int32)
    wl = BASE.with_(Hq=4, Hkv=Hkv, rotary_dim=R, style=style, theta=1e4, qk_norm=norm)
    tl = int(kpos.max()) + 1
    cos, sin = g.rope_tables(spec(wl), tl) if R else (None, None)
    cfg = cfg_of("bf16", D, 4, Hkv, R, style, cos, sin, norm, wl.eps,
                       dev(kw) if norm else None, dev(kw) if norm else None)
    kv = _paged_kv(kp, vp, table)
    g.paged_append(cfg, kv, dev(k_new), dev(v_new), dev(kpos, torch.int32),
                   dev(start, torch.int32))
    torch.cuda.synchronize()
    got_k = kv.k_pool.float().cpu().numpy()
    got_v = kv.v_pool.float().cpu().numpy()
    rows = oracle.append_rows(k_new, kpos, inv_freq=inv_freq(wl), style=style,
                              k_norm_w=kw if norm else None, eps=wl.eps)
    ref_k = oracle.paged_update(kp, table, start, rows, bs)
    ref_v = oracle.paged_update(vp, table, start, v_new, bs)
    np.testing.assert_array_equal(got_v, ref_v)                       # values: copied
    np.testing.assert_allclose(got_k, ref_k, rtol=2 ** -8, atol=1e-6)  # keys: one bf16 rounding
    written = oracle.paged_update(np.zeros(kp.shape, bool), table, start,
                                  np.ones(k_new.shape, bool), bs)
    np.testing.assert_array_equal(got_k[~written], kp[~written])      # other slots untouched


PAGED_DEC = {
    "bs16": (16, {}),
    "bs32_window": (32, dict(window=300)),
    "bs256_sinks_chunk": (256, dict(chunk=500, chunk_lookback=1, sinks=True)),
    "bs16_window_recycled": (16, dict(window=100)),
    "bs64_cap_G16_recycled": (64, dict(softcap=5.0, Hq=32, Hkv=2, window=700)),
    "bs128_qknorm_interleaved": (128, dict(qk_norm=True, rotary_dim=64, style="interleaved",
                                           rope_kind="default", theta=1e4)),
}


@pytest.mark.parametrize("split", ["auto", "decode_long"])
@pytest.mark.parametrize("name", list(PAGED_DEC))
def test_paged_decode_matches_oracle(name, split):
    bs, kw = PAGED_DEC[name]
    wl = DEC.with_(**kw)
    say("paged decode", name, split)
    lens, q, qw = decode_lens_q(wl, seed=29)
    lens[0], lens[1] = 1, wl.S
    max_blocks = (wl.S + bs - 1) // bs
    kp, vp, table = paged_pool_inputs(wl.B, wl.Hkv, wl.D, bs, max_blocks, spare=1, seed=bs)
    gpu_table = table.copy()
    if name.endswith("recycled"):
        # the one spare block is poisoned with NaN; blocks wholly before a sequence's window and
        # wholly past its length point there, as recycled (or unused) entries may: the kernel must
        # never read them
        nan_blk = kp.shape[0] - 1
        kp[nan_blk] = np.nan
        vp[nan_blk] = np.nan
        for b in range(wl.B):
            n = int(lens[b])
            first = max(0, n - wl.window) if wl.window else 0
            for i in range(max_blocks):
                if (i + 1) * bs <= first or i * bs >= n:
                    gpu_table[b, i] = nan_blk
    cos, sin = g.rope_tables(spec(wl), wl.S)
    cfg = cfg_of(wl.dtype, wl.D, wl.Hq, wl.Hkv, wl.rotary_dim, wl.style, cos, sin,
                       wl.qk_norm, wl.eps, dev(qw) if wl.qk_norm else None,
                       dev(qw) if wl.qk_norm else None, 0.0, wl.softcap, **cfg_extra(wl), kernel=split)
    out = g.attn_decode_paged(cfg, dev(q), _paged_kv(kp, vp, gpu_table), dev(lens, torch.int32),
                              wl.window)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    kpf = np.nan_to_num(kp)
    vpf = np.nan_to_num(vp)
    ref = oracle.attn_decode_paged(q, kpf, vpf, table, lens, bs, inv_freq=inv_freq(wl),
                                   style=wl.style, window=wl.window, q_norm_w=qw, eps=wl.eps,
                                   softcap=wl.softcap, **mask_kw(wl))
    check(got, ref, head_axis=1)


# ----------------------------------------------------------------------------------------------
# Absorbed latent-attention decode core
# ----------------------------------------------------------------------------------------------
MLA = WORKLOADS["deepseek_mla_decode_bf16"]
# DeepSeek-V3: qk_head_dim 192, YaRN factor 40 with mscale_all_dim 1 sharpens the scale by m^2
MLA_SCALE = oracle.yarn_softmax_scale(192, 40.0, 1.0)


# (many short sequences: shares span several of them; 33 x <= 3 blocks: fewer blocks than shares,
# so some shares are empty; 144 heads: a second, partly idle head group)
@pytest.mark.parametrize("H,Smax,B", [(16, 5000, 4), (128, 2100, 3), (64, 100, 2), (32, 4096, 1),
                                      (128, 300, 40), (16, 70, 33), (144, 700, 3)])
def test_mla_decode_matches_oracle(H, Smax, B):
    wl = MLA.with_(B=B, Hq=H, S=Smax, lens_lo=1, lens_hi=Smax)
    say("mla decode", H, Smax, B)
    lens, q, _ = decode_lens_q(wl, seed=31)
    lens[0] = 1
    if B > 1:
        lens[-1] = Smax
    if B > 2:
        lens[1] = 0          # a sequence with no cached row: zero output
    cache = np.full((B, Smax, 576), np.nan, np.float32)  # slots past a length are never read
    for b in range(B):
        if lens[b]:
            kk, _ = decode_cache_seq(wl, b, int(lens[b]), seed=31)
            cache[b, :lens[b]] = kk[0]
    out = g.mla_decode(dev(q), dev(cache), dev(lens, torch.int32), MLA_SCALE)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    ref = oracle.mla_decode(q, np.nan_to_num(cache), lens, MLA_SCALE)
    check(got, ref, head_axis=1)


# A key aligned with one head's query, scaled by c, scores far above everything before it in its
# sequence: by about 40 log2 units at c = 0.5 (weights up to 2^40 against the reference the first
# block set, taken in place) and by several hundred at c = 4 (past 2^64: the share is flagged and
# computed again by the rescaling kernel).
@pytest.mark.parametrize("c", [0.5, 4.0])
def test_mla_decode_score_jump(c):
    H, Smax, B = 32, 300, 2
    wl = MLA.with_(B=B, Hq=H, S=Smax, lens_lo=1, lens_hi=Smax)
    say("mla decode score jump", c)
    lens, q, _ = decode_lens_q(wl, seed=37)
    lens[:] = [Smax, 200]
    cache = np.zeros((B, Smax, 576), np.float32)
    for b in range(B):
        kk, _ = decode_cache_seq(wl, b, int(lens[b]), seed=37)
        cache[b, :lens[b]] = kk[0]
        qb = torch.as_tensor(q[b, 5]).to(torch.bfloat16).float().numpy()
        cache[b, lens[b] - 1] = c * qb
    out = g.mla_decode(dev(q), dev(cache), dev(lens, torch.int32), MLA_SCALE)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    cache_b = torch.as_tensor(cache).to(torch.bfloat16).float().numpy()
    ref = oracle.mla_decode(q, cache_b, lens, MLA_SCALE)
    check(got, ref, head_axis=1)


def test_full_size_mla_decode_sampled():
    # the bench's DeepSeek-V3-shaped batch and launch, sampled sequences checked by the oracle
    import bench
    mx, _, _, _ = bench.run_mla(MLA, 1, 0, torch, g)
    lens = mx["lens"]
    got = mx["out"].float().cpu().numpy()
    assert np.isfinite(got).all()
    for b in sorted({int(np.argmin(lens)), int(np.argmax(lens)), 0}):
        n = int(lens[b])
        ref = oracle.mla_decode_one(mx["q"][b].float().cpu().numpy(),
                                    mx["cache"][b, :n].float().cpu().numpy(), n, mx["scale"])
        check(got[b][None], ref[None], head_axis=1)
