"""CPU tests of the C ABI: the library loads, exports every declared symbol, validates host-side
arguments before launching anything, and computes the rotary frequency schedule on the host
exactly as the oracle does.  No call here reaches a kernel launch."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
g = pytest.importorskip("gqa_scaled_rope_amd")

if not os.path.exists(g.LIB_PATH):
    pytest.skip("libgqa_rope.so not built", allow_module_level=True)

lib = g.library()


def test_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "gqa_rope.h")).read()
    declared = set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(gqa_[a-z_0-9]+)\s*\(", header,
                              re.M))
    assert declared, "no declarations parsed"
    assert declared == set(g.EXPORTS), (declared ^ set(g.EXPORTS))
    for name in declared:
        assert hasattr(lib, name)


def test_version():
    assert b"gfx950" in lib.gqa_version()


def _cfg(**kw):
    base = dict(dtype=1, head_dim=128, num_q_heads=32, num_kv_heads=8, rotary_dim=0, rot_style=0,
                cos_table=None, sin_table=None, table_len=0, qk_norm=0, eps=1e-6, q_norm_w=None,
                k_norm_w=None, scale=0.0, softcap=0.0, sinks=None, chunk_size=0, chunk_lookback=0,
                kernel=0, reserved=0)
    base.update(kw)
    c = g._AttnCfg()
    for k, v in base.items():
        setattr(c, k, v)
    return c


FAKE = 1 << 20  # aligned non-null host-side stand-in; validation fails before any use


def _prefill(c, B=1, L=4, S=4, n_cached=0, window=0, q=FAKE, k=FAKE, v=FAKE, pos=FAKE, kpos=FAKE,
             out=FAKE, ws=None, ws_bytes=0):
    return lib.gqa_attn_prefill(ctypes.byref(c) if c is not None else None, q, k, v, pos, 0, kpos,
                                0, B, L, S, n_cached, window, out, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(dtype=5), 3, "dtype"),
    (dict(head_dim=100), 2, "head_dim"),
    (dict(head_dim=512), 2, "head_dim"),
    (dict(num_kv_heads=7), 2, "multiple of num_kv_heads"),
    (dict(num_q_heads=0), 2, "num_q_heads"),
    (dict(rotary_dim=63), 2, "rotary_dim"),
    (dict(rotary_dim=256), 2, "rotary_dim"),
    (dict(rotary_dim=64), 1, "cos_table"),
    (dict(rotary_dim=64, cos_table=FAKE, sin_table=FAKE, table_len=0), 2, "table_len"),
    (dict(rotary_dim=64, cos_table=FAKE + 4, sin_table=FAKE, table_len=8), 7, "aligned"),
    (dict(rot_style=3), 7, "rot_style"),
    (dict(qk_norm=1), 1, "q_norm_w"),
    (dict(qk_norm=1, q_norm_w=FAKE, k_norm_w=FAKE, eps=-1.0), 7, "eps"),
    (dict(scale=-1.0), 7, "scale"),
    (dict(softcap=float("nan")), 7, "softcap"),
    (dict(sinks=FAKE + 2), 7, "sinks"),
    (dict(chunk_size=-1), 2, "chunk_size"),
    (dict(chunk_size=64, chunk_lookback=-1), 2, "chunk_lookback"),
    (dict(kernel=6), 7, "kernel"),
    (dict(kernel=-1), 7, "kernel"),
    (dict(reserved=1), 7, "reserved"),
])
def test_prefill_rejects_bad_cfg(kw, status, msg):
    st = _prefill(_cfg(**kw))
    assert st == status
    assert msg in g.last_error()


def test_prefill_rejects_bad_sizes_and_pointers():
    c = _cfg()
    assert _prefill(None) == 1
    assert _prefill(c, B=-1) == 2
    assert _prefill(c, n_cached=5, S=4) == 2 and "n_cached" in g.last_error()
    assert _prefill(c, window=-3) == 2
    assert _prefill(c, q=None) == 1
    assert _prefill(c, k=None) == 1
    assert _prefill(c, q=FAKE + 2) == 7
    # an empty problem is a no-op: returns OK without touching any pointer
    assert _prefill(c, B=0, q=None, k=None, v=None, pos=None, kpos=None, out=None) == 0
    assert _prefill(c, L=0, q=None, k=None, v=None, pos=None, kpos=None, out=None) == 0
    assert g.last_error() == ""
    # workspace: null with bytes, misaligned, too small for a shape that needs key preparation
    assert _prefill(c, ws=None, ws_bytes=64) == 5
    assert _prefill(c, ws=FAKE + 16, ws_bytes=1 << 20) == 5
    cr = _cfg(rotary_dim=128, cos_table=FAKE, sin_table=FAKE, table_len=8)
    need = lib.gqa_prefill_workspace_bytes(ctypes.byref(cr), 2, 300, 100)
    # new keys plus the last 31 cached rows (so that a 32-key tile reads one source), bf16,
    # rounded up to 256 bytes; then room for split partials: 128 query blocks x 2 halves x 66
    # values x 512 threads x 4 bytes
    keys = 2 * (200 + 31) * 8 * 128 * 2
    split = 128 * 2 * 66 * 512 * 4
    assert need == (keys + 255) // 256 * 256 + split
    # too small for the prepared keys: refused (a size between the two would run, unsplit)
    assert _prefill(cr, B=2, L=300, S=300, n_cached=100, ws=FAKE, ws_bytes=keys - 2) == 5
    assert lib.gqa_prefill_workspace_bytes(ctypes.byref(cr), 2, 300, 300) == split  # all cached
    assert lib.gqa_prefill_workspace_bytes(ctypes.byref(_cfg()), 2, 300, 0) == split  # no prep
    assert lib.gqa_prefill_workspace_bytes(ctypes.byref(cr), 2, 300, 301) == 0
    assert "n_cached" in g.last_error()


def test_decode_validation_and_workspace():
    c = _cfg()
    need = lib.gqa_decode_workspace_bytes(ctypes.byref(c), 64, 32768)
    # split partials, B * Hkv * ceil(Smax/1024) * G * (D + 2) floats, each part 256-aligned,
    # then the prepared queries, B * Hq * D bf16 (256-aligned), then one int32 per split launch
    # (the split size it chose, for the combine kernel)
    items = 64 * 8 * 32 * 4
    align = lambda x: (x + 255) // 256 * 256
    assert need == align(items * 128 * 4) + align(items * 2 * 4) + align(64 * 32 * 128 * 2) + 4
    # more than 2048 sequences take several split launches: one flag each
    need3 = lib.gqa_decode_workspace_bytes(ctypes.byref(c), 4100, 64)
    items3 = 4100 * 8 * 1 * 4
    assert need3 == (align(items3 * 128 * 4) + align(items3 * 2 * 4) + align(4100 * 32 * 128 * 2)
                     + 3 * 4)
    st = lib.gqa_attn_decode(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, 64, 32768, 0, FAKE, None,
                             0, None)
    assert st == 5 and "workspace" in g.last_error()
    st = lib.gqa_attn_decode(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, 64, 32768, 0, FAKE, FAKE,
                             need - 1, None)
    assert st == 5
    st = lib.gqa_attn_decode(ctypes.byref(c), FAKE, FAKE, FAKE, None, 2, 16, 0, FAKE, FAKE,
                             need, None)
    assert st == 1 and "lens" in g.last_error()
    assert lib.gqa_attn_decode(ctypes.byref(c), None, None, None, None, 0, 16, 0, None, None, 0,
                               None) == 0
    assert lib.gqa_attn_decode(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, 1, 0, 0, FAKE, FAKE, need,
                               None) == 2
    # fp32 runs on the generic kernel, which needs no workspace
    c32 = _cfg(dtype=0)
    assert lib.gqa_decode_workspace_bytes(ctypes.byref(c32), 64, 32768) == 0


def test_rope_param_validation():
    def st(**kw):
        p = g.RopeSpec(**{**dict(rotary_dim=64), **kw}).c_struct()
        return lib.gqa_rope_tables(ctypes.byref(p), 16, FAKE, FAKE, None)
    assert st(rotary_dim=63) == 2
    assert st(theta=0.0) == 7
    assert st(kind="linear", factor=0.0) == 7
    assert st(kind="llama3", factor=8.0, low_freq_factor=4.0, high_freq_factor=1.0) == 7
    p = g.RopeSpec(64).c_struct()
    p.kind = 9
    assert lib.gqa_rope_tables(ctypes.byref(p), 16, FAKE, FAKE, None) == 4
    assert "unknown rope kind" in g.last_error()
    p = g.RopeSpec(64).c_struct()
    assert lib.gqa_rope_tables(ctypes.byref(p), 0, FAKE, FAKE, None) == 2
    with pytest.raises(g.GQAError):
        g.RopeSpec(64, kind="dynamic").c_struct()
    assert st(kind="yarn", factor=0.0) == 7
    assert st(kind="yarn", factor=4.0, beta_fast=1.0, beta_slow=2.0) == 7
    assert st(kind="yarn", factor=4.0, original_max_pos=0.0) == 7
    assert st(kind="longrope") == 1                       # no short table
    assert "short_factor" in g.last_error()
    assert st(kind="longrope", short_factor=[1.0] * 32, seq_len=9000) == 1   # needs the long one
    assert st(kind="longrope", short_factor=[1.0] * 31 + [0.0]) == 7
    with pytest.raises(g.GQAError):
        g.RopeSpec(64, kind="longrope", short_factor=[1.0] * 31).c_struct()
    p = g.RopeSpec(64).c_struct()
    p.reserved = 1
    assert lib.gqa_rope_tables(ctypes.byref(p), 16, FAKE, FAKE, None) == 7


@pytest.mark.parametrize("R,kind,theta,factor", [
    (128, "default", 1e6, 1.0), (64, "default", 1e4, 1.0), (32, "linear", 1e4, 4.0),
    (128, "llama3", 5e5, 8.0), (64, "llama3", 5e5, 8.0), (2, "default", 1e4, 1.0),
])
def test_host_inv_freq_matches_oracle(R, kind, theta, factor):
    got = np.array(g.rope_inv_freq(g.RopeSpec(R, kind, theta, factor, 1.0, 4.0, 8192.0)))
    ref = oracle.rope_inv_freq(R, theta, kind, factor, 1.0, 4.0, 8192.0)
    np.testing.assert_allclose(got, ref, rtol=1e-15, atol=0)


_LONG = [1.0 + 0.05 * i for i in range(32)]
_SHORT = [1.0 + 0.01 * i for i in range(32)]


@pytest.mark.parametrize("kw,okw", [
    (dict(rotary_dim=128, theta=1e4, factor=4.0, original_max_pos=4096.0), {}),
    (dict(rotary_dim=64, theta=1e4, factor=40.0, original_max_pos=4096.0, beta_fast=32.0,
          beta_slow=1.0), dict(beta_fast=32.0, beta_slow=1.0)),
    (dict(rotary_dim=128, theta=5e5, factor=8.0, original_max_pos=8192.0, truncate=False),
     dict(truncate=False)),
    (dict(rotary_dim=32, theta=1e6, factor=16.0, original_max_pos=2048.0, beta_fast=16.0,
          beta_slow=2.0, truncate=False), dict(beta_fast=16.0, beta_slow=2.0, truncate=False)),
])
def test_host_yarn_matches_oracle(kw, okw):
    spec = g.RopeSpec(kind="yarn", **kw)
    got = np.array(g.rope_inv_freq(spec))
    ref = oracle.rope_inv_freq(kw["rotary_dim"], kw["theta"], "yarn", kw["factor"],
                               original_max_position_embeddings=kw["original_max_pos"], **okw)
    np.testing.assert_allclose(got, ref, rtol=1e-15, atol=0)


@pytest.mark.parametrize("seq_len", [0, 4096, 4097, 131072])
def test_host_longrope_matches_oracle(seq_len):
    spec = g.RopeSpec(64, "longrope", 1e4, original_max_pos=4096.0, short_factor=_SHORT,
                      long_factor=_LONG, seq_len=seq_len)
    got = np.array(g.rope_inv_freq(spec))
    ref = oracle.rope_inv_freq(64, 1e4, "longrope", original_max_position_embeddings=4096.0,
                               short_factor=_SHORT, long_factor=_LONG, seq_len=seq_len)
    np.testing.assert_allclose(got, ref, rtol=1e-15, atol=0)


@pytest.mark.parametrize("kind,factor,extra", [
    ("default", 1.0, {}), ("llama3", 8.0, {}), ("yarn", 4.0, {}), ("yarn", 0.5, {}),
    ("yarn", 40.0, dict(mscale=1.0, mscale_all_dim=0.707)),
    ("yarn", 40.0, dict(mscale=0.707, mscale_all_dim=0.707)),
    ("yarn", 40.0, dict(mscale_all_dim=1.0)),
    ("yarn", 16.0, dict(attention_factor=1.25)), ("longrope", 1.0, {}),
    ("longrope", 1.0, dict(attention_factor=1.19)),
])
def test_host_attention_factor_and_softmax_scale_match_oracle(kind, factor, extra):
    spec = g.RopeSpec(64, kind, 1e4, factor, original_max_pos=4096.0, short_factor=_SHORT,
                      **extra)
    ref = oracle.rope_attention_factor(kind, factor, **extra)
    assert g.rope_attention_factor(spec) == pytest.approx(ref, rel=1e-15)
    for qk_dim in (64, 128, 192):
        ref_sc = (oracle.yarn_softmax_scale(qk_dim, factor, extra.get("mscale_all_dim"))
                  if kind == "yarn" else qk_dim ** -0.5)
        assert g.rope_softmax_scale(spec, qk_dim) == pytest.approx(ref_sc, rel=1e-15)
    with pytest.raises(g.GQAError):
        g.rope_softmax_scale(spec, 0)


def test_noalloc_decode_validates_before_touching_the_gpu():
    # sizes whose partials exceed the fixed scratch are refused on the host, as are the ordinary
    # argument errors of gqa_attn_decode
    c = _cfg()
    assert lib.gqa_decode_workspace_bytes(ctypes.byref(c), 64, 65536) > g.DECODE_NOALLOC_MAX_BYTES
    st = lib.gqa_attn_decode_noalloc(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, 64, 65536, 0, FAKE,
                                     None)
    assert st == 5 and "no-allocation" in g.last_error()
    st = lib.gqa_attn_decode_noalloc(ctypes.byref(c), FAKE, FAKE, FAKE, None, 2, 16, 0, FAKE, None)
    assert st == 1 and "lens" in g.last_error()
    assert lib.gqa_attn_decode_noalloc(ctypes.byref(c), None, None, None, None, 0, 16, 0, None,
                                       None) == 0
    assert lib.gqa_attn_decode_noalloc(ctypes.byref(_cfg(kernel=9)), FAKE, FAKE, FAKE, FAKE, 1, 16,
                                       0, FAKE, None) == 7


def test_kernel_choice_is_per_call():
    # the library exports no selection state: the choice travels in each call's cfg
    assert not any("policy" in name for name in g.EXPORTS)
    with pytest.raises(g.GQAError):
        g.AttnConfig("bf16", 128, 32, 8, kernel="fastest").c_struct()
    for name, val in g.KERNELS.items():
        assert g.AttnConfig("bf16", 128, 32, 8, kernel=name).c_struct().kernel == val
    # a generic-kernel call needs no decode workspace; the forced split sizes use the MFMA one
    c = _cfg()
    need = lib.gqa_decode_workspace_bytes(ctypes.byref(c), 4, 4096)
    assert need > 0
    assert lib.gqa_decode_workspace_bytes(ctypes.byref(_cfg(kernel=1)), 4, 4096) == 0
    assert lib.gqa_decode_workspace_bytes(ctypes.byref(_cfg(kernel=2)), 4, 4096) == need
    assert lib.gqa_decode_workspace_bytes(ctypes.byref(_cfg(kernel=3)), 4, 4096) == need
    # prefill: the generic kernel needs no key-preparation workspace
    cr = dict(rotary_dim=128, cos_table=FAKE, sin_table=FAKE, table_len=8)
    assert lib.gqa_prefill_workspace_bytes(ctypes.byref(_cfg(**cr)), 2, 300, 100) > 0
    assert lib.gqa_prefill_workspace_bytes(ctypes.byref(_cfg(kernel=1, **cr)), 2, 300, 100) == 0


def _prefill_kernel(c, B, L, S, n_cached=0, window=0, ws=1):
    which = ctypes.c_int32(-1)
    assert lib.gqa_prefill_kernel(ctypes.byref(c), B, L, S, n_cached, window, ws,
                                  ctypes.byref(which)) == 0, g.last_error()
    return g.PREFILL_KERNELS[which.value]


def test_prefill_kernel_choice():
    # the benchmark prefill shapes: long key bands on the eight-wavefront streaming kernel, the
    # 128-key window (about 160 keys per workgroup) on the four-wavefront one
    from synth import WORKLOADS
    want = {"qwen3_prefill_bf16": "stream_long", "mistral_swa_prefill_bf16": "stream_long",
            "chunked_prefill_bf16_w4096": "stream_long", "chunked_prefill_bf16_full": "stream_long",
            "sinks_swa128_prefill_bf16": "stream_short"}
    for name, kern in want.items():
        wl = WORKLOADS[name]
        c = _cfg(num_q_heads=wl.Hq, num_kv_heads=wl.Hkv, rotary_dim=wl.rotary_dim,
                 rot_style=0 if wl.style == "half" else 1, cos_table=FAKE, sin_table=FAKE,
                 table_len=8, qk_norm=int(wl.qk_norm), q_norm_w=FAKE if wl.qk_norm else None,
                 k_norm_w=FAKE if wl.qk_norm else None)
        assert _prefill_kernel(c, wl.B, wl.L, wl.S, wl.n_cached, wl.window) == kern, name
    cr = dict(rotary_dim=128, cos_table=FAKE, sin_table=FAKE, table_len=8)
    # forced either way; without a workspace the fused kernel; generic and fp32 on generic
    assert _prefill_kernel(_cfg(kernel=5, **cr), 2, 8192, 8192, 0, 4096) == "stream_short"
    assert _prefill_kernel(_cfg(kernel=4, **cr), 4, 4096, 4096, 0, 128) == "stream_long"
    assert _prefill_kernel(_cfg(**cr), 2, 8192, 8192, 0, 4096, ws=0) == "fused"
    assert _prefill_kernel(_cfg(kernel=1, **cr), 2, 8192, 8192, 0, 4096) == "generic"
    assert _prefill_kernel(_cfg(dtype=0, **cr), 2, 64, 64) == "generic"
    # nothing to prepare (no rotation, no norm): the stream kernels need no workspace
    assert _prefill_kernel(_cfg(), 2, 8192, 8192, 0, 0, ws=0) == "stream_long"
    which = ctypes.c_int32(-1)
    assert lib.gqa_prefill_kernel(ctypes.byref(_cfg()), 1, 4, 4, 5, 0, 1, ctypes.byref(which)) == 2


def test_second_hip_runtime_is_detected():
    # two different libamdhip64 files mapped into one process is the state in which torch's
    # streams are invalid for the library; the loader refuses it
    one = ("7f00-7f10 r-xp 00000000 08:01 11 /opt/x/torch/lib/libamdhip64.so\n"
           "7f10-7f20 r--p 00010000 08:01 11 /opt/x/torch/lib/libamdhip64.so\n"
           "7f30-7f40 r-xp 00000000 08:01 12 /usr/lib/libc.so.6\n")
    two = one + "7f50-7f60 r-xp 00000000 08:01 13 /opt/rocm/lib/libamdhip64.so.7.2.0\n"
    assert len(g.hip_runtimes_mapped(one)) == 1
    assert len(g.hip_runtimes_mapped(two)) == 2
    assert len(g.hip_runtimes_mapped("")) == 0
    # this process (torch imported first, library loaded) holds at most one
    assert len(g.hip_runtimes_mapped()) <= 1


def test_decode_byte_model_matches_page(golden):
    # the decode traffic model used by the bench: 2 (K, V) * Hkv * D * bytes per cached token
    # per layer; the page prints the per-token KV size of whole models
    import bench
    for row in golden("kv_bytes_per_token.json")["rows"]:
        per_layer = bench.kv_bytes_per_token_per_layer(row["kv_heads"], row["head_dim"],
                                                       row["bytes_per_elem"])
        kib = row["layers"] * per_layer / 1024
        assert kib == row["kv_KiB_per_token"]
        assert row["layers"] * per_layer * 32768 / 2 ** 30 == pytest.approx(row["GiB_for_32k_tokens"])


def test_counter_traffic_only_for_its_workload():
    # the HBM byte counters are kept per (kernel, workload): a bench line for a workload without
    # counters reports no traffic rather than another workload's bytes
    import bench
    import json
    with open(os.path.join(os.path.dirname(bench.__file__), "profiles", "traffic.json")) as f:
        kernels = json.load(f)["kernels"]
    assert kernels
    for kernel, per_workload in kernels.items():
        for workload, rec in per_workload.items():
            assert bench.measured_traffic(kernel, workload + "_other") is None
            got = bench.measured_traffic(kernel, workload)
            # None once the kernel's source has changed since the counters were taken
            assert got is None or got == int(rec["hbm_bytes_per_launch"])


def test_prefill_flop_model():
    # allowed (query, key) pairs per (b, h) for the workloads, counted by brute force over
    # positions at a reduced size and by the closed form used in the bench
    import bench
    for L, S, w, nc in ((64, 64, 0, 0), (64, 64, 16, 0), (16, 64, 0, 48), (16, 64, 32, 48)):
        qp = np.arange(S - L, S) if nc else np.arange(L)
        brute = int(oracle.allowed_mask(qp, np.arange(S), w).sum())
        assert bench.allowed_pairs(L, S, w, nc) == brute
    for L, S, w, nc, c, lb in ((64, 64, 0, 0, 8, 0), (64, 64, 0, 0, 7, 1), (16, 64, 5, 48, 6, 2),
                               (64, 64, 0, 0, 1, 0), (64, 64, 0, 0, 1000, 0)):
        qp = np.arange(S - L, S) if nc else np.arange(L)
        brute = int(oracle.allowed_mask(qp, np.arange(S), w, c, lb).sum())
        assert bench.allowed_pairs(L, S, w, nc, c, lb) == brute
    assert bench.allowed_pairs(16384, 16384, 0, 0, 8192, 0) == 2 * 8192 * 8193 // 2
    assert bench.allowed_pairs(2048, 2048, 0, 0) == 2098176
    assert bench.allowed_pairs(8192, 8192, 4096, 0) == 25167872
    assert bench.allowed_pairs(512, 4096, 4096, 3584) == 1966336
    assert bench.allowed_pairs(512, 4096, 0, 3584) == 1966336
    assert math.isclose(4 * 4 * 32 * 128 * 2098176, 1.3751e11, rel_tol=1e-4)


def test_decode_key_count_model():
    # rows a decode query reads = allowed keys of the last row, by the oracle's mask
    import bench
    from synth import WORKLOADS
    for kw in (dict(window=0), dict(window=100), dict(chunk=64), dict(chunk=64, chunk_lookback=1),
               dict(chunk=50, window=70)):
        wl = WORKLOADS["llama31_decode_bf16"].with_(**kw)
        for n in (1, 63, 64, 65, 129, 1000):
            want = int(oracle.allowed_mask([n - 1], np.arange(n), wl.window, wl.chunk,
                                           wl.chunk_lookback).sum())
            assert bench.decode_keys(wl, n) == want


def test_c_struct_layout_matches_ctypes(tmp_path):
    # the ctypes mirrors of the two public structs have the header's sizes and offsets
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    fields = {"gqa_attn_cfg": g._AttnCfg, "gqa_rope_params": g._RopeParams,
              "gqa_paged_kv": g._PagedKV}
    lines = []
    for cname, py in fields.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    src = tmp_path / "lay.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "gqa_rope.h"\n'
                   "int main(void) {" + "".join(lines) + "return 0;}\n")
    exe = tmp_path / "lay"
    r = subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(root, "include"),
                        "-I", "/opt/rocm/include", str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("header needs the HIP runtime headers: " + r.stderr[-200:])
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    for line in filter(None, out):
        cname, what, val = line.split()
        py = fields[cname]
        want = ctypes.sizeof(py) if what == "size" else getattr(py, what).offset
        assert int(val) == want, line


def _paged(**kw):
    base = dict(k_pool=FAKE, v_pool=FAKE, block_table=FAKE, max_blocks=8, block_size=16,
                num_blocks=32, reserved=0)
    base.update(kw)
    p = g._PagedKV()
    for k, v in base.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("kw,status,msg", [
    (dict(block_size=24), 7, "power of two"),
    (dict(block_size=8), 7, "power of two"),
    (dict(block_size=2048), 7, "power of two"),
    (dict(max_blocks=0), 2, "max_blocks"),
    (dict(num_blocks=0), 2, "num_blocks"),
    (dict(k_pool=None), 1, "k_pool"),
    (dict(block_table=None), 1, "block_table"),
    (dict(v_pool=FAKE + 8), 7, "aligned"),
    (dict(reserved=3), 7, "reserved"),
])
def test_paged_validation(kw, status, msg):
    c = _cfg()
    kv = _paged(**kw)
    st = lib.gqa_attn_decode_paged(ctypes.byref(c), FAKE, ctypes.byref(kv), FAKE, 2, 0, FAKE, FAKE,
                                   1 << 30, None)
    assert st == status and msg in g.last_error()
    st = lib.gqa_paged_append(ctypes.byref(c), ctypes.byref(kv), FAKE, FAKE, FAKE, 0, FAKE, 2, 1,
                              None)
    assert st == status and msg in g.last_error()
    assert lib.gqa_paged_decode_workspace_bytes(ctypes.byref(c), ctypes.byref(kv), 2) == 0


def test_paged_workspace_and_support():
    c = _cfg()
    kv = _paged()
    # same split partials as a contiguous cache of max_blocks * block_size slots
    assert (lib.gqa_paged_decode_workspace_bytes(ctypes.byref(c), ctypes.byref(kv), 64) ==
            lib.gqa_decode_workspace_bytes(ctypes.byref(c), 64, 8 * 16))
    assert lib.gqa_attn_decode_paged(ctypes.byref(_cfg(dtype=0)), FAKE, ctypes.byref(kv), FAKE, 2,
                                     0, FAKE, FAKE, 1 << 30, None) == 4
    assert lib.gqa_attn_decode_paged(ctypes.byref(_cfg(num_q_heads=64, num_kv_heads=2)), FAKE,
                                     ctypes.byref(kv), FAKE, 2, 0, FAKE, FAKE, 1 << 30, None) == 4
    need = lib.gqa_paged_decode_workspace_bytes(ctypes.byref(c), ctypes.byref(kv), 2)
    assert lib.gqa_attn_decode_paged(ctypes.byref(c), FAKE, ctypes.byref(kv), FAKE, 2, 0, FAKE,
                                     FAKE, need - 1, None) == 5
    # empty problems are no-ops
    assert lib.gqa_attn_decode_paged(ctypes.byref(c), None, ctypes.byref(kv), None, 0, 0, None,
                                     None, 0, None) == 0
    assert lib.gqa_paged_append(ctypes.byref(c), ctypes.byref(kv), None, None, None, 0, None, 3, 0,
                                None) == 0


def test_mla_validation_and_workspace():
    assert lib.gqa_mla_decode_workspace_bytes(2, 24, 100) == 0 and "multiple of 16" in g.last_error()
    assert lib.gqa_mla_decode_workspace_bytes(2, 16, 0) == 0
    n = lib.gqa_mla_decode_workspace_bytes(2, 16, 4096)
    # per (piece slot, head) a 512-wide partial and (m, l); 256 shares + B sequences of slots;
    # then one recompute flag per (head group, share, wavefront of the 32-head kernel)
    a256 = lambda x: (x + 255) // 256 * 256
    assert n == a256((256 + 2) * 16 * 512 * 4) + a256((256 + 2) * 16 * 2 * 4) + 1 * 256 * 4 * 4
    assert lib.gqa_mla_decode_workspace_bytes(2, 144, 4096) == (
        a256((256 + 2) * 144 * 512 * 4) + a256((256 + 2) * 144 * 2 * 4) + 2 * 256 * 4 * 4)
    assert lib.gqa_mla_decode_workspace_bytes(2, 16, 100000) == n  # independent of Smax
    call = lambda **kw: lib.gqa_mla_decode(*[kw.get(k, d) for k, d in (
        ("q", FAKE), ("c", FAKE), ("lens", FAKE), ("B", 2), ("H", 16), ("S", 4096),
        ("scale", 0.1), ("out", FAKE), ("ws", FAKE), ("nb", n), ("st", None))])
    assert call(H=8) == 2
    assert call(scale=0.0) == 7 and "scale" in g.last_error()
    assert call(q=None) == 1
    assert call(out=FAKE + 4) == 7
    assert call(nb=n - 1) == 5
    assert call(ws=FAKE + 16) == 5
    assert call(B=0, q=None, c=None, lens=None, out=None, ws=None, nb=0) == 0
    assert call(B=65535, S=1 << 21) == 2 and "32 bits" in g.last_error()
