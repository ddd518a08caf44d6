"""Benchmark of the rotary grouped-query attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --only NAME [--steps K] [--warmup W]      (one workload, for the profiler)

One step = one pass of the whole hot path over one batch of synthetic input, inputs resident in
HBM: the rotary tables (gqa_rope_tables), the key preparation that norms and rotates the new keys
into the K cache (gqa_prep_keys), and the attention over the cache (gqa_attn_prefill with every
key used as stored), replayed as one HIP graph.  The headline workload is the largest prefill
that fits one GPU, the Mistral-style sliding-window prefill (B=2, L=S=8192, Hq=32, Hkv=8, D=128,
window 4096).  Every other workload of the scope is timed in the same run and reported under
"configs" with its own roofline and CPU baseline: the tiny fp32 causal prefill (latency only),
the Qwen3-style prefill, the chunked prefill in both layer kinds (window 4096, full) and the
Llama-3.1-style split-KV decode; the paged-pool decode and the latent-attention decode follow
under "extras".

Prints ONE JSON line on stdout (progress goes to stderr).  FLOPs count only allowed
(query, key) pairs, 4 * D per pair per head; decode bytes are the K and V rows each sequence
actually reads plus q, out and lens.  Kernel times come from HIP events recorded on the stream
the kernels are launched on, around K back-to-back launches of the timed call.  Before each timed
region the W warmup calls run, continued until at least 50 ms of GPU work has run back to back
(the clock's ramp after an idle gap; "warmup_min_gpu_ms" in the line).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3           # MI355X fp32 vector
HBM_PEAK_GBS = 8000.0              # MI355X HBM3E
METRIC = "prefill attn TFLOP/s (% MFMA peak); decode KV GB/s (% HBM peak)"


# ---- work models (pure functions; pinned by tests/test_abi_cpu.py) -----------------------------
def allowed_pairs(L, S, window, n_cached, chunk=0, chunk_lookback=0):
    """Allowed (query, key) pairs of one (sequence, head): queries at positions S-L..S-1 when
    keys before them are cached, else 0..L-1; keys at 0..S-1.  With chunks each query sees
    its own chunk and chunk_lookback chunks before it (and at most `window` keys)."""
    start = S - L if n_cached else 0
    if chunk > 0:
        import numpy as np
        p = np.arange(start, start + L, dtype=np.int64)
        lo = np.maximum(0, (p // chunk - chunk_lookback) * chunk)
        if window > 0:
            lo = np.maximum(lo, p - window + 1)
        return int(np.maximum(np.minimum(p, S - 1) - lo + 1, 0).sum())

    def upto(n):  # sum over positions p < n of min(p + 1, w), w = infinity when 0
        if n <= 0:
            return 0
        if window <= 0 or n <= window:
            return n * (n + 1) // 2
        return window * (window + 1) // 2 + (n - window) * window
    return upto(start + L) - upto(start)


def prefill_flops(wl):
    return 4 * wl.B * wl.Hq * wl.D * allowed_pairs(wl.L, wl.S, wl.window, wl.n_cached, wl.chunk,
                                                   wl.chunk_lookback)


def kv_bytes_per_token_per_layer(kv_heads, head_dim, bytes_per_elem):
    return 2 * kv_heads * head_dim * bytes_per_elem


def decode_keys(wl, n):
    """Cache rows a decode query at position n - 1 reads: its window and chunks."""
    first = 0
    if wl.window:
        first = max(first, n - wl.window)
    if wl.chunk:
        first = max(first, ((n - 1) // wl.chunk - wl.chunk_lookback) * wl.chunk)
    return n - first


def decode_bytes(wl, lens):
    eb = 2 if wl.dtype == "bf16" else 4
    keys = sum(decode_keys(wl, int(n)) for n in lens)
    return (keys * kv_bytes_per_token_per_layer(wl.Hkv, wl.D, eb)
            + 2 * wl.B * wl.Hq * wl.D * eb + 4 * wl.B)


# symbol names of the prefill kernels, by gqa_prefill_kernel's answer
PREFILL_KERNEL_NAMES = {"stream_long": "prefill_stream_kernel", "stream_short": "prefill_short_kernel",
                        "fused": "prefill_mfma_kernel", "generic": "attn_generic_kernel"}


def profile_record(kernel, workload):
    """The committed counter summary of `kernel` on `workload` (profiles/traffic.json), or None
    when no counters were taken on that workload or the kernel's source has changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)["kernels"][kernel][workload]
        with open(os.path.join(ROOT, rec["source"]), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != rec["source_sha256"]:
                return None
        return rec
    except (OSError, KeyError, ValueError, TypeError):
        return None


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter runs
    (FETCH_SIZE and WRITE_SIZE scaled by a known-size copy), or None (see profile_record)."""
    rec = profile_record(kernel, workload)
    try:
        return int(rec["hbm_bytes_per_launch"]) if rec else None
    except (KeyError, ValueError, TypeError):
        return None


def measured_mfma(kernel, workload):
    """MFMA busy share of SIMD cycles (SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs x GRBM_GUI_ACTIVE
    per XCD) and the clock of that counter run, from the committed counters, or (None, None)."""
    rec = profile_record(kernel, workload) or {}
    return rec.get("mfma_busy"), rec.get("clock_ghz_counter_run")


# ---- helpers ---------------------------------------------------------------------------------
def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _rope_spec(g, wl):
    return g.RopeSpec(wl.rotary_dim, wl.rope_kind, wl.theta, wl.factor, wl.low_freq_factor,
                      wl.high_freq_factor, wl.original_max_pos)


def _mask_cfg(wl, torch):
    """Learned sinks (seeded draw) and chunking of a workload, as AttnConfig fields."""
    from synth import draw_sinks
    sk = draw_sinks(wl)
    return dict(sinks=None if sk is None else torch.from_numpy(sk).to("cuda"),
                chunk_size=wl.chunk, chunk_lookback=wl.chunk_lookback)


def _prefill_setup(wl, torch, g):
    from synth import device_normal
    dev = "cuda"
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    q = device_normal((wl.B, wl.L, wl.Hq, wl.D), wl.seed * 10 + 1, wl.dtype)
    k = device_normal((wl.B, wl.S, wl.Hkv, wl.D), wl.seed * 10 + 2, wl.dtype)
    v = device_normal((wl.B, wl.S, wl.Hkv, wl.D), wl.seed * 10 + 3, wl.dtype)
    qw = kw = None
    if wl.qk_norm:
        qw = (1.0 + 0.02 * device_normal((wl.D,), wl.seed * 10 + 4, "f32")).to(dt)
        kw = (1.0 + 0.02 * device_normal((wl.D,), wl.seed * 10 + 5, "f32")).to(dt)
    start = wl.S - wl.L if wl.n_cached else 0
    pos = torch.arange(start, start + wl.L, dtype=torch.int32, device=dev)
    kpos = torch.arange(wl.S, dtype=torch.int32, device=dev)
    table_len = wl.S
    cos = torch.empty((table_len, wl.rotary_dim // 2), dtype=torch.float32, device=dev)
    sin = torch.empty_like(cos)
    cfg = g.AttnConfig(wl.dtype, wl.D, wl.Hq, wl.Hkv, wl.rotary_dim, wl.style, cos, sin,
                       wl.qk_norm, wl.eps, qw, kw, 0.0, wl.softcap, **_mask_cfg(wl, torch))
    out = torch.empty_like(q)
    kcache = k.clone()   # rows < n_cached: the cache as stored; the rest is rewritten each step
    # the attention call's workspace (its keys are prepared: n_cached = S), allocated once: room
    # for the split key walks of a last, partial round of query blocks
    nws = g.prefill_workspace_bytes(cfg, wl.B, wl.S, wl.S) if wl.dtype == "bf16" else 0
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    return dict(q=q, k=k, v=v, qw=qw, kw=kw, pos=pos, kpos=kpos, cos=cos, sin=sin, cfg=cfg,
                out=out, table_len=table_len, kcache=kcache, ws=ws)


SETTLE_MS = 50.0   # least GPU time of untimed warmup before a timed region


def _warm_up(fn, warmup, torch):
    """The W untimed warmup calls, continued in batches until at least SETTLE_MS of GPU time has
    run back to back: after an idle gap (a graph capture, a check, the CPU baseline) MI355X
    raises its clock over the first tens of milliseconds of load, and a timed region that starts
    inside that ramp reads up to 15% slow (measured: 0.94 ms for the first Mistral-style steps
    after 0.5 s idle, 0.79 ms after 40 steps)."""
    n, ms = 0, 0.0
    while n < warmup or ms < SETTLE_MS:
        ms += _time_calls(fn, 4, torch) * 4
        n += 4
    return n


def _time_calls(fn, n, torch):
    """Average ms of n back-to-back calls of fn, from HIP events on the current stream (the
    stream every library call here is launched on)."""
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(n):
        fn()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / n


def run_prefill(wl, steps, warmup, torch, g, graph=True):
    """The prefill step (tables, key preparation, attention) of workload wl: returns the inputs
    and outputs, the step time (ms, as replayed) and the time of each call alone (ms, n calls of
    that call back to back).  fp32 problems have no key-preparation pass (the attention call
    prepares the keys itself)."""
    x = _prefill_setup(wl, torch, g)
    spec = _rope_spec(g, wl)
    stream = torch.cuda.current_stream()
    bf16 = wl.dtype == "bf16"

    def tables():
        g.rope_tables(spec, x["table_len"], x["cos"], x["sin"])

    def prep():
        g.prep_keys(x["cfg"], x["k"], x["kpos"], wl.n_cached, k_out=x["kcache"])

    def attention():
        if bf16:
            g.attn_prefill(x["cfg"], x["q"], x["kcache"], x["v"], x["pos"], x["kpos"], wl.S,
                           wl.window, x["out"], workspace=x["ws"])
        else:
            g.attn_prefill(x["cfg"], x["q"], x["k"], x["v"], x["pos"], x["kpos"], wl.n_cached,
                           wl.window, x["out"], workspace=None)

    def launches():
        tables()
        if bf16:
            prep()
        attention()

    for _ in range(warmup):
        launches()
    torch.cuda.synchronize()
    step_fn = launches
    if graph:
        # the step's launches captured once as a HIP graph and replayed (no memset or allocation
        # is recorded: every buffer exists before the capture); the replayed output must match
        # the eager one bit for bit
        eager = x["out"].clone()
        hg = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            x["out"].zero_()
            torch.cuda.synchronize()
            with torch.cuda.graph(hg, stream=cap):
                launches()
        stream.wait_stream(cap)
        for _ in range(3):
            x["out"].zero_()
            hg.replay()
            torch.cuda.synchronize()
            if not torch.equal(x["out"], eager):
                raise RuntimeError("graph replay differs from the eager step")
        x["graph"] = hg
        step_fn = hg.replay
    _warm_up(step_fn, warmup, torch)
    step_ms = _time_calls(step_fn, steps, torch)
    # each call alone, back to back (the attention call reads the cache the step left)
    parts = {"rope_tables": _time_calls(tables, steps, torch)}
    if bf16:
        parts["prep_keys"] = _time_calls(prep, steps, torch)
    parts["attention"] = _time_calls(attention, steps, torch)
    return x, step_ms, parts


def prefill_record(wl, steps, warmup, torch, g, graph, cpu, budget_s):
    """Bench record of one prefill workload: step throughput, the attention kernel's roofline and,
    unless cpu is False, the oracle's rate on a bounded sample with parity on the timed outputs."""
    x, step_ms, parts = run_prefill(wl, steps, warmup, torch, g, graph=graph)
    flops = prefill_flops(wl)
    kern_ms = parts["attention"]
    achieved = flops / (kern_ms * 1e-3) / 1e12
    value = flops / (step_ms * 1e-3) / 1e12
    bf16 = wl.dtype == "bf16"
    log(f"[bench] {wl.name}: step {step_ms:.4f} ms ("
        + ", ".join(f"{k} {v:.4f}" for k, v in parts.items())
        + f") -> step {value:.1f}, attention {achieved:.1f} TFLOP/s")
    if bf16:
        # the kernel the attention call runs (it reads prepared keys: n_cached = S)
        kern = PREFILL_KERNEL_NAMES[g.prefill_kernel(x["cfg"], wl.B, wl.L, wl.S, wl.S, wl.window,
                                                     workspace=True)]
        roof = {"bound": "mfma", "kernel": kern, "achieved": round(achieved, 2),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(kern, wl.name),
                "kernel_ms_mean": round(kern_ms, 4), "algorithmic_flop": flops}
        # MFMA busy as rocprof counts it (at the clock the chip runs under this load, below the
        # 2.4 GHz of the peak figure)
        roof["mfma_busy_rocprof"], roof["clock_ghz_counter_run"] = measured_mfma(kern, wl.name)
    else:
        # 16 query rows: far too small to load any unit of the chip; reported against the fp32
        # vector peak for completeness, no roofline claim
        roof = {"bound": "alu", "kernel": "attn_generic_kernel", "achieved": round(achieved, 6),
                "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / FP32_PEAK_TFLOPS, 8), "traffic": None,
                "kernel_ms_mean": round(kern_ms, 5), "algorithmic_flop": flops,
                "note": "latency-bound (16 query rows); no roofline claim"}
    rec = {"workload": wl.name, "value": round(value, 4 if bf16 else 8), "unit": "TFLOP/s",
           "ms_per_step": round(step_ms, 5), "dtype": wl.dtype,
           "step_parts_ms": {k: round(v, 5) for k, v in parts.items()},
           "config": _config(wl), "roofline": roof}
    if not bf16:
        rec["latency_us"] = round(step_ms * 1e3, 2)
    if cpu:
        rec["cpu_baseline"] = cpu_baseline_prefill(wl, x, torch, budget_s)
        log(f"[bench] {wl.name}: cpu baseline {rec['cpu_baseline']['value']:.4g} TFLOP/s, parity "
            f"{rec['cpu_baseline']['parity_ok']}")
    del x
    torch.cuda.empty_cache()
    return rec


def _config(wl):
    return {"workload": wl.name, "B": wl.B, "L": wl.L, "S": wl.S, "Hq": wl.Hq, "Hkv": wl.Hkv,
            "head_dim": wl.D, "rotary_dim": wl.rotary_dim, "rot_style": wl.style,
            "rope": wl.rope_kind, "theta": wl.theta, "qk_norm": wl.qk_norm, "window": wl.window,
            "softcap": wl.softcap, "n_cached": wl.n_cached, "chunk": wl.chunk,
            "chunk_lookback": wl.chunk_lookback, "sinks": wl.sinks}


def run_decode(wl, steps, warmup, torch, g):
    from synth import decode_device_inputs
    x = decode_device_inputs(wl)
    spec = _rope_spec(g, wl)
    cos, sin = g.rope_tables(spec, wl.S)
    cfg = g.AttnConfig(wl.dtype, wl.D, wl.Hq, wl.Hkv, wl.rotary_dim, wl.style, cos, sin,
                       wl.qk_norm, wl.eps, x.get("qw"), x.get("kw"), 0.0, wl.softcap,
                       **_mask_cfg(wl, torch))
    ws = torch.empty(g.decode_workspace_bytes(cfg, wl.B, wl.S), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x["q"])

    def call():
        g.attn_decode(cfg, x["q"], x["k"], x["v"], x["lens"], wl.window, out, ws)

    _warm_up(call, warmup, torch)
    ms = _time_calls(call, steps, torch)
    x.update(cfg=cfg, out=out, cos=cos, sin=sin)
    return x, ms


def decode_record(wl, steps, warmup, torch, g, cpu, budget_s):
    dx, dms = run_decode(wl, steps, warmup, torch, g)
    lens = dx["lens"].cpu().tolist()
    nbytes = decode_bytes(wl, lens)
    gbs = nbytes / (dms * 1e-3) / 1e9
    log(f"[bench] {wl.name}: {dms:.4f} ms per call -> {gbs:.0f} GB/s")
    rec = {"workload": wl.name, "value": round(gbs, 1), "unit": "GB/s", "ms_per_call": round(dms, 4),
           "algorithmic_bytes": nbytes, "dtype": wl.dtype, "config": _config(wl),
           "roofline": {"bound": "hbm",
                        "kernel": "decode_prep_q_kernel + decode_split_kernel + "
                                  "decode_combine_kernel (one gqa_attn_decode call)",
                        "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic("decode_split_kernel", wl.name),
                        "kernel_ms_mean": round(dms, 4)}}
    if cpu:
        rec["cpu_baseline"] = cpu_baseline_decode(wl, dx, torch, budget_s)
        log(f"[bench] {wl.name}: cpu baseline {rec['cpu_baseline']['value']:.4g} GB/s, parity "
            f"{rec['cpu_baseline']['parity_ok']}")
    return rec, dx, nbytes


def run_decode_paged(wl, dx, block_size, steps, warmup, torch, g):
    """The decode workload again, its cache rows moved into a paged pool of block_size slots per
    block whose blocks are laid out in a seeded random order (a block table per sequence)."""
    B, Hkv, Smax, D = (int(t) for t in dx["k"].shape)
    nbps = (Smax + block_size - 1) // block_size
    gen = torch.Generator(device="cpu")
    gen.manual_seed(1234 + block_size)
    perm = torch.randperm(B * nbps, generator=gen).to("cuda")
    table = perm.view(B, nbps).to(torch.int32).contiguous()

    def to_pool(cache):
        blocks = cache.view(B, Hkv, nbps, block_size, D).permute(0, 2, 1, 3, 4).reshape(
            B * nbps, Hkv, block_size, D)
        pool = torch.empty_like(blocks)
        pool[perm] = blocks
        return pool
    kv = g.PagedKV(to_pool(dx["k"]), to_pool(dx["v"]), table)
    cfg = dx["cfg"]
    ws = torch.empty(g.paged_decode_workspace_bytes(cfg, kv, B), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dx["q"])
    def call():
        g.attn_decode_paged(cfg, dx["q"], kv, dx["lens"], wl.window, out, ws)

    _warm_up(call, warmup, torch)
    ms = _time_calls(call, steps, torch)
    same = bool(torch.equal(out, dx["out"]))
    del kv, ws
    return ms, same


MLA_ROW_BYTES = 576 * 2
MLA_FLOP_PER_KEY_HEAD = 2 * 576 + 2 * 512   # scores over 576 features, values over 512


def mla_scale():
    """DeepSeek-V3's softmax scale: qk_head_dim 192, YaRN factor 40 with mscale_all_dim 1."""
    import math
    m = 0.1 * 1.0 * math.log(40.0) + 1.0
    return 192 ** -0.5 * m * m


def run_mla(wl, steps, warmup, torch, g):
    """The absorbed latent-attention decode core over a DeepSeek-V3-shaped batch."""
    from synth import device_normal
    import numpy as np
    rng = np.random.default_rng(wl.seed)
    lens = rng.integers(wl.lens_lo, wl.lens_hi + 1, size=wl.B).astype(np.int32)
    q = device_normal((wl.B, wl.Hq, wl.D), wl.seed * 10 + 1, "bf16")
    cache = device_normal((wl.B, wl.S, wl.D), wl.seed * 10 + 2, "bf16")
    dl = torch.from_numpy(lens).to("cuda")
    scale = mla_scale()
    ws = torch.empty(g.mla_decode_workspace_bytes(wl.B, wl.Hq, wl.S), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((wl.B, wl.Hq, 512), dtype=torch.bfloat16, device="cuda")
    def call():
        g.mla_decode(q, cache, dl, scale, out, ws)

    _warm_up(call, warmup, torch)
    ms = _time_calls(call, steps, torch)
    keys = int(lens.sum())
    nbytes = keys * MLA_ROW_BYTES + wl.B * wl.Hq * (576 + 512) * 2 + 4 * wl.B
    flops = keys * wl.Hq * MLA_FLOP_PER_KEY_HEAD
    return dict(lens=lens, q=q, cache=cache, out=out, scale=scale), ms, nbytes, flops


def cpu_baseline_prefill(wl, x, torch, budget_s=15.0):
    """Time the oracle on a bounded sample -- whole sequences, in order, until about budget_s of
    CPU time -- check the GPU output on the same sample, and report the rate in TFLOP/s."""
    import numpy as np
    import oracle
    inv = oracle.rope_inv_freq(wl.rotary_dim, wl.theta, wl.rope_kind, wl.factor,
                               wl.low_freq_factor, wl.high_freq_factor, wl.original_max_pos)
    qw = x["qw"].float().cpu().numpy() if x["qw"] is not None else None
    kw = x["kw"].float().cpu().numpy() if x["kw"] is not None else None
    pos = x["pos"].cpu().numpy()[None]
    kpos = x["kpos"].cpu().numpy()[None]
    from synth import draw_sinks
    sinks = draw_sinks(wl)
    t_total, nseq, ok, maxerr = 0.0, 0, True, 0.0
    for b in range(wl.B):
        q = x["q"][b:b + 1].float().cpu().numpy()
        k = x["k"][b:b + 1].float().cpu().numpy()
        v = x["v"][b:b + 1].float().cpu().numpy()
        t = time.perf_counter()
        ref = oracle.attn_prefill(q, k, v, pos, kpos, inv_freq=inv, style=wl.style,
                                  n_cached=wl.n_cached, window=wl.window, q_norm_w=qw,
                                  k_norm_w=kw, eps=wl.eps, softcap=wl.softcap, sinks=sinks,
                                  chunk=wl.chunk, chunk_lookback=wl.chunk_lookback)
        t_total += time.perf_counter() - t
        got = x["out"][b:b + 1].float().cpu().numpy()
        err = np.abs(got - ref)
        maxerr = max(maxerr, float(err.max()))
        tol = 1e-4 if wl.dtype == "f32" else 2e-2 + 2e-2 * np.abs(ref)
        ok &= bool(np.all(err <= tol))
        nseq += 1
        if t_total >= budget_s:
            break
    flops = 4 * nseq * wl.Hq * wl.D * allowed_pairs(wl.L, wl.S, wl.window, wl.n_cached,
                                                    wl.chunk, wl.chunk_lookback)
    return dict(value=flops / t_total / 1e12, unit="TFLOP/s", cores=_blas_threads(),
                host_cpu_count=os.cpu_count(), kind="oracle",
                sample=f"{nseq} of {wl.B} sequences of {wl.name}, all rows and heads "
                       f"({flops / 1e9:.1f} GFLOP in {t_total:.1f} s)",
                parity_ok=ok, max_abs_err=maxerr)


def cpu_baseline_decode(wl, x, torch, budget_s=15.0):
    import numpy as np
    import oracle
    lens = x["lens"].cpu().numpy()
    inv = oracle.rope_inv_freq(wl.rotary_dim, wl.theta, wl.rope_kind, wl.factor,
                               wl.low_freq_factor, wl.high_freq_factor, wl.original_max_pos)
    eb = 2
    from synth import draw_sinks
    sinks = draw_sinks(wl)
    t_total, nbytes, ok, maxerr, nseq = 0.0, 0, True, 0.0, 0
    for b in range(wl.B):
        n = int(lens[b])
        kk = x["k"][b, :, :n].float().cpu().numpy()
        vv = x["v"][b, :, :n].float().cpu().numpy()
        qq = x["q"][b].float().cpu().numpy()
        t = time.perf_counter()
        ref = oracle.attn_decode_one(qq, kk, vv, n, inv_freq=inv, style=wl.style,
                                     window=wl.window, softcap=wl.softcap, sinks=sinks,
                                     chunk=wl.chunk, chunk_lookback=wl.chunk_lookback)
        t_total += time.perf_counter() - t
        got = x["out"][b].float().cpu().numpy()
        err = np.abs(got - ref)
        maxerr = max(maxerr, float(err.max()))
        ok &= bool(np.all(err <= 2e-2 + 2e-2 * np.abs(ref)))
        keys = decode_keys(wl, n)
        nbytes += keys * kv_bytes_per_token_per_layer(wl.Hkv, wl.D, eb)
        nseq += 1
        if t_total >= budget_s:
            break
    return dict(value=nbytes / t_total / 1e9, unit="GB/s", cores=_blas_threads(),
                host_cpu_count=os.cpu_count(), kind="oracle",
                sample=f"{nseq} of {wl.B} sequences of {wl.name} ({nbytes / 1e6:.0f} MB of K/V "
                       f"in {t_total:.1f} s)", parity_ok=ok, max_abs_err=maxerr)


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        n = max((i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"), default=1)
        return int(n)
    except Exception:
        return os.cpu_count() or 1


CONFIGS = ("tiny_causal_f32", "qwen3_prefill_bf16", "chunked_prefill_bf16_w4096",
           "chunked_prefill_bf16_full")
# the widened rows' workloads: gpt-oss-style sinks with a 128-key window, Llama-4-style chunks of
# 8192, and the Llama-3.1-style decode with chunks of 8192 and sinks
WIDENED = ("sinks_swa128_prefill_bf16", "llama4_chunked_prefill_bf16", "sinks_chunk_decode_bf16")
DECODE_CONFIG = "llama31_decode_bf16"


def run_only(name, steps, warmup, torch, g):
    """One workload's timed loop, eager launches, for a profiler run (no CPU baseline)."""
    from synth import WORKLOADS
    wl = WORKLOADS[name]
    if wl.name == "deepseek_mla_decode_bf16":
        _, ms, nbytes, _ = run_mla(wl, steps, warmup, torch, g)
        rec = {"workload": name, "ms_per_call": ms, "GB/s": nbytes / (ms * 1e-3) / 1e9}
    elif wl.kind == "decode":
        dx, ms = run_decode(wl, steps, warmup, torch, g)
        nbytes = decode_bytes(wl, dx["lens"].cpu().tolist())
        rec = {"workload": name, "ms_per_call": ms, "GB/s": nbytes / (ms * 1e-3) / 1e9}
    else:
        _, step_ms, parts = run_prefill(wl, steps, warmup, torch, g, graph=False)
        rec = {"workload": name, "ms_per_step": step_ms, "parts_ms": parts,
               "attention_TFLOP/s": prefill_flops(wl) / (parts["attention"] * 1e-3) / 1e12}
    print(json.dumps(rec), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mistral_swa_prefill_bf16",
                    help="headline prefill workload")
    ap.add_argument("--configs", default=",".join(CONFIGS + (DECODE_CONFIG,)),
                    help="comma-separated workloads timed beside the headline ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle time on the headline's sample (sub-records get half)")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch the step's kernels one by one instead of replaying a HIP graph")
    ap.add_argument("--mla-workload", default="deepseek_mla_decode_bf16",
                    help="latent-attention decode workload timed as an extra ('' to skip)")
    ap.add_argument("--widened", default=",".join(WIDENED),
                    help="workloads of the widened rows (sinks, chunked masks) timed as extras, "
                         "each with its roofline and an oracle check on a bounded sample")
    ap.add_argument("--paged-block", type=int, default=16, metavar="N",
                    help="also time the decode workload through a paged pool of N-slot blocks "
                         "(0: skip)")
    ap.add_argument("--only", default="", metavar="NAME",
                    help="run only this workload's timed loop (eager) and print its times")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (three times), the "
                         "known-size reference for scaling HBM byte counters")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (this build has no multi-GPU path); got --gpus "
              f"{args.gpus}", file=sys.stderr)
        return 2

    import torch

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 3}), flush=True)
        return 0

    import gqa_scaled_rope_amd as g
    from synth import WORKLOADS

    g.library()
    if args.only:
        return run_only(args.only, args.steps, args.warmup, torch, g)
    cpu = not args.no_cpu_baseline
    graph = not args.no_graph
    wl = WORKLOADS[args.workload]
    log(f"[bench] headline prefill workload {wl.name}: warmup {args.warmup}, steps {args.steps}")
    head = prefill_record(wl, args.steps, args.warmup, torch, g, graph, cpu, args.cpu_budget)
    line = {
        "metric": METRIC, "value": head["value"], "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) draws, device-generated)",
        "config": {**head["config"], "parallelism": "none (1 GPU)",
                   "launch": "eager" if args.no_graph else "HIP graph of the step's kernels"},
        "roofline": head["roofline"],
        "step_parts_ms": head["step_parts_ms"],
        # every timed region follows its W warmup calls, continued until this much GPU time ran
        "warmup_min_gpu_ms": SETTLE_MS,
    }
    if cpu:
        line["cpu_baseline"] = head["cpu_baseline"]
    configs = {}
    dx = None
    for name in filter(None, args.configs.split(",")):
        cwl = WORKLOADS[name]
        log(f"[bench] config {name}")
        if cwl.kind == "decode":
            rec, dx, nbytes = decode_record(cwl, args.steps, args.warmup, torch, g, cpu,
                                            args.cpu_budget / 2)
            if args.paged_block:
                pms, same = run_decode_paged(cwl, dx, args.paged_block, args.steps, args.warmup,
                                             torch, g)
                pgbs = nbytes / (pms * 1e-3) / 1e9
                log(f"[bench] paged decode (blocks of {args.paged_block}) {pms:.3f} ms -> "
                    f"{pgbs:.0f} GB/s, bit-identical to the contiguous cache: {same}")
                rec["paged"] = {"block_size": args.paged_block, "value": round(pgbs, 1),
                                "unit": "GB/s", "ms_per_call": round(pms, 4),
                                "frac": round(pgbs / HBM_PEAK_GBS, 4),
                                "identical_to_contiguous": same}
            del dx
            torch.cuda.empty_cache()
        else:
            rec = prefill_record(cwl, args.steps, args.warmup, torch, g, graph, cpu,
                                 args.cpu_budget / 2)
        configs[name] = rec
    line["configs"] = configs
    extras = {}
    if args.mla_workload:
        mwl = WORKLOADS[args.mla_workload]
        log(f"[bench] latent-attention decode workload {mwl.name}")
        mx, mms, mbytes, mflops = run_mla(mwl, args.steps, args.warmup, torch, g)
        mgbs = mbytes / (mms * 1e-3) / 1e9
        mtf = mflops / (mms * 1e-3) / 1e12
        log(f"[bench] latent-attention decode {mms:.3f} ms -> {mgbs:.0f} GB/s, {mtf:.1f} TFLOP/s")
        extras["mla_decode"] = {
            "workload": mwl.name, "value": round(mgbs, 1), "unit": "GB/s",
            "ms_per_call": round(mms, 4), "algorithmic_bytes": mbytes, "algorithmic_flop": mflops,
            "roofline": {"bound": "hbm",
                         "kernel": "mla_split32_kernel + mla_split16_kernel (flagged shares only) + "
                                   "mla_combine_kernel (one gqa_mla_decode call)",
                         "achieved": round(mgbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(mgbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("mla_split32_kernel", mwl.name),
                         "mfma_busy_rocprof": measured_mfma("mla_split32_kernel", mwl.name)[0],
                         "mfma_tflops": round(mtf, 1),
                         "mfma_frac": round(mtf / MFMA_BF16_PEAK_TFLOPS, 4)}}
        del mx
    for name in filter(None, args.widened.split(",")):
        wwl = WORKLOADS[name]
        log(f"[bench] widened row {name}")
        if wwl.kind == "decode":
            rec, wdx, _ = decode_record(wwl, args.steps, args.warmup, torch, g, cpu,
                                        args.cpu_budget / 3)
            del wdx
        else:
            rec = prefill_record(wwl, args.steps, args.warmup, torch, g, graph, cpu,
                                 args.cpu_budget / 3)
        extras[name] = rec
        torch.cuda.empty_cache()
    line["extras"] = extras
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
