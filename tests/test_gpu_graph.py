"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Each graph is replayed several times, with the program's own eager work (filling the output with
NaN, drawing unrelated random numbers) and a synchronization between replays, and every replay
must reproduce the eager result bit for bit: the kernels are deterministic and record no memset,
so a replay that differs would mean the capture lost or reordered work.  The bench replays the
prefill step this way.
"""
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
g = pytest.importorskip("gqa_scaled_rope_amd")

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import bench  # noqa: E402
from synth import WORKLOADS, decode_device_inputs, device_normal  # noqa: E402


def _replays_match_eager(fn, out, replays=3):
    fn()
    torch.cuda.synchronize()
    eager = out.clone()
    hg = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(hg, stream=cap):
            fn()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for i in range(replays):
        out.fill_(float("nan"))
        torch.randn(1 << 16, device="cuda").sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        hg.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from the eager call"


@pytest.mark.parametrize("name", ["qwen3_prefill_bf16", "chunked_prefill_bf16_w4096",
                                  "sinks_swa128_prefill_bf16"])
def test_prefill_step_graph(name):
    # rope tables + key preparation + attention, as one captured step (smaller batch)
    wl = WORKLOADS[name]
    wl = wl.with_(B=1, L=min(wl.L, 512), S=min(wl.S, 1024) if wl.n_cached else min(wl.S, 512),
                  n_cached=max(min(wl.S, 1024) - min(wl.L, 512), 0) if wl.n_cached else 0)
    print("graph prefill", wl.name, wl.B, wl.L, wl.S, wl.n_cached, flush=True)
    x = bench._prefill_setup(wl, torch, g)
    spec = bench._rope_spec(g, wl)

    def step():
        g.rope_tables(spec, x["table_len"], x["cos"], x["sin"])
        g.prep_keys(x["cfg"], x["k"], x["kpos"], wl.n_cached, k_out=x["kcache"])
        g.attn_prefill(x["cfg"], x["q"], x["kcache"], x["v"], x["pos"], x["kpos"], wl.S,
                       wl.window, x["out"], workspace=None)

    _replays_match_eager(step, x["out"])


def test_decode_graph():
    wl = WORKLOADS["llama31_decode_bf16"].with_(B=8, S=4096, lens_lo=1, lens_hi=4096)
    print("graph decode", wl.B, wl.S, flush=True)
    x = decode_device_inputs(wl)
    cos, sin = g.rope_tables(bench._rope_spec(g, wl), wl.S)
    cfg = g.AttnConfig(wl.dtype, wl.D, wl.Hq, wl.Hkv, wl.rotary_dim, wl.style, cos, sin,
                       wl.qk_norm, wl.eps, x.get("qw"), x.get("kw"), 0.0, wl.softcap,
                       **bench._mask_cfg(wl, torch))
    ws = torch.empty(g.decode_workspace_bytes(cfg, wl.B, wl.S), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x["q"])
    _replays_match_eager(
        lambda: g.attn_decode(cfg, x["q"], x["k"], x["v"], x["lens"], wl.window, out, ws), out)


def test_latent_attention_decode_graph():
    B, H, S = 6, 128, 3000
    print("graph latent attention", B, H, S, flush=True)
    q = device_normal((B, H, 576), 71, "bf16")
    cache = device_normal((B, S, 576), 72, "bf16")
    lens = torch.tensor([1, 0, 3000, 777, 2048, 33], dtype=torch.int32, device="cuda")
    ws = torch.empty(g.mla_decode_workspace_bytes(B, H, S), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, H, 512), dtype=torch.bfloat16, device="cuda")
    _replays_match_eager(lambda: g.mla_decode(q, cache, lens, bench.mla_scale(), out, ws), out)
