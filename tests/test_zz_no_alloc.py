"""The decode entry point that allocates nothing (gqa_attn_decode_noalloc), called through the C
ABI, against gqa_attn_decode with a caller workspace on the same inputs: the same kernels run
on the same data, so the outputs must be bit-identical.  Two calls in a row, the second smaller,
so that what the first leaves in the shared scratch cannot leak into the second; then a third
call with the forced long decode splits.  Sequences of the second call are also checked against
the oracle."""
import ctypes

import numpy as np
import pytest

import oracle
from synth import WORKLOADS, decode_device_inputs, draw_sinks

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
g = pytest.importorskip("gqa_scaled_rope_amd")

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _cfg(wl, kernel="auto"):
    spec = g.RopeSpec(wl.rotary_dim, wl.rope_kind, wl.theta, wl.factor, wl.low_freq_factor,
                      wl.high_freq_factor, wl.original_max_pos)
    cos, sin = g.rope_tables(spec, wl.S)
    sk = draw_sinks(wl)
    return g.AttnConfig(wl.dtype, wl.D, wl.Hq, wl.Hkv, wl.rotary_dim, wl.style, cos, sin,
                        sinks=None if sk is None else torch.from_numpy(sk).to("cuda"),
                        chunk_size=wl.chunk, chunk_lookback=wl.chunk_lookback, kernel=kernel)


def _noalloc(cfg, x, window):
    out = torch.full_like(x["q"], float("nan"))
    c = cfg.c_struct()
    B, Smax = int(x["q"].shape[0]), int(x["k"].shape[2])
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = g.library().gqa_attn_decode_noalloc(
        ctypes.byref(c), x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(),
        x["lens"].data_ptr(), B, Smax, int(window), out.data_ptr(), stream)
    assert st == 0, g.last_error()
    return out


def _compare(wl, kernel="auto", seed=None):
    print("noalloc decode", wl.name, wl.B, wl.S, kernel, flush=True)
    x = decode_device_inputs(wl, seed=seed)
    cfg = _cfg(wl, kernel)
    need = g.decode_workspace_bytes(cfg, wl.B, wl.S)
    assert 0 < need <= g.DECODE_NOALLOC_MAX_BYTES
    ref = g.attn_decode(cfg, x["q"], x["k"], x["v"], x["lens"], wl.window)
    got = _noalloc(cfg, x, wl.window)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    return x, got


def test_noalloc_decode_matches_workspace_decode():
    # 1: the Llama-3.1-style batch (64 sequences, up to 32768 keys: ~34 MiB of partials)
    _compare(WORKLOADS["llama31_decode_bf16"])
    # 2: a smaller batch with a window, sinks and chunks, after the large one
    wl = WORKLOADS["llama31_decode_bf16"].with_(B=5, S=2600, lens_lo=1, lens_hi=2600, window=1500,
                                                 chunk=2048, sinks=True, seed=44)
    x, got = _compare(wl)
    lens = x["lens"].cpu().numpy()
    inv = oracle.rope_inv_freq(wl.rotary_dim, wl.theta, wl.rope_kind, wl.factor,
                               wl.low_freq_factor, wl.high_freq_factor, wl.original_max_pos)
    out = got.float().cpu().numpy()
    for b in range(wl.B):
        n = int(lens[b])
        ref = oracle.attn_decode_one(x["q"][b].float().cpu().numpy(),
                                     x["k"][b, :, :n].float().cpu().numpy(),
                                     x["v"][b, :, :n].float().cpu().numpy(), n, inv_freq=inv,
                                     window=wl.window, sinks=draw_sinks(wl), chunk=wl.chunk)
        err = np.abs(out[b] - ref)
        assert np.all(err <= 2e-2 + 2e-2 * np.abs(ref)), err.max()
    # 3: forced long splits, smaller again
    _compare(WORKLOADS["llama31_decode_bf16"].with_(B=3, S=5000, lens_lo=2000, lens_hi=5000,
                                                     seed=45), kernel="decode_long")


def test_noalloc_decode_rejects_sizes_past_the_limit():
    wl = WORKLOADS["llama31_decode_bf16"]
    cfg = _cfg(wl)
    c = cfg.c_struct()
    # 64 sequences of 65536 keys need ~67 MiB of partials: refused before any launch
    st = g.library().gqa_attn_decode_noalloc(ctypes.byref(c), 1 << 20, 1 << 20, 1 << 20, 1 << 20,
                                             64, 65536, 0, 1 << 20, None)
    assert st == 5 and "no-allocation" in g.last_error()
