"""Python binding of libgqa_rope (rotary grouped-query causal attention for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP kernels of
``libgqa_rope.so`` behind the C ABI declared in ``include/gqa_rope.h``.  PyTorch supplies device
memory and the current stream.  There is no fallback: if the library is not built, every call
raises.

The functions mirror the C entry points: :func:`rope_tables`, :func:`attn_prefill`,
:func:`attn_decode`, :func:`decode_workspace_bytes`, :func:`rope_inv_freq`,
:func:`rope_attention_factor`, :func:`rope_softmax_scale`, :func:`last_error`.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

__all__ = [
    "GQAError", "RopeSpec", "AttnConfig", "library", "rope_inv_freq", "rope_tables",
    "rope_attention_factor", "rope_softmax_scale",
    "attn_prefill", "attn_decode", "decode_workspace_bytes", "PagedKV", "paged_append",
    "paged_decode_workspace_bytes", "attn_decode_paged", "mla_decode_workspace_bytes",
    "mla_decode", "prefill_workspace_bytes", "prefill_kernel", "PREFILL_KERNELS", "prep_keys",
    "last_error", "KERNELS",
    "hip_runtimes_mapped", "attn_decode_noalloc", "DECODE_NOALLOC_MAX_BYTES", "LIB_PATH",
    "EXPORTS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgqa_rope.so")

GQA_F32, GQA_BF16 = 0, 1
ROPE_KINDS = {"default": 0, "linear": 1, "llama3": 2, "yarn": 3, "longrope": 4}
ROT_STYLES = {"half": 0, "interleaved": 1}
# gqa_attn_cfg.kernel (gqa_kernel_select): per-call kernel choice, "auto" in production
KERNELS = {"auto": 0, "generic": 1, "decode_short": 2, "decode_long": 3, "prefill_long": 4,
           "prefill_short": 5}
STATUS = {0: "GQA_OK", 1: "GQA_E_NULL", 2: "GQA_E_SHAPE", 3: "GQA_E_DTYPE",
          4: "GQA_E_UNSUPPORTED", 5: "GQA_E_WORKSPACE", 6: "GQA_E_HIP", 7: "GQA_E_VALUE"}


class GQAError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


class _RopeParams(ctypes.Structure):
    _fields_ = [("rotary_dim", ctypes.c_int32), ("kind", ctypes.c_int32),
                ("theta", ctypes.c_double), ("factor", ctypes.c_double),
                ("low_freq_factor", ctypes.c_double), ("high_freq_factor", ctypes.c_double),
                ("original_max_pos", ctypes.c_double), ("beta_fast", ctypes.c_double),
                ("beta_slow", ctypes.c_double), ("yarn_no_truncate", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("mscale", ctypes.c_double),
                ("mscale_all_dim", ctypes.c_double), ("attention_factor", ctypes.c_double),
                ("short_factor", ctypes.POINTER(ctypes.c_double)),
                ("long_factor", ctypes.POINTER(ctypes.c_double)), ("seq_len", ctypes.c_int64)]


class _AttnCfg(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("rotary_dim", ctypes.c_int32), ("rot_style", ctypes.c_int32),
                ("cos_table", ctypes.c_void_p), ("sin_table", ctypes.c_void_p),
                ("table_len", ctypes.c_int32), ("qk_norm", ctypes.c_int32),
                ("eps", ctypes.c_double), ("q_norm_w", ctypes.c_void_p),
                ("k_norm_w", ctypes.c_void_p), ("scale", ctypes.c_double),
                ("softcap", ctypes.c_double), ("sinks", ctypes.c_void_p),
                ("chunk_size", ctypes.c_int32), ("chunk_lookback", ctypes.c_int32),
                ("kernel", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class _PagedKV(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("max_blocks", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


_P = ctypes.c_void_p
_I32, _I64, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
# name -> (restype, argtypes); every function declared in include/gqa_rope.h
EXPORTS = {
    "gqa_rope_tables": (_I32, [ctypes.POINTER(_RopeParams), _I32, _P, _P, _P]),
    "gqa_rope_inv_freq": (_I32, [ctypes.POINTER(_RopeParams), ctypes.POINTER(ctypes.c_double)]),
    "gqa_rope_attention_factor": (_I32, [ctypes.POINTER(_RopeParams),
                                         ctypes.POINTER(ctypes.c_double)]),
    "gqa_rope_softmax_scale": (_I32, [ctypes.POINTER(_RopeParams), _I32,
                                      ctypes.POINTER(ctypes.c_double)]),
    "gqa_prep_keys": (_I32, [ctypes.POINTER(_AttnCfg), _P, _P, _I64, _I32, _I32, _I32, _P, _P]),
    "gqa_prefill_workspace_bytes": (_SZ, [ctypes.POINTER(_AttnCfg), _I32, _I32, _I32]),
    "gqa_prefill_kernel": (_I32, [ctypes.POINTER(_AttnCfg), _I32, _I32, _I32, _I32, _I32, _I32,
                                  ctypes.POINTER(_I32)]),
    "gqa_attn_prefill": (_I32, [ctypes.POINTER(_AttnCfg), _P, _P, _P, _P, _I64, _P, _I64, _I32,
                                _I32, _I32, _I32, _I32, _P, _P, _SZ, _P]),
    "gqa_decode_workspace_bytes": (_SZ, [ctypes.POINTER(_AttnCfg), _I32, _I32]),
    "gqa_attn_decode": (_I32, [ctypes.POINTER(_AttnCfg), _P, _P, _P, _P, _I32, _I32, _I32, _P, _P,
                               _SZ, _P]),
    "gqa_attn_decode_noalloc": (_I32, [ctypes.POINTER(_AttnCfg), _P, _P, _P, _P, _I32, _I32,
                                       _I32, _P, _P]),
    "gqa_paged_append": (_I32, [ctypes.POINTER(_AttnCfg), ctypes.POINTER(_PagedKV), _P, _P, _P,
                                _I64, _P, _I32, _I32, _P]),
    "gqa_paged_decode_workspace_bytes": (_SZ, [ctypes.POINTER(_AttnCfg), ctypes.POINTER(_PagedKV),
                                               _I32]),
    "gqa_attn_decode_paged": (_I32, [ctypes.POINTER(_AttnCfg), _P, ctypes.POINTER(_PagedKV), _P,
                                     _I32, _I32, _P, _P, _SZ, _P]),
    "gqa_mla_decode_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "gqa_mla_decode": (_I32, [_P, _P, _P, _I32, _I32, _I32, ctypes.c_double, _P, _P, _SZ, _P]),
    "gqa_last_error": (ctypes.c_char_p, []),
    "gqa_version": (ctypes.c_char_p, []),
}

_lib = None


def hip_runtimes_mapped(maps_text=None):
    """Distinct HIP runtime files (libamdhip64) mapped into this process, read from
    /proc/self/maps (or from the given text)."""
    if maps_text is None:
        try:
            with open("/proc/self/maps") as f:
                maps_text = f.read()
        except OSError:
            return set()
    found = set()
    for line in maps_text.splitlines():
        parts = line.split(None, 5)
        if len(parts) == 6 and os.path.basename(parts[5]).startswith("libamdhip64.so"):
            path = parts[5].strip()
            try:
                path = os.path.realpath(path)
            except OSError:
                pass
            found.add(path)
    return found


def library():
    """Load libgqa_rope.so (built in-tree by __graft_entry__.build()); raise if it is missing, or
    if loading it left two HIP runtimes in the process."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -c 'import __graft_entry__ as "
                               f"g; g.build()'` (hipcc, gfx950)")
        # torch ships its own HIP runtime (same soname as ROCm's).  Loading torch first makes the
        # library resolve to that runtime, so torch's streams and allocations are valid in it; the
        # other order would bring a second HIP runtime into the process, in which torch's streams
        # are invalid and the first call crashes or fails.  That state is detected and refused.
        import torch  # noqa: F401
        lib = ctypes.CDLL(LIB_PATH)
        runtimes = hip_runtimes_mapped()
        if len(runtimes) > 1:
            raise RuntimeError("two HIP runtimes are mapped into this process ("
                               + ", ".join(sorted(runtimes)) + "): import torch before anything "
                               "that loads libamdhip64, so that libgqa_rope binds to torch's")
        for name, (res, args) in EXPORTS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def last_error() -> str:
    return library().gqa_last_error().decode()


def _check(status):
    if status != 0:
        raise GQAError(status, last_error())


# ------------------------------------------------------------------------------------------------
@dataclass
class RopeSpec:
    rotary_dim: int
    kind: str = "default"
    theta: float = 1e4
    factor: float = 1.0
    low_freq_factor: float = 1.0
    high_freq_factor: float = 4.0
    original_max_pos: float = 8192.0
    # yarn (None selects the schedule's default or "absent")
    beta_fast: Optional[float] = None
    beta_slow: Optional[float] = None
    truncate: bool = True
    mscale: Optional[float] = None
    mscale_all_dim: Optional[float] = None
    # yarn and longrope
    attention_factor: Optional[float] = None
    # longrope: per-pair factor tables (R/2 each) and the sequence length that picks one
    short_factor: Optional[Sequence[float]] = None
    long_factor: Optional[Sequence[float]] = None
    seq_len: int = 0

    def c_struct(self):
        if self.kind not in ROPE_KINDS:
            raise GQAError(4, f"unknown rope kind {self.kind!r}; known: {', '.join(ROPE_KINDS)}")

        def table(v):
            return None if v is None else (ctypes.c_double * len(v))(*[float(x) for x in v])

        short, long_ = table(self.short_factor), table(self.long_factor)
        dbl = ctypes.POINTER(ctypes.c_double)
        st = _RopeParams(
            self.rotary_dim, ROPE_KINDS[self.kind], self.theta, self.factor,
            self.low_freq_factor, self.high_freq_factor, self.original_max_pos,
            self.beta_fast or 0.0, self.beta_slow or 0.0, 0 if self.truncate else 1, 0,
            self.mscale or 0.0, self.mscale_all_dim or 0.0, self.attention_factor or 0.0,
            ctypes.cast(short, dbl) if short is not None else dbl(),
            ctypes.cast(long_, dbl) if long_ is not None else dbl(), int(self.seq_len))
        half = self.rotary_dim // 2
        for name, t in (("short_factor", short), ("long_factor", long_)):
            if t is not None and len(t) != half:
                raise GQAError(2, f"{name} has {len(t)} entries, expected {half}")
        st._tables = (short, long_)   # the arrays live as long as the struct
        return st


def rope_inv_freq(spec: RopeSpec):
    """Host copy of the pair frequencies the tables use (list of R/2 floats)."""
    st = spec.c_struct()
    buf = (ctypes.c_double * max(1, spec.rotary_dim // 2))()
    _check(library().gqa_rope_inv_freq(ctypes.byref(st), buf))
    return list(buf)[: spec.rotary_dim // 2]


def rope_attention_factor(spec: RopeSpec) -> float:
    """Factor the cos/sin tables are multiplied by (1 unless yarn or longrope)."""
    st = spec.c_struct()
    out = ctypes.c_double()
    _check(library().gqa_rope_attention_factor(ctypes.byref(st), ctypes.byref(out)))
    return out.value


def rope_softmax_scale(spec: RopeSpec, qk_dim: int) -> float:
    """qk_dim^-0.5, with YaRN's temperature when the schedule is yarn with mscale_all_dim."""
    st = spec.c_struct()
    out = ctypes.c_double()
    _check(library().gqa_rope_softmax_scale(ctypes.byref(st), int(qk_dim), ctypes.byref(out)))
    return out.value


def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, shape, dtype, device=True):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise GQAError(2, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise GQAError(3, f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise GQAError(2, f"{name} must be contiguous")
    if device and not t.is_cuda:
        raise GQAError(1, f"{name} must be a device tensor")
    return ctypes.c_void_p(t.data_ptr())


def rope_tables(spec: RopeSpec, table_len: int, cos=None, sin=None, stream=None):
    """cos/sin tables [table_len, R/2] fp32 on the current device (allocated if not given)."""
    torch = _torch()
    half = spec.rotary_dim // 2
    if cos is None:
        cos = torch.empty((table_len, half), dtype=torch.float32, device="cuda")
    if sin is None:
        sin = torch.empty((table_len, half), dtype=torch.float32, device="cuda")
    pc = _need(cos, "cos", (table_len, half), torch.float32)
    ps = _need(sin, "sin", (table_len, half), torch.float32)
    st = spec.c_struct()
    _check(library().gqa_rope_tables(ctypes.byref(st), int(table_len), pc, ps, _stream(stream)))
    return cos, sin


# ------------------------------------------------------------------------------------------------
@dataclass
class AttnConfig:
    dtype: str                      # "bf16" | "f32"
    head_dim: int
    num_q_heads: int
    num_kv_heads: int
    rotary_dim: int = 0
    rot_style: str = "half"
    cos: Optional[object] = None    # device tensor [table_len, R/2] fp32
    sin: Optional[object] = None
    qk_norm: bool = False
    eps: float = 1e-6
    q_norm_w: Optional[object] = None   # device tensor [D] in dtype
    k_norm_w: Optional[object] = None
    scale: float = 0.0
    softcap: float = 0.0
    sinks: Optional[object] = None      # device tensor [num_q_heads] fp32: learned sink logits
    chunk_size: int = 0                 # chunked attention: chunk length in positions (0 = off)
    chunk_lookback: int = 0             # chunks before the query's own that stay visible
    kernel: str = "auto"                # per-call kernel choice (KERNELS); "auto" in production

    @property
    def torch_dtype(self):
        torch = _torch()
        return {"bf16": torch.bfloat16, "f32": torch.float32}[self.dtype]

    def c_struct(self):
        torch = _torch()
        if self.dtype not in ("bf16", "f32"):
            raise GQAError(3, f"dtype must be 'bf16' or 'f32', got {self.dtype!r}")
        if self.rot_style not in ROT_STYLES:
            raise GQAError(7, f"rot_style must be 'half' or 'interleaved', got {self.rot_style!r}")
        half = self.rotary_dim // 2
        pc = ps = None
        tl = 0
        if self.rotary_dim > 0:
            if self.cos is None or self.sin is None:
                raise GQAError(1, "cos/sin tables are required when rotary_dim > 0")
            tl = int(self.cos.shape[0])
            pc = _need(self.cos, "cos", (tl, half), torch.float32).value
            ps = _need(self.sin, "sin", (tl, half), torch.float32).value
        qw = kw = None
        if self.qk_norm:
            if self.q_norm_w is None or self.k_norm_w is None:
                raise GQAError(1, "q_norm_w and k_norm_w are required when qk_norm is set")
            qw = _need(self.q_norm_w, "q_norm_w", (self.head_dim,), self.torch_dtype).value
            kw = _need(self.k_norm_w, "k_norm_w", (self.head_dim,), self.torch_dtype).value
        if self.kernel not in KERNELS:
            raise GQAError(7, f"kernel must be one of {sorted(KERNELS)}, got {self.kernel!r}")
        sk = None
        if self.sinks is not None:
            sk = _need(self.sinks, "sinks", (self.num_q_heads,), torch.float32).value
        return _AttnCfg(GQA_BF16 if self.dtype == "bf16" else GQA_F32, self.head_dim,
                        self.num_q_heads, self.num_kv_heads, self.rotary_dim,
                        ROT_STYLES[self.rot_style], pc, ps, tl, int(bool(self.qk_norm)), self.eps,
                        qw, kw, self.scale, self.softcap, sk, int(self.chunk_size),
                        int(self.chunk_lookback), KERNELS[self.kernel], 0)


def prep_keys(cfg: AttnConfig, k, key_positions, n_cached=0, k_out=None, stream=None):
    """Norm and rotate key rows [n_cached, S) of k [B, S, Hkv, D] into k_out (same layout; may be
    k itself).  Returns k_out."""
    torch = _torch()
    B, S = k.shape[0], k.shape[1]
    dt = cfg.torch_dtype
    pk = _need(k, "k", (B, S, cfg.num_kv_heads, cfg.head_dim), dt)
    if key_positions.dim() == 1:
        pkp, kstride = _need(key_positions, "key_positions", (S,), torch.int32), 0
    else:
        pkp, kstride = _need(key_positions, "key_positions", (B, S), torch.int32), S
    if k_out is None:
        k_out = k.clone()
    po = _need(k_out, "k_out", tuple(k.shape), dt)
    c = cfg.c_struct()
    _check(library().gqa_prep_keys(ctypes.byref(c), pk, pkp, kstride, B, S, int(n_cached), po,
                                   _stream(stream)))
    return k_out


def prefill_workspace_bytes(cfg: AttnConfig, B: int, S: int, n_cached: int = 0) -> int:
    c = cfg.c_struct()
    n = library().gqa_prefill_workspace_bytes(ctypes.byref(c), int(B), int(S), int(n_cached))
    err = last_error()
    if n == 0 and err:
        raise GQAError(2, err)
    return int(n)


PREFILL_KERNELS = {0: "generic", 1: "fused", 2: "stream_long", 3: "stream_short"}


def prefill_kernel(cfg: AttnConfig, B: int, L: int, S: int, n_cached: int = 0, window: int = 0,
                   workspace: bool = True) -> str:
    """Name of the kernel gqa_attn_prefill runs for these sizes (host-only query)."""
    c = cfg.c_struct()
    which = ctypes.c_int32(-1)
    _check(library().gqa_prefill_kernel(ctypes.byref(c), int(B), int(L), int(S), int(n_cached),
                                        int(window), int(bool(workspace)), ctypes.byref(which)))
    return PREFILL_KERNELS[which.value]


def attn_prefill(cfg: AttnConfig, q, k, v, positions, key_positions, n_cached=0, window=0,
                 out=None, workspace="auto", stream=None):
    """q [B, L, Hq, D], k/v [B, S, Hkv, D], positions [B, L] or [L], key_positions [B, S] or [S]
    (int32, nondecreasing).  Returns out [B, L, Hq, D].

    workspace: "auto" allocates gqa_prefill_workspace_bytes (prepared keys and room for split
    key walks) when the streaming kernels apply; None runs without one (the fused kernel when
    keys need preparing); or a uint8 device tensor."""
    torch = _torch()
    B, L, Hq, D = q.shape
    S = k.shape[1]
    dt = cfg.torch_dtype
    pq = _need(q, "q", (B, L, cfg.num_q_heads, cfg.head_dim), dt)
    pk = _need(k, "k", (B, S, cfg.num_kv_heads, cfg.head_dim), dt)
    pv = _need(v, "v", (B, S, cfg.num_kv_heads, cfg.head_dim), dt)
    if positions.dim() == 1:
        pp, pstride = _need(positions, "positions", (L,), torch.int32), 0
    else:
        pp, pstride = _need(positions, "positions", (B, L), torch.int32), L
    if key_positions.dim() == 1:
        pkp, kstride = _need(key_positions, "key_positions", (S,), torch.int32), 0
    else:
        pkp, kstride = _need(key_positions, "key_positions", (B, S), torch.int32), S
    if out is None:
        out = torch.empty_like(q)
    po = _need(out, "out", tuple(q.shape), dt)
    if isinstance(workspace, str):
        need = prefill_workspace_bytes(cfg, B, S, n_cached)
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device) if need else None
    pw, nbytes = ctypes.c_void_p(None), 0
    if workspace is not None:
        pw = _need(workspace, "workspace", (workspace.numel(),), torch.uint8)
        nbytes = workspace.numel()
    c = cfg.c_struct()
    _check(library().gqa_attn_prefill(ctypes.byref(c), pq, pk, pv, pp, pstride, pkp, kstride, B, L,
                                      S, int(n_cached), int(window), po, pw, nbytes,
                                      _stream(stream)))
    return out


def decode_workspace_bytes(cfg: AttnConfig, B: int, Smax: int) -> int:
    c = cfg.c_struct()
    n = library().gqa_decode_workspace_bytes(ctypes.byref(c), int(B), int(Smax))
    err = last_error()
    if n == 0 and err:
        raise GQAError(2, err)
    return int(n)


def attn_decode(cfg: AttnConfig, q, kcache, vcache, lens, window=0, out=None, workspace=None,
                stream=None):
    """q [B, Hq, D], kcache/vcache [B, Hkv, Smax, D], lens [B] int32.  Returns out [B, Hq, D]."""
    torch = _torch()
    B = q.shape[0]
    Smax = kcache.shape[2]
    dt = cfg.torch_dtype
    pq = _need(q, "q", (B, cfg.num_q_heads, cfg.head_dim), dt)
    pk = _need(kcache, "kcache", (B, cfg.num_kv_heads, Smax, cfg.head_dim), dt)
    pv = _need(vcache, "vcache", (B, cfg.num_kv_heads, Smax, cfg.head_dim), dt)
    pl = _need(lens, "lens", (B,), torch.int32)
    if out is None:
        out = torch.empty_like(q)
    po = _need(out, "out", tuple(q.shape), dt)
    need = decode_workspace_bytes(cfg, B, Smax)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    pw, nbytes = ctypes.c_void_p(None), 0
    if workspace is not None:
        pw = _need(workspace, "workspace", (workspace.numel(),), torch.uint8)
        nbytes = workspace.numel()
    c = cfg.c_struct()
    _check(library().gqa_attn_decode(ctypes.byref(c), pq, pk, pv, pl, B, Smax, int(window), po, pw,
                                     nbytes, _stream(stream)))
    return out


DECODE_NOALLOC_MAX_BYTES = 64 << 20   # GQA_DECODE_NOALLOC_MAX_BYTES


def attn_decode_noalloc(cfg: AttnConfig, q, kcache, vcache, lens, window=0, out=None,
                        stream=None):
    """attn_decode whose split partials live in the library's fixed per-GPU scratch (no device
    allocation by the library; `out` is allocated here only when not given).  Calls that overlap
    on one GPU race."""
    torch = _torch()
    B = q.shape[0]
    Smax = kcache.shape[2]
    dt = cfg.torch_dtype
    pq = _need(q, "q", (B, cfg.num_q_heads, cfg.head_dim), dt)
    pk = _need(kcache, "kcache", (B, cfg.num_kv_heads, Smax, cfg.head_dim), dt)
    pv = _need(vcache, "vcache", (B, cfg.num_kv_heads, Smax, cfg.head_dim), dt)
    pl = _need(lens, "lens", (B,), torch.int32)
    if out is None:
        out = torch.empty_like(q)
    po = _need(out, "out", tuple(q.shape), dt)
    c = cfg.c_struct()
    _check(library().gqa_attn_decode_noalloc(ctypes.byref(c), pq, pk, pv, pl, B, Smax, int(window),
                                             po, _stream(stream)))
    return out


# ------------------------------------------------------------------------------------------------
@dataclass
class PagedKV:
    """Paged KV pool: k_pool, v_pool [num_blocks, Hkv, block_size, D] and block_table int32
    [B, max_blocks] (device tensors); slot j of sequence b is row j % block_size of block
    block_table[b, j // block_size]."""
    k_pool: object
    v_pool: object
    block_table: object

    def c_struct(self, cfg: AttnConfig):
        torch = _torch()
        nb, hkv, bs, d = (int(x) for x in self.k_pool.shape)
        pk = _need(self.k_pool, "k_pool", (nb, cfg.num_kv_heads, bs, cfg.head_dim), cfg.torch_dtype)
        pv = _need(self.v_pool, "v_pool", (nb, cfg.num_kv_heads, bs, cfg.head_dim), cfg.torch_dtype)
        if self.block_table.dim() != 2:
            raise GQAError(2, "block_table must be [B, max_blocks]")
        pt = _need(self.block_table, "block_table", tuple(self.block_table.shape), torch.int32)
        return _PagedKV(pk.value, pv.value, pt.value, int(self.block_table.shape[1]), bs, nb, 0)


def paged_append(cfg: AttnConfig, kv: PagedKV, k_new, v_new, key_positions, start, stream=None):
    """cache.update with the key preparation fused in: k_new, v_new [B, L, Hkv, D] go to slots
    start[b] .. start[b] + L - 1 (keys normed and rotated at key_positions [B, L] or [L])."""
    torch = _torch()
    B, L = int(k_new.shape[0]), int(k_new.shape[1])
    dt = cfg.torch_dtype
    pk = _need(k_new, "k_new", (B, L, cfg.num_kv_heads, cfg.head_dim), dt)
    pv = _need(v_new, "v_new", (B, L, cfg.num_kv_heads, cfg.head_dim), dt)
    if key_positions.dim() == 1:
        pp, stride = _need(key_positions, "key_positions", (L,), torch.int32), 0
    else:
        pp, stride = _need(key_positions, "key_positions", (B, L), torch.int32), L
    ps = _need(start, "start", (B,), torch.int32)
    c = cfg.c_struct()
    k = kv.c_struct(cfg)
    _check(library().gqa_paged_append(ctypes.byref(c), ctypes.byref(k), pk, pv, pp, stride, ps, B,
                                      L, _stream(stream)))


def paged_decode_workspace_bytes(cfg: AttnConfig, kv: PagedKV, B: int) -> int:
    c = cfg.c_struct()
    k = kv.c_struct(cfg)
    n = library().gqa_paged_decode_workspace_bytes(ctypes.byref(c), ctypes.byref(k), int(B))
    err = last_error()
    if n == 0 and err:
        raise GQAError(2, err)
    return int(n)


def attn_decode_paged(cfg: AttnConfig, q, kv: PagedKV, lens, window=0, out=None, workspace=None,
                      stream=None):
    """q [B, Hq, D] against a paged pool, lens [B] int32.  Returns out [B, Hq, D]."""
    torch = _torch()
    B = int(q.shape[0])
    dt = cfg.torch_dtype
    pq = _need(q, "q", (B, cfg.num_q_heads, cfg.head_dim), dt)
    pl = _need(lens, "lens", (B,), torch.int32)
    if out is None:
        out = torch.empty_like(q)
    po = _need(out, "out", tuple(q.shape), dt)
    if workspace is None:
        workspace = torch.empty(paged_decode_workspace_bytes(cfg, kv, B), dtype=torch.uint8,
                                device=q.device)
    pw = _need(workspace, "workspace", (workspace.numel(),), torch.uint8)
    c = cfg.c_struct()
    k = kv.c_struct(cfg)
    _check(library().gqa_attn_decode_paged(ctypes.byref(c), pq, ctypes.byref(k), pl, B,
                                           int(window), po, pw, workspace.numel(),
                                           _stream(stream)))
    return out


# ------------------------------------------------------------------------------------------------
MLA_WIDTH, MLA_LATENT = 576, 512


def mla_decode_workspace_bytes(B: int, H: int, Smax: int) -> int:
    n = library().gqa_mla_decode_workspace_bytes(int(B), int(H), int(Smax))
    err = last_error()
    if n == 0 and err:
        raise GQAError(2, err)
    return int(n)


def mla_decode(q, cache, lens, scale, out=None, workspace=None, stream=None):
    """Absorbed latent-attention decode core: q [B, H, 576] bf16, cache [B, Smax, 576] bf16, lens
    [B] int32.  Returns out [B, H, 512] bf16 (before W_uv)."""
    torch = _torch()
    B, H = int(q.shape[0]), int(q.shape[1])
    Smax = int(cache.shape[1])
    pq = _need(q, "q", (B, H, MLA_WIDTH), torch.bfloat16)
    pc = _need(cache, "cache", (B, Smax, MLA_WIDTH), torch.bfloat16)
    pl = _need(lens, "lens", (B,), torch.int32)
    if out is None:
        out = torch.empty((B, H, MLA_LATENT), dtype=torch.bfloat16, device=q.device)
    po = _need(out, "out", (B, H, MLA_LATENT), torch.bfloat16)
    if workspace is None:
        workspace = torch.empty(mla_decode_workspace_bytes(B, H, Smax), dtype=torch.uint8,
                                device=q.device)
    pw = _need(workspace, "workspace", (workspace.numel(),), torch.uint8)
    _check(library().gqa_mla_decode(pq, pc, pl, B, H, Smax, float(scale), po, pw, workspace.numel(),
                                    _stream(stream)))
    return out
