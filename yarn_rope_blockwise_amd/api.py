"""Thin ctypes binding of libyrb.so (C ABI in include/yrb.h).

Marshalling only: tensors are passed as raw device pointers plus element
strides, the stream is torch's current stream, and every step of the path
runs in the library's HIP kernels.  Importing fails loudly when the library
has not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libyrb.so")

PLAIN, PI, NTK, YARN = 0, 1, 2, 3
BF16, F32, FP8_E4M3 = 0, 1, 2
LAYOUT_HALF, LAYOUT_INTERLEAVED = 0, 1
ACC_FIRST, ACC_FINALIZE = 1, 2
WORKSPACE_BYTES = 64      # YRB_WORKSPACE_BYTES
EXPORTS = ("rope_tables_build", "rope_tables_build_factors", "rope_apply", "attn_prefill_blockwise",
           "attn_prefill_blockwise_noalloc", "attn_prefill_sink_window", "attn_prefill_sink_window_chunk",
           "attn_block_accumulate", "attn_decode_sink_window", "attn_decode_sink_window_fp8",
           "rope_apply_ex", "attn_decode_sink_window_ex", "yrb_status_str")

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_vp = ctypes.c_void_p
_i64p = ctypes.POINTER(ctypes.c_int64)
_dp = ctypes.POINTER(ctypes.c_double)


class YrbRopeConfig(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("base", ctypes.c_double), ("scale", ctypes.c_double),
                ("orig_ctx", ctypes.c_int64), ("alpha", ctypes.c_double),
                ("beta", ctypes.c_double)]


@dataclass(frozen=True)
class RopeConfig:
    kind: int
    head_dim: int
    base: float = 10000.0
    scale: float = 1.0
    orig_ctx: int = 4096
    alpha: float = 1.0
    beta: float = 32.0

    @classmethod
    def of(cls, r) -> "RopeConfig":
        return cls(r.kind, r.head_dim, r.base, r.scale, r.orig_ctx, r.alpha, r.beta)

    def c(self) -> YrbRopeConfig:
        return YrbRopeConfig(self.kind, self.head_dim, self.base, self.scale, self.orig_ctx,
                             self.alpha, self.beta)


class YrbError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({_status_str(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libyrb.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m yarn_rope_blockwise_amd.build`")
        # torch first: libyrb.so then binds to the HIP runtime torch already
        # loaded, so both work on the same devices, streams and allocations
        # (loaded the other way round, a process ends up with two runtimes and
        # the library's launches fail).
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        L.yrb_status_str.argtypes = [ctypes.c_int]
        L.yrb_status_str.restype = ctypes.c_char_p
        L.rope_tables_build.argtypes = [ctypes.POINTER(YrbRopeConfig), _i64, _i64, _vp, _dp, _dp,
                                        _vp]
        L.rope_tables_build_factors.argtypes = [_i32, ctypes.c_double, _dp, _i64, _i64, _vp, _dp,
                                                _vp]
        L.rope_apply.argtypes = [_vp, _vp, _i32, _i64, _i64, _i64, _i64, _i64p, _i64p, _vp, _i64,
                                 _i64, _vp, _vp]
        L.attn_prefill_blockwise.argtypes = [_vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _i64,
                                             _i64, _i64p, _vp, _i64, ctypes.c_float, _i32, _vp,
                                             _vp, _vp]
        L.attn_prefill_blockwise_noalloc.argtypes = [_vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64,
                                                     _i64, _i64, _i64p, _vp, _i64, ctypes.c_float,
                                                     _i32, _vp, _vp]
        L.attn_prefill_sink_window.argtypes = [_vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _i64,
                                               _i64, _i64p, _vp, _i64, ctypes.c_float, _i64, _i64,
                                               _vp, _vp, _vp]
        L.attn_prefill_sink_window_chunk.argtypes = [_vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _i64,
                                                     _i64, _i64, _i64p, _i64, _vp, _i64, ctypes.c_float,
                                                     _i64, _i64, _vp, _vp, _vp]
        L.attn_block_accumulate.argtypes = [_vp, _vp, _vp, _i32, _i64, _i64, _i64, _i64, _i64,
                                            _i64, _i64p, _i64, _i64, _vp, _i64, ctypes.c_float,
                                            _i32, _vp, _vp, _vp, _i32, _vp, _i64p, _vp, _vp]
        L.attn_decode_sink_window.argtypes = [_vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _i64,
                                              _i64, _i64, _i64p, _i64p, _i64p, _vp, _vp, _vp,
                                              _i64, ctypes.c_float, _vp]
        L.attn_decode_sink_window_fp8.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                                  _i64, _i64, _i64p, _i64p, _i64p, _vp, _vp, _vp,
                                                  _vp, _vp, _i64, ctypes.c_float, _vp]
        L.rope_apply_ex.argtypes = [_vp, _vp, _i32, _i64, _i64, _i64, _i64, _i64p, _i64p, _vp,
                                    _i64, _i64, _vp, _i32, _vp]
        L.attn_decode_sink_window_ex.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, _i64, _i64, _i64,
                                                 _i64, _i64, _i64, _i64p, _i64p, _i64p, _vp, _vp,
                                                 _vp, _vp, _vp, _i64, ctypes.c_float, _vp]
        for name in EXPORTS[:-1]:
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _status_str(status: int) -> str:
    try:
        return lib().yrb_status_str(status).decode()
    except Exception:  # pragma: no cover - only while reporting another error
        return "?"


def _check(fn: str, status: int):
    if status != 0:
        raise YrbError(fn, status)


def _arr(vals):
    a = (ctypes.c_int64 * len(vals))(*[int(v) for v in vals])
    return a


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _bsh_strides(t):
    """(b, s, h) element strides of a [B, S, H, D] tensor with unit dim stride."""
    if t.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous")
    return [t.stride(0), t.stride(1), t.stride(2)]


# ----------------------------------------------------------------------------
# rope_tables_build
# ----------------------------------------------------------------------------

def rope_frequencies(cfg: RopeConfig):
    """theta'_i (fp64, host) and attn_factor from the library, no launch."""
    th = (ctypes.c_double * (cfg.head_dim // 2))()
    af = ctypes.c_double()
    c = cfg.c()
    _check("rope_tables_build", lib().rope_tables_build(ctypes.byref(c), 0, 0, None, th,
                                                          ctypes.byref(af), None))
    return np.array(th[:], dtype=np.float64), af.value


def rope_tables_build(cfg: RopeConfig, n_pos: int, pos0: int = 0, out=None, device="cuda"):
    """cos/sin table [n_pos, d/2, 2] fp32 on the GPU; returns (table, theta', attn_factor)."""
    import torch
    if out is None:
        out = torch.empty((n_pos, cfg.head_dim // 2, 2), dtype=torch.float32, device=device)
    th = (ctypes.c_double * (cfg.head_dim // 2))()
    af = ctypes.c_double()
    c = cfg.c()
    _check("rope_tables_build", lib().rope_tables_build(ctypes.byref(c), pos0, n_pos, _ptr(out),
                                                          th, ctypes.byref(af), _stream()))
    return out, np.array(th[:], dtype=np.float64), af.value


def _factor_array(head_dim: int, factors):
    f = np.ascontiguousarray(np.asarray(factors, dtype=np.float64).reshape(-1))
    if f.size != head_dim // 2:
        raise ValueError(f"need {head_dim // 2} factors, got {f.size}")
    return f


def rope_frequencies_factors(head_dim: int, base: float, factors):
    """theta'_i = theta_i / lambda_i (fp64, host) from the library, no launch."""
    f = _factor_array(head_dim, factors)
    th = (ctypes.c_double * (head_dim // 2))()
    _check("rope_tables_build_factors", lib().rope_tables_build_factors(
        head_dim, base, f.ctypes.data_as(_dp), 0, 0, None, th, None))
    return np.array(th[:], dtype=np.float64)


def rope_tables_build_factors(head_dim: int, base: float, factors, n_pos: int, pos0: int = 0,
                              out=None, device="cuda"):
    """cos/sin table [n_pos, d/2, 2] fp32 from per-pair factors; returns (table, theta')."""
    import torch
    f = _factor_array(head_dim, factors)
    if out is None:
        out = torch.empty((n_pos, head_dim // 2, 2), dtype=torch.float32, device=device)
    th = (ctypes.c_double * (head_dim // 2))()
    _check("rope_tables_build_factors", lib().rope_tables_build_factors(
        head_dim, base, f.ctypes.data_as(_dp), pos0, n_pos, _ptr(out), th, _stream()))
    return out, np.array(th[:], dtype=np.float64)


# ----------------------------------------------------------------------------
# rope_apply
# ----------------------------------------------------------------------------

def rope_apply(x, cos_sin, pos_offset: int = 0, pos_ids=None, out=None):
    """Rotate half-split pairs of x [B, S, H, D] (bf16 or fp32)."""
    import torch
    if out is None:
        out = torch.empty_like(x)
    B, S, H, D = x.shape
    if pos_ids is not None:
        pos_ids = pos_ids.to(torch.int32).contiguous()
    _check("rope_apply", lib().rope_apply(
        _ptr(x), _ptr(out), _dtype_code(x), B, S, H, D, _arr(_bsh_strides(x)),
        _arr(_bsh_strides(out)), _ptr(cos_sin), cos_sin.shape[0], pos_offset, _ptr(pos_ids),
        _stream()))
    return out


# ----------------------------------------------------------------------------
# attn_prefill_blockwise
# ----------------------------------------------------------------------------

def new_workspace(device="cuda"):
    """A zeroed workspace for the prefill calls and attn_block_accumulate.
    One serves any number of calls in sequence on a stream; calls that may
    run at the same time need one each."""
    import torch
    return torch.zeros(WORKSPACE_BYTES // 4, dtype=torch.int32, device=device)


def attn_prefill_blockwise(q, k, v, softmax_scale: float, cos_sin=None, causal: bool = True,
                           out=None, lse=None, workspace=None):
    """Causal (or full) attention, q rotated on load when ``cos_sin`` is given.

    q [B,S,Hq,D] (raw), k [B,S,Hkv,D] already rotated (rope_apply), v [B,S,Hkv,D].
    ``workspace`` (new_workspace()) lets the grid balance its last items at
    run time; None takes a fixed schedule with the same results.
    """
    import torch
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if out is None:
        out = torch.empty_like(q)
    strides = _arr(_bsh_strides(q) + _bsh_strides(k) + _bsh_strides(v) + _bsh_strides(out))
    n_rows = 0 if cos_sin is None else cos_sin.shape[0]
    _check("attn_prefill_blockwise", lib().attn_prefill_blockwise(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _dtype_code(q), B, S, Hq, Hkv, D, strides,
        _ptr(cos_sin), n_rows, float(softmax_scale), int(bool(causal)), _ptr(lse),
        _ptr(workspace), _stream()))
    return out


def attn_prefill_blockwise_noalloc(q, k, v, softmax_scale: float, cos_sin=None,
                                   causal: bool = True, out=None, lse=None):
    """attn_prefill_blockwise with the claim counter in the library's static
    per-GPU array instead of a workspace (for callers that cannot allocate;
    calls that overlap on one GPU race on it).  ``out`` must be given when
    the caller cannot allocate it here."""
    import torch
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if out is None:
        out = torch.empty_like(q)
    strides = _arr(_bsh_strides(q) + _bsh_strides(k) + _bsh_strides(v) + _bsh_strides(out))
    n_rows = 0 if cos_sin is None else cos_sin.shape[0]
    _check("attn_prefill_blockwise_noalloc", lib().attn_prefill_blockwise_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _dtype_code(q), B, S, Hq, Hkv, D, strides,
        _ptr(cos_sin), n_rows, float(softmax_scale), int(bool(causal)), _ptr(lse), _stream()))
    return out


def attn_prefill_sink_window(q, k, v, softmax_scale: float, n_sink: int, window: int,
                             cos_sin=None, out=None, lse=None, workspace=None):
    """attn_prefill_blockwise under the sink+window mask: key n is visible to
    query t iff n <= t and (n < n_sink or n > t - window); bf16 only."""
    import torch
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if out is None:
        out = torch.empty_like(q)
    strides = _arr(_bsh_strides(q) + _bsh_strides(k) + _bsh_strides(v) + _bsh_strides(out))
    n_rows = 0 if cos_sin is None else cos_sin.shape[0]
    _check("attn_prefill_sink_window", lib().attn_prefill_sink_window(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _dtype_code(q), B, S, Hq, Hkv, D, strides,
        _ptr(cos_sin), n_rows, float(softmax_scale), int(n_sink), int(window), _ptr(lse),
        _ptr(workspace), _stream()))
    return out


def attn_prefill_sink_window_chunk(q, k, v, softmax_scale: float, n_sink: int, window: int,
                                   q_offset: int, cos_sin=None, out=None, lse=None, workspace=None):
    """One chunk of a sink+window prefill: q [B,Sq,Hq,D] at positions
    q_offset.., k/v [B,Sk,Hkv,D] at positions 0.. (k already rotated); key t
    is visible to query position p iff t <= p and (t < n_sink or t > p -
    window).  bf16 only."""
    import torch
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    if out is None:
        out = torch.empty_like(q)
    strides = _arr(_bsh_strides(q) + _bsh_strides(k) + _bsh_strides(v) + _bsh_strides(out))
    n_rows = 0 if cos_sin is None else cos_sin.shape[0]
    _check("attn_prefill_sink_window_chunk", lib().attn_prefill_sink_window_chunk(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _dtype_code(q), B, Sq, Sk, Hq, Hkv, D, strides,
        int(q_offset), _ptr(cos_sin), n_rows, float(softmax_scale), int(n_sink), int(window), _ptr(lse),
        _ptr(workspace), _stream()))
    return out


# ----------------------------------------------------------------------------
# attn_block_accumulate
# ----------------------------------------------------------------------------

@dataclass
class AccState:
    """Online-softmax state of one query block: o_acc [B,Sq,Hq,D], m/l [B,Hq,Sq] (fp32)."""
    o_acc: object
    m: object
    l: object

    @classmethod
    def empty(cls, B, Sq, Hq, D, device="cuda"):
        import torch
        return cls(torch.empty((B, Sq, Hq, D), dtype=torch.float32, device=device),
                   torch.empty((B, Hq, Sq), dtype=torch.float32, device=device),
                   torch.empty((B, Hq, Sq), dtype=torch.float32, device=device))


def attn_block_accumulate(q, k_blk, v_blk, state: AccState, q_offset: int, k_offset: int,
                          softmax_scale: float, cos_sin=None, causal: bool = True,
                          first: bool = False, finalize: bool = False, out=None,
                          workspace=None):
    """Fold one (already rotated) key/value block into the state; q is rotated
    on load when ``cos_sin`` is given.  Returns ``out`` when finalizing."""
    import torch
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k_blk.shape[1], k_blk.shape[2]
    if finalize and out is None:
        out = torch.empty_like(q)
    strides = _arr(_bsh_strides(q) + _bsh_strides(k_blk) + _bsh_strides(v_blk))
    flags = (ACC_FIRST if first else 0) | (ACC_FINALIZE if finalize else 0)
    o_str = _arr(_bsh_strides(out)) if finalize else None
    n_rows = 0 if cos_sin is None else cos_sin.shape[0]
    _check("attn_block_accumulate", lib().attn_block_accumulate(
        _ptr(q), _ptr(k_blk), _ptr(v_blk), _dtype_code(q), B, Sq, Sk, Hq, Hkv, D, strides,
        q_offset, k_offset, _ptr(cos_sin), n_rows, float(softmax_scale), int(bool(causal)),
        _ptr(state.o_acc), _ptr(state.m), _ptr(state.l), flags, _ptr(out), o_str,
        _ptr(workspace), _stream()))
    return out


# ----------------------------------------------------------------------------
# attn_decode_sink_window
# ----------------------------------------------------------------------------

def attn_decode_sink_window(q, k_cache, v_cache, cache_len, n_sink: int, window: int, cos_sin,
                            softmax_scale: float, ring_head=None, out=None):
    """q [B,Hq,D]; caches [B,Hkv,C,D] (un-rotated keys); cache_len/ring_head int32 [B]."""
    import torch
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    if out is None:
        out = torch.empty_like(q)
    if q.stride(2) != 1 or k_cache.stride(3) != 1 or v_cache.stride(3) != 1 or out.stride(2) != 1:
        raise ValueError("the head dimension must be contiguous")
    if tuple(k_cache.stride()) != tuple(v_cache.stride()):
        raise ValueError("k_cache and v_cache must share strides")
    cache_len = cache_len.to(torch.int32).contiguous()
    if ring_head is not None:
        ring_head = ring_head.to(torch.int32).contiguous()
    _check("attn_decode_sink_window", lib().attn_decode_sink_window(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _dtype_code(q), B, Hq, Hkv, D,
        n_sink, window, _arr([q.stride(0), q.stride(1)]),
        _arr([k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)]),
        _arr([out.stride(0), out.stride(1)]), _ptr(cache_len), _ptr(ring_head), _ptr(cos_sin),
        cos_sin.shape[0], float(softmax_scale), _stream()))
    return out


def attn_decode_sink_window_fp8(q, k_codes, v_codes, cache_len, n_sink: int, window: int, cos_sin,
                                softmax_scale: float, ring_head=None, out=None, k_scale=None,
                                v_scale=None):
    """q [B,Hq,D] bf16; caches [B,Hkv,C,D] uint8 OCP E4M3 codes (un-rotated keys);
    k_scale / v_scale fp32 [B,Hkv] dequantisation scales or None (1)."""
    import torch
    B, Hq, D = q.shape
    Hkv = k_codes.shape[1]
    if k_codes.dtype != torch.uint8 or v_codes.dtype != torch.uint8:
        raise ValueError("fp8 caches are passed as uint8 codes")
    if out is None:
        out = torch.empty_like(q)
    if q.stride(2) != 1 or k_codes.stride(3) != 1 or v_codes.stride(3) != 1 or out.stride(2) != 1:
        raise ValueError("the head dimension must be contiguous")
    if tuple(k_codes.stride()) != tuple(v_codes.stride()):
        raise ValueError("k and v caches must share strides")
    cache_len = cache_len.to(torch.int32).contiguous()
    if ring_head is not None:
        ring_head = ring_head.to(torch.int32).contiguous()
    if k_scale is not None:
        k_scale = k_scale.to(torch.float32).contiguous()
    if v_scale is not None:
        v_scale = v_scale.to(torch.float32).contiguous()
    _check("attn_decode_sink_window_fp8", lib().attn_decode_sink_window_fp8(
        _ptr(q), _ptr(k_codes), _ptr(v_codes), _ptr(out), B, Hq, Hkv, D, n_sink, window,
        _arr([q.stride(0), q.stride(1)]),
        _arr([k_codes.stride(0), k_codes.stride(1), k_codes.stride(2)]),
        _arr([out.stride(0), out.stride(1)]), _ptr(cache_len), _ptr(ring_head), _ptr(k_scale),
        _ptr(v_scale), _ptr(cos_sin), cos_sin.shape[0], float(softmax_scale), _stream()))
    return out


def rope_apply_ex(x, cos_sin, layout: int = LAYOUT_HALF, pos_offset: int = 0, pos_ids=None,
                  out=None):
    """rope_apply with a pair layout: LAYOUT_HALF (i, i+d/2) or LAYOUT_INTERLEAVED (2i, 2i+1)."""
    import torch
    if out is None:
        out = torch.empty_like(x)
    B, S, H, D = x.shape
    if pos_ids is not None:
        pos_ids = pos_ids.to(torch.int32).contiguous()
    _check("rope_apply_ex", lib().rope_apply_ex(
        _ptr(x), _ptr(out), _dtype_code(x), B, S, H, D, _arr(_bsh_strides(x)),
        _arr(_bsh_strides(out)), _ptr(cos_sin), cos_sin.shape[0], pos_offset, _ptr(pos_ids),
        layout, _stream()))
    return out


def attn_decode_sink_window_ex(q, k_cache, v_cache, cache_len, n_sink: int, window: int, cos_sin,
                               softmax_scale: float, layout: int = LAYOUT_HALF, ring_head=None,
                               out=None, k_scale=None, v_scale=None):
    """The decode with the cache type taken from k_cache (bf16, or uint8 E4M3 codes with
    optional k_scale / v_scale [B,Hkv]) and the key/query pair layout."""
    import torch
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    cache_dtype = FP8_E4M3 if k_cache.dtype == torch.uint8 else _dtype_code(k_cache)
    if out is None:
        out = torch.empty_like(q)
    if q.stride(2) != 1 or k_cache.stride(3) != 1 or v_cache.stride(3) != 1 or out.stride(2) != 1:
        raise ValueError("the head dimension must be contiguous")
    if tuple(k_cache.stride()) != tuple(v_cache.stride()):
        raise ValueError("k and v caches must share strides")
    cache_len = cache_len.to(torch.int32).contiguous()
    if ring_head is not None:
        ring_head = ring_head.to(torch.int32).contiguous()
    if k_scale is not None:
        k_scale = k_scale.to(torch.float32).contiguous()
    if v_scale is not None:
        v_scale = v_scale.to(torch.float32).contiguous()
    _check("attn_decode_sink_window_ex", lib().attn_decode_sink_window_ex(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), cache_dtype, layout, B, Hq, Hkv, D,
        n_sink, window, _arr([q.stride(0), q.stride(1)]),
        _arr([k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)]),
        _arr([out.stride(0), out.stride(1)]), _ptr(cache_len), _ptr(ring_head), _ptr(k_scale),
        _ptr(v_scale), _ptr(cos_sin), cos_sin.shape[0], float(softmax_scale), _stream()))
    return out
