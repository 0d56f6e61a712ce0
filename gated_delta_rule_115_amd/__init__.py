"""MI355X (gfx950) Gated DeltaNet token mixer: thin Python binding of libgdn.so.

The functions below carry the names of the C entry points declared in
include/gdn.h and do argument marshalling only: they check device, dtype,
shape and contiguity of torch tensors, allocate outputs / workspace when the
caller does not pass them, and call the library on the current HIP stream.
Every step of the computation runs in the library's HIP kernels; there is no
CPU or PyTorch fallback.  If libgdn.so is missing or fails to load, every
entry point raises.

Operation ("The Key to Going Linear: Analysis-Driven Transformer
Linearization", section 3.1.2): per (batch, head), a key-major f32 state
S in R^{Dk x Dv} is updated per token as
    S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
and read as out_t = scale * S_t^T q_t.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "GDN_BF16", "GDN_F32", "GdnError", "lib", "library_path",
    "gdn_abi_version", "gdn_prefill_workspace_bytes", "gdn_prefill_chunked",
    "gdn_decode_step", "gdn_short_conv_silu", "gdn_short_conv_step",
    "gdn_swa_sink_decode", "gdn_swa_sink_prefill", "gdn_swa_cache_fill",
    "gdn_hybrid_prefill_workspace_bytes", "gdn_hybrid_prefill",
    "gdn_prefill_chgate_workspace_bytes", "gdn_prefill_chunked_chgate", "gdn_decode_step_chgate",
    "gdn_prefill_backward_workspace_bytes", "gdn_prefill_backward",
    "gdn_prefill_chunked_noalloc", "GDN_NOALLOC_SCRATCH_BYTES",
    "gdn_prefill_chunked_kgla", "gdn_decode_step_kgla", "gdn_prefill_chunked_conv",
    "EXPORTED_SYMBOLS",
]

GDN_BF16 = 0
GDN_F32 = 1
_STATUS = {0: "GDN_OK", 1: "GDN_ERR_INVALID_ARG", 2: "GDN_ERR_UNSUPPORTED",
           3: "GDN_ERR_HIP"}

# Every function the C header declares.
EXPORTED_SYMBOLS = (
    "gdn_abi_version", "gdn_last_error", "gdn_prefill_workspace_bytes",
    "gdn_prefill_chunked", "gdn_decode_step", "gdn_short_conv_silu",
    "gdn_short_conv_step", "gdn_swa_sink_decode", "gdn_swa_sink_prefill",
    "gdn_swa_cache_fill", "gdn_hybrid_prefill_workspace_bytes", "gdn_hybrid_prefill",
    "gdn_prefill_chgate_workspace_bytes", "gdn_prefill_chunked_chgate", "gdn_decode_step_chgate",
    "gdn_prefill_backward_workspace_bytes", "gdn_prefill_backward",
    "gdn_prefill_chunked_noalloc", "gdn_prefill_chunked_kgla", "gdn_decode_step_kgla",
    "gdn_prefill_chunked_conv",
)

# Size of the static scratch of gdn_prefill_chunked_noalloc (gdn.h).
GDN_NOALLOC_SCRATCH_BYTES = 64 << 20

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libgdn.so")
_lib = None


class GdnError(RuntimeError):
    """A library call returned a non-zero gdn_status."""

    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: {_STATUS.get(status, status)}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libgdn.so (built by gated_delta_rule_115_amd.build); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise ImportError(
            f"{library_path} is missing: build it with "
            "`python -m gated_delta_rule_115_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(library_path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.gdn_abi_version.restype = i
    L.gdn_last_error.restype = ctypes.c_char_p
    L.gdn_prefill_workspace_bytes.restype = sz
    L.gdn_prefill_workspace_bytes.argtypes = [i] * 7
    L.gdn_prefill_chunked.restype = i
    L.gdn_prefill_chunked.argtypes = [vp] * 8 + [i] * 8 + [f, vp, sz, vp]
    L.gdn_decode_step.restype = i
    L.gdn_prefill_chunked_noalloc.restype = i
    L.gdn_prefill_chunked_noalloc.argtypes = [vp] * 8 + [i] * 8 + [f, vp]
    L.gdn_prefill_chunked_conv.restype = i
    L.gdn_prefill_chunked_conv.argtypes = [vp] * 6 + [i, f] + [vp] * 5 + [i] * 8 + [f, vp, sz, vp]
    L.gdn_decode_step.argtypes = [vp] * 8 + [i] * 6 + [f, vp]
    L.gdn_short_conv_silu.restype = i
    L.gdn_short_conv_silu.argtypes = [vp] * 3 + [i] * 5 + [f, i, i, vp]
    L.gdn_short_conv_step.restype = i
    L.gdn_short_conv_step.argtypes = [vp] * 4 + [i] * 4 + [f, i, i, vp]
    L.gdn_swa_sink_decode.restype = i
    L.gdn_swa_sink_decode.argtypes = [vp] * 6 + [i] * 5 + [f, i, vp, i, i, vp]
    L.gdn_swa_sink_prefill.restype = i
    L.gdn_swa_sink_prefill.argtypes = [vp] * 4 + [i] * 6 + [f, i, i, i, vp]
    L.gdn_swa_cache_fill.restype = i
    L.gdn_swa_cache_fill.argtypes = [vp] * 4 + [i] * 7 + [vp]
    L.gdn_hybrid_prefill_workspace_bytes.restype = sz
    L.gdn_hybrid_prefill_workspace_bytes.argtypes = [i] * 6
    L.gdn_hybrid_prefill.restype = i
    L.gdn_hybrid_prefill.argtypes = [vp] * 12 + [i] * 6 + [f, f, i, i, vp, sz, vp]
    L.gdn_prefill_chgate_workspace_bytes.restype = sz
    L.gdn_prefill_chgate_workspace_bytes.argtypes = [i] * 3
    L.gdn_prefill_chunked_chgate.restype = i
    L.gdn_prefill_chunked_chgate.argtypes = [vp] * 8 + [i] * 7 + [f, vp, sz, vp]
    L.gdn_decode_step_chgate.restype = i
    L.gdn_decode_step_chgate.argtypes = [vp] * 8 + [i] * 6 + [f, vp]
    L.gdn_prefill_chunked_kgla.restype = i
    L.gdn_prefill_chunked_kgla.argtypes = [vp] * 8 + [i] * 7 + [f, vp, sz, vp]
    L.gdn_decode_step_kgla.restype = i
    L.gdn_decode_step_kgla.argtypes = [vp] * 8 + [i] * 6 + [f, vp]
    L.gdn_prefill_backward_workspace_bytes.restype = sz
    L.gdn_prefill_backward_workspace_bytes.argtypes = [i] * 5
    L.gdn_prefill_backward.restype = i
    L.gdn_prefill_backward.argtypes = [vp] * 14 + [i] * 6 + [f, vp, sz, vp]
    _lib = L
    return L


def gdn_abi_version() -> int:
    return lib().gdn_abi_version()


def _check(fn, status):
    if status != 0:
        raise GdnError(fn, status, lib().gdn_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _out_dtype(x_dtype, out_dtype):
    return x_dtype if out_dtype is None else out_dtype


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name, dtype=None, shape=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def gdn_prefill_workspace_bytes(B, T, H, Dk, Dv, chunk=64, dtype=GDN_BF16) -> int:
    return int(lib().gdn_prefill_workspace_bytes(B, T, H, Dk, Dv, chunk, dtype))


def gdn_prefill_chunked(q, k, v, alpha, beta, state_in=None, *, chunk=64,
                        scale=1.0, out=None, out_dtype=None, state_out=None,
                        workspace=None, want_state=True, stream=None):
    """Chunk-parallel prefill.  q, k [B,T,H,Dk], v [B,T,H,Dv] (bf16 or f32),
    alpha, beta [B,T,H] f32, state_in [B,H,Dk,Dv] f32 or None.  out_dtype
    (default: q's dtype) may be float32 with bf16 inputs.
    Returns (out [B,T,H,Dv], state_out [B,H,Dk,Dv] or None)."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dt = _dtype_code(q)
    _dev(q, "q")
    _dev(k, "k", q.dtype, (B, T, H, Dk))
    _dev(v, "v", q.dtype, (B, T, H, Dv))
    _dev(alpha, "alpha", torch.float32, (B, T, H))
    _dev(beta, "beta", torch.float32, (B, T, H))
    _dev(state_in, "state_in", torch.float32, (B, H, Dk, Dv))
    odt = _out_dtype(q.dtype, out_dtype) if out is None else out.dtype
    if out is None:
        out = torch.empty((B, T, H, Dv), dtype=odt, device=q.device)
    _dev(out, "out", odt, (B, T, H, Dv))
    if state_out is None and want_state:
        state_out = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
    _dev(state_out, "state_out", torch.float32, (B, H, Dk, Dv))
    need = gdn_prefill_workspace_bytes(B, T, H, Dk, Dv, chunk, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace", torch.uint8)
    st = lib().gdn_prefill_chunked(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state_in),
        _ptr(state_out), _ptr(out), B, T, H, Dk, Dv, chunk, dt, _dtype_code(out),
        float(scale), _ptr(workspace), workspace.numel(), _stream(stream))
    _check("gdn_prefill_chunked", st)
    return out, state_out


def gdn_prefill_chunked_noalloc(q, k, v, alpha, beta, state_in, out, state_out=None, *,
                                chunk=64, scale=1.0, stream=None):
    """gdn_prefill_chunked with the library's static scratch instead of a
    workspace: allocates nothing (the caller passes out, and state_out or
    None).  Calls on one GPU share the scratch: order them on one stream."""
    if out is None:
        raise ValueError("gdn_prefill_chunked_noalloc allocates nothing: pass out")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    _dev(q, "q")
    _dev(k, "k", q.dtype, (B, T, H, Dk))
    _dev(v, "v", q.dtype, (B, T, H, Dv))
    _dev(alpha, "alpha", torch.float32, (B, T, H))
    _dev(beta, "beta", torch.float32, (B, T, H))
    _dev(state_in, "state_in", torch.float32, (B, H, Dk, Dv))
    _dev(out, "out", out.dtype, (B, T, H, Dv))
    _dev(state_out, "state_out", torch.float32, (B, H, Dk, Dv))
    st = lib().gdn_prefill_chunked_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state_in),
        _ptr(state_out), _ptr(out), B, T, H, Dk, Dv, chunk, _dtype_code(q), _dtype_code(out),
        float(scale), _stream(stream))
    _check("gdn_prefill_chunked_noalloc", st)
    return out, state_out


def gdn_prefill_chunked_conv(xq, xk, xv, taps_q, taps_k, taps_v, alpha, beta, state_in=None, *,
                             conv_eps=1e-6, chunk=64, scale=1.0, out=None, out_dtype=None,
                             state_out=None, workspace=None, want_state=True, stream=None):
    """gdn_prefill_chunked on the raw projections: xq, xk, xv [B,T,H,128]
    bf16 pass through the causal short convolution (taps_* [H*128, 4] f32,
    taps[:, 3] on the current token) and SiLU, and q, k through the per-head
    L2 normalisation (eps conv_eps), inside the prefill kernels.  Returns
    (out [B,T,H,128], state_out [B,H,128,128] or None)."""
    B, T, H, Dk = xq.shape
    Dv = xv.shape[-1]
    dt = _dtype_code(xq)
    _dev(xq, "xq")
    _dev(xk, "xk", xq.dtype, (B, T, H, Dk))
    _dev(xv, "xv", xq.dtype, (B, T, H, Dv))
    K = taps_q.shape[-1]
    _dev(taps_q, "taps_q", torch.float32, (H * Dk, K))
    _dev(taps_k, "taps_k", torch.float32, (H * Dk, K))
    _dev(taps_v, "taps_v", torch.float32, (H * Dv, K))
    _dev(alpha, "alpha", torch.float32, (B, T, H))
    _dev(beta, "beta", torch.float32, (B, T, H))
    _dev(state_in, "state_in", torch.float32, (B, H, Dk, Dv))
    odt = _out_dtype(xq.dtype, out_dtype) if out is None else out.dtype
    if out is None:
        out = torch.empty((B, T, H, Dv), dtype=odt, device=xq.device)
    _dev(out, "out", odt, (B, T, H, Dv))
    if state_out is None and want_state:
        state_out = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=xq.device)
    _dev(state_out, "state_out", torch.float32, (B, H, Dk, Dv))
    need = gdn_prefill_workspace_bytes(B, T, H, Dk, Dv, chunk, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=xq.device)
    _dev(workspace, "workspace", torch.uint8)
    st = lib().gdn_prefill_chunked_conv(
        _ptr(xq), _ptr(xk), _ptr(xv), _ptr(taps_q), _ptr(taps_k), _ptr(taps_v), K,
        float(conv_eps), _ptr(alpha), _ptr(beta), _ptr(state_in), _ptr(state_out), _ptr(out),
        B, T, H, Dk, Dv, chunk, dt, _dtype_code(out), float(scale), _ptr(workspace),
        workspace.numel(), _stream(stream))
    _check("gdn_prefill_chunked_conv", st)
    return out, state_out


def gdn_decode_step(q, k, v, alpha, beta, state_in, *, state_out=None,
                    scale=1.0, out=None, out_dtype=None, stream=None):
    """One token per sequence.  q, k [B,H,Dk], v [B,H,Dv], alpha, beta [B,H],
    state_in [B,H,Dk,Dv] f32.  state_out=state_in updates in place.
    Returns (out [B,H,Dv], state_out)."""
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    dt = _dtype_code(q)
    _dev(q, "q")
    _dev(k, "k", q.dtype, (B, H, Dk))
    _dev(v, "v", q.dtype, (B, H, Dv))
    _dev(alpha, "alpha", torch.float32, (B, H))
    _dev(beta, "beta", torch.float32, (B, H))
    _dev(state_in, "state_in", torch.float32, (B, H, Dk, Dv))
    if state_out is None:
        state_out = torch.empty_like(state_in)
    _dev(state_out, "state_out", torch.float32, (B, H, Dk, Dv))
    odt = _out_dtype(q.dtype, out_dtype) if out is None else out.dtype
    if out is None:
        out = torch.empty((B, H, Dv), dtype=odt, device=q.device)
    _dev(out, "out", odt, (B, H, Dv))
    st = lib().gdn_decode_step(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state_in),
        _ptr(state_out), _ptr(out), B, H, Dk, Dv, dt, _dtype_code(out),
        float(scale), _stream(stream))
    _check("gdn_decode_step", st)
    return out, state_out


def gdn_short_conv_silu(x, taps, *, l2norm_group=0, eps=1e-6, out=None,
                        out_dtype=None, stream=None):
    """Causal depthwise conv + SiLU (+ per-group L2 norm).  x [B,T,Ch],
    taps [Ch,K] f32 (taps[:, K-1] on the current token).  Returns y [B,T,Ch]."""
    B, T, Ch = x.shape
    K = taps.shape[1]
    dt = _dtype_code(x)
    _dev(x, "x")
    _dev(taps, "taps", torch.float32, (Ch, K))
    odt = _out_dtype(x.dtype, out_dtype) if out is None else out.dtype
    if out is None:
        out = torch.empty((B, T, Ch), dtype=odt, device=x.device)
    _dev(out, "out", odt, (B, T, Ch))
    st = lib().gdn_short_conv_silu(_ptr(x), _ptr(taps), _ptr(out), B, T, Ch, K,
                                   int(l2norm_group), float(eps), dt,
                                   _dtype_code(out), _stream(stream))
    _check("gdn_short_conv_silu", st)
    return out


def gdn_short_conv_step(x, taps, conv_state, *, l2norm_group=0, eps=1e-6, out=None,
                        out_dtype=None, stream=None):
    """One decode step of the short conv.  x [B,Ch], taps [Ch,K] f32,
    conv_state [B,K-1,Ch] (x's dtype; the previous K-1 inputs, oldest first),
    updated in place.  Returns y [B,Ch]."""
    B, Ch = x.shape
    K = taps.shape[1]
    dt = _dtype_code(x)
    _dev(x, "x")
    _dev(taps, "taps", torch.float32, (Ch, K))
    _dev(conv_state, "conv_state", x.dtype, (B, K - 1, Ch))
    odt = _out_dtype(x.dtype, out_dtype) if out is None else out.dtype
    if out is None:
        out = torch.empty((B, Ch), dtype=odt, device=x.device)
    _dev(out, "out", odt, (B, Ch))
    st = lib().gdn_short_conv_step(_ptr(x), _ptr(taps), _ptr(conv_state), _ptr(out), B, Ch,
                                   K, int(l2norm_group), float(eps), dt, _dtype_code(out),
                                   _stream(stream))
    _check("gdn_short_conv_step", st)
    return out


def gdn_swa_sink_decode(q, k_cache, v_cache, n_tokens, *, n_sink, window,
                        k_new=None, v_new=None, softmax_scale=None,
                        accumulate=False, out=None, out_dtype=None, stream=None):
    """Softmax over sinks + sliding window for the current token.
    q [B,H,D]; k_cache, v_cache [B,H,n_sink+window,D]; n_tokens [B] int32
    (tokens seen including the current).  k_new/v_new [B,H,D] are written
    into the current slot first when given.  accumulate=True adds into out."""
    B, H, D = q.shape
    dt = _dtype_code(q)
    nslot = n_sink + window
    _dev(q, "q")
    _dev(k_cache, "k_cache", q.dtype, (B, H, nslot, D))
    _dev(v_cache, "v_cache", q.dtype, (B, H, nslot, D))
    _dev(n_tokens, "n_tokens", torch.int32, (B,))
    _dev(k_new, "k_new", q.dtype, (B, H, D))
    _dev(v_new, "v_new", q.dtype, (B, H, D))
    odt = _out_dtype(q.dtype, out_dtype) if out is None else out.dtype
    if out is None:
        if accumulate:
            raise ValueError("accumulate=True needs out")
        out = torch.empty((B, H, D), dtype=odt, device=q.device)
    _dev(out, "out", odt, (B, H, D))
    if softmax_scale is None:
        softmax_scale = D ** -0.5
    st = lib().gdn_swa_sink_decode(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
        _ptr(n_tokens), B, H, D, int(n_sink), int(window), float(softmax_scale),
        int(bool(accumulate)), _ptr(out), dt, _dtype_code(out), _stream(stream))
    _check("gdn_swa_sink_decode", st)
    return out


def gdn_swa_sink_prefill(q, k, v, *, n_sink, window, softmax_scale=None,
                         accumulate_from=None, out=None, out_dtype=None, stream=None):
    """Softmax over sinks + sliding window at every position of a sequence.
    q, k, v [B,T,H,D] bf16 (D = 128).  Rows t >= accumulate_from add into out
    (None: write every row)."""
    B, T, H, D = q.shape
    _dev(q, "q")
    _dev(k, "k", q.dtype, q.shape)
    _dev(v, "v", q.dtype, q.shape)
    odt = _out_dtype(q.dtype, out_dtype) if out is None else out.dtype
    if out is None:
        if accumulate_from is not None and accumulate_from < T:
            raise ValueError("accumulate_from < T needs out")
        out = torch.empty((B, T, H, D), dtype=odt, device=q.device)
    _dev(out, "out", odt, (B, T, H, D))
    if softmax_scale is None:
        softmax_scale = D ** -0.5
    acc = T if accumulate_from is None else int(accumulate_from)
    st = lib().gdn_swa_sink_prefill(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, T, H, D, int(n_sink), int(window),
        float(softmax_scale), acc, _dtype_code(q), _dtype_code(out), _stream(stream))
    _check("gdn_swa_sink_prefill", st)
    return out


def gdn_swa_cache_fill(k, v, k_cache, v_cache, *, n_sink, window, stream=None):
    """Fill the [B,H,n_sink+window,D] decode caches from k, v [B,T,H,D]."""
    B, T, H, D = k.shape
    _dev(k, "k")
    _dev(v, "v", k.dtype, k.shape)
    _dev(k_cache, "k_cache", k.dtype, (B, H, n_sink + window, D))
    _dev(v_cache, "v_cache", k.dtype, (B, H, n_sink + window, D))
    st = lib().gdn_swa_cache_fill(_ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), B, T, H, D,
                                  int(n_sink), int(window), _dtype_code(k), _stream(stream))
    _check("gdn_swa_cache_fill", st)
    return k_cache, v_cache


def gdn_hybrid_prefill_workspace_bytes(B, T, H, D, n_sink, window) -> int:
    return lib().gdn_hybrid_prefill_workspace_bytes(B, T, H, D, int(n_sink), int(window))


def gdn_hybrid_prefill(q_lin, k_lin, v_lin, alpha, beta, q_swa, k_swa, v_swa, *, n_sink,
                       window, lin_scale=1.0, softmax_scale=None, state_out=None, out=None,
                       out_dtype=None, k_cache=None, v_cache=None, workspace=None,
                       stream=None):
    """Hybrid layer over a sequence: linear state over the tokens outside the
    sinks and the window, read with q_lin, plus the sink/window softmax of
    (q_swa, k_swa, v_swa).  All token tensors [B,T,H,D] bf16 (D = 128);
    alpha, beta [B,T,H] f32.  Returns (out, state_out)."""
    B, T, H, D = q_lin.shape
    shp = (B, T, H, D)
    for t, n in ((q_lin, "q_lin"), (k_lin, "k_lin"), (v_lin, "v_lin"), (q_swa, "q_swa"),
                 (k_swa, "k_swa"), (v_swa, "v_swa")):
        _dev(t, n, q_lin.dtype, shp)
    _dev(alpha, "alpha", torch.float32, (B, T, H))
    _dev(beta, "beta", torch.float32, (B, T, H))
    odt = _out_dtype(q_lin.dtype, out_dtype) if out is None else out.dtype
    if out is None:
        out = torch.empty(shp, dtype=odt, device=q_lin.device)
    _dev(out, "out", odt, shp)
    if state_out is None:
        state_out = torch.empty((B, H, D, D), dtype=torch.float32, device=q_lin.device)
    _dev(state_out, "state_out", torch.float32, (B, H, D, D))
    nslot = n_sink + window
    _dev(k_cache, "k_cache", q_lin.dtype, (B, H, nslot, D))
    _dev(v_cache, "v_cache", q_lin.dtype, (B, H, nslot, D))
    need = gdn_hybrid_prefill_workspace_bytes(B, T, H, D, n_sink, window)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_lin.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if softmax_scale is None:
        softmax_scale = D ** -0.5
    st = lib().gdn_hybrid_prefill(
        _ptr(q_lin), _ptr(k_lin), _ptr(v_lin), _ptr(alpha), _ptr(beta), _ptr(q_swa),
        _ptr(k_swa), _ptr(v_swa), _ptr(state_out), _ptr(out), _ptr(k_cache), _ptr(v_cache),
        B, T, H, D, int(n_sink), int(window), float(lin_scale), float(softmax_scale),
        _dtype_code(q_lin), _dtype_code(out), _ptr(workspace), wbytes, _stream(stream))
    _check("gdn_hybrid_prefill", st)
    return out, state_out


def gdn_prefill_chgate_workspace_bytes(B, T, H) -> int:
    return int(lib().gdn_prefill_chgate_workspace_bytes(B, T, H))


def _prefill_chgate(fn, q, k, v, alpha, beta, state_in, scale, out, out_dtype, state_out,
                    workspace, stream):
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    _dev(q, "q")
    _dev(k, "k", q.dtype, q.shape)
    _dev(v, "v", q.dtype, (B, T, H, Dv))
    _dev(alpha, "alpha", torch.float32, (B, T, H, Dk))
    _dev(beta, "beta", torch.float32, (B, T, H))
    _dev(state_in, "state_in", torch.float32, (B, H, Dk, Dv))
    odt = _out_dtype(q.dtype, out_dtype) if out is None else out.dtype
    if out is None:
        out = torch.empty((B, T, H, Dv), dtype=odt, device=q.device)
    _dev(out, "out", odt, (B, T, H, Dv))
    if state_out is None:
        state_out = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
    _dev(state_out, "state_out", torch.float32, (B, H, Dk, Dv))
    need = gdn_prefill_chgate_workspace_bytes(B, T, H)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = getattr(lib(), fn)(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state_in), _ptr(state_out),
        _ptr(out), B, T, H, Dk, Dv, _dtype_code(q), _dtype_code(out), float(scale),
        _ptr(workspace), wbytes, _stream(stream))
    _check(fn, st)
    return out, state_out


def _decode_chgate(fn, q, k, v, alpha, beta, state_in, state_out, out, out_dtype, scale,
                   stream):
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    _dev(q, "q")
    _dev(k, "k", q.dtype, q.shape)
    _dev(v, "v", q.dtype, (B, H, Dv))
    _dev(alpha, "alpha", torch.float32, (B, H, Dk))
    _dev(beta, "beta", torch.float32, (B, H))
    _dev(state_in, "state_in", torch.float32, (B, H, Dk, Dv))
    if state_out is None:
        state_out = torch.empty_like(state_in)
    _dev(state_out, "state_out", torch.float32, (B, H, Dk, Dv))
    odt = _out_dtype(q.dtype, out_dtype) if out is None else out.dtype
    if out is None:
        out = torch.empty((B, H, Dv), dtype=odt, device=q.device)
    _dev(out, "out", odt, (B, H, Dv))
    st = getattr(lib(), fn)(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state_in), _ptr(state_out),
        _ptr(out), B, H, Dk, Dv, _dtype_code(q), _dtype_code(out), float(scale),
        _stream(stream))
    _check(fn, st)
    return out, state_out


def gdn_prefill_chunked_chgate(q, k, v, alpha, beta, state_in=None, *, scale=1.0, out=None,
                               out_dtype=None, state_out=None, workspace=None, stream=None):
    """Chunked GDN prefill with a channel-wise gate G_t = diag(alpha_t):
    q, k, alpha [B,T,H,Dk] (alpha f32), v [B,T,H,Dv], beta [B,T,H] f32.
    Returns (out [B,T,H,Dv], S_T [B,H,Dk,Dv])."""
    return _prefill_chgate("gdn_prefill_chunked_chgate", q, k, v, alpha, beta, state_in, scale,
                           out, out_dtype, state_out, workspace, stream)


def gdn_decode_step_chgate(q, k, v, alpha, beta, state_in, *, state_out=None, out=None,
                           out_dtype=None, scale=1.0, stream=None):
    """One channel-gated step: q, k, alpha [B,H,Dk] (alpha f32), v [B,H,Dv],
    beta [B,H]; state [B,H,Dk,Dv] (state_out may be state_in).  Returns (out, S')."""
    return _decode_chgate("gdn_decode_step_chgate", q, k, v, alpha, beta, state_in, state_out,
                          out, out_dtype, scale, stream)


def gdn_prefill_chunked_kgla(q, k, v, alpha, beta, state_in=None, *, scale=1.0, out=None,
                             out_dtype=None, state_out=None, workspace=None, stream=None):
    """Gated linear attention with a key-dependent gate (kGLA): per-channel
    gate alpha o (1 - beta k o k), write k v^T.  Shapes as for
    gdn_prefill_chunked_chgate.  Returns (out [B,T,H,Dv], S_T [B,H,Dk,Dv])."""
    return _prefill_chgate("gdn_prefill_chunked_kgla", q, k, v, alpha, beta, state_in, scale,
                           out, out_dtype, state_out, workspace, stream)


def gdn_decode_step_kgla(q, k, v, alpha, beta, state_in, *, state_out=None, out=None,
                         out_dtype=None, scale=1.0, stream=None):
    """One kGLA step; shapes as for gdn_decode_step_chgate.  Returns (out, S')."""
    return _decode_chgate("gdn_decode_step_kgla", q, k, v, alpha, beta, state_in, state_out,
                          out, out_dtype, scale, stream)


def gdn_prefill_backward_workspace_bytes(B, T, H, Dk, Dv) -> int:
    return int(lib().gdn_prefill_backward_workspace_bytes(B, T, H, Dk, Dv))


def gdn_prefill_backward(q, k, v, alpha, beta, dout, state_in=None, dstate_out=None, *,
                         scale=1.0, workspace=None, stream=None):
    """Gradients of gdn_prefill_chunked (scalar gate): returns dict dq, dk, dv,
    dalpha, dbeta, dstate_in (f32).  dout [B,T,H,Dv] f32; dstate_out
    [B,H,Dk,Dv] f32 or None."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    _dev(q, "q")
    _dev(k, "k", q.dtype, q.shape)
    _dev(v, "v", q.dtype, (B, T, H, Dv))
    _dev(alpha, "alpha", torch.float32, (B, T, H))
    _dev(beta, "beta", torch.float32, (B, T, H))
    _dev(state_in, "state_in", torch.float32, (B, H, Dk, Dv))
    _dev(dout, "dout", torch.float32, (B, T, H, Dv))
    _dev(dstate_out, "dstate_out", torch.float32, (B, H, Dk, Dv))
    f32 = dict(dtype=torch.float32, device=q.device)
    r = dict(dq=torch.empty((B, T, H, Dk), **f32), dk=torch.empty((B, T, H, Dk), **f32),
             dv=torch.empty((B, T, H, Dv), **f32), dalpha=torch.empty((B, T, H), **f32),
             dbeta=torch.empty((B, T, H), **f32), dstate_in=torch.empty((B, H, Dk, Dv), **f32))
    need = gdn_prefill_backward_workspace_bytes(B, T, H, Dk, Dv)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    st = lib().gdn_prefill_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state_in), _ptr(dout),
        _ptr(dstate_out), _ptr(r["dq"]), _ptr(r["dk"]), _ptr(r["dv"]), _ptr(r["dalpha"]),
        _ptr(r["dbeta"]), _ptr(r["dstate_in"]), B, T, H, Dk, Dv, _dtype_code(q),
        float(scale), _ptr(workspace), wbytes, _stream(stream))
    _check("gdn_prefill_backward", st)
    return r
