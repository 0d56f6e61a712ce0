"""CPU oracle for the Gated DeltaNet token mixer (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this module.  The GPU library never imports, links or calls it,
and this module imports nothing from the GPU library.

The arithmetic lives in ``gdn_oracle.c`` (plain C, double precision, OpenMP
over independent (batch, head) pairs); this file only compiles it with gcc and
marshals numpy arrays.  Every function takes and returns float64 arrays in the
layouts documented in the C file:

    q, k [B, T, H, Dk]    v, out [B, T, H, Dv]    alpha, beta [B, T, H]
    state [B, H, Dk, Dv]

Sources followed ("The Key to Going Linear: Analysis-Driven Transformer
Linearization"): section 3.1.2 (GDN update and read-out), section 3.2.2
(gated linear attention with a key-dependent gate), section 3.1
(softmax), section 4 (disjoint sliding window + sinks; short convolutions),
appendix B.1 (key normalisation), appendix B.1 "Approximation error" (nMSE).

Pins (tests/test_oracle.py): every function here is checked against closed
forms, invariants, library routines or brute force; see the test file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)


def build(force: bool = False) -> str:
    """Compile gdn_oracle.c into liboracle.so next to it (gcc -O2 -fopenmp)."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC",
                               "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        i = ctypes.c_int
        d = ctypes.c_double
        lib.gdn_oracle_recurrence_f64.argtypes = [_dp] * 8 + [i] * 5 + [d, i]
        lib.gdn_oracle_recurrence_f32.argtypes = [_dp] * 8 + [i] * 5 + [d, i]
        lib.gdn_oracle_swa_sink_f64.argtypes = [_dp] * 4 + [i] * 6 + [d, i]
        lib.gdn_oracle_recurrence_chgate_f64.argtypes = [_dp] * 8 + [i] * 5 + [d, i]
        lib.gdn_oracle_recurrence_bwd_f64.argtypes = [_dp] * 14 + [i] * 5 + [d]
        lib.gdn_oracle_kgla_f64.argtypes = [_dp] * 8 + [i] * 5 + [d]
        lib.gdn_oracle_hybrid_f64.argtypes = [_dp] * 9 + [i] * 7 + [d, d]
        lib.gdn_oracle_short_conv_silu_f64.argtypes = [_dp] * 3 + [i] * 5 + [d]
        lib.gdn_oracle_short_conv_step_f64.argtypes = [_dp] * 5 + [i] * 4 + [d]
        lib.gdn_oracle_num_threads.restype = i
        _lib = lib
    return _lib


def _arr(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def num_threads() -> int:
    """OpenMP threads the oracle runs with (OMP_NUM_THREADS or all cores)."""
    return _load().gdn_oracle_num_threads()


def gdn_recurrence(q, k, v, alpha, beta, state_in=None, scale=1.0,
                   erase=True, precision="f64"):
    """Token-by-token GDN (section 3.1.2).  Returns (out [B,T,H,Dv], S_T).

    erase=False removes the (I - beta k k^T) factor: test hook for the
    gated-accumulation (GLA) special case.  precision="f32" rounds every
    operation to float (used only to bound the oracle's own rounding).
    """
    q, k, v, alpha, beta = map(_arr, (q, k, v, alpha, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, T, H)
    assert alpha.shape == (B, T, H) and beta.shape == (B, T, H)
    s_in = None if state_in is None else _arr(state_in)
    if s_in is not None:
        assert s_in.shape == (B, H, Dk, Dv)
    out = np.zeros((B, T, H, Dv))
    s_out = np.zeros((B, H, Dk, Dv))
    fn = {"f64": _load().gdn_oracle_recurrence_f64,
          "f32": _load().gdn_oracle_recurrence_f32}[precision]
    fn(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(s_in),
       _ptr(s_out), _ptr(out), B, T, H, Dk, Dv, float(scale), int(bool(erase)))
    return out, s_out


def decode_step(q, k, v, alpha, beta, state_in, scale=1.0):
    """One recurrence step per (b, h): q, k [B,H,Dk], v [B,H,Dv], gates [B,H].

    This is the recurrence at T = 1 ([B,1,H,D] and [B,H,D] are the same
    memory).  Returns (out [B,H,Dv], S' [B,H,Dk,Dv]).
    """
    q, k, v = (_arr(x)[:, None] for x in (q, k, v))
    a, b = (_arr(x)[:, None] for x in (alpha, beta))
    out, s = gdn_recurrence(q, k, v, a, b, state_in, scale)
    return out[:, 0], s


def gdn_recurrence_backward(q, k, v, alpha, beta, dout, state_in=None, dstate_out=None,
                            scale=1.0):
    """Gradients of gdn_recurrence (section 3.1.2, scalar gate) by the adjoint
    of the token loop.  dout [B,T,H,Dv], dstate_out [B,H,Dk,Dv] or None.
    Returns dict dq, dk, dv, dalpha, dbeta, dstate_in."""
    q, k, v, alpha, beta, dout = map(_arr, (q, k, v, alpha, beta, dout))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    s_in = None if state_in is None else _arr(state_in)
    ds = None if dstate_out is None else _arr(dstate_out)
    r = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
             dalpha=np.zeros_like(alpha), dbeta=np.zeros_like(beta),
             dstate_in=np.zeros((B, H, Dk, Dv)))
    _load().gdn_oracle_recurrence_bwd_f64(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(s_in), _ptr(dout), _ptr(ds),
        _ptr(r["dq"]), _ptr(r["dk"]), _ptr(r["dv"]), _ptr(r["dalpha"]), _ptr(r["dbeta"]),
        _ptr(r["dstate_in"]), B, T, H, Dk, Dv, float(scale))
    return r


def gdn_recurrence_chgate(q, k, v, alpha, beta, state_in=None, scale=1.0, gate_first=True):
    """GDN with a channel-wise gate G_t = diag(alpha_t) (section 3.2's diag
    gates in the section 3.1.2 update), alpha [B,T,H,Dk].  Returns (out, S_T).

    gate_first=False applies the erase before the gate: a test hook that shows
    the order matters once the gate is not a multiple of I.
    """
    q, k, v, alpha, beta = map(_arr, (q, k, v, alpha, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == q.shape and alpha.shape == q.shape and beta.shape == (B, T, H)
    s_in = None if state_in is None else _arr(state_in)
    out = np.zeros((B, T, H, Dv))
    s_out = np.zeros((B, H, Dk, Dv))
    _load().gdn_oracle_recurrence_chgate_f64(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(s_in), _ptr(s_out),
        _ptr(out), B, T, H, Dk, Dv, float(scale), int(bool(gate_first)))
    return out, s_out


def decode_step_chgate(q, k, v, alpha, beta, state_in, scale=1.0):
    """One channel-gated step per (b, h): q, k, alpha [B,H,Dk], v [B,H,Dv],
    beta [B,H].  Returns (out [B,H,Dv], S')."""
    q, k, v, a = (_arr(x)[:, None] for x in (q, k, v, alpha))
    b = _arr(beta)[:, None]
    out, s = gdn_recurrence_chgate(q, k, v, a, b, state_in, scale)
    return out[:, 0], s


def kgla(q, k, v, alpha, beta, state_in=None, scale=1.0):
    """Gated linear attention with a key-dependent gate (section 3.2.2):
    per-channel gate alpha_t o (1 - beta_t k_t o k_t), write k_t v_t^T, read
    after the write.  q, k, alpha [B,T,H,Dk], v [B,T,H,Dv], beta [B,T,H].
    Returns (out [B,T,H,Dv], S_T [B,H,Dk,Dv])."""
    q, k, v, alpha, beta = map(_arr, (q, k, v, alpha, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == q.shape and alpha.shape == q.shape and beta.shape == (B, T, H)
    s_in = None if state_in is None else _arr(state_in)
    out = np.zeros((B, T, H, Dv))
    s_out = np.zeros((B, H, Dk, Dv))
    _load().gdn_oracle_kgla_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                _ptr(s_in), _ptr(s_out), _ptr(out), B, T, H, Dk, Dv,
                                float(scale))
    return out, s_out


def kgla_step(q, k, v, alpha, beta, state_in, scale=1.0):
    """One kGLA step per (b, h): q, k, alpha [B,H,Dk], v [B,H,Dv], beta [B,H]."""
    q, k, v, a = (_arr(x)[:, None] for x in (q, k, v, alpha))
    b = _arr(beta)[:, None]
    out, s = kgla(q, k, v, a, b, state_in, scale)
    return out[:, 0], s


def swa_sink_attention(q, k, v, n_sink, window, softmax_scale, last_only=False):
    """Softmax over sinks {0..s-1} and window {t-w+1..t} at every t.

    q, k, v [B,T,H,D] -> [B,T,H,D] (section 3.1 softmax on section 4's set I).
    last_only=True computes only position T-1 (a decode step) and returns
    [B,H,D].
    """
    q, k, v = map(_arr, (q, k, v))
    B, T, H, D = q.shape
    out = np.zeros((B, T, H, D))
    t_begin = T - 1 if last_only else 0
    _load().gdn_oracle_swa_sink_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                    B, T, H, D, int(n_sink), int(window),
                                    float(softmax_scale), int(t_begin))
    return out[:, -1] if last_only else out


def hybrid(ql, kl, vl, alpha, beta, qs, ks, vs, n_sink, window,
           lin_scale=1.0, softmax_scale=None):
    """Disjoint linear + sink/window softmax layer output (section 4).

    y_t = lin_scale * S_lin(t)^T ql_t + softmax over I_t with (qs, ks, vs),
    where S_lin(t) holds tokens {n_sink .. t-window} (0-based).
    """
    ql, kl, vl, alpha, beta, qs, ks, vs = map(
        _arr, (ql, kl, vl, alpha, beta, qs, ks, vs))
    B, T, H, Dk = ql.shape
    Dv = vl.shape[-1]
    assert qs.shape == (B, T, H, Dv) and ks.shape == qs.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(Dv)
    out = np.zeros((B, T, H, Dv))
    _load().gdn_oracle_hybrid_f64(_ptr(ql), _ptr(kl), _ptr(vl), _ptr(alpha),
                                  _ptr(beta), _ptr(qs), _ptr(ks), _ptr(vs),
                                  _ptr(out), B, T, H, Dk, Dv, int(n_sink),
                                  int(window), float(lin_scale),
                                  float(softmax_scale))
    return out


def short_conv_silu(x, taps, l2norm_group=0, eps=1e-6):
    """Causal depthwise conv (taps[c, K-1] on the current token) + SiLU.

    x [B,T,Ch], taps [Ch,K] -> [B,T,Ch]; optional per-group L2 normalisation.
    """
    x, taps = _arr(x), _arr(taps)
    B, T, Ch = x.shape
    K = taps.shape[1]
    assert taps.shape == (Ch, K)
    y = np.zeros_like(x)
    _load().gdn_oracle_short_conv_silu_f64(_ptr(x), _ptr(taps), _ptr(y), B, T,
                                           Ch, K, int(l2norm_group), float(eps))
    return y


def short_conv_step(x, taps, state, l2norm_group=0, eps=1e-6):
    """One decode step of short_conv_silu from the previous K-1 inputs.

    x [B,Ch], taps [Ch,K], state [B,K-1,Ch] (oldest row first) ->
    (y [B,Ch], new state [B,K-1,Ch] = previous rows 1.. followed by x).
    """
    x, taps, state = _arr(x), _arr(taps), _arr(state)
    B, Ch = x.shape
    K = taps.shape[1]
    assert taps.shape == (Ch, K) and state.shape == (B, K - 1, Ch)
    y = np.zeros_like(x)
    new_state = np.zeros_like(state)
    _load().gdn_oracle_short_conv_step_f64(_ptr(x), _ptr(taps), _ptr(state),
                                           _ptr(new_state), _ptr(y), B, Ch, K,
                                           int(l2norm_group), float(eps))
    return y, new_state


def rms_normalised_max_error(got, ref) -> float:
    """max |got - ref| / RMS(ref) over the whole tensor (the parity statistic)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-300)


def nmse(got, ref) -> float:
    """Normalised MSE of appendix B.1: mean((got-ref)^2) / Var(ref)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.mean((got - ref) ** 2) / max(np.var(ref), 1e-300))
