"""C-ABI contract on the CPU: the library loads, exports every function that
include/gdn.h declares, and rejects bad arguments on the host with the
documented status codes before anything touches a GPU.  No call here passes
validation with real work, so no kernel is launched."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_115_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")
OK, INVALID, UNSUPPORTED = 0, 1, 2
BF16, F32 = 0, 1
A = 4096  # a 16-byte-aligned fake address (never dereferenced: validation fails first)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 7
    L = gdn.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(gdn.EXPORTED_SYMBOLS)


def test_abi_version_matches_header():
    m = re.search(r"#define\s+GDN_ABI_VERSION\s+(\d+)", open(HEADER).read())
    assert gdn.gdn_abi_version() == int(m.group(1))


def _prefill(**kw):
    a = dict(q=A, k=A, v=A, alpha=A, beta=A, s_in=None, s_out=None, out=A, B=1, T=64,
             H=2, Dk=128, Dv=128, chunk=64, dt=BF16, odt=BF16, scale=1.0, ws=A,
             wsb=1 << 40)
    a.update(kw)
    return gdn.lib().gdn_prefill_chunked(
        a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["s_in"], a["s_out"], a["out"],
        a["B"], a["T"], a["H"], a["Dk"], a["Dv"], a["chunk"], a["dt"], a["odt"],
        a["scale"], a["ws"], a["wsb"], None)


def _err():
    return gdn.lib().gdn_last_error().decode()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(Dk=100), UNSUPPORTED, "head dims"),
    (dict(Dv=256), UNSUPPORTED, "head dims"),
    (dict(chunk=48), UNSUPPORTED, "chunk"),
    (dict(dt=7), INVALID, "dtype"),
    (dict(odt=5), INVALID, "out_dtype"),
    (dict(dt=F32, odt=BF16), UNSUPPORTED, "bf16 output"),
    (dict(B=-1), INVALID, "bad sizes"),
    (dict(H=0), INVALID, "bad sizes"),
    (dict(q=None), INVALID, "q is NULL"),
    (dict(out=None), INVALID, "out is NULL"),
    (dict(k=A + 2), INVALID, "aligned"),
    (dict(s_in=A + 4), INVALID, "aligned"),
    (dict(alpha=None), INVALID, "alpha"),
    # chunk 32 needs a workspace (chunk 64 with bf16, Dk = 128 needs none)
    (dict(chunk=32, ws=None), INVALID, "workspace is NULL"),
    (dict(chunk=32, ws=A + 16), INVALID, "256-byte"),
    (dict(chunk=32, wsb=100), INVALID, "too small"),
    (dict(dt=F32, odt=F32, ws=None), INVALID, "workspace is NULL"),
])
def test_prefill_validation(kw, code, msg):
    assert _prefill(**kw) == code
    assert msg in _err()


def test_prefill_empty_batch_is_ok_without_gpu():
    assert _prefill(B=0, q=None, k=None, v=None, out=None, ws=None) == OK
    assert _err() == ""


def test_workspace_bytes():
    f = gdn.gdn_prefill_workspace_bytes
    # bf16, Dk = Dv = 128, chunk 64: the per-head kernels in one pass, no workspace
    assert f(2, 65, 3, 128, 128, 64, BF16) == 0
    # bf16, Dk = 128, Dv < 128: the two-kernel form's per-chunk records
    for dv in (16, 32, 64):
        assert f(2, 65, 3, 128, dv, 64, BF16) == 2 * 3 * 2 * (2 * 64 * 64 * 2 + 256)
    # otherwise, per chunk: two C x C operand matrices + C f32 log gates,
    # padded to 256 B
    assert f(1, 64, 1, 128, 128, 32, BF16) == 2 * (2 * 32 * 32 * 2 + 256)
    assert f(2, 65, 3, 64, 128, 64, BF16) == 2 * 3 * 2 * (2 * 64 * 64 * 2 + 256)
    assert f(1, 64, 1, 128, 128, 64, F32) == 2 * 64 * 64 * 4 + 256
    assert f(1, 16, 1, 16, 16, 16, F32) == 2304
    assert f(1, 16, 1, 100, 16, 16, F32) == 0


def test_decode_validation():
    L = gdn.lib()
    call = lambda **kw: L.gdn_decode_step(
        kw.get("q", A), A, A, A, A, kw.get("s", A), A, A, kw.get("B", 2), 2,
        kw.get("Dk", 64), 64, kw.get("dt", BF16), kw.get("odt", BF16), 1.0, None)
    assert call(Dk=48) == UNSUPPORTED
    assert call(q=None) == INVALID and "q is NULL" in _err()
    assert call(s=A + 8) == INVALID and "aligned" in _err()
    assert call(dt=F32, odt=BF16) == UNSUPPORTED
    assert call(B=0, q=None) == OK


def test_prefill_conv_validation():
    """gdn_prefill_chunked_conv: argument checks only (nothing is launched)."""
    L = gdn.lib()

    def call(**kw):
        a = dict(x=A, taps=A, K=4, eps=1e-6, B=1, T=64, H=2, Dk=128, Dv=128, chunk=64,
                 dt=BF16, ws=A)
        a.update(kw)
        return L.gdn_prefill_chunked_conv(
            a["x"], A, A, a["taps"], A, A, a["K"], a["eps"], A, A, None, None, A, a["B"],
            a["T"], a["H"], a["Dk"], a["Dv"], a["chunk"], a["dt"], BF16, 1.0, a["ws"], 1 << 40,
            None)
    assert call(K=3) == UNSUPPORTED and "4 taps" in _err()
    assert call(Dk=64, Dv=64) == UNSUPPORTED and "Dk = Dv = 128" in _err()
    assert call(chunk=32) == UNSUPPORTED
    assert call(dt=F32) == UNSUPPORTED
    assert call(eps=-1.0) == INVALID and "conv_eps" in _err()
    assert call(taps=None) == INVALID and "taps" in _err()
    assert call(x=None) == INVALID and "is NULL" in _err()
    assert call(B=0, x=None, taps=None) == OK


def test_conv_validation():
    L = gdn.lib()
    call = lambda **kw: L.gdn_short_conv_silu(
        kw.get("x", A), A, kw.get("y", A + (1 << 30)), 1, kw.get("T", 10),
        kw.get("Ch", 256), kw.get("K", 4), kw.get("g", 0), 1e-6, BF16, BF16, None)
    assert call(K=9) == UNSUPPORTED
    assert call(Ch=12) == UNSUPPORTED
    assert call(g=24) == UNSUPPORTED
    assert call(g=512, Ch=256) == UNSUPPORTED
    assert call(y=A + 16) == INVALID and "overlaps" in _err()
    assert call(x=None) == INVALID
    assert call(T=0, x=None) == OK


def test_conv_step_validation():
    L = gdn.lib()
    call = lambda **kw: L.gdn_short_conv_step(
        kw.get("x", A), A, kw.get("s", A + (2 << 30)), kw.get("y", A + (1 << 30)),
        kw.get("B", 4), kw.get("Ch", 256), kw.get("K", 4), kw.get("g", 0), 1e-6, BF16,
        BF16, None)
    assert call(K=9) == UNSUPPORTED
    assert call(K=0) == UNSUPPORTED
    assert call(Ch=12) == UNSUPPORTED
    assert call(g=24) == UNSUPPORTED
    assert call(y=A + 16) == INVALID and "overlaps x" in _err()
    assert call(s=A + 16) == INVALID and "x overlaps conv_state" in _err()
    assert call(y=A + (2 << 30) + 64) == INVALID and "conv_state" in _err()
    assert call(s=None) == INVALID
    assert call(x=None) == INVALID
    assert call(B=-1) == INVALID
    assert call(B=0, x=None, s=None) == OK


def test_swa_validation():
    L = gdn.lib()
    call = lambda **kw: L.gdn_swa_sink_decode(
        A, kw.get("kn", None), kw.get("vn", None), A, A, kw.get("nt", A), 2, 2,
        kw.get("D", 128), kw.get("s", 4), kw.get("w", 8), 0.1, kw.get("acc", 0), A,
        BF16, BF16, None)
    assert call(D=96) == UNSUPPORTED
    assert call(w=0) == INVALID
    assert call(s=-1) == INVALID
    assert call(kn=A) == INVALID and "both" in _err()
    assert call(acc=2) == INVALID
    assert call(nt=None) == INVALID


def test_swa_prefill_validation():
    L = gdn.lib()
    call = lambda **kw: L.gdn_swa_sink_prefill(
        kw.get("q", A), A, A, A, kw.get("B", 2), kw.get("T", 64), 2, kw.get("D", 128),
        kw.get("s", 4), kw.get("w", 8), 0.1, 64, kw.get("dt", BF16), kw.get("odt", BF16), None)
    assert call(D=64) == UNSUPPORTED
    assert call(dt=F32, odt=F32) == UNSUPPORTED
    assert call(w=0) == INVALID
    assert call(s=-1) == INVALID
    assert call(q=None) == INVALID and "q" in _err()
    assert call(q=A + 8) == INVALID and "aligned" in _err()
    assert call(T=0, q=None) == OK
    assert L.gdn_swa_sink_prefill(A, A, A, A, 2, 64, 2, 128, 4, 8, -0.1, 64, BF16, BF16,
                                  None) == INVALID and "softmax_scale" in _err()


def test_swa_cache_fill_validation():
    L = gdn.lib()
    call = lambda **kw: L.gdn_swa_cache_fill(
        A, A, kw.get("kc", A), A, 2, kw.get("T", 64), 2, kw.get("D", 128), 4,
        kw.get("w", 8), kw.get("dt", BF16), None)
    assert call(D=96) == UNSUPPORTED
    assert call(w=0) == INVALID
    assert call(dt=3) == INVALID
    assert call(kc=None) == INVALID
    assert call(T=0, kc=None) == OK


def test_hybrid_prefill_validation():
    L = gdn.lib()
    ws = L.gdn_hybrid_prefill_workspace_bytes(4, 4096, 32, 128, 4, 512)
    assert ws > 0 and ws % 256 == 0
    assert L.gdn_hybrid_prefill_workspace_bytes(4, 4096, 32, 64, 4, 512) == 0
    assert L.gdn_hybrid_prefill_workspace_bytes(1, 500, 32, 128, 4, 512) == 0  # no linear set

    def call(**kw):
        a = dict(ql=A, al=A, qs=A, so=None, out=A, kc=None, vc=None, B=4, T=4096, H=32, D=128,
                 s=4, w=512, dt=BF16, odt=BF16, ws=A, wsb=ws)
        a.update(kw)
        return L.gdn_hybrid_prefill(a["ql"], A, A, a["al"], A, a["qs"], A, A, a["so"], a["out"],
                                    a["kc"], a["vc"], a["B"], a["T"], a["H"], a["D"], a["s"],
                                    a["w"], 1.0, 0.1, a["dt"], a["odt"], a["ws"], a["wsb"], None)
    assert call(D=64) == UNSUPPORTED
    assert call(dt=F32, odt=F32) == UNSUPPORTED
    assert call(w=0) == INVALID
    assert call(kc=A) == INVALID and "both" in _err()
    assert call(wsb=ws - 256) == INVALID and "workspace too small" in _err()
    assert call(ws=None) == INVALID and "workspace" in _err()
    assert call(ql=None) == INVALID and "q_lin" in _err()
    assert call(al=None) == INVALID and "alpha" in _err()
    assert call(qs=None) == INVALID and "q_swa" in _err()
    assert call(so=A + 4) == INVALID and "state_out" in _err()
    assert call(B=0, ql=None, qs=None, out=None) == OK


def test_chgate_validation():
    L = gdn.lib()
    ws = L.gdn_prefill_chgate_workspace_bytes(2, 100, 3)
    assert ws > 0 and ws % 256 == 0
    assert L.gdn_prefill_chgate_workspace_bytes(2, 0, 3) == 0

    def pre(**kw):
        a = dict(q=A, al=A, B=2, T=100, H=3, Dk=128, Dv=128, ws=A, wsb=ws, dt=BF16, odt=BF16)
        a.update(kw)
        return L.gdn_prefill_chunked_chgate(a["q"], A, A, a["al"], A, None, None, A, a["B"],
                                            a["T"], a["H"], a["Dk"], a["Dv"], a["dt"], a["odt"],
                                            1.0, a["ws"], a["wsb"], None)
    assert pre(Dk=16) == UNSUPPORTED
    assert pre(Dv=48) == UNSUPPORTED
    assert pre(wsb=ws - 256) == INVALID and "workspace too small" in _err()
    assert pre(ws=None) == INVALID
    assert pre(al=None) == INVALID
    assert pre(q=None) == INVALID
    assert pre(dt=F32, odt=BF16) == UNSUPPORTED
    assert pre(B=0, q=None) == OK

    def dec(**kw):
        a = dict(q=A, al=A, B=2, Dk=128)
        a.update(kw)
        return L.gdn_decode_step_chgate(a["q"], A, A, a["al"], A, A, A, A, a["B"], 3, a["Dk"],
                                        128, BF16, BF16, 1.0, None)
    assert dec(Dk=100) == UNSUPPORTED
    assert dec(al=None) == INVALID
    assert dec(q=None) == INVALID
    assert dec(B=0, q=None) == OK


def test_backward_validation():
    L = gdn.lib()
    ws = L.gdn_prefill_backward_workspace_bytes(2, 100, 3, 64, 64)
    # the state every 4 tokens per (b, h, 32-column slice), then per-slice
    # partials of dq, dk [B,T,H,Dk] and dalpha, dbeta [B,T,H]
    ns = 64 // 32
    assert ws == (2 * 3 * ns * 25 * 64 * 32 + ns * 2 * 100 * 3 * (2 * 64 + 2)) * 4
    assert L.gdn_prefill_backward_workspace_bytes(1, 10, 1, 16, 16) == 3 * 16 * 16 * 4
    assert L.gdn_prefill_backward_workspace_bytes(2, 100, 3, 100, 64) == 0

    def call(**kw):
        a = dict(q=A, ds=A, Dk=64, Dv=64, ws=A, wsb=ws, dt=F32, B=2)
        a.update(kw)
        return L.gdn_prefill_backward(a["q"], A, A, A, A, None, A, None, A, A, A, A, A, a["ds"],
                                      a["B"], 100, 3, a["Dk"], a["Dv"], a["dt"], 1.0, a["ws"],
                                      a["wsb"], None)
    assert call(Dk=96) == UNSUPPORTED
    assert call(dt=5) == INVALID
    assert call(wsb=ws - 1) == INVALID and "workspace too small" in _err()
    assert call(ws=None) == INVALID
    assert call(q=None) == INVALID
    assert call(ds=None) == INVALID
    assert call(B=0, q=None) == OK


def test_missing_library_raises(monkeypatch, tmp_path):
    monkeypatch.setattr(gdn, "_lib", None)
    monkeypatch.setattr(gdn, "library_path", str(tmp_path / "absent.so"))
    with pytest.raises(ImportError):
        gdn.lib()
