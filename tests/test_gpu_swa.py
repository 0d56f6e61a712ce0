"""GPU parity: the sink + sliding-window softmax decode step and the hybrid
(disjoint linear + softmax) decode step ("The Key to Going Linear:
Analysis-Driven Transformer Linearization", section 4, "Adding Sliding Window
Attention").

The KV cache is filled from a token history with the slot rule the C header
documents (sinks in slots 0..s-1, later positions p in slot s + (p-s) % w);
slots that hold no attended token are filled with junk first, so a kernel
reading the wrong slots fails.  The oracle sees only the token history.
"""
import math

import numpy as np
import pytest
import torch

import gated_delta_rule_115_amd as gdn
import oracle
import synthetic
from common import TOL, assert_bf16_is_rounded_f32, dev, err, f64, say

pytestmark = pytest.mark.gpu


def slot_of(p, s, w):
    return p if p < s else s + (p - s) % w


def build_cache(k_hist, v_hist, n_tok, s, w, upto_exclusive_last, seed):
    """Cache [B,H,s+w,D] holding positions 0..n_tok[b]-1 (or -2 when the last
    token is passed as k_new), over junk."""
    B, T, H, D = k_hist.shape
    g = torch.Generator().manual_seed(seed)
    kc = (torch.randn(B, H, s + w, D, generator=g) * 3).to(k_hist.dtype)
    vc = (torch.randn(B, H, s + w, D, generator=g) * 3).to(v_hist.dtype)
    for b in range(B):
        last = n_tok[b] - (1 if upto_exclusive_last else 0)
        for p in range(last):
            kc[b, :, slot_of(p, s, w)] = k_hist[b, p]
            vc[b, :, slot_of(p, s, w)] = v_hist[b, p]
    return kc.contiguous(), vc.contiguous()


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 128), ("bf16", 64), ("f32", 128)])
@pytest.mark.parametrize("use_new", [False, True])
def test_swa_decode_matches_oracle(dtype, D, use_new):
    s, w, H = 4, 8, 3
    n_tok = [1, 3, 4, 5, 11, 12, 13, 40]
    B, T = len(n_tok), max(n_tok)
    say(f"swa {dtype} D={D} new={use_new}")
    g = torch.Generator().manual_seed(D + (7 if use_new else 0))
    dt = synthetic.TORCH_DTYPE[dtype]
    qh, kh, vh = (torch.randn(B, T, H, D, generator=g).to(dt) for _ in range(3))
    kc, vc = build_cache(kh, vh, n_tok, s, w, use_new, seed=5)
    q = torch.stack([qh[b, n_tok[b] - 1] for b in range(B)]).contiguous()
    kn = torch.stack([kh[b, n_tok[b] - 1] for b in range(B)]).contiguous() if use_new else None
    vn = torch.stack([vh[b, n_tok[b] - 1] for b in range(B)]).contiguous() if use_new else None
    nt = torch.tensor(n_tok, dtype=torch.int32)
    kcd, vcd = dev(kc), dev(vc)
    y = gdn.gdn_swa_sink_decode(dev(q), kcd, vcd, dev(nt), n_sink=s, window=w,
                                k_new=dev(kn), v_new=dev(vn), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = np.stack([oracle.swa_sink_attention(f64(qh[b:b + 1, :n_tok[b]]),
                                              f64(kh[b:b + 1, :n_tok[b]]),
                                              f64(vh[b:b + 1, :n_tok[b]]), s, w,
                                              1 / math.sqrt(D), last_only=True)[0]
                    for b in range(B)])
    assert err(y, ref) <= TOL[dtype]
    if use_new:  # the current token now sits in its slot
        for b in range(B):
            sl = slot_of(n_tok[b] - 1, s, w)
            assert torch.equal(kcd[b, :, sl].cpu(), kn[b]) and torch.equal(vcd[b, :, sl].cpu(), vn[b])
    # accumulate=1 adds into an existing output
    base = torch.randn(B, H, D, generator=g).to(torch.float32)
    acc = dev(base.clone())
    gdn.gdn_swa_sink_decode(dev(q), kcd, vcd, dev(nt), n_sink=s, window=w,
                            accumulate=True, out=acc)
    torch.cuda.synchronize()
    assert err(acc, ref + f64(base)) <= TOL[dtype]
    if dtype == "bf16":
        yb = gdn.gdn_swa_sink_decode(dev(q), kcd, vcd, dev(nt), n_sink=s, window=w)
        y2 = gdn.gdn_swa_sink_decode(dev(q), kcd, vcd, dev(nt), n_sink=s, window=w,
                                     out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert_bf16_is_rounded_f32(yb, y2)


def test_swa_full_batch_256x32_window512_sinks4():
    """Full decode batch: B=256, H=32, d=128, 4 sinks + 512-token window, bf16
    cache, 4096-token context (every slot attended)."""
    B, H, D, s, w = 256, 32, 128, 4, 512
    t = 4097
    say("swa full 256x32, 516 slots")
    q, kc, vc = synthetic.swa_inputs(B, H, D, s + w, dtype="bf16", seed=5, device="cuda")
    kn, vn = (x[:, :, 0].contiguous() for x in synthetic.swa_inputs(B, H, D, 1, seed=6,
                                                                     device="cuda")[1:])
    nt = torch.full((B,), t, dtype=torch.int32, device="cuda")
    y = gdn.gdn_swa_sink_decode(q, kc, vc, nt, n_sink=s, window=w, k_new=kn, v_new=vn,
                                out_dtype=torch.float32)
    torch.cuda.synchronize()
    cur = slot_of(t - 1, s, w)
    assert torch.equal(kc[:, :, cur], kn)
    e = _swa_all_heads_err(q, kc, vc, y, s, w)
    say(f"  all {B * H} heads: err {e:.3e}")
    assert e <= TOL["bf16"]


def _swa_all_heads_err(q, kc, vc, y, s, w, group=512):
    """Max error / RMS of y [B,H,D] against the oracle's softmax over every
    (b, h)'s cache, taken as a sequence of its s + w attended tokens with the
    query at the last position (the order of the window's keys does not
    change the softmax), in groups of `group` heads."""
    B, H, D = q.shape
    n = s + w
    qf, kf, vf = (t.reshape(B * H, *t.shape[2:]) for t in (q, kc, vc))
    ref = np.zeros((B * H, D))
    for g0 in range(0, B * H, group):
        g1 = min(B * H, g0 + group)
        ks = f64(kf[g0:g1]).transpose(1, 0, 2)[None]    # [1, n, heads, D]
        vs = f64(vf[g0:g1]).transpose(1, 0, 2)[None]
        qs = np.zeros_like(ks)
        qs[0, n - 1] = f64(qf[g0:g1])
        ref[g0:g1] = oracle.swa_sink_attention(qs, ks, vs, s, w, 1 / math.sqrt(D),
                                               last_only=True)[0]
    return oracle.rms_normalised_max_error(f64(y).reshape(B * H, D), ref)


# ---------------------------------------------------------------------------
# Hybrid decode step: GDN step on the token leaving the window + softmax over
# sinks and window, summed (section 4).  The linear state before the step is
# produced by the GPU prefill over tokens s .. P-w-1.
# ---------------------------------------------------------------------------
def _hybrid_step_gpu(lin, sm, P, s, w, dtype):
    """lin: dict of linear-path tensors [B,T,H,D]; sm: softmax q/k/v [B,T,H,D]."""
    B, T, H, D = lin["q"].shape
    n_lin = max(0, P - w - s)  # tokens s .. P-w-1
    st = torch.zeros(B, H, D, D, device="cuda")
    if n_lin > 0:
        part = {n: dev(lin[n][:, s:s + n_lin].contiguous()) for n in lin}
        gdn.gdn_prefill_chunked(part["q"], part["k"], part["v"], part["alpha"],
                                part["beta"], st, state_out=st, chunk=64,
                                out_dtype=torch.float32)
    j = P - w
    qP = dev(lin["q"][:, P].contiguous())
    if j >= s:
        kj, vj = dev(lin["k"][:, j].contiguous()), dev(lin["v"][:, j].contiguous())
        aj, bj = dev(lin["alpha"][:, j].contiguous()), dev(lin["beta"][:, j].contiguous())
    else:  # nothing leaves the window yet: identity token, read only
        kj, vj = torch.zeros_like(qP), torch.zeros_like(qP)
        aj, bj = torch.ones(B, H, device="cuda"), torch.zeros(B, H, device="cuda")
    o, _ = gdn.gdn_decode_step(qP, kj, vj, aj, bj, st, state_out=st,
                               out_dtype=torch.float32)
    n_tok = [P + 1] * B
    kc, vc = build_cache(sm["k"], sm["v"], n_tok, s, w, True, seed=P)
    gdn.gdn_swa_sink_decode(dev(sm["q"][:, P].contiguous()), dev(kc), dev(vc),
                            dev(torch.tensor(n_tok, dtype=torch.int32)), n_sink=s,
                            window=w, k_new=dev(sm["k"][:, P].contiguous()),
                            v_new=dev(sm["v"][:, P].contiguous()), accumulate=True, out=o)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hybrid_decode_step_matches_oracle(dtype):
    B, T, H, D, s, w = 2, 90, 2, 64, 4, 8
    lin = synthetic.gdn_inputs(B, T, H, D, D, dtype=dtype, seed=31)
    lin.pop("state0")
    sq, sk, sv = (synthetic.gdn_inputs(B, T, H, D, D, dtype=dtype, seed=40 + i,
                                       normalise_qk=False)["v"] for i in range(3))
    sm = {"q": sq, "k": sk, "v": sv}
    ref = oracle.hybrid(*(f64(lin[n]) for n in ("q", "k", "v", "alpha", "beta")),
                        f64(sq), f64(sk), f64(sv), s, w)
    for P in (0, 3, 5, 11, 12, 13, 40, 89):
        say(f"hybrid {dtype} P={P}")
        o = _hybrid_step_gpu(lin, sm, P, s, w, dtype)
        assert err(o, ref[:, P]) <= TOL[dtype], P


def test_hybrid_full_decode_batch_all_heads():
    """Full hybrid decode step: B=256, H=32, d=128, 4096-token context, 4 sinks,
    512-token window.  The state entering the step comes from the GPU prefill
    of tokens 4..3583; the step inserts token 3584 and reads with q_4096.

    Every head of the step is checked: the oracle's decode step starts from
    the same state buffer (read back before the step) and its softmax runs
    over each head's cache.  The state buffer itself is checked against the
    oracle's recurrence over the 3,580 linear tokens on 16 sampled heads (a
    full oracle prefill of 8,192 heads is ~2.4e12 multiply-adds)."""
    B, H, D, s, w = 256, 32, 128, 4, 512
    P = 4096
    n_lin = P - w - s           # 3580 tokens in the state before the step
    T_lin = P - w + 1           # linear-path tokens 0..3584
    say("hybrid full-size: prefill 256x3580x32 then one step")
    names = ("q", "k", "v", "alpha", "beta")
    lin = synthetic.gdn_inputs(B, T_lin, H, D, D, dtype="bf16", seed=5, device="cuda")
    q_lin = synthetic.gdn_inputs(B, 1, H, D, D, dtype="bf16", seed=55, device="cuda")["q"][:, 0]
    st = torch.zeros(B, H, D, D, device="cuda")
    gdn.gdn_prefill_chunked(*(lin[n][:, s:s + n_lin].contiguous() for n in names),
                            st, state_out=st, chunk=64, want_state=True)
    torch.cuda.synchronize()
    st_before = f64(st)
    j = P - w
    step_in = [q_lin.contiguous()] + [lin[n][:, j].contiguous() for n in names[1:]]
    o, _ = gdn.gdn_decode_step(*step_in, st, state_out=st, out_dtype=torch.float32)
    qs, kc, vc = synthetic.swa_inputs(B, H, D, s + w, dtype="bf16", seed=56, device="cuda")
    nt = torch.full((B,), P + 1, dtype=torch.int32, device="cuda")
    y = gdn.gdn_swa_sink_decode(qs, kc, vc, nt, n_sink=s, window=w, out_dtype=torch.float32)
    gdn.gdn_swa_sink_decode(qs, kc, vc, nt, n_sink=s, window=w, accumulate=True, out=o)
    torch.cuda.synchronize()
    # every head: oracle step from the same state + oracle softmax over the cache
    ro, rs = oracle.decode_step(*(f64(t) for t in step_in), st_before)
    e_state = oracle.rms_normalised_max_error(f64(st), rs)
    e_swa = _swa_all_heads_err(qs, kc, vc, y, s, w)
    e_lin = oracle.rms_normalised_max_error(f64(o) - f64(y), ro)
    say(f"  all {B * H} heads: step state {e_state:.2e}, linear read {e_lin:.2e}, "
        f"softmax {e_swa:.2e}")
    assert e_state <= TOL["bf16"] and e_lin <= TOL["bf16"] and e_swa <= TOL["bf16"]
    # the summed output against the oracle's two paths
    ref_sum = ro + (f64(y))  # y itself is checked above against the oracle
    assert oracle.rms_normalised_max_error(f64(o), ref_sum) <= TOL["bf16"]
    # the state entering the step, sampled heads against the oracle prefill
    rng = np.random.default_rng(3)
    picks = rng.choice(B * H, size=16, replace=False)
    bs, hs = picks // H, picks % H
    gsel = lambda t: torch.stack([t[b, s:s + n_lin, h] for b, h in zip(bs, hs)], dim=1)[None]
    _, rs0 = oracle.gdn_recurrence(*(f64(gsel(lin[n])) for n in names))
    got0 = np.stack([st_before[b, h] for b, h in zip(bs, hs)])[None]
    e0 = oracle.rms_normalised_max_error(got0, rs0)
    say(f"  prefilled state, 16 sampled heads: {e0:.2e}")
    assert e0 <= TOL["bf16"]
