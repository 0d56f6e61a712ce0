"""GPU parity: GDN with a channel-wise gate G_t = diag(alpha_t) (section 3.2's
diagonal gates in the section 3.1.2 update of "The Key to Going Linear:
Analysis-Driven Transformer Linearization"), chunked prefill and decode step,
against the CPU oracle's channel-gate recurrence."""
import numpy as np
import pytest
import torch

import gated_delta_rule_115_amd as gdn
import oracle
import synthetic
from common import TOL, assert_bf16_is_rounded_f32, dev, err, f64, say

pytestmark = pytest.mark.gpu
NAMES = ("q", "k", "v", "alpha", "beta")


def _gpu(x, state_in=None, **kw):
    return gdn.gdn_prefill_chunked_chgate(*(dev(x[n]) for n in NAMES), dev(state_in), **kw)


def _ref(x, state_in=None, scale=1.0):
    return oracle.gdn_recurrence_chgate(*(f64(x[n]) for n in NAMES), f64(state_in), scale=scale)


# (dtype, B, T, H, Dk, Dv, gate_scale): a ragged tail (100 = 3 x 32 + 4), Dk != Dv both
# ways, T = 1, strong gates (per-channel log-gate ranges up to ~70 within a
# chunk: midpoint-factored Gram blocks) and very strong ones (ranges past 80:
# the exact per-element path); bf16 inputs (f16 MFMA operands in the
# recurrence) at every Dk and with 32- and 64-column value slices.
@pytest.mark.parametrize("dtype,B,T,H,Dk,Dv,gs", [
    ("f32", 2, 100, 2, 32, 32, 0.1), ("f32", 1, 64, 2, 64, 128, 0.1),
    ("f32", 1, 96, 2, 128, 32, 0.1), ("bf16", 2, 130, 3, 128, 128, 0.1),
    ("bf16", 1, 1, 2, 128, 64, 0.1), ("f32", 2, 70, 2, 64, 64, 2.0),
    ("bf16", 1, 200, 2, 128, 128, 2.0), ("f32", 1, 96, 2, 64, 64, 5.0),
    ("bf16", 2, 70, 2, 32, 32, 0.1), ("bf16", 1, 99, 2, 64, 128, 0.1),
    ("bf16", 1, 64, 2, 128, 32, 2.0),
    # Dk = 32 (one row per thread of the per-chunk pass) with strong and very
    # strong gates: the exact-range exchange and the per-element path
    ("f32", 1, 70, 2, 32, 32, 2.0), ("bf16", 1, 96, 2, 32, 64, 5.0),
    # bf16, Dk = Dv = 128: the tiled recurrence (one work-group per head) --
    # one token, one chunk plus one token, very strong gates (exact path)
    ("bf16", 2, 1, 2, 128, 128, 0.1), ("bf16", 1, 33, 3, 128, 128, 0.1),
    ("bf16", 1, 96, 2, 128, 128, 5.0)])
def test_chgate_prefill_matches_oracle(dtype, B, T, H, Dk, Dv, gs):
    say(f"chgate prefill {dtype} B{B} T{T} H{H} Dk{Dk} Dv{Dv} gate {gs}")
    x = synthetic.chgate_inputs(B, T, H, Dk, Dv, dtype=dtype, seed=T + Dk, state0="randn",
                                gate_scale=gs)
    o, s = _gpu(x, x["state0"], scale=0.5, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rs = _ref(x, x["state0"], scale=0.5)
    eo, es = err(o, ro), err(s, rs)
    say(f"  out err {eo:.2e}, state err {es:.2e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]
    if dtype == "bf16":
        ob, _ = _gpu(x, x["state0"], scale=0.5)
        torch.cuda.synchronize()
        assert_bf16_is_rounded_f32(ob.cpu(), o.cpu())


def test_chgate_equal_channels_matches_scalar_oracle():
    """A gate equal on every channel is the scalar gate alpha_t I."""
    x = synthetic.gdn_inputs(2, 90, 2, 64, 64, dtype="f32", seed=4, state0="randn")
    xc = dict(x, alpha=x["alpha"][..., None].expand(2, 90, 2, 64).contiguous())
    o, s = _gpu(xc, x["state0"])
    torch.cuda.synchronize()
    ro, rs = oracle.gdn_recurrence(*(f64(x[n]) for n in NAMES), f64(x["state0"]))
    assert err(o, ro) <= TOL["f32"] and err(s, rs) <= TOL["f32"]


def test_chgate_split_resume_and_aliasing():
    x = synthetic.chgate_inputs(1, 150, 2, 64, 64, dtype="f32", seed=11, state0="randn")
    a = {n: x[n][:, :70].contiguous() for n in NAMES}
    b = {n: x[n][:, 70:].contiguous() for n in NAMES}
    _, s1 = _gpu(a, x["state0"])
    st = s1.clone()
    o2, _ = gdn.gdn_prefill_chunked_chgate(*(dev(b[n]) for n in NAMES), st, state_out=st)
    torch.cuda.synchronize()
    ro, rs = _ref(x, x["state0"])
    assert err(o2, ro[:, 70:]) <= TOL["f32"] and err(st, rs) <= TOL["f32"]


@pytest.mark.parametrize("dtype,B,H,Dk,Dv", [("f32", 3, 2, 16, 32), ("f32", 2, 3, 128, 64),
                                             ("bf16", 4, 2, 128, 128), ("bf16", 2, 2, 32, 16)])
def test_chgate_decode_matches_oracle(dtype, B, H, Dk, Dv):
    x = synthetic.chgate_inputs(B, 1, H, Dk, Dv, dtype=dtype, seed=Dk + Dv, state0="randn")
    step = [dev(x[n][:, 0].contiguous()) for n in NAMES]
    s0 = dev(x["state0"])
    o, s1 = gdn.gdn_decode_step_chgate(*step, s0, out_dtype=torch.float32)
    st = s0.clone()
    o2, _ = gdn.gdn_decode_step_chgate(*step, st, state_out=st, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rs = oracle.decode_step_chgate(*(f64(x[n][:, 0]) for n in NAMES), f64(x["state0"]))
    assert err(o, ro) <= TOL[dtype] and err(s1, rs) <= TOL[dtype]
    assert torch.equal(o, o2) and torch.equal(s1, st)


def test_chgate_prefill_then_decode_steps():
    B, T, H, D = 2, 77, 2, 128
    x = synthetic.chgate_inputs(B, T + 3, H, D, D, dtype="bf16", seed=5)
    pre = {n: x[n][:, :T].contiguous() for n in NAMES}
    _, st = _gpu(pre)
    outs = []
    for t in range(T, T + 3):
        o, _ = gdn.gdn_decode_step_chgate(*(dev(x[n][:, t].contiguous()) for n in NAMES), st,
                                          state_out=st, out_dtype=torch.float32)
        outs.append(o)
    torch.cuda.synchronize()
    ro, rs = _ref(x)
    for i, o in enumerate(outs):
        assert err(o, ro[:, T + i]) <= TOL["bf16"]
    assert err(st, rs) <= TOL["bf16"]


def test_chgate_full_size_all_heads():
    """The channel-gate workload the bench times (B4 H32 T4096 d128, bf16):
    every head against the oracle, outputs and final state."""
    c = synthetic.CONFIGS["chgate_llama8b"]
    B, T, H, D = c["B"], c["T"], c["H"], c["Dk"]
    x = synthetic.chgate_inputs(B, T, H, D, D, dtype="bf16", seed=c["seed"], device="cuda")
    o, st = gdn.gdn_prefill_chunked_chgate(*(x[n] for n in NAMES), None,
                                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rs = oracle.gdn_recurrence_chgate(*(f64(x[n]) for n in NAMES))
    e, es = err(o, ro), err(st, rs)
    say(f"  all {B * H} heads: out err {e:.2e}, state err {es:.2e}")
    assert e <= TOL["bf16"] and es <= TOL["bf16"]
