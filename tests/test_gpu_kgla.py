"""GPU parity: gated linear attention with a key-dependent gate (kGLA;
"The Key to Going Linear: Analysis-Driven Transformer Linearization",
section 3.2.2), chunked prefill and decode step, against the oracle's kGLA
recurrence (itself pinned to the printed sum by brute force)."""
import pytest
import torch

import gated_delta_rule_115_amd as gdn
import oracle
import synthetic
from common import TOL, assert_bf16_is_rounded_f32, dev, err, f64, say

pytestmark = pytest.mark.gpu
NAMES = ("q", "k", "v", "alpha", "beta")


def _gpu(x, state_in=None, **kw):
    return gdn.gdn_prefill_chunked_kgla(*(dev(x[n]) for n in NAMES), dev(state_in), **kw)


def _ref(x, state_in=None, scale=1.0):
    return oracle.kgla(*(f64(x[n]) for n in NAMES), f64(state_in), scale=scale)


# (dtype, B, T, H, Dk, Dv, gate_scale, key_cos): ragged tails, Dk != Dv both
# ways, T = 1, 32- and 64-column value slices, strong gates (midpoint-factored
# Gram blocks) and very strong ones (per-element ratios), keys concentrated
# around one direction.
@pytest.mark.parametrize("dtype,B,T,H,Dk,Dv,gs,cos", [
    ("f32", 2, 100, 2, 32, 32, 0.1, None), ("f32", 1, 64, 2, 64, 128, 0.1, None),
    ("f32", 1, 96, 2, 128, 32, 0.1, None), ("bf16", 2, 130, 3, 128, 128, 0.1, None),
    ("bf16", 1, 1, 2, 128, 64, 0.1, None), ("f32", 2, 70, 2, 64, 64, 2.0, None),
    ("bf16", 1, 200, 2, 128, 128, 2.0, None), ("f32", 1, 96, 2, 64, 64, 5.0, None),
    ("f32", 1, 300, 2, 128, 64, 0.1, 0.97), ("bf16", 1, 300, 2, 128, 128, 0.1, 0.9),
    ("f32", 1, 70, 2, 32, 32, 2.0, None), ("bf16", 1, 96, 2, 32, 64, 5.0, None)])
def test_kgla_prefill_matches_oracle(dtype, B, T, H, Dk, Dv, gs, cos):
    say(f"kgla prefill {dtype} B{B} T{T} H{H} Dk{Dk} Dv{Dv} gate {gs} cos {cos}")
    x = synthetic.chgate_inputs(B, T, H, Dk, Dv, dtype=dtype, seed=T + Dk + 1, state0="randn",
                                gate_scale=gs, key_cos=cos)
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


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_kgla_prefill_then_decode_steps(dtype):
    """Prefill T tokens, then three decode steps in place: equal to the oracle
    over T + 3 tokens."""
    B, T, H, D = 2, 77, 3, 64
    x = synthetic.chgate_inputs(B, T + 3, H, D, D, dtype=dtype, seed=9, state0="randn")
    pre = {n: x[n][:, :T].contiguous() for n in NAMES}
    _, st = _gpu(pre, x["state0"])
    outs = []
    for t in range(T, T + 3):
        o, _ = gdn.gdn_decode_step_kgla(*(dev(x[n][:, t].contiguous()) for n in NAMES), st,
                                        state_out=st, out_dtype=torch.float32)
        outs.append(o)
    torch.cuda.synchronize()
    ro, rs = _ref(x, x["state0"])
    for i, o in enumerate(outs):
        assert err(o, ro[:, T + i]) <= TOL[dtype]
    assert err(st, rs) <= TOL[dtype]


def test_kgla_decode_step_batch():
    """The decode batch shape (B256 H32 d128), one step from a random state,
    every head against the oracle step."""
    B, H, D = 256, 32, 128
    x = synthetic.chgate_inputs(B, 1, H, D, D, dtype="bf16", seed=12, state0="randn",
                                device="cuda")
    step = {n: x[n][:, 0].contiguous() for n in NAMES}
    s0 = x["state0"]
    o, s1 = gdn.gdn_decode_step_kgla(*(step[n] for n in NAMES), s0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rs = oracle.kgla_step(*(f64(step[n]) for n in NAMES), f64(s0))
    eo, es = err(o, ro), err(s1, rs)
    say(f"kgla decode batch: out {eo:.2e} state {es:.2e}")
    assert eo <= TOL["f32"] and es <= TOL["f32"]


def test_kgla_full_size_all_heads():
    """The Llama-3-8B-shaped layer (B4 H32 T4096 d128, bf16) with the kGLA
    mixer: every head against the oracle, outputs and final state."""
    c = synthetic.CONFIGS["chgate_llama8b"]
    B, T, H, D = c["B"], c["T"], c["H"], c["Dk"]
    x = synthetic.chgate_inputs(B, T, H, D, D, dtype="bf16", seed=c["seed"] + 100, device="cuda")
    o, st = gdn.gdn_prefill_chunked_kgla(*(x[n] for n in NAMES), None, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rs = oracle.kgla(*(f64(x[n]) for n in NAMES))
    e, es = err(o, ro), err(st, rs)
    say(f"  kgla all {B * H} heads: out err {e:.2e}, state err {es:.2e}")
    assert e <= TOL["bf16"] and es <= TOL["bf16"]
