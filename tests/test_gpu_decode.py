"""GPU parity: gdn_decode_step against the oracle's recurrence at T = 1.

Passage: "The Key to Going Linear: Analysis-Driven Transformer
Linearization", section 3.1.2 (recurrent form).
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_115_amd as gdn
import oracle
import synthetic
from common import TOL, assert_bf16_is_rounded_f32, dev, err, f64, say

pytestmark = pytest.mark.gpu


def _inputs(B, H, Dk, Dv, dtype, seed):
    x = synthetic.gdn_inputs(B, 1, H, Dk, Dv, dtype=dtype, seed=seed, state0="randn")
    q, k, v = (x[n][:, 0].contiguous() for n in ("q", "k", "v"))
    a, b = (x[n][:, 0].contiguous() for n in ("alpha", "beta"))
    return q, k, v, a, b, x["state0"]


@pytest.mark.parametrize("dtype,B,H,Dk,Dv", [
    ("f32", 3, 2, 16, 16), ("f32", 2, 3, 32, 16), ("f32", 2, 2, 16, 64),
    ("f32", 2, 4, 128, 32), ("f32", 4, 8, 128, 128),
    ("bf16", 8, 4, 128, 128), ("bf16", 5, 3, 64, 32), ("bf16", 3, 2, 16, 128),
])
def test_decode_matches_oracle(dtype, B, H, Dk, Dv):
    say(f"decode dtype={dtype} B={B} H={H} Dk={Dk} Dv={Dv}")
    q, k, v, a, b, s0 = _inputs(B, H, Dk, Dv, dtype, seed=B * 100 + Dk + Dv)
    scale = 0.7
    args = [dev(t) for t in (q, k, v, a, b, s0)]
    o, s = gdn.gdn_decode_step(*args, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rs = oracle.decode_step(f64(q), f64(k), f64(v), f64(a), f64(b), f64(s0), scale=scale)
    assert err(o, ro) <= TOL[dtype]
    assert err(s, rs) <= TOL[dtype]
    if dtype == "bf16":
        ob, sb = gdn.gdn_decode_step(*args, scale=scale)
        torch.cuda.synchronize()
        assert_bf16_is_rounded_f32(ob, o)
        assert torch.equal(sb, s)


def test_decode_in_place_equals_out_of_place():
    q, k, v, a, b, s0 = _inputs(4, 4, 128, 128, "bf16", seed=7)
    args = [dev(t) for t in (q, k, v, a, b)]
    s_in = dev(s0)
    o1, s1 = gdn.gdn_decode_step(*args, s_in.clone())
    s_inplace = s_in.clone()
    o2, s2 = gdn.gdn_decode_step(*args, s_inplace, state_out=s_inplace)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2) and s2 is s_inplace


def test_decode_full_batch_256x32():
    """Full decode batch (256 sequences, 32 heads, d = 128, bf16 I/O, f32 state)."""
    say("decode full 256x32x128")
    q, k, v, a, b, s0 = _inputs(256, 32, 128, 128, "bf16", seed=5)
    args = [dev(t) for t in (q, k, v, a, b, s0)]
    o, s = gdn.gdn_decode_step(*args, out_dtype=torch.float32)
    ob, _ = gdn.gdn_decode_step(*args)
    torch.cuda.synchronize()
    assert_bf16_is_rounded_f32(ob, o)
    ro, rs = oracle.decode_step(f64(q), f64(k), f64(v), f64(a), f64(b), f64(s0))
    assert err(o, ro) <= TOL["bf16"]
    assert err(s, rs) <= TOL["bf16"]


def test_decode_empty_batch_is_noop():
    z = torch.empty((0, 2, 16), device="cuda")
    s = torch.empty((0, 2, 16, 16), device="cuda")
    o, s2 = gdn.gdn_decode_step(z, z, z, torch.empty((0, 2), device="cuda"),
                                torch.empty((0, 2), device="cuda"), s)
    assert o.shape == (0, 2, 16)


def test_decode_beta_zero_is_pure_decay_and_readout():
    """beta = 0: S' = alpha S and out = alpha S^T q exactly as the oracle."""
    q, k, v, a, b, s0 = _inputs(2, 3, 32, 32, "f32", seed=11)
    b = torch.zeros_like(b)
    o, s = gdn.gdn_decode_step(dev(q), dev(k), dev(v), dev(a), dev(b), dev(s0))
    torch.cuda.synchronize()
    ro, rs = oracle.decode_step(f64(q), f64(k), f64(v), f64(a), f64(b), f64(s0))
    assert err(s, rs) <= 1e-6 and err(o, ro) <= 1e-5
