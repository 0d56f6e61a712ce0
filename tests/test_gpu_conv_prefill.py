"""GPU parity of the fused projection adaptation, gdn_prefill_chunked_conv:
the causal short convolution + SiLU on the raw q, k, v projections and the
per-head L2 normalisation of q and k, done inside the prefill's tile loads
("The Key to Going Linear: Analysis-Driven Transformer Linearization",
section 4 "Adapting Q/K/V"; key normalisation of appendix B.1, "Metric 1").

The reference is the oracle chain with nothing rounded between its steps:
oracle.short_conv_silu in f64 on the raw bf16 projections, then
oracle.gdn_recurrence on those f64 results.  Cases: one pass per head, the
segment split (halo rows taken across segment boundaries), several
sequences, ragged lengths, sequences shorter than the convolution window,
T = 0, and the full Qwen-32B-shaped layer on every head.
"""
import pytest
import torch

import gated_delta_rule_115_amd as gdn
import oracle
import synthetic
from common import TOL, assert_bf16_is_rounded_f32, err, f64, say

pytestmark = pytest.mark.gpu
D = 128
EPS = 1e-6


def _inputs(B, T, H, seed, state0="zero"):
    g = synthetic.gdn_inputs(B, T, H, D, D, dtype="bf16", seed=seed, normalise_qk=False,
                             state0=state0, device="cuda")
    taps = {n: synthetic.conv_inputs(1, 1, H * D, 4, seed=seed * 10 + i, device="cuda")[1]
            for i, n in enumerate(("q", "k", "v"))}
    return g, taps


def _fused(g, taps, scale=1.0, out_dtype=torch.float32):
    return gdn.gdn_prefill_chunked_conv(g["q"], g["k"], g["v"], taps["q"], taps["k"], taps["v"],
                                        g["alpha"], g["beta"], g["state0"], conv_eps=EPS,
                                        scale=scale, out_dtype=out_dtype)


def _chain(g, taps, B, T, H, scale=1.0):
    qkv = {}
    for n, grp in (("q", D), ("k", D), ("v", 0)):
        qkv[n] = oracle.short_conv_silu(f64(g[n]).reshape(B, T, H * D), f64(taps[n]),
                                        l2norm_group=grp, eps=EPS).reshape(B, T, H, D)
    s0 = None if g["state0"] is None else f64(g["state0"])
    return oracle.gdn_recurrence(qkv["q"], qkv["k"], qkv["v"], f64(g["alpha"]),
                                 f64(g["beta"]), s0, scale=scale)


@pytest.mark.parametrize("B,T,H,segmented", [
    (2, 1000, 2, False), (1, 3000, 2, True), (2, 2500, 1, True), (1, 3001, 1, True),
    (3, 130, 2, False), (1, 65, 3, False), (2, 64, 1, False), (1, 63, 2, False),
    (1, 5, 2, False), (1, 1, 1, False), (1, 3, 1, False),
])
def test_fused_conv_prefill_matches_oracle_chain(B, T, H, segmented):
    say(f"fused conv prefill B={B} T={T} H={H}")
    assert (gdn.gdn_prefill_workspace_bytes(B, T, H, D, D, 64) > 0) == segmented
    g, taps = _inputs(B, T, H, seed=T + 7 * B + H, state0="randn")
    o, s = _fused(g, taps, scale=0.9)
    torch.cuda.synchronize()
    ro, rs = _chain(g, taps, B, T, H, scale=0.9)
    eo, es = err(o, ro), err(s, rs)
    say(f"  out {eo:.2e} state {es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    ob, sb = _fused(g, taps, scale=0.9, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_bf16_is_rounded_f32(ob, o)
    assert torch.equal(sb, s)


def test_fused_conv_prefill_empty_sequence_copies_state():
    g, taps = _inputs(2, 1, 2, seed=5, state0="randn")
    z = {n: g[n][:, :0].contiguous() for n in ("q", "k", "v", "alpha", "beta")}
    z["state0"] = g["state0"]
    o, s = _fused(z, taps)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 2, D)
    assert torch.equal(s, g["state0"])


def test_fused_conv_prefill_qwen32b_all_heads():
    """The Qwen-32B-shaped layer (B=2, T=16384, 40 heads of 128, conv kernel
    4): every element of the output and the final state of all 80 heads
    against the unrounded oracle chain."""
    c = synthetic.CONFIGS["qwen32b_conv"]
    B, T, H = c["B"], c["T"], c["H"]
    say(f"fused conv prefill qwen32b B={B} T={T} H={H}")
    g, taps = _inputs(B, T, H, seed=c["seed"])
    o, s = _fused(g, taps)
    torch.cuda.synchronize()
    ro, rs = _chain(g, taps, B, T, H)
    eo, es = err(o, ro), err(s, rs)
    say(f"  all {B * H} heads: out {eo:.3e} state {es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
