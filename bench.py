#!/usr/bin/env python3
"""Benchmark of the GDN token mixer on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  leg "prefill_long32k": gdn_prefill_chunked on B=1, H=32, T=32768, d=128,
                         bf16 q/k/v/out, f32 gates and state, chunk 64
                         (512 sequential chunks per head; final state written)
  leg "decode_b256":     the hybrid decode step on B=256, H=32, d=128:
                         gdn_decode_step (in place, on the token leaving the
                         512-token window) + gdn_swa_sink_decode (4 sinks +
                         512 window slots, bf16 KV, writes the new token,
                         adds into the same output); the f32 state comes from
                         a GPU prefill of the 4096-token context (set-up)
  leg "hybrid_prefill":  the hybrid layer over whole sequences, B=4, H=32,
                         T=4096, d=128, 4 sinks + 512 window, bf16:
                         gdn_hybrid_prefill (linear state over the tokens
                         outside sinks and window, read with q shifted by the
                         window; sink/window softmax added; decode caches and
                         final state written)
  leg "chgate_llama8b":  GDN with a channel-wise gate diag(alpha_t), B=4, H=32,
                         T=4096, d=128, bf16 in/out, f32 gates [B,T,H,128]:
                         gdn_prefill_chunked_chgate (chunks of 32, f32)
  leg "backward_t1024":  gradients of the scalar-gate prefill (dq, dk, dv,
                         dalpha, dbeta, dS0) for B=4, H=32, T=1024, d=128,
                         bf16 inputs, f32 gradients: gdn_prefill_backward
                         (chunked reverse mode, f32 MFMA)
  leg "conv_qwen32b":    Qwen-32B-shaped layer with projection adaptation,
                         B=2, H=40, T=16384: gdn_prefill_chunked_conv (short
                         convolution + SiLU on the raw q, k, v and the L2 norm
                         of q, k inside the prefill kernels' tile loads)
  leg "conv_qwen32b_twocall": the same layer as separate calls:
                         gdn_short_conv_silu on q, k, v (bf16 results in HBM),
                         then gdn_prefill_chunked

The headline value is the prefill leg's throughput in tokens/s (B*T per call,
all heads), with the decode leg's tokens/s (B per step) reported beside it.
Inputs are resident in HBM before timing starts; every leg is timed with HIP
events on the stream the kernels run on (torch's current stream).  The CPU
oracle (plain C, f64) is timed on a bounded sample of the same workloads on
this host's cores as a reported baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

import gated_delta_rule_115_amd as gdn  # noqa: E402
import synthetic  # noqa: E402

# MI355X published peaks (dense).
PEAK_BF16_FLOPS = 2.5e15   # bf16 and f16 MFMA
PEAK_F32_MFMA_FLOPS = 157.3e12
PEAK_HBM_BPS = 8.0e12

# Algorithmic work per unit (fixed definitions; d = Dk = Dv, chunk C = 64):
#   prefill flops per token-head: dense-tile count of the chunked form
#     2C(3d + 2d) + 6 d^2 = 180,224 at d = 128
#   prefill bytes per token-head: bf16 q, k, v + f32 alpha, beta + bf16 out
#     2(3d) + 8 + 2d = 1,032 at d = 128; plus the f32 final state per head.
def prefill_flops_per_token_head(d, C=64):
    return 2 * C * (3 * d + 2 * d) + 6 * d * d


def prefill_bytes(B, T, H, d, esize=2):
    return B * T * H * (esize * 3 * d + 8 + esize * d) + B * H * d * d * 4


# Hybrid decode bytes per (b, h): GDN step reads and writes the f32 state,
# reads bf16 q, k, v and f32 alpha, beta, writes bf16 out; the softmax path
# streams the bf16 cache slots except the current one, reads and stores the
# new k, v, reads q, and reads + writes the (bf16) output it adds into.
def decode_gdn_bytes(d, esize=2):
    return 8 * d * d + esize * 3 * d + 8 + esize * d


# Channel-gate prefill, chunks of C = 32, per token-head: the per-chunk pass
# forms the gate-ratio Gram blocks A and Pm (4 C dk) on f32 MFMA; the
# recurrence forms K S, Q S and the state update (6 dk dv), T Y and Pm U
# (4 C dv), on f16 MFMA for bf16 inputs: 16,384 + 114,688 flop at d = 128.
def chgate_prep_flops_per_token_head(dk, C=32):
    return 4 * C * dk


def chgate_recur_flops_per_token_head(dk, dv, C=32):
    return 6 * dk * dv + 4 * C * dv


# bf16 q, k, v, out + f32 per-channel alpha and beta per token-head.
def chgate_bytes(B, T, H, dk, dv, esize=2):
    return B * T * H * (esize * (2 * dk + 2 * dv) + 4 * dk + 4) + B * H * dk * dv * 4


# Backward per token-head at d = d_k = d_v, chunk C = 64: dense-tile count of
# the chunked reverse mode (products on lower block triangles counted at
# 10/16 of the square):
#   C d^2 products (2 C d^2 flops each): K S and K^T (d U) in the state
#   sweep; K dSn and Q^T dO + K^T dX (two) in the reverse sweep; dO S^T,
#   dX S^T, (d U) dSn^T in the gradient pass -> 16 C d^2;
#   C^2 d products: K K^T, Q K^T (lower), Tm Y, P^T dO, Tm^T dU, dO U^T,
#   dU Y^T (lower), E1 K, E1^T Q, (E2 + E2^T) K -> 14.75 C^2 d;
#   C^3 products: dTm Tm^T and Tm^T M1 -> 4 C^3;
# divided by C: 16 d^2 + 14.75 C d + 4 C^2 = 399,360 at d = 128.
def backward_flops_per_token_head(d, C=64):
    return int(16 * d * d + 14.75 * C * d + 4 * C * C)


def swa_set_sizes(T, n_sink, window):
    """|I_t| for t = 0..T-1: sinks {0..s-1} and window {t-w+1..t}, each once."""
    t = torch.arange(T, dtype=torch.int64)
    sinks = torch.clamp(t + 1, max=n_sink)
    lo = torch.clamp(t - window + 1, min=n_sink)
    return sinks + torch.clamp(t - lo + 1, min=0)


# Softmax path over a sequence: q.k and p.v per attended pair, 2 d flops each.
def swa_prefill_flops(B, T, H, d, n_sink, window):
    return int(4 * d * swa_set_sizes(T, n_sink, window).sum().item()) * B * H


# bf16 q, k, v read once; out written, and read back on the rows it adds to.
def swa_prefill_bytes(B, T, H, d, acc_rows, esize=2):
    return B * H * (T * (3 * d * esize + d * esize) + acc_rows * d * esize)


def decode_swa_bytes(d, n_slots, esize=2):
    return esize * (2 * d * (n_slots - 1) + 2 * d + 2 * d + d + 2 * d)


# HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch)
# scaled by the copy calibration (read x2.00, write x1.00), recorded with the
# SHA-1 of the kernel source they were taken on: a kernel whose source has
# changed since reports traffic null.  Each figure is copied from the profile
# summary named in "profile".
PROFILE = "profiles/gdn_kernels_bench_workloads.md"
# The long32k prefill call launches three kernels (segment transition pass,
# combine pass, output pass); its entry sums them.
PREFILL_KERNELS = "prefill_lead_kernel<bf16> + segment_combine_kernel + prefill_out_kernel<bf16>"
# The fused-convolution prefill of the Qwen-32B-shaped layer: the same three
# kernels, instantiated with the convolution in their tile loads.
PREFILL_CONV_KERNELS = ("prefill_lead_kernel<bf16,conv> + segment_combine_kernel + "
                        "prefill_out_kernel<bf16,conv>")
CHGATE_KERNELS = ("chgate_prep_kernel (f32) + chgate_recur_tile_kernel (bf16 inputs: f16 MFMA "
                  "operands, f32 accumulation and state)")
# The backward call (d = 128) launches the chunked reverse mode's four kernels,
# every product on f32 MFMA.
BWD_KERNELS = ("bwdc_prep_kernel + bwdc_fwd_kernel + bwdc_dstate_kernel + bwdc_grad_kernel "
               "(bf16 inputs, f32 MFMA)")
COUNTERS = {
    PREFILL_KERNELS: dict(
        src="gated_delta_rule_115_amd/csrc/gdn_prefill_head.hip",
        sha1="7d272a8c4a3e61df3fc2b8b4e2b998427123eb32",
        fetch_kib=248642 + 15389 + 371797, write_kib=55305 + 14336 + 239618,
        profile=PROFILE),
    PREFILL_CONV_KERNELS: dict(
        src="gated_delta_rule_115_amd/csrc/gdn_prefill_head.hip",
        sha1="7d272a8c4a3e61df3fc2b8b4e2b998427123eb32",
        fetch_kib=318663 + 12834 + 423939, write_kib=102722 + 10240 + 258828,
        profile=PROFILE),
    "decode_step_kernel<bf16,bf16,128,128>": dict(
        src="gated_delta_rule_115_amd/csrc/gdn_decode.hip",
        sha1="d0e70d0a01d4633fac0a955eda54f3bd69f01b62",
        fetch_kib=265758, write_kib=526637, profile=PROFILE),
    "swa_sink_decode_kernel<bf16,bf16,128>": dict(
        src="gated_delta_rule_115_amd/csrc/gdn_swa.hip",
        sha1="afa1a0eccd2a4fdf0d91fdc379ee91e97784c24f",
        fetch_kib=1062046, write_kib=6144, profile=PROFILE),
    # mean of the three launches of the counter run (same inputs)
    "swa_sink_prefill_kernel<bf16>": dict(
        src="gated_delta_rule_115_amd/csrc/gdn_swa_prefill.hip",
        sha1="37b818d402e8140a9ccfde193dc53fe2b22252c0",
        fetch_kib=(254840 + 254984 + 255142) / 3, write_kib=(132055 + 132042 + 132151) / 3,
        profile=PROFILE),
    CHGATE_KERNELS: dict(
        src="gated_delta_rule_115_amd/csrc/gdn_chgate.hip",
        sha1="c48cc347bf8361d2ce70ab62068c985f38dbf84f",
        fetch_kib=264722 + 361550, write_kib=329728 + 139264, profile=PROFILE),
    BWD_KERNELS: dict(
        src="gated_delta_rule_115_amd/csrc/gdn_bwd_chunk.hip",
        sha1="bad5dce9c0ea52a578d39c2b7f9c04dd69beec37",
        fetch_kib=33369 + 51536 + 100695 + 370170, write_kib=101575 + 262145 + 335881 + 132178,
        profile=PROFILE),
    # the three projections of the leg together
    "short_conv_silu_kernel<bf16,bf16,4> (x3)": dict(
        src="gated_delta_rule_115_amd/csrc/gdn_conv.hip",
        sha1="26dcd19fe2422c955fb54847fe44d26b1569afa6",
        fetch_kib=168102 + 168094 + 168099, write_kib=327682 + 327680 + 327702, profile=PROFILE),
    # the three projections' decode-time steps together
    "short_conv_step_kernel<bf16,bf16,4> (x3)": dict(
        src="gated_delta_rule_115_amd/csrc/gdn_conv.hip",
        sha1="26dcd19fe2422c955fb54847fe44d26b1569afa6",
        fetch_kib=5460 + 5460 + 5460, write_kib=10240 + 10240 + 10240, profile=PROFILE),
}
READ_FACTOR, WRITE_FACTOR = 2.00, 1.00


def traffic_bytes(kernel):
    rec = COUNTERS.get(kernel)
    if rec is None:
        return None
    path = os.path.join(HERE, rec["src"])
    with open(path, "rb") as f:
        if hashlib.sha1(f.read()).hexdigest() != rec["sha1"]:
            return None
    return (rec["fetch_kib"] * READ_FACTOR + rec["write_kib"] * WRITE_FACTOR) * 1024


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--legs", default="prefill_long32k,decode_b256,hybrid_prefill,"
                                      "chgate_llama8b,backward_t1024,conv_qwen32b,"
                                      "conv_qwen32b_twocall,convstep_b256")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (5 times) "
                         "and exit: the reference reading for HBM byte counters")
    return ap.parse_args()


class Leg:
    def __init__(self, name):
        self.name = name
        self.ms = []

    def timed(self, fn, stream):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        return (a, b)


def make_prefill_leg():
    c = synthetic.CONFIGS["long32k"]
    B, T, H, d = c["B"], c["T"], c["H"], c["Dk"]
    x = synthetic.gdn_inputs(B, T, H, d, d, dtype="bf16", seed=c["seed"], device="cuda")
    out = torch.empty(B, T, H, d, dtype=torch.bfloat16, device="cuda")
    st = torch.empty(B, H, d, d, dtype=torch.float32, device="cuda")
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(B, T, H, d, d, 64), dtype=torch.uint8,
                     device="cuda")

    def run(mark):
        gdn.gdn_prefill_chunked(x["q"], x["k"], x["v"], x["alpha"], x["beta"], None,
                                chunk=64, out=out, state_out=st, workspace=ws)
        mark("prefill")

    info = dict(B=B, T=T, H=H, d=d, tokens=B * T,
                flops=prefill_flops_per_token_head(d) * B * T * H,
                bytes=prefill_bytes(B, T, H, d))
    return run, info, x


def make_decode_leg():
    c = synthetic.CONFIGS["hybrid_decode"]
    B, H, d, s, w, ctx = c["B"], c["H"], c["Dk"], c["n_sink"], c["window"], c["context"]
    # f32 state from the GPU prefill of tokens s .. ctx-w-1 (the linear set of
    # the 4096-token context before this step); set-up, not timed.
    n_lin = ctx - w - s
    pre = synthetic.gdn_inputs(B, n_lin, H, d, d, dtype="bf16", seed=c["seed"], device="cuda")
    st = torch.empty(B, H, d, d, dtype=torch.float32, device="cuda")
    gdn.gdn_prefill_chunked(pre["q"], pre["k"], pre["v"], pre["alpha"], pre["beta"], None,
                            chunk=64, state_out=st)
    torch.cuda.synchronize()
    del pre
    torch.cuda.empty_cache()
    tok = synthetic.gdn_inputs(B, 1, H, d, d, dtype="bf16", seed=c["seed"] + 100, device="cuda")
    q, k, v = (tok[n][:, 0].contiguous() for n in ("q", "k", "v"))
    a, b = (tok[n][:, 0].contiguous() for n in ("alpha", "beta"))
    qs, kc, vc = synthetic.swa_inputs(B, H, d, s + w, dtype="bf16", seed=c["seed"] + 200,
                                      device="cuda")
    kn, vn = (z[:, :, 0].contiguous() for z in
              synthetic.swa_inputs(B, H, d, 1, seed=c["seed"] + 300, device="cuda")[1:])
    nt = torch.full((B,), ctx + 1, dtype=torch.int32, device="cuda")
    out = torch.empty(B, H, d, dtype=torch.bfloat16, device="cuda")

    def run(mark):
        gdn.gdn_decode_step(q, k, v, a, b, st, state_out=st, out=out)
        mark("decode_step")
        gdn.gdn_swa_sink_decode(qs, kc, vc, nt, n_sink=s, window=w, k_new=kn, v_new=vn,
                                accumulate=True, out=out)
        mark("swa_sink_decode")

    info = dict(B=B, H=H, d=d, tokens=B, n_slots=s + w,
                bytes=B * H * (decode_gdn_bytes(d) + decode_swa_bytes(d, s + w)),
                bytes_gdn=B * H * decode_gdn_bytes(d),
                bytes_swa=B * H * decode_swa_bytes(d, s + w))
    return run, info, dict(q=q, k=k, v=v, alpha=a, beta=b, state=st)


def make_hybrid_prefill_leg():
    c = synthetic.CONFIGS["hybrid_prefill"]
    B, T, H, d, s, w = c["B"], c["T"], c["H"], c["Dk"], c["n_sink"], c["window"]
    x = synthetic.gdn_inputs(B, T, H, d, d, dtype="bf16", seed=c["seed"], device="cuda")
    qs, ks, vs = synthetic.swa_seq_inputs(B, T, H, d, seed=c["seed"] + 1000, device="cuda")
    out = torch.empty(B, T, H, d, dtype=torch.bfloat16, device="cuda")
    st = torch.empty(B, H, d, d, dtype=torch.float32, device="cuda")
    kc = torch.empty(B, H, s + w, d, dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    ws = torch.empty(max(1, gdn.gdn_hybrid_prefill_workspace_bytes(B, T, H, d, s, w)),
                     dtype=torch.uint8, device="cuda")

    def run(mark):
        gdn.gdn_hybrid_prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], qs, ks, vs,
                               n_sink=s, window=w, state_out=st, out=out, k_cache=kc,
                               v_cache=vc, workspace=ws)
        mark("hybrid_prefill")

    def swa_only():
        gdn.gdn_swa_sink_prefill(qs, ks, vs, n_sink=s, window=w, accumulate_from=s + w,
                                 out=out)

    t_lin = T - w - s
    swa_f = swa_prefill_flops(B, T, H, d, s, w)
    swa_b = swa_prefill_bytes(B, T, H, d, T - s - w)
    lin_f = prefill_flops_per_token_head(d) * B * t_lin * H
    lin_b = prefill_bytes(B, t_lin, H, d)
    info = dict(B=B, T=T, H=H, d=d, tokens=B * T, flops=lin_f + swa_f,
                bytes=lin_b + swa_b + 2 * 2 * B * H * (s + w) * d * 2,
                swa_flops=swa_f, swa_bytes=swa_b, swa_only=swa_only)
    return run, info


def make_chgate_leg():
    c = synthetic.CONFIGS["chgate_llama8b"]
    B, T, H, d = c["B"], c["T"], c["H"], c["Dk"]
    x = synthetic.chgate_inputs(B, T, H, d, d, dtype="bf16", seed=c["seed"], device="cuda")
    out = torch.empty(B, T, H, d, dtype=torch.bfloat16, device="cuda")
    st = torch.empty(B, H, d, d, dtype=torch.float32, device="cuda")
    ws = torch.empty(gdn.gdn_prefill_chgate_workspace_bytes(B, T, H), dtype=torch.uint8,
                     device="cuda")

    def run(mark):
        gdn.gdn_prefill_chunked_chgate(x["q"], x["k"], x["v"], x["alpha"], x["beta"], None,
                                       out=out, state_out=st, workspace=ws)
        mark("chgate_prefill")

    n = B * T * H
    info = dict(B=B, T=T, H=H, d=d, tokens=B * T,
                prep_flops=chgate_prep_flops_per_token_head(d) * n,
                recur_flops=chgate_recur_flops_per_token_head(d, d) * n,
                bytes=chgate_bytes(B, T, H, d, d))
    return run, info


def make_backward_leg():
    B, T, H, d = 4, 1024, 32, 128
    x = synthetic.gdn_inputs(B, T, H, d, d, dtype="bf16", seed=8, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(9)
    dout = torch.randn(B, T, H, d, generator=gen, device="cuda")
    ws = torch.empty(gdn.gdn_prefill_backward_workspace_bytes(B, T, H, d, d), dtype=torch.uint8,
                     device="cuda")

    def run(mark):
        gdn.gdn_prefill_backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], dout,
                                 workspace=ws)
        mark("backward")

    info = dict(B=B, T=T, H=H, d=d, tokens=B * T,
                flops=backward_flops_per_token_head(d) * B * T * H,
                peak_flops=PEAK_F32_MFMA_FLOPS,
                bytes=B * T * H * (2 * 3 * d + 8 + 4 * d + 4 * (3 * d + 2)))
    return run, info


def make_conv_leg():
    c = synthetic.CONFIGS["qwen32b_conv"]
    B, T, H, d = c["B"], c["T"], c["H"], c["Dk"]
    g = synthetic.gdn_inputs(B, T, H, d, d, dtype="bf16", seed=c["seed"], normalise_qk=False,
                             device="cuda")
    taps = {n: synthetic.conv_inputs(1, 1, H * d, 4, seed=c["seed"] * 10 + i, device="cuda")[1]
            for i, n in enumerate(("q", "k", "v"))}
    out = torch.empty(B, T, H, d, dtype=torch.bfloat16, device="cuda")
    st = torch.empty(B, H, d, d, dtype=torch.float32, device="cuda")
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(B, T, H, d, d, 64), dtype=torch.uint8,
                     device="cuda")

    def run(mark):
        gdn.gdn_prefill_chunked_conv(g["q"], g["k"], g["v"], taps["q"], taps["k"], taps["v"],
                                     g["alpha"], g["beta"], None, out=out, state_out=st,
                                     workspace=ws)
        mark("prefill_conv")

    info = dict(B=B, T=T, H=H, d=d, tokens=B * T,
                flops=prefill_flops_per_token_head(d) * B * T * H,
                bytes=prefill_bytes(B, T, H, d))
    return run, info


def make_conv_twocall_leg():
    c = synthetic.CONFIGS["qwen32b_conv"]
    B, T, H, d = c["B"], c["T"], c["H"], c["Dk"]
    g = synthetic.gdn_inputs(B, T, H, d, d, dtype="bf16", seed=c["seed"], normalise_qk=False,
                             device="cuda")
    raw = {n: g[n].reshape(B, T, H * d) for n in ("q", "k", "v")}
    taps = {n: synthetic.conv_inputs(1, 1, H * d, 4, seed=c["seed"] * 10 + i, device="cuda")[1]
            for i, n in enumerate(("q", "k", "v"))}
    conv = {n: torch.empty_like(raw[n]) for n in raw}
    out = torch.empty(B, T, H, d, dtype=torch.bfloat16, device="cuda")
    st = torch.empty(B, H, d, d, dtype=torch.float32, device="cuda")
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(B, T, H, d, d, 64), dtype=torch.uint8,
                     device="cuda")

    def run(mark):
        for n, grp in (("q", d), ("k", d), ("v", 0)):
            gdn.gdn_short_conv_silu(raw[n], taps[n], l2norm_group=grp, out=conv[n])
        mark("conv")
        gdn.gdn_prefill_chunked(conv["q"].view(B, T, H, d), conv["k"].view(B, T, H, d),
                                conv["v"].view(B, T, H, d), g["alpha"], g["beta"], None,
                                chunk=64, out=out, state_out=st, workspace=ws)
        mark("prefill")

    info = dict(B=B, T=T, H=H, d=d, tokens=B * T,
                conv_bytes=3 * B * T * H * d * 2 * 2,
                flops=prefill_flops_per_token_head(d) * B * T * H,
                bytes=prefill_bytes(B, T, H, d))
    return run, info


def make_convstep_leg():
    """Decode-time short conv of the Qwen-32B-shaped layer: one new token for
    each of 256 sequences through the q, k, v convolutions (K = 4, per-head L2
    norm on q and k), each with its K - 1 = 3 previous inputs as state."""
    c = synthetic.CONFIGS["qwen32b_conv"]
    H, d, K, B = c["H"], c["Dk"], 4, 256
    Ch = H * d
    xs = {n: synthetic.conv_inputs(B, K, Ch, K, seed=c["seed"] * 100 + i, device="cuda")
          for i, n in enumerate(("q", "k", "v"))}
    x = {n: xs[n][0][:, K - 1].contiguous() for n in xs}
    state = {n: xs[n][0][:, :K - 1].contiguous() for n in xs}
    taps = {n: xs[n][1] for n in xs}
    y = {n: torch.empty_like(x[n]) for n in xs}

    def run(mark):
        for n, grp in (("q", d), ("k", d), ("v", 0)):
            gdn.gdn_short_conv_step(x[n], taps[n], state[n], l2norm_group=grp, out=y[n])
        mark("conv_step")

    # per projection: x read, y written, the K - 1 history rows read and written (bf16)
    info = dict(B=B, Ch=Ch, K=K, tokens=B, bytes=3 * B * Ch * 2 * (2 + 2 * (K - 1)))
    return run, info


def cpu_baseline(prefill_x, decode_x):
    """The oracle as it stands, on a bounded sample of each workload."""
    import numpy as np
    import oracle

    f64 = synthetic.to_f64
    res = {}
    # Prefill: the whole 32k-token workload (all 32 heads, every token).
    Ts = prefill_x["q"].shape[1]
    ins = [f64(prefill_x[n][:, :Ts]) for n in ("q", "k", "v", "alpha", "beta")]
    t0 = time.perf_counter()
    oracle.gdn_recurrence(*ins)
    dt = time.perf_counter() - t0
    res["prefill"] = dict(value=Ts / dt, unit="tokens/s", seconds=dt,
                          sample=f"the whole prefill workload: 32 heads x {Ts} tokens (B=1)")
    # Decode: the GDN step of all 256 x 32 heads.
    d_ins = [f64(decode_x[n]) for n in ("q", "k", "v", "alpha", "beta", "state")]
    t0 = time.perf_counter()
    oracle.decode_step(*d_ins)
    dt = time.perf_counter() - t0
    res["decode"] = dict(value=d_ins[0].shape[0] / dt, unit="tokens/s", seconds=dt,
                         sample="GDN step of all 256 x 32 heads (softmax path not timed)")
    res["cores"] = oracle.num_threads()
    return res


def copy_calibration(mib):
    """A plain copy kernel of known size: reads and writes mib MiB per launch.
    Profiling it with the FETCH_SIZE / WRITE_SIZE counters gives the factor
    between those counters and real HBM bytes on this machine."""
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 5}), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); every "
              "(batch, head) of this workload is independent, so several GPUs would run "
              "independent copies of this one-GPU measurement.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    legs_wanted = args.legs.split(",")

    legs = {}
    infos = {}
    keep = {}
    if "prefill_long32k" in legs_wanted:
        run, info, x = make_prefill_leg()
        legs["prefill_long32k"], infos["prefill_long32k"], keep["prefill"] = run, info, x
    if "decode_b256" in legs_wanted:
        run, info, x = make_decode_leg()
        legs["decode_b256"], infos["decode_b256"], keep["decode"] = run, info, x
    if "hybrid_prefill" in legs_wanted:
        run, info = make_hybrid_prefill_leg()
        legs["hybrid_prefill"], infos["hybrid_prefill"] = run, info
    if "chgate_llama8b" in legs_wanted:
        run, info = make_chgate_leg()
        legs["chgate_llama8b"], infos["chgate_llama8b"] = run, info
    if "backward_t1024" in legs_wanted:
        run, info = make_backward_leg()
        legs["backward_t1024"], infos["backward_t1024"] = run, info
    if "conv_qwen32b" in legs_wanted:
        run, info = make_conv_leg()
        legs["conv_qwen32b"], infos["conv_qwen32b"] = run, info
    if "conv_qwen32b_twocall" in legs_wanted:
        run, info = make_conv_twocall_leg()
        legs["conv_qwen32b_twocall"], infos["conv_qwen32b_twocall"] = run, info
    if "convstep_b256" in legs_wanted:
        run, info = make_convstep_leg()
        legs["convstep_b256"], infos["convstep_b256"] = run, info
    torch.cuda.synchronize()

    def step(record):
        """One pass of every leg.  With record, HIP events on the kernels'
        stream bracket each leg and each kernel segment inside it."""
        evs = {}
        for name, fn in legs.items():
            if not record:
                fn(lambda seg: None)
                continue
            a = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            marks = [("", a)]

            def mark(seg, marks=marks):
                e = torch.cuda.Event(enable_timing=True)
                e.record(stream)
                marks.append((seg, e))

            fn(mark)
            evs[name] = marks
        return evs

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    all_evs = [step(True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # The softmax-path kernel of the hybrid prefill on its own (same inputs and
    # launch shape as inside gdn_hybrid_prefill), for its roofline line.
    swa_pref_ms = None
    if "hybrid_prefill" in legs:
        fn = infos["hybrid_prefill"]["swa_only"]
        fn()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        swa_pref_ms = a.elapsed_time(b) / args.steps
    leg_ms = {n: [e[n][0][1].elapsed_time(e[n][-1][1]) for e in all_evs] for n in legs}
    # per-kernel segment times (ms), averaged over the timed steps
    seg_ms = {}
    for n in legs:
        for i in range(1, len(all_evs[0][n])):
            seg = all_evs[0][n][i][0]
            vals = [e[n][i - 1][1].elapsed_time(e[n][i][1]) for e in all_evs]
            seg_ms[(n, seg)] = sum(vals) / len(vals)

    out_legs = {}
    for n, ms in leg_ms.items():
        inf = infos[n]
        avg = sum(ms) / len(ms)
        sec = avg / 1e3
        rec = dict(ms_avg=avg, ms_min=min(ms), tokens_per_s=inf["tokens"] / sec)
        if "flops" in inf:
            rec["tflops"] = inf["flops"] / sec / 1e12
            rec["mfma_frac"] = inf["flops"] / sec / inf.get("peak_flops", PEAK_BF16_FLOPS)
            rec["hbm_gbps_algorithmic"] = inf["bytes"] / sec / 1e9
            rec["hbm_frac"] = inf["bytes"] / sec / PEAK_HBM_BPS
        else:
            rec["hbm_gbps_algorithmic"] = inf["bytes"] / sec / 1e9
            rec["hbm_frac"] = inf["bytes"] / sec / PEAK_HBM_BPS
        out_legs[n] = rec

    for (n, seg), ms in seg_ms.items():
        out_legs[n].setdefault("kernel_ms", {})[seg] = ms

    def hbm_roof(kernel, nbytes, ms):
        sec = ms / 1e3
        t = traffic_bytes(kernel)
        return dict(bound="hbm", kernel=kernel, achieved=nbytes / sec / 1e9,
                    peak=PEAK_HBM_BPS / 1e9, unit="GB/s", frac=nbytes / sec / PEAK_HBM_BPS,
                    traffic=t, bytes_per_launch=nbytes, ms_per_launch=ms)

    head = out_legs.get("prefill_long32k")
    value = head["tokens_per_s"] if head else None
    roofline = None
    if head:
        inf = infos["prefill_long32k"]
        ms = seg_ms[("prefill_long32k", "prefill")]
        sec = ms / 1e3
        kern = PREFILL_KERNELS
        roofline = dict(bound="mfma", kernel=kern, achieved=inf["flops"] / sec / 1e12,
                        peak=PEAK_BF16_FLOPS / 1e12, unit="TFLOP/s",
                        frac=inf["flops"] / sec / PEAK_BF16_FLOPS, traffic=traffic_bytes(kern),
                        ms_per_launch=ms, flops_per_launch=inf["flops"],
                        flops_per_token_head=prefill_flops_per_token_head(inf["d"]),
                        hbm_bytes_algorithmic=inf["bytes"],
                        hbm_frac_algorithmic=inf["bytes"] / sec / PEAK_HBM_BPS)
    roof_dec = None
    if "decode_b256" in out_legs:
        inf = infos["decode_b256"]
        roof_dec = [hbm_roof("decode_step_kernel<bf16,bf16,128,128>", inf["bytes_gdn"],
                             seg_ms[("decode_b256", "decode_step")]),
                    hbm_roof("swa_sink_decode_kernel<bf16,bf16,128>", inf["bytes_swa"],
                             seg_ms[("decode_b256", "swa_sink_decode")])]
    roof_swa_pref = None
    if swa_pref_ms is not None:
        inf = infos["hybrid_prefill"]
        sec = swa_pref_ms / 1e3
        kern = "swa_sink_prefill_kernel<bf16>"
        # q, k, v and the output move 1,280 B per token-head against 264 kflop
        # (516 attended keys): below the ridge, so HBM bounds it.
        roof_swa_pref = dict(bound="hbm", kernel=kern, achieved=inf["swa_bytes"] / sec / 1e9,
                             peak=PEAK_HBM_BPS / 1e9, unit="GB/s",
                             frac=inf["swa_bytes"] / sec / PEAK_HBM_BPS,
                             traffic=traffic_bytes(kern), bytes_per_launch=inf["swa_bytes"],
                             ms_per_launch=swa_pref_ms, flops_per_launch=inf["swa_flops"],
                             tflops=inf["swa_flops"] / sec / 1e12,
                             mfma_frac=inf["swa_flops"] / sec / PEAK_BF16_FLOPS)
    roof_chgate = None
    if "chgate_llama8b" in out_legs:
        inf = infos["chgate_llama8b"]
        ms = seg_ms[("chgate_llama8b", "chgate_prefill")]
        sec = ms / 1e3
        kern = CHGATE_KERNELS
        # Each kernel against the pipe its products use: the per-chunk pass's
        # Gram blocks on f32 MFMA, the recurrence on f16 MFMA.  The call's peak
        # is the flop-weighted one: total flops over the time both would take
        # at their peaks.
        flops = inf["prep_flops"] + inf["recur_flops"]
        t_min = inf["prep_flops"] / PEAK_F32_MFMA_FLOPS + inf["recur_flops"] / PEAK_BF16_FLOPS
        peak = flops / t_min
        roof_chgate = dict(bound="mfma", kernel=kern,
                           achieved=flops / sec / 1e12, peak=peak / 1e12, unit="TFLOP/s",
                           frac=t_min / sec, traffic=traffic_bytes(kern),
                           peak_note="flop-weighted: per-chunk pass on f32 MFMA (157.3 TFLOP/s), "
                                     "recurrence on f16 MFMA (2.5 PFLOP/s)",
                           ms_per_launch=ms, flops_per_launch=flops,
                           prep_flops_per_launch=inf["prep_flops"],
                           recur_flops_per_launch=inf["recur_flops"],
                           hbm_bytes_algorithmic=inf["bytes"],
                           hbm_frac_algorithmic=inf["bytes"] / sec / PEAK_HBM_BPS)
    roof_bwd = None
    if "backward_t1024" in out_legs:
        inf = infos["backward_t1024"]
        ms = seg_ms[("backward_t1024", "backward")]
        sec = ms / 1e3
        roof_bwd = dict(bound="mfma", kernel=BWD_KERNELS,
                        achieved=inf["flops"] / sec / 1e12,
                        peak=PEAK_F32_MFMA_FLOPS / 1e12, unit="TFLOP/s",
                        frac=inf["flops"] / sec / PEAK_F32_MFMA_FLOPS,
                        traffic=traffic_bytes(BWD_KERNELS),
                        ms_per_launch=ms, flops_per_launch=inf["flops"],
                        hbm_bytes_algorithmic=inf["bytes"],
                        hbm_frac_algorithmic=inf["bytes"] / sec / PEAK_HBM_BPS)
    roof_conv = None
    if "conv_qwen32b" in out_legs:
        inf = infos["conv_qwen32b"]
        ms = seg_ms[("conv_qwen32b", "prefill_conv")]
        sec = ms / 1e3
        kern = PREFILL_CONV_KERNELS
        roof_conv = dict(bound="mfma", kernel=kern, achieved=inf["flops"] / sec / 1e12,
                         peak=PEAK_BF16_FLOPS / 1e12, unit="TFLOP/s",
                         frac=inf["flops"] / sec / PEAK_BF16_FLOPS, traffic=traffic_bytes(kern),
                         ms_per_launch=ms, flops_per_launch=inf["flops"],
                         hbm_bytes_algorithmic=inf["bytes"],
                         hbm_frac_algorithmic=inf["bytes"] / sec / PEAK_HBM_BPS)
    roof_conv_kernel = None
    if "conv_qwen32b_twocall" in out_legs:
        inf = infos["conv_qwen32b_twocall"]
        roof_conv_kernel = hbm_roof("short_conv_silu_kernel<bf16,bf16,4> (x3)",
                                    inf["conv_bytes"], seg_ms[("conv_qwen32b_twocall", "conv")])

    roof_convstep = None
    if "convstep_b256" in out_legs:
        inf = infos["convstep_b256"]
        roof_convstep = hbm_roof("short_conv_step_kernel<bf16,bf16,4> (x3)", inf["bytes"],
                                 seg_ms[("convstep_b256", "conv_step")])

    cpu = None
    if not args.no_cpu_baseline and "prefill" in keep and "decode" in keep:
        cb = cpu_baseline(keep["prefill"], keep["decode"])
        cpu = dict(value=cb["prefill"]["value"], unit="tokens/s", cores=cb["cores"],
                   kind="oracle", sample=cb["prefill"]["sample"],
                   seconds=cb["prefill"]["seconds"],
                   decode=dict(value=cb["decode"]["value"], unit="tokens/s",
                               sample=cb["decode"]["sample"],
                               seconds=cb["decode"]["seconds"]))

    step_ms = wall * 1e3 / args.steps
    line = {
        "metric": "GDN layer tokens/s (prefill T=32k, decode B=256) + % MFMA / HBM peak",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 I/O, f16 MFMA operands, f32 accumulation and state",
        "data": "synthetic (seeded torch.Generator; Llama/Qwen-shaped layers, random init)",
        "config": {
            "workload": "long32k prefill (B1 H32 T32768 d128, chunk 64) + hybrid decode "
                        "(B256 H32 d128, 4 sinks + 512 window) + hybrid prefill (B4 H32 "
                        "T4096 d128, 4 sinks + 512 window) + channel-gate prefill (B4 H32 "
                        "T4096 d128) + backward (B4 H32 T1024 d128) + qwen32b fused "
                        "conv+prefill (B2 H40 T16384 d128), and as separate calls + "
                        "decode-time conv step (B256, 3 x 5120 channels, K 4)",
            "global_batch": 1, "seq_len": 32768, "parallelism": "single-gpu",
        },
        "decode_tokens_per_s": out_legs.get("decode_b256", {}).get("tokens_per_s"),
        "legs": out_legs,
        "roofline": roofline,
        "roofline_decode": roof_dec,
        "roofline_swa_prefill": roof_swa_pref,
        "roofline_chgate": roof_chgate,
        "roofline_backward": roof_bwd,
        "roofline_conv": roof_conv,
        "roofline_conv_kernel": roof_conv_kernel,
        "roofline_conv_step": roof_convstep,
        "cpu_baseline": cpu,
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
