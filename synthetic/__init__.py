"""Seeded synthetic inputs for the GDN token mixer.

This module only draws random tensors with the shapes and distributions of
the workloads (Llama-3-8B- and Qwen-shaped attention layers, as used by "The
Key to Going Linear: Analysis-Driven Transformer Linearization", sections 3.3
and 5).  It holds none of the token mixer's arithmetic; both the GPU tests /
benchmark and the CPU oracle consume what it returns.  No dataset, checkpoint
or trained weight is involved: every tensor is drawn from a seeded
``torch.Generator``.

Recipe (per (token, head) unless stated):
  q, k  ~ N(0, 1), divided by (||.||_2 + 1e-6) in float32, then cast
  v     ~ N(0, 1), cast
  beta  = sigmoid(N(0, 1))                      float32, in (0, 1)
  alpha = exp(-softplus(N(0, 1)) * 0.1)         float32, in (~0.6, 1)
  S0    = 0, or N(0, 1) / sqrt(Dk) per element  float32 [B, H, Dk, Dv]
Concentrated keys (key_cos = c): each head draws one unit direction mu, and
every key is c mu + sqrt(1 - c^2) z with z a random unit vector orthogonal to
mu, so cos(k_t, mu) = c and the running mean key points along mu (the key
concentration of appendix B.1, Metric 1); beta_shift b draws beta =
sigmoid(N(0, 1) + b) (b > 0 pushes the step sizes towards 1).
Short-convolution inputs: raw q, k, v ~ N(0, 1) and taps ~ N(0, 0.5^2).
Sliding-window inputs: raw q and k/v cache ~ N(0, 1) (logits ~ N(0, 1)).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

# Workloads: name -> shapes and recipe.  "chunk" is the prefill chunk size.
CONFIGS = {
    "tiny": dict(B=1, H=2, T=64, Dk=16, Dv=16, dtype="f32", chunk=16,
                 state0="zero", seed=1),
    "llama8b": dict(B=4, H=32, T=4096, Dk=128, Dv=128, dtype="bf16", chunk=64,
                    state0="randn", seed=2),
    "long32k": dict(B=1, H=32, T=32768, Dk=128, Dv=128, dtype="bf16",
                    chunk=64, state0="zero", seed=3),
    "qwen32b_conv": dict(B=2, H=40, T=16384, Dk=128, Dv=128, dtype="bf16",
                         chunk=64, state0="zero", seed=4, conv_kernel=4),
    "hybrid_decode": dict(B=256, H=32, T=1, Dk=128, Dv=128, dtype="bf16",
                          n_sink=4, window=512, context=4096, seed=5),
    "hybrid_prefill": dict(B=4, H=32, T=4096, Dk=128, Dv=128, dtype="bf16",
                           n_sink=4, window=512, seed=6),
    "chgate_llama8b": dict(B=4, H=32, T=4096, Dk=128, Dv=128, dtype="bf16", chunk=32,
                           state0="zero", seed=7),
}

TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, g, device):
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32)


def _unit(x):
    return x / (torch.linalg.vector_norm(x, dim=-1, keepdim=True) + 1e-6)


def concentrated_unit(x, cos, g, device):
    """Unit vectors along the last axis of x's shape [B, T, H, D] at cosine
    `cos` to one random unit direction per (batch, head)."""
    B, T, H, D = x.shape
    mu = _unit(_randn((B, 1, H, D), g, device))
    z = x - (x * mu).sum(-1, keepdim=True) * mu
    z = z / torch.linalg.vector_norm(z, dim=-1, keepdim=True)
    return cos * mu + math.sqrt(max(0.0, 1.0 - cos * cos)) * z


def gdn_inputs(B, T, H, Dk, Dv, dtype="bf16", seed=0, state0="zero",
               normalise_qk=True, key_cos=None, beta_shift=0.0, device="cpu"):
    """q, k [B,T,H,Dk], v [B,T,H,Dv] in `dtype`; alpha, beta [B,T,H] f32;
    state0 [B,H,Dk,Dv] f32 or None.  key_cos: keys concentrated around a
    per-head direction at that cosine (see the module docstring)."""
    g = _gen(seed, device)
    dt = TORCH_DTYPE[dtype]
    q = _randn((B, T, H, Dk), g, device)
    k = _randn((B, T, H, Dk), g, device)
    if normalise_qk:
        q, k = _unit(q), _unit(k)
    v = _randn((B, T, H, Dv), g, device)
    beta = torch.sigmoid(_randn((B, T, H), g, device) + beta_shift)
    alpha = torch.exp(-torch.nn.functional.softplus(_randn((B, T, H), g, device)) * 0.1)
    s0 = None
    if state0 == "randn":
        s0 = _randn((B, H, Dk, Dv), g, device) / math.sqrt(Dk)
    if key_cos is not None:
        k = _unit(concentrated_unit(k, float(key_cos), _gen(seed + 104729, device), device))
    return dict(q=q.to(dt).contiguous(), k=k.to(dt).contiguous(),
                v=v.to(dt).contiguous(), alpha=alpha.contiguous(),
                beta=beta.contiguous(), state0=s0)


def chgate_inputs(B, T, H, Dk, Dv, dtype="bf16", seed=0, state0="zero", gate_scale=0.1,
                  key_cos=None, beta_shift=0.0, device="cpu"):
    """gdn_inputs with a channel-wise gate: alpha [B,T,H,Dk] f32, each entry
    exp(-gate_scale * softplus(N(0,1))) (the scalar gate's distribution per
    channel)."""
    x = gdn_inputs(B, T, H, Dk, Dv, dtype=dtype, seed=seed, state0=state0, key_cos=key_cos,
                   beta_shift=beta_shift, device=device)
    g = _gen(seed + 7919, device)
    x["alpha"] = torch.exp(-torch.nn.functional.softplus(_randn((B, T, H, Dk), g, device))
                           * gate_scale).contiguous()
    return x


def conv_inputs(B, T, Ch, K=4, dtype="bf16", seed=0, device="cpu"):
    """Raw projection output x [B,T,Ch] ~ N(0,1) and taps [Ch,K] ~ N(0,0.25)."""
    g = _gen(seed, device)
    x = _randn((B, T, Ch), g, device).to(TORCH_DTYPE[dtype]).contiguous()
    taps = (_randn((Ch, K), g, device) * 0.5).contiguous()
    return x, taps


def swa_inputs(B, H, D, n_slots, dtype="bf16", seed=0, device="cpu"):
    """Raw softmax-path query [B,H,D] and k/v caches [B,H,n_slots,D] ~ N(0,1)."""
    g = _gen(seed, device)
    dt = TORCH_DTYPE[dtype]
    q = _randn((B, H, D), g, device).to(dt).contiguous()
    kc = _randn((B, H, n_slots, D), g, device).to(dt).contiguous()
    vc = _randn((B, H, n_slots, D), g, device).to(dt).contiguous()
    return q, kc, vc


def swa_seq_inputs(B, T, H, D, dtype="bf16", seed=0, device="cpu"):
    """Raw softmax-path q, k, v [B,T,H,D] ~ N(0,1) over a whole sequence."""
    g = _gen(seed, device)
    dt = TORCH_DTYPE[dtype]
    return tuple(_randn((B, T, H, D), g, device).to(dt).contiguous() for _ in range(3))


def to_f64(x):
    """Exact upcast of the bits a kernel receives (bf16/f32 -> f64 numpy)."""
    return None if x is None else x.detach().to("cpu", torch.float64).numpy()
