"""Pins for the CPU oracle (runs on CPU, no GPU).

Each test ties an oracle routine to something that is not the oracle itself:
a closed form, an invariant, a textbook routine from torch/numpy, or brute
force with explicit matrices.  Passages ("The Key to Going Linear:
Analysis-Driven Transformer Linearization"):
  section 3.1.2  GDN update / read-out
  section 3.2    GLA and GDN unrolled weights (P^GLA, P^Delta)
  section 3.1    causal softmax attention
  section 4      disjoint sliding window + sinks; short convolutions
  appendix A.3   rank-1 expansion M_t = I - sum beta k k^T + E_t, E_t = O(beta^2)
  appendix B.1   nMSE
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(12345)


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_gdn(B, T, H, Dk, Dv, rng, beta_scale=1.0, s0=True):
    q = _unit_rows(rng.standard_normal((B, T, H, Dk)))
    k = _unit_rows(rng.standard_normal((B, T, H, Dk)))
    v = rng.standard_normal((B, T, H, Dv))
    beta = beta_scale / (1 + np.exp(-rng.standard_normal((B, T, H))))
    alpha = np.exp(-0.1 * np.log1p(np.exp(rng.standard_normal((B, T, H)))))
    S0 = rng.standard_normal((B, H, Dk, Dv)) / math.sqrt(Dk) if s0 else None
    return q, k, v, alpha, beta, S0


# --------------------------------------------------------------------------
# P-i: beta = 0 -> pure decay of S0; o_t = (prod_{j<=t} alpha_j) S0^T q_t.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("Dk,Dv", [(4, 3), (3, 5), (8, 8)])
def test_beta_zero_is_pure_decay(Dk, Dv):
    B, T, H = 2, 9, 3
    q, k, v, alpha, beta, S0 = _rand_gdn(B, T, H, Dk, Dv, RNG)
    beta[:] = 0.0
    out, ST = oracle.gdn_recurrence(q, k, v, alpha, beta, S0)
    cum = np.cumprod(alpha, axis=1)  # [B,T,H]
    for b, t, h in itertools.product(range(B), range(T), range(H)):
        expect = cum[b, t, h] * (S0[b, h].T @ q[b, t, h])
        np.testing.assert_allclose(out[b, t, h], expect, atol=1e-12, rtol=0)
    np.testing.assert_allclose(ST, cum[:, -1, :, None, None] * S0, atol=1e-12,
                               rtol=0)
    out0, ST0 = oracle.gdn_recurrence(q, k, v, alpha, beta, None)
    assert np.all(out0 == 0) and np.all(ST0 == 0)


# --------------------------------------------------------------------------
# P-ii: without the erase factor the update is gated accumulation; compare
# with the unrolled GLA form of section 3.2 (scalar gates):
#   o_t = sum_{i<=t} (prod_{j=i+1}^t alpha_j) beta_i (q_t.k_i) v_i
#         + (prod_{j<=t} alpha_j) S0^T q_t
# --------------------------------------------------------------------------
def test_no_erase_equals_gla_unrolled():
    B, T, H, Dk, Dv = 1, 11, 2, 5, 3
    q, k, v, alpha, beta, S0 = _rand_gdn(B, T, H, Dk, Dv, RNG)
    out, _ = oracle.gdn_recurrence(q, k, v, alpha, beta, S0, erase=False)
    for b, h, t in itertools.product(range(B), range(H), range(T)):
        acc = np.prod(alpha[b, :t + 1, h]) * (S0[b, h].T @ q[b, t, h])
        for i in range(t + 1):
            w = np.prod(alpha[b, i + 1:t + 1, h]) * beta[b, i, h]
            acc = acc + w * (q[b, t, h] @ k[b, i, h]) * v[b, i, h]
        np.testing.assert_allclose(out[b, t, h], acc, atol=1e-12, rtol=0)


# --------------------------------------------------------------------------
# P-ii-b: appendix A.3 -- the erase factor differs from gated accumulation
# only at second order in beta: ||o_GDN - o_GLA|| = O(eps^2) for beta -> eps*beta.
# Halving eps must divide the gap by ~4.
# --------------------------------------------------------------------------
def test_gdn_minus_gla_is_second_order_in_beta():
    B, T, H, Dk, Dv = 1, 16, 2, 8, 4
    q, k, v, alpha, beta, _ = _rand_gdn(B, T, H, Dk, Dv, RNG, s0=False)

    def gap(eps):
        o1, _ = oracle.gdn_recurrence(q, k, v, alpha, eps * beta, None)
        o0, _ = oracle.gdn_recurrence(q, k, v, alpha, eps * beta, None,
                                      erase=False)
        return np.linalg.norm(o1 - o0)

    for eps in (1e-2, 5e-3):
        ratio = gap(eps) / gap(eps / 2)
        assert 3.5 <= ratio <= 4.5, ratio
    # ... and the gap itself is not zero (the erase term is really there).
    assert gap(1.0) > 1e-3


# --------------------------------------------------------------------------
# P-iii: alpha = 1, beta = 1, orthonormal keys -> exact associative memory:
# querying with an earlier key returns its value; rewriting a key overwrites.
# --------------------------------------------------------------------------
def test_orthonormal_keys_exact_retrieval_and_overwrite():
    Dk, Dv = 8, 5
    Qm, _ = np.linalg.qr(RNG.standard_normal((Dk, Dk)))
    keys = Qm.T  # rows orthonormal
    T = 2 * Dk
    k = np.zeros((1, T, 1, Dk))
    v = RNG.standard_normal((1, T, 1, Dv))
    q = np.zeros((1, T, 1, Dk))
    # first Dk tokens write key j, value v_j; query with key (j*3) % (j+1)
    for t in range(Dk):
        k[0, t, 0] = keys[t]
        q[0, t, 0] = keys[(t * 3) % (t + 1)]
    # next Dk tokens overwrite key (t - Dk) with a fresh value, query with it
    for t in range(Dk, T):
        k[0, t, 0] = keys[t - Dk]
        q[0, t, 0] = keys[t - Dk]
    ones = np.ones((1, T, 1))
    out, ST = oracle.gdn_recurrence(q, k, v, ones, ones, None)
    for t in range(Dk):
        np.testing.assert_allclose(out[0, t, 0], v[0, (t * 3) % (t + 1), 0],
                                   atol=1e-12, rtol=0)
    for t in range(Dk, T):
        np.testing.assert_allclose(out[0, t, 0], v[0, t, 0], atol=1e-12, rtol=0)
    # final state is exactly sum_j key_j (newest value_j)^T
    expect = sum(np.outer(keys[j], v[0, Dk + j, 0]) for j in range(Dk))
    np.testing.assert_allclose(ST[0, 0], expect, atol=1e-12, rtol=0)


# --------------------------------------------------------------------------
# P-iv: brute force with explicit d x d matrices (section 3.2 unrolled form).
# D_j = alpha_j (I - beta_j k_j k_j^T); latest token leftmost:
#   S_t = D_t ... D_1 S0 + sum_i D_t ... D_{i+1} beta_i k_i v_i^T
#   o_t = S_t^T q_t  ==  sum_i P^Delta_i v_i + (D_t...D_1 S0)^T q_t
# --------------------------------------------------------------------------
@pytest.mark.parametrize("Dk,Dv", [(3, 2), (5, 4), (3, 4), (5, 2)])
def test_brute_force_matrix_products(Dk, Dv):
    B, T, H = 1, 8, 2
    q, k, v, alpha, beta, S0 = _rand_gdn(B, T, H, Dk, Dv, RNG)
    scale = 0.75
    out, ST = oracle.gdn_recurrence(q, k, v, alpha, beta, S0, scale=scale)
    I = np.eye(Dk)
    for h in range(H):
        D = [alpha[0, j, h] * (I - beta[0, j, h] * np.outer(k[0, j, h], k[0, j, h]))
             for j in range(T)]

        def prod(lo, hi):  # D_hi ... D_lo (inclusive), identity if empty
            M = np.eye(Dk)
            for j in range(lo, hi + 1):
                M = D[j] @ M
            return M

        for t in range(T):
            S = prod(0, t) @ S0[0, h]
            o_pdelta = (prod(0, t) @ S0[0, h]).T @ q[0, t, h]
            for i in range(t + 1):
                S = S + prod(i + 1, t) @ (beta[0, i, h] * np.outer(k[0, i, h], v[0, i, h]))
                # P^Delta_i = beta_i q^T W_i (prod_{j=i+1}^t (I - beta_j k_j k_j^T)) k_i
                p_delta = beta[0, i, h] * (q[0, t, h] @ prod(i + 1, t) @ k[0, i, h])
                o_pdelta = o_pdelta + p_delta * v[0, i, h]
            np.testing.assert_allclose(out[0, t, h], scale * (S.T @ q[0, t, h]),
                                       atol=1e-12, rtol=0)
            np.testing.assert_allclose(out[0, t, h], scale * o_pdelta,
                                       atol=1e-12, rtol=0)
        np.testing.assert_allclose(ST[0, h], S, atol=1e-12, rtol=0)


# --------------------------------------------------------------------------
# P-v: the sink/window softmax equals a dense masked softmax (torch), and with
# no sinks and a window covering the sequence it is full causal attention
# (section 3.1 display).
# --------------------------------------------------------------------------
def _dense_masked_softmax(q, k, v, mask, scale):
    qt, kt, vt = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
    logits = (qt @ kt.transpose(-1, -2)) * scale
    logits = logits.masked_fill(~mask, float("-inf"))
    return (torch.softmax(logits, dim=-1) @ vt).permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("s,w", [(0, 100), (2, 3), (4, 5), (0, 1), (3, 1), (6, 2)])
def test_swa_sink_equals_dense_masked_softmax(s, w):
    B, T, H, D = 2, 13, 3, 6
    q, k, v = (RNG.standard_normal((B, T, H, D)) for _ in range(3))
    scale = 1 / math.sqrt(D)
    got = oracle.swa_sink_attention(q, k, v, s, w, scale)
    t = torch.arange(T)[:, None]
    i = torch.arange(T)[None, :]
    mask = (i <= t) & ((i < s) | (i >= t - w + 1))
    ref = _dense_masked_softmax(q, k, v, mask, scale)
    np.testing.assert_allclose(got, ref, atol=1e-12, rtol=0)
    if s == 0 and w >= T:
        causal = torch.nn.functional.scaled_dot_product_attention(
            *(torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v)),
            is_causal=True).permute(0, 2, 1, 3).numpy()
        np.testing.assert_allclose(got, causal, atol=1e-12, rtol=0)


# --------------------------------------------------------------------------
# P-vi: disjointness of sinks / window / linear state in the hybrid output.
# With alpha = beta = 1 and orthonormal one-hot keys the linear read returns
# twice the indicator of the linear set (lin_scale = 2); with zero softmax
# keys the softmax path returns the indicator of the exact set divided by its
# size (at most 1).  Every earlier
# token must appear in exactly one of the two, no later token in either.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("s,w", [(2, 4), (0, 3), (3, 1), (1, 20)])
def test_hybrid_sets_are_disjoint_and_cover(s, w):
    T = 14
    D = T
    eye = np.eye(D)
    kl = eye[None, :, None, :].copy()          # k_i = e_i
    vl = eye[None, :, None, :].copy()          # v_i = e_i
    ql = np.ones((1, T, 1, D))                 # q . k_i = 1 for all i
    ones = np.ones((1, T, 1))
    qs = RNG.standard_normal((1, T, 1, D))
    ks = np.zeros((1, T, 1, D))                # uniform softmax weights
    vs = eye[None, :, None, :].copy()
    out = oracle.hybrid(ql, kl, vl, ones, ones, qs, ks, vs, s, w,
                        lin_scale=2.0)[0, :, 0]
    for t in range(T):
        lin = {i for i in range(D) if abs(out[t, i] - 2.0) < 1e-12}
        exact = {i for i in range(D) if 1e-12 < out[t, i] < 1.0 + 1e-12}
        zero = {i for i in range(D) if abs(out[t, i]) < 1e-12}
        assert lin | exact | zero == set(range(D))
        assert lin | exact == set(range(t + 1)), (t, lin, exact)
        assert not (lin & exact)
        assert exact == {i for i in range(t + 1) if i < s or i >= t - w + 1}
        np.testing.assert_allclose(out[t, sorted(exact)], 1.0 / len(exact),
                                   atol=1e-12)


# The hybrid's linear term is the recurrence read one window late:
# lin(t) = S_{t-w}^T q_t where S_{t-w} has seen tokens n_sink..t-w.
def test_hybrid_linear_term_is_shifted_recurrence():
    B, T, H, D = 1, 20, 2, 6
    s, w = 3, 4
    q, k, v, alpha, beta, _ = _rand_gdn(B, T, H, D, D, RNG, s0=False)
    qs = RNG.standard_normal((B, T, H, D))
    ks = RNG.standard_normal((B, T, H, D))
    vs = RNG.standard_normal((B, T, H, D))
    hyb = oracle.hybrid(q, k, v, alpha, beta, qs, ks, vs, s, w)
    swa = oracle.swa_sink_attention(qs, ks, vs, s, w, 1 / math.sqrt(D))
    lin = hyb - swa
    # recurrence over tokens s..T-1, reading token j's state with q_{j+w}
    n = T - w - s
    qq = q[:, s + w:s + w + n]
    o, _ = oracle.gdn_recurrence(qq, k[:, s:s + n], v[:, s:s + n],
                                 alpha[:, s:s + n], beta[:, s:s + n])
    np.testing.assert_allclose(lin[:, s + w:], o, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lin[:, :s + w], 0.0, atol=1e-12)


# --------------------------------------------------------------------------
# P-vii: short convolution = torch conv1d (groups=Ch, left pad K-1) + SiLU;
# identity taps give SiLU(x); the L2 option rescales each group to norm
# ||y||/(||y||+eps) without changing its direction.
# --------------------------------------------------------------------------
def test_short_conv_equals_torch_conv1d():
    B, T, Ch, K = 2, 17, 12, 4
    x = RNG.standard_normal((B, T, Ch))
    taps = 0.5 * RNG.standard_normal((Ch, K))
    got = oracle.short_conv_silu(x, taps)
    xt = torch.from_numpy(x).permute(0, 2, 1)
    ref = torch.nn.functional.conv1d(xt, torch.from_numpy(taps)[:, None, :],
                                     padding=K - 1, groups=Ch)[..., :T]
    ref = torch.nn.functional.silu(ref).permute(0, 2, 1).numpy()
    np.testing.assert_allclose(got, ref, atol=1e-12, rtol=0)
    ident = np.zeros((Ch, K))
    ident[:, K - 1] = 1.0
    np.testing.assert_allclose(oracle.short_conv_silu(x, ident),
                               torch.nn.functional.silu(torch.from_numpy(x)).numpy(),
                               atol=1e-12, rtol=0)
    eps, grp = 1e-3, 4
    yn = oracle.short_conv_silu(x, taps, l2norm_group=grp, eps=eps)
    for g0 in range(0, Ch, grp):
        a = ref[..., g0:g0 + grp]
        bnorm = np.linalg.norm(yn[..., g0:g0 + grp], axis=-1)
        anorm = np.linalg.norm(a, axis=-1)
        np.testing.assert_allclose(bnorm, anorm / (anorm + eps), atol=1e-12)
        cos = (a * yn[..., g0:g0 + grp]).sum(-1) / (anorm * bnorm)
        np.testing.assert_allclose(cos, 1.0, atol=1e-12)


# --------------------------------------------------------------------------
# P-vii': one decode step of the short convolution.  Stepping a zero history
# through a sequence reproduces torch conv1d token by token and leaves the
# last K-1 inputs as the state; a one-hot tap j reads the input K-1-j tokens
# back; a prefix in sequence form followed by steps from the prefix's last
# K-1 inputs equals the whole sequence (with the L2 option too); K = 1 has
# an empty history.
# --------------------------------------------------------------------------
def test_short_conv_step_chains_to_conv1d():
    B, T, Ch, K = 3, 11, 16, 4
    x = RNG.standard_normal((B, T, Ch))
    taps = 0.5 * RNG.standard_normal((Ch, K))
    xt = torch.from_numpy(x).permute(0, 2, 1)
    ref = torch.nn.functional.conv1d(xt, torch.from_numpy(taps)[:, None, :],
                                     padding=K - 1, groups=Ch)[..., :T]
    ref = torch.nn.functional.silu(ref).permute(0, 2, 1).numpy()
    st = np.zeros((B, K - 1, Ch))
    for t in range(T):
        y, st = oracle.short_conv_step(x[:, t], taps, st)
        np.testing.assert_allclose(y, ref[:, t], atol=1e-12, rtol=0)
    np.testing.assert_array_equal(st, x[:, T - K + 1:])
    for j in range(K):
        oh = np.zeros((Ch, K))
        oh[:, j] = 1.0
        s0 = RNG.standard_normal((B, K - 1, Ch))
        x0 = RNG.standard_normal((B, Ch))
        y, _ = oracle.short_conv_step(x0, oh, s0)
        src = s0[:, j] if j < K - 1 else x0
        np.testing.assert_allclose(y, src / (1.0 + np.exp(-src)), atol=1e-15, rtol=0)
    T1 = 6
    full = oracle.short_conv_silu(x, taps, l2norm_group=8, eps=1e-3)
    st = x[:, T1 - K + 1:T1].copy()
    for t in range(T1, T):
        y, st = oracle.short_conv_step(x[:, t], taps, st, l2norm_group=8, eps=1e-3)
        np.testing.assert_allclose(y, full[:, t], atol=1e-12, rtol=0)
    t1 = RNG.standard_normal((Ch, 1))
    y, s1 = oracle.short_conv_step(x[:, 0], t1, np.zeros((B, 0, Ch)))
    a = t1[:, 0] * x[:, 0]
    np.testing.assert_allclose(y, a / (1.0 + np.exp(-a)), atol=1e-15, rtol=0)
    assert s1.shape == (B, 0, Ch)


# --------------------------------------------------------------------------
# P-viii: the oracle's own rounding: float32 vs float64 on the tiny workload.
# --------------------------------------------------------------------------
def test_oracle_f32_vs_f64_on_tiny():
    import synthetic
    c = synthetic.CONFIGS["tiny"]
    x = synthetic.gdn_inputs(c["B"], c["T"], c["H"], c["Dk"], c["Dv"],
                             dtype="f32", seed=c["seed"])
    args = [synthetic.to_f64(x[n]) for n in ("q", "k", "v", "alpha", "beta")]
    o64, s64 = oracle.gdn_recurrence(*args)
    o32, s32 = oracle.gdn_recurrence(*args, precision="f32")
    assert oracle.rms_normalised_max_error(o32, o64) <= 1e-5
    assert oracle.rms_normalised_max_error(s32, s64) <= 1e-5


# --------------------------------------------------------------------------
# P-ix: an identity token (alpha=1, beta=0, q=k=v=0) leaves S bitwise
# unchanged and reads 0 -- the padding used for ragged chunk tails.
# --------------------------------------------------------------------------
def test_identity_token_is_exact_noop():
    B, T, H, Dk, Dv = 1, 7, 2, 6, 5
    q, k, v, alpha, beta, S0 = _rand_gdn(B, T, H, Dk, Dv, RNG)
    _, S_a = oracle.gdn_recurrence(q, k, v, alpha, beta, S0)
    pad = lambda x, val: np.concatenate([x, np.full_like(x[:, :1], val)], axis=1)
    o_b, S_b = oracle.gdn_recurrence(pad(q, 0), pad(k, 0), pad(v, 0),
                                     pad(alpha, 1), pad(beta, 0), S0)
    assert np.array_equal(S_a, S_b)
    assert np.all(o_b[:, -1] == 0)


# --------------------------------------------------------------------------
# P-x: split / resume.  Running T1 tokens, then T2 tokens from the returned
# state, is bitwise the same as running T1+T2 tokens.
# --------------------------------------------------------------------------
def test_split_resume_is_bitwise():
    B, T, H, Dk, Dv = 2, 23, 2, 6, 4
    q, k, v, alpha, beta, S0 = _rand_gdn(B, T, H, Dk, Dv, RNG)
    o, S = oracle.gdn_recurrence(q, k, v, alpha, beta, S0)
    c = 9
    sl = lambda x, a, b: x[:, a:b]
    o1, S1 = oracle.gdn_recurrence(*(sl(x, 0, c) for x in (q, k, v, alpha, beta)), S0)
    o2, S2 = oracle.gdn_recurrence(*(sl(x, c, T) for x in (q, k, v, alpha, beta)), S1)
    assert np.array_equal(np.concatenate([o1, o2], axis=1), o)
    assert np.array_equal(S2, S)


# The decode wrapper is the recurrence at T = 1 and chains like it.
def test_decode_steps_chain_to_recurrence():
    B, T, H, Dk, Dv = 3, 5, 2, 4, 6
    q, k, v, alpha, beta, S0 = _rand_gdn(B, T, H, Dk, Dv, RNG)
    o, S = oracle.gdn_recurrence(q, k, v, alpha, beta, S0, scale=0.5)
    St = S0
    for t in range(T):
        ot, St = oracle.decode_step(q[:, t], k[:, t], v[:, t], alpha[:, t],
                                    beta[:, t], St, scale=0.5)
        assert np.array_equal(ot, o[:, t])
    assert np.array_equal(St, S)


# Error statistics used by the parity tests.
def test_error_statistics():
    ref = np.array([1.0, -1.0, 1.0, -1.0])
    got = ref + np.array([0.0, 0.1, 0.0, 0.0])
    assert abs(oracle.rms_normalised_max_error(got, ref) - 0.1) < 1e-15
    # appendix B.1: nMSE = MSE / Var(ref)
    assert abs(oracle.nmse(got, ref) - (0.01 / 4) / 1.0) < 1e-15


# The decode-step form of the softmax path is the last row of the full one.
def test_swa_last_only_matches_full():
    B, T, H, D = 2, 11, 2, 4
    q, k, v = (RNG.standard_normal((B, T, H, D)) for _ in range(3))
    full = oracle.swa_sink_attention(q, k, v, 2, 3, 0.5)
    last = oracle.swa_sink_attention(q, k, v, 2, 3, 0.5, last_only=True)
    assert np.array_equal(last, full[:, -1])


# --------------------------------------------------------------------------
# Channel-wise gate G_t = diag(alpha_t) (section 3.2's diag gates in the
# section 3.1.2 update; G_t applied before the erase, as the page orders it).
# --------------------------------------------------------------------------
def _rand_chgate(B, T, H, Dk, Dv, rng):
    q, k, v, alpha, beta, S0 = _rand_gdn(B, T, H, Dk, Dv, rng)
    a_ch = np.exp(-0.5 * rng.random((B, T, H, Dk)))  # per-channel gates in (0.6, 1]
    return q, k, v, a_ch, beta, S0


def test_chgate_equal_channels_is_the_scalar_gate():
    """A gate that is the same on every channel is alpha_t I: the pinned
    scalar-gate recurrence."""
    B, T, H, Dk, Dv = 2, 9, 2, 6, 5
    q, k, v, alpha, beta, S0 = _rand_gdn(B, T, H, Dk, Dv, RNG)
    a_ch = np.repeat(alpha[..., None], Dk, axis=-1)
    o1, s1 = oracle.gdn_recurrence_chgate(q, k, v, a_ch, beta, S0, scale=0.5)
    o2, s2 = oracle.gdn_recurrence(q, k, v, alpha, beta, S0, scale=0.5)
    np.testing.assert_allclose(o1, o2, atol=1e-13, rtol=0)
    np.testing.assert_allclose(s1, s2, atol=1e-13, rtol=0)


def test_chgate_beta_zero_is_per_channel_decay():
    """beta = 0: S_t = diag(prod_{j<=t} alpha_j) S0, so o_t = S0^T (g_t * q_t)."""
    B, T, H, Dk, Dv = 1, 7, 2, 5, 3
    q, k, v, a_ch, beta, S0 = _rand_chgate(B, T, H, Dk, Dv, RNG)
    beta = np.zeros_like(beta)
    out, ST = oracle.gdn_recurrence_chgate(q, k, v, a_ch, beta, S0)
    g = np.cumprod(a_ch, axis=1)
    for h in range(H):
        for t in range(T):
            np.testing.assert_allclose(out[0, t, h], S0[0, h].T @ (g[0, t, h] * q[0, t, h]),
                                       atol=1e-12, rtol=0)
        np.testing.assert_allclose(ST[0, h], g[0, T - 1, h][:, None] * S0[0, h],
                                   atol=1e-12, rtol=0)


@pytest.mark.parametrize("Dk,Dv", [(3, 2), (5, 4), (4, 4)])
def test_chgate_brute_force_matrix_products(Dk, Dv):
    """S_t = D_t ... D_1 S0 + sum_i D_t ... D_{i+1} beta_i k_i v_i^T with the
    explicit D_j = (I - beta_j k_j k_j^T) diag(alpha_j), latest leftmost."""
    B, T, H = 1, 8, 2
    q, k, v, a_ch, beta, S0 = _rand_chgate(B, T, H, Dk, Dv, RNG)
    out, ST = oracle.gdn_recurrence_chgate(q, k, v, a_ch, beta, S0, scale=0.75)
    I = np.eye(Dk)
    for h in range(H):
        D = [(I - beta[0, j, h] * np.outer(k[0, j, h], k[0, j, h])) @ np.diag(a_ch[0, j, h])
             for j in range(T)]

        def prod(lo, hi):
            M = np.eye(Dk)
            for j in range(lo, hi + 1):
                M = D[j] @ M
            return M

        for t in range(T):
            S = prod(0, t) @ S0[0, h]
            for i in range(t + 1):
                S = S + prod(i + 1, t) @ (beta[0, i, h] * np.outer(k[0, i, h], v[0, i, h]))
            np.testing.assert_allclose(out[0, t, h], 0.75 * (S.T @ q[0, t, h]),
                                       atol=1e-12, rtol=0)
        np.testing.assert_allclose(ST[0, h], S, atol=1e-12, rtol=0)


def test_chgate_order_matters_and_scalar_gates_commute():
    """With a diagonal gate, gate-then-erase and erase-then-gate differ; with
    a scalar gate they agree (the reason the order is a reading only here)."""
    B, T, H, Dk, Dv = 1, 6, 1, 4, 3
    q, k, v, a_ch, beta, S0 = _rand_chgate(B, T, H, Dk, Dv, RNG)
    o1, _ = oracle.gdn_recurrence_chgate(q, k, v, a_ch, beta, S0, gate_first=True)
    o2, _ = oracle.gdn_recurrence_chgate(q, k, v, a_ch, beta, S0, gate_first=False)
    assert np.max(np.abs(o1 - o2)) > 1e-3
    a_eq = np.repeat(a_ch[..., :1], Dk, axis=-1)
    o3, _ = oracle.gdn_recurrence_chgate(q, k, v, a_eq, beta, S0, gate_first=True)
    o4, _ = oracle.gdn_recurrence_chgate(q, k, v, a_eq, beta, S0, gate_first=False)
    np.testing.assert_allclose(o3, o4, atol=1e-13, rtol=0)


def test_chgate_decode_steps_chain_to_recurrence():
    B, T, H, Dk, Dv = 2, 5, 2, 4, 3
    q, k, v, a_ch, beta, S0 = _rand_chgate(B, T, H, Dk, Dv, RNG)
    out, ST = oracle.gdn_recurrence_chgate(q, k, v, a_ch, beta, S0)
    S = S0
    for t in range(T):
        o, S = oracle.decode_step_chgate(q[:, t], k[:, t], v[:, t], a_ch[:, t], beta[:, t], S)
        np.testing.assert_array_equal(o, out[:, t])
    np.testing.assert_array_equal(S, ST)


# --------------------------------------------------------------------------
# Gated linear attention with a key-dependent gate (kGLA, section 3.2.2):
# y_t = sum_{i<=t} (q_t^T [prod_{j=i+1}^{t} diag(alpha_j)(I - beta_j
# Diag(k_j o k_j))] k_i) v_i.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("Dk,Dv", [(3, 2), (5, 4)])
def test_kgla_equals_the_printed_sum(Dk, Dv):
    """The printed sum, with the explicit diagonal factors multiplied as full
    matrices (no state), against the oracle from a zero state; and with a
    state S0 the extra term q_t^T (prod_{j<=t} D_j) S0."""
    B, T, H = 1, 7, 2
    q, k, v, a_ch, beta, S0 = _rand_chgate(B, T, H, Dk, Dv, RNG)
    out0, _ = oracle.kgla(q, k, v, a_ch, beta, None, scale=0.5)
    out1, S1 = oracle.kgla(q, k, v, a_ch, beta, S0)
    I = np.eye(Dk)
    for h in range(H):
        D = [np.diag(a_ch[0, j, h]) @ (I - beta[0, j, h] * np.diag(k[0, j, h] * k[0, j, h]))
             for j in range(T)]

        def prod(lo, hi):
            M = np.eye(Dk)
            for j in range(lo, hi + 1):
                M = D[j] @ M
            return M

        for t in range(T):
            y = sum((q[0, t, h] @ prod(i + 1, t) @ k[0, i, h]) * v[0, i, h] for i in range(t + 1))
            np.testing.assert_allclose(out0[0, t, h], 0.5 * y, atol=1e-12, rtol=0)
            y1 = y + q[0, t, h] @ prod(0, t) @ S0[0, h]
            np.testing.assert_allclose(out1[0, t, h], y1, atol=1e-12, rtol=0)
        S = prod(0, T - 1) @ S0[0, h] + sum(
            prod(i + 1, T - 1) @ np.outer(k[0, i, h], v[0, i, h]) for i in range(T))
        np.testing.assert_allclose(S1[0, h], S, atol=1e-12, rtol=0)


def test_kgla_beta_zero_scalar_gate_is_gla():
    """beta = 0 and one gate value on every channel: scalar-gated linear
    attention, i.e. the GDN oracle's no-erase hook with a unit write (pinned
    above), and for a constant gate a the closed form sum a^(t-i) (q.k_i) v_i."""
    B, T, H, Dk, Dv = 2, 9, 2, 6, 5
    q, k, v, alpha, beta, S0 = _rand_gdn(B, T, H, Dk, Dv, RNG)
    a_ch = np.repeat(alpha[..., None], Dk, axis=-1)
    o1, s1 = oracle.kgla(q, k, v, a_ch, np.zeros_like(beta), S0)
    o2, s2 = oracle.gdn_recurrence(q, k, v, alpha, np.ones_like(beta), S0, erase=False)
    np.testing.assert_allclose(o1, o2, atol=1e-13, rtol=0)
    np.testing.assert_allclose(s1, s2, atol=1e-13, rtol=0)
    a = 0.9
    o3, _ = oracle.kgla(q, k, v, np.full_like(a_ch, a), np.zeros_like(beta))
    for t in range(T):
        y = sum(a ** (t - i) * np.einsum("bhd,bhd->bh", q[:, t], k[:, i])[..., None] * v[:, i]
                for i in range(t + 1))
        np.testing.assert_allclose(o3[:, t], y, atol=1e-12, rtol=0)


def test_kgla_one_hot_keys_with_unit_step_equal_gdn():
    """For a one-hot key e_c, Diag(k o k) = k k^T, so with beta = 1 (the GDN
    write beta k v^T is then k v^T) kGLA is the channel-gated GDN update."""
    B, T, H, Dk, Dv = 1, 12, 2, 5, 3
    q, _, v, a_ch, beta, S0 = _rand_chgate(B, T, H, Dk, Dv, RNG)
    k = np.eye(Dk)[RNG.integers(0, Dk, (B, T, H))]
    ones = np.ones_like(beta)
    o1, s1 = oracle.kgla(q, k, v, a_ch, ones, S0)
    o2, s2 = oracle.gdn_recurrence_chgate(q, k, v, a_ch, ones, S0)
    np.testing.assert_allclose(o1, o2, atol=1e-13, rtol=0)
    np.testing.assert_allclose(s1, s2, atol=1e-13, rtol=0)
    # and with beta < 1 the two differ (the write is not scaled by beta in kGLA)
    o3, _ = oracle.kgla(q, k, v, a_ch, beta, S0)
    o4, _ = oracle.gdn_recurrence_chgate(q, k, v, a_ch, beta, S0)
    assert np.max(np.abs(o3 - o4)) > 1e-2


def test_kgla_steps_chain_to_recurrence():
    B, T, H, Dk, Dv = 2, 5, 2, 4, 3
    q, k, v, a_ch, beta, S0 = _rand_chgate(B, T, H, Dk, Dv, RNG)
    out, ST = oracle.kgla(q, k, v, a_ch, beta, S0, scale=0.7)
    S = S0
    for t in range(T):
        o, S = oracle.kgla_step(q[:, t], k[:, t], v[:, t], a_ch[:, t], beta[:, t], S, scale=0.7)
        np.testing.assert_array_equal(o, out[:, t])
    np.testing.assert_array_equal(S, ST)


# --------------------------------------------------------------------------
# Backward of the recurrence (the gradients a layer trained through the mixer
# needs).  Pinned by torch autograd over a plain token loop (fp64, CPU) and by
# central finite differences of the oracle's own forward.
# --------------------------------------------------------------------------
def _torch_forward(q, k, v, a, b, S0, scale):
    B, T, H, Dk = q.shape
    outs, S = [], S0
    for t in range(T):
        kt, vt, qt = k[:, t], v[:, t], q[:, t]                    # [B,H,D]
        at, bt = a[:, t][..., None, None], b[:, t][..., None, None]
        p = torch.einsum("bhi,bhij->bhj", kt, S)
        S = at * (S - bt * kt[..., :, None] * p[..., None, :]) + bt * kt[..., :, None] * vt[..., None, :]
        outs.append(scale * torch.einsum("bhij,bhi->bhj", S, qt))
    return torch.stack(outs, 1), S


@pytest.mark.parametrize("Dk,Dv", [(4, 3), (3, 5)])
def test_backward_matches_torch_autograd(Dk, Dv):
    B, T, H = 2, 7, 2
    q, k, v, alpha, beta, S0 = _rand_gdn(B, T, H, Dk, Dv, RNG)
    dout = RNG.standard_normal((B, T, H, Dv))
    dST = RNG.standard_normal((B, H, Dk, Dv))
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True)
          for x in (q, k, v, alpha, beta, S0)]
    o, ST = _torch_forward(*ts, 0.7)
    ((o * torch.from_numpy(dout)).sum() + (ST * torch.from_numpy(dST)).sum()).backward()
    r = oracle.gdn_recurrence_backward(q, k, v, alpha, beta, dout, S0, dST, scale=0.7)
    for name, t in zip(("dq", "dk", "dv", "dalpha", "dbeta", "dstate_in"), ts):
        np.testing.assert_allclose(r[name], t.grad.numpy(), atol=1e-11, rtol=1e-9, err_msg=name)


def test_backward_matches_finite_differences():
    B, T, H, Dk, Dv = 1, 6, 1, 3, 2
    q, k, v, alpha, beta, S0 = _rand_gdn(B, T, H, Dk, Dv, RNG)
    dout = RNG.standard_normal((B, T, H, Dv))
    r = oracle.gdn_recurrence_backward(q, k, v, alpha, beta, dout, S0)

    def loss(xs):
        o, _ = oracle.gdn_recurrence(*xs)
        return float((o * dout).sum())

    xs = [q, k, v, alpha, beta, S0]
    names = ("dq", "dk", "dv", "dalpha", "dbeta", "dstate_in")
    eps = 1e-6
    for i, name in enumerate(names):
        d = RNG.standard_normal(xs[i].shape)
        plus = [x.copy() for x in xs]
        minus = [x.copy() for x in xs]
        plus[i] = plus[i] + eps * d
        minus[i] = minus[i] - eps * d
        fd = (loss(plus) - loss(minus)) / (2 * eps)
        np.testing.assert_allclose(float((r[name] * d).sum()), fd, rtol=1e-6, atol=1e-8,
                                   err_msg=name)
