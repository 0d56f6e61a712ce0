"""The chunked reverse mode that the d = 128 backward kernels implement,
written out in f64 numpy (per chunk: the forward chunk form, the state sweep,
the reverse state-gradient sweep and the per-chunk gradients, in the
kernels' order), checked against the oracle's token-loop adjoint of the
section 3.1.2 update ("The Key to Going Linear: Analysis-Driven Transformer
Linearization").  It pins the derivation on the CPU: a dropped term or a
wrong sign in any gradient formula fails here before any kernel runs.  The
numpy code below is test code only; the kernels share nothing with it."""
import numpy as np
import pytest

import oracle
import synthetic


def _chunked_backward(q, k, v, alpha, beta, dout, s0, dsT, scale, C):
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    NC = (T + C - 1) // C
    res = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
               dalpha=np.zeros_like(alpha), dbeta=np.zeros_like(beta),
               dstate_in=np.zeros((B, H, Dk, Dv)))
    for b in range(B):
        for h in range(H):
            def pad(x, fill):
                out = np.full((NC * C,) + x.shape[1:], fill, dtype=np.float64)
                out[:T] = x
                return out
            Q, K, V = pad(q[b, :, h], 0.), pad(k[b, :, h], 0.), pad(v[b, :, h], 0.)
            A_, Bt, dO = pad(alpha[b, :, h], 1.), pad(beta[b, :, h], 0.), pad(dout[b, :, h], 0.)
            # per-chunk record: gates, Gram matrices, Tm, P
            rec = []
            for c in range(NC):
                sl = slice(c * C, (c + 1) * C)
                gam = np.cumsum(np.log(A_[sl]))
                G = np.exp(gam[:, None] - gam[None, :])
                Gk = K[sl] @ K[sl].T
                A = np.tril(Bt[sl][:, None] * G * Gk, -1)
                Tm = np.linalg.inv(np.eye(C) + A)
                P = np.tril(scale * G * (Q[sl] @ K[sl].T))
                rec.append((gam, G, Gk, A, Tm, P))
            # state sweep: S entering each chunk, Vm, U
            S = np.zeros((Dk, Dv)) if s0 is None else s0[b, h].copy()
            fw = []
            for c in range(NC):
                sl = slice(c * C, (c + 1) * C)
                gam, G, Gk, A, Tm, P = rec[c]
                g, d = np.exp(gam), np.exp(gam[-1] - gam)
                Vm = V[sl] - g[:, None] * (K[sl] @ S)
                U = Tm @ (Bt[sl][:, None] * Vm)
                fw.append((S.copy(), Vm, U))
                S = g[-1] * S + (d[:, None] * K[sl]).T @ U
            # reverse sweep of the state gradient
            dS = np.zeros((Dk, Dv)) if dsT is None else dsT[b, h].copy()
            bw = [None] * NC
            for c in reversed(range(NC)):
                sl = slice(c * C, (c + 1) * C)
                gam, G, Gk, A, Tm, P = rec[c]
                g, d = np.exp(gam), np.exp(gam[-1] - gam)
                dU = P.T @ dO[sl] + d[:, None] * (K[sl] @ dS)
                dY = Tm.T @ dU
                bw[c] = (dS.copy(), dU, dY)
                dX = -(Bt[sl] * g)[:, None] * dY
                dS = g[-1] * dS + (scale * g[:, None] * Q[sl]).T @ dO[sl] + K[sl].T @ dX
            res["dstate_in"][b, h] = dS
            # per-chunk gradients
            for c in range(NC):
                sl = slice(c * C, (c + 1) * C)
                n = min(T, (c + 1) * C) - c * C
                gam, G, Gk, A, Tm, P = rec[c]
                g, d = np.exp(gam), np.exp(gam[-1] - gam)
                S, Vm, U = fw[c]
                dSn, dU, dY = bw[c]
                Kc, Qc, bc = K[sl], Q[sl], Bt[sl]
                dX = -(bc * g)[:, None] * dY
                dQS = (scale * g[:, None] * dO[sl]) @ S.T
                Z1 = dX @ S.T
                Z2 = (d[:, None] * U) @ dSn.T
                dP = np.tril(dO[sl] @ U.T)
                dT = np.tril(dU @ (bc[:, None] * Vm).T, -1)
                dA = np.tril(-(Tm.T @ dT @ Tm.T), -1)
                E1 = dP * scale * np.tril(G)
                E2 = bc[:, None] * dA * G
                dq = dQS + E1 @ Kc
                dk = Z1 + Z2 + E1.T @ Qc + (E2 + E2.T) @ Kc
                F = dP * P + dA * A
                dgam = ((dQS * Qc).sum(1) + (Z1 * Kc).sum(1) - (Z2 * Kc).sum(1)
                        + F.sum(1) - F.sum(0))
                dgam[-1] += g[-1] * (dSn * S).sum() + (Z2 * Kc).sum()
                dbeta = (dY * Vm).sum(1) + (dA * G * Gk).sum(1)
                dla = np.cumsum(dgam[::-1])[::-1]
                res["dq"][b, c * C:c * C + n, h] = dq[:n]
                res["dk"][b, c * C:c * C + n, h] = dk[:n]
                res["dv"][b, c * C:c * C + n, h] = (bc[:, None] * dY)[:n]
                res["dbeta"][b, c * C:c * C + n, h] = dbeta[:n]
                res["dalpha"][b, c * C:c * C + n, h] = (dla / A_[sl])[:n]
    return res


# (B, T, H, Dk, Dv, chunk, initial state, key concentration): ragged tails, one
# exact chunk, Dk != Dv, keys at mean-key cosine 0.9 and 1.0 with beta near 1.
@pytest.mark.parametrize("B,T,H,Dk,Dv,C,s0,cos,bshift", [
    (1, 100, 2, 16, 8, 16, "randn", None, 0.0),
    (2, 70, 1, 32, 32, 32, "zero", None, 0.0),
    (1, 64, 1, 16, 16, 64, "randn", None, 0.0),
    (1, 130, 1, 32, 16, 64, "randn", 0.9, 0.0),
    (1, 90, 1, 16, 24, 32, "randn", 1.0, 3.0),
])
def test_chunked_reverse_mode_matches_token_adjoint(B, T, H, Dk, Dv, C, s0, cos, bshift):
    x = synthetic.gdn_inputs(B, T, H, Dk, Dv, dtype="f32", seed=T + C, state0=s0, key_cos=cos,
                             beta_shift=bshift)
    f = lambda t: None if t is None else t.double().numpy()  # noqa: E731
    rng = np.random.default_rng(T)
    dout = rng.standard_normal((B, T, H, Dv))
    dsT = rng.standard_normal((B, H, Dk, Dv))
    args = [f(x[n]) for n in ("q", "k", "v", "alpha", "beta")]
    ref = oracle.gdn_recurrence_backward(*args, dout, f(x["state0"]), dsT, scale=0.7)
    got = _chunked_backward(*args, dout, f(x["state0"]), dsT, 0.7, C)
    for n in ref:
        assert oracle.rms_normalised_max_error(got[n], ref[n]) < 1e-9, n
