"""The gated delta rule in chunks, in numpy fp64 -- the chunkwise algorithm of [Kazeia]
"Chunkwise (delta rule)" / "P1 -- chunk f32", derived here from the token recurrence;
used only to pin the oracle's token-by-token recurrence (an independent algorithm that
must reach the same result up to rounding).

Within a chunk of n tokens with entry state S0, let lg_t = alpha_1 + ... + alpha_t (the
log of the cumulative gate) and R[t, s] = exp(lg_t - lg_s) for s <= t.  Unrolling
S_t = g_t S_{t-1} + k_t d_t^T gives S_t = e^{lg_t} S0 + sum_{s<=t} R[t,s] k_s d_s^T, and
the delta updates d satisfy (I + A) D = diag(beta) (V - diag(e^lg) K S0) with A strictly
lower triangular, A[t,s] = beta_t R[t,s] k_t.k_s.  So, with T = (I + A)^-1:
    U = T diag(beta) V,   W = T diag(beta e^lg) K,   D = U - W S0
    O = diag(e^lg) Q S0 + (tril(R) * Q K^T) D
    S = e^{lg_n} S0 + K^T diag(R[n, :]) D
"""
import numpy as np


def gdn_chunkwise(q, k, v, beta, alpha, s0=None, C=64):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    beta, alpha = np.asarray(beta, np.float64), np.asarray(alpha, np.float64)
    B, H, P, dk = q.shape
    dv = v.shape[3]
    out = np.zeros((B, H, P, dv))
    st = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if s0 is None else np.asarray(s0[b, h], np.float64).copy()
            for c0 in range(0, P, C):
                n = min(C, P - c0)
                Q, K, V = q[b, h, c0:c0 + n], k[b, h, c0:c0 + n], v[b, h, c0:c0 + n]
                be = beta[b, h, c0:c0 + n]
                lg = np.cumsum(alpha[b, h, c0:c0 + n])
                R = np.exp(lg[:, None] - lg[None, :])
                A = np.tril(be[:, None] * R * (K @ K.T), -1)
                T = np.linalg.inv(np.eye(n) + A)
                U = T @ (be[:, None] * V)
                W = T @ ((be * np.exp(lg))[:, None] * K)
                Dl = U - W @ S
                out[b, h, c0:c0 + n] = np.exp(lg)[:, None] * (Q @ S) + (np.tril(R) * (Q @ K.T)) @ Dl
                S = np.exp(lg[-1]) * S + K.T @ (R[-1][:, None] * Dl)
            st[b, h] = S
    return out, st
