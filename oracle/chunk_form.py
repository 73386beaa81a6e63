"""Chunk-parallel (UT transform) form of the Gated Delta Rule in float64.

TEST INFRASTRUCTURE ONLY — pins the token-loop oracle through the method's
central claim: processing C tokens at a time through the entering state gives
the same outputs and final state as the token loop (Gated DeltaNet blog post,
torch_chunk_gated_delta_rule; lite_boost.ops.chunk_gated_delta_rule, formula
section; inferencelayer deltanet.rs, core_chunk).

For one chunk of n <= C tokens with entering state S0 and in-chunk cumulative
log decay gamma_r = g_0 + ... + g_r (all zeros when g is absent):

  A[r, i] = beta_r (k_r . k_i) exp(gamma_r - gamma_i)  for i < r, else 0
  T       = (I + A)^-1                                   unit lower triangular
  Vnew    = T diag(beta) (V - diag(exp(gamma)) K S0)     pseudo-values
  P[r, i] = (q_r . k_i) exp(gamma_r - gamma_i)           for i <= r, else 0
  O       = scale (diag(exp(gamma)) Q S0 + P Vnew)
  S_next  = exp(gamma_{n-1}) S0 + (diag(exp(gamma_{n-1} - gamma)) K)^T Vnew

The pseudo-value u_r is what the token at r actually writes once every earlier
token of the chunk and the entering state are accounted for; decay ratios are
taken as differences of log decays before exponentiating. The solve uses a
library triangular solve. A final partial chunk uses n < C.
"""
import numpy as np
from scipy.linalg import solve_triangular


def chunked(q, k, v, beta, g=None, state=None, scale=1.0, chunk=64):
    """One sequence on one head. q, k: (L, Dk); v: (L, Dv); beta, g: (L,).
    Returns (out (L, Dv), final state (Dk, Dv))."""
    q, k, v, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, beta))
    L, Dk = k.shape
    Dv = v.shape[1]
    S = np.zeros((Dk, Dv)) if state is None else np.array(state, dtype=np.float64, copy=True)
    out = np.zeros((L, Dv))
    for c0 in range(0, L, chunk):
        c1 = min(c0 + chunk, L)
        n = c1 - c0
        Q, K, V, b = q[c0:c1], k[c0:c1], v[c0:c1], beta[c0:c1]
        gam = np.zeros(n) if g is None else np.cumsum(np.asarray(g[c0:c1], dtype=np.float64))
        diff = gam[:, None] - gam[None, :]
        lower_strict = np.tril(np.ones((n, n), dtype=bool), -1)
        lower = np.tril(np.ones((n, n), dtype=bool), 0)
        decay = np.where(lower, np.exp(np.where(lower, diff, 0.0)), 0.0)
        A = np.where(lower_strict, b[:, None] * (K @ K.T) * decay, 0.0)
        rhs = b[:, None] * (V - np.exp(gam)[:, None] * (K @ S))
        Vnew = solve_triangular(np.eye(n) + A, rhs, lower=True, unit_diagonal=True)
        P = np.where(lower, (Q @ K.T) * decay, 0.0)
        out[c0:c1] = scale * (np.exp(gam)[:, None] * (Q @ S) + P @ Vnew)
        S = np.exp(gam[-1]) * S + (np.exp(gam[-1] - gam)[:, None] * K).T @ Vnew
    return out, S
