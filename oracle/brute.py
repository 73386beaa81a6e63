"""Brute-force unrolled form of the Gated Delta Rule (float64, tiny sizes only).

TEST INFRASTRUCTURE ONLY — pins the token-loop oracle.

Every token is an affine map of the state (ssm_lab.py, delta_rule_recurrent,
matrix form of the gated delta rule; inferencelayer deltanet.rs, core_chunk
derivation):

    S_t = M_t S_{t-1} + N_t,   M_t = (I - beta_t k_t k_t^T) D_t,   N_t = beta_t k_t v_t^T,

with D_t = exp(g_t) * diag(exp(gk_t)) the decay (identity scale when g is
absent, no per-key factor when gk is absent). Here each S_t is rebuilt from
scratch as the explicit sum

    S_t = (M_t ... M_1) S_0 + sum_{i<=t} (M_t ... M_{i+1}) N_i,

using dense Dk x Dk matrices, and o_t = scale * S_t^T q_t. Nothing is carried
from one t to the next except the inputs.
"""
import numpy as np


def transitions(k, v, beta, g=None, gk=None):
    L, Dk = k.shape
    Ms, Ns = [], []
    for t in range(L):
        d = np.ones(Dk) * (np.exp(g[t]) if g is not None else 1.0)
        if gk is not None:
            d = d * np.exp(gk[t])
        Dt = np.diag(d)
        kt = k[t][:, None]
        Ms.append((np.eye(Dk) - beta[t] * (kt @ kt.T)) @ Dt)
        Ns.append(beta[t] * (kt @ v[t][None, :]))
    return Ms, Ns


def unrolled(q, k, v, beta, g=None, gk=None, state=None, scale=1.0):
    """Returns (out (L, Dv), all states (L, Dk, Dv))."""
    q, k, v, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, beta))
    L, Dk = k.shape
    Dv = v.shape[1]
    S0 = np.zeros((Dk, Dv)) if state is None else np.asarray(state, dtype=np.float64)
    Ms, Ns = transitions(k, v, beta, g, gk)
    outs, states = [], []
    for t in range(L):
        prod = np.eye(Dk)
        for j in range(t, -1, -1):       # prod = M_t ... M_{j}
            prod = prod @ Ms[j]
        St = prod @ S0
        for i in range(t + 1):
            P = np.eye(Dk)
            for j in range(t, i, -1):    # P = M_t ... M_{i+1}
                P = P @ Ms[j]
            St = St + P @ Ns[i]
        states.append(St)
        outs.append(scale * (St.T @ q[t]))
    return np.array(outs).reshape(L, Dv), np.array(states).reshape(L, Dk, Dv)
