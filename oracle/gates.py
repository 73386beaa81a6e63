"""Fused preprocessing of the Gated DeltaNet layer, in float64 — TEST
INFRASTRUCTURE ONLY: the gates, and the optional q/k normalisation.

The Gated DeltaNet blog post's layer code forms the write strength and the log
decay right before the recurrence, from the gate projections b and a and the
per-value-head parameters A_log and dt_bias:

    beta = sigmoid(b),    g = -exp(A_log) * softplus(a + dt_bias)

inferencelayer deltanet.rs states the same in its module header and forms
them per token in its recurrent step, its chunk form and its step/chunk
kernels. Written out here from those definitions, with
sigmoid(x) = 1 / (1 + e^-x) and softplus(x) = ln(1 + e^x). The recurrence
oracle then takes beta and g as usual.

With use_qk_l2norm_in_kernel the blog post's recurrent and chunk functions
first replace q and k by l2norm(x) = x / sqrt(sum(x^2) + 1e-6) over the head
dimension; deltanet.rs's l2norm is the same, eps inside the square root.
"""
import numpy as np


def sigmoid(x):
    """1 / (1 + e^-x), elementwise in float64 (e^-x is formed only for x >= 0
    and e^x only for x < 0, so no intermediate overflows)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def softplus(x):
    """ln(1 + e^x), elementwise in float64: max(x, 0) + ln(1 + e^-|x|)."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def gates(beta_logits, a, A_log, dt_bias):
    """beta and g of the fused-gate call.

    beta_logits, a: (..., Nv, S); A_log, dt_bias: (Nv,) per value head.
    Returns (beta, g), each (..., Nv, S) float64.
    """
    b = np.asarray(beta_logits, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    A_log = np.asarray(A_log, dtype=np.float64)[:, None]
    dt_bias = np.asarray(dt_bias, dtype=np.float64)[:, None]
    return sigmoid(b), -np.exp(A_log) * softplus(a + dt_bias)


def l2norm(x, eps=1e-6):
    """x / sqrt(sum(x^2) + eps) over the last axis, in float64."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + eps)
