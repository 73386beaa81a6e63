"""Gated RMSNorm output epilogue, in float64 — TEST INFRASTRUCTURE ONLY.

inferencelayer deltanet.rs (module header; the per-head gated RMSNorm of its
recurrent step and chunk form, and of its DN_STEP / DN_CHUNK kernels) ends the
layer's core with, per token and value head, on the output row o of Dv values:

    out_j = o_j * w_j * silu(z_j) / sqrt(mean_j(o_j^2) + eps),
    silu(x) = x / (1 + e^-x) = x * sigmoid(x),

w being one weight vector of Dv values shared by all heads and z the gate
projection of the same shape as o. The mean runs over the head's Dv columns
(not their sum) and eps sits inside the square root. The Gated DeltaNet blog
post's layer comment writes sigmoid(z) for the gate factor; its code (like
deltanet.rs and the model's hidden activation) uses silu, which is what is
written here. A row with mean + eps == 0 (o all zeros and eps = 0) is taken to
stay zero rather than 0/0.
"""
import numpy as np

from .gates import sigmoid


def silu(x):
    """x * sigmoid(x), elementwise in float64."""
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)


def gated_rmsnorm(o, z, w, eps):
    """The epilogue over the last axis: o, z (..., Dv); w (Dv,); eps >= 0."""
    o = np.asarray(o, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    m = (o * o).mean(-1, keepdims=True) + float(eps)
    safe = np.where(m > 0.0, m, 1.0)
    inv = np.where(m > 0.0, 1.0 / np.sqrt(safe), 0.0)
    return o * inv * w * silu(z)
