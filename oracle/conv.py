"""Depthwise causal conv1d + SiLU ahead of the recurrence, in float64 — TEST
INFRASTRUCTURE ONLY.

The Gated DeltaNet layer (the blog post's layer code; inferencelayer
deltanet.rs, the conv ring of its step and chunk code and the DN_CONV kernel)
runs the fused q/k/v projection, C = 2 Nk Dk + Nv Dv channels per token,
through a depthwise causal convolution of K taps followed by SiLU, then
splits the channels into q (Nk heads of Dk), k (Nk x Dk) and v (Nv x Dv):

    y_t[c] = silu(bias[c] + sum_{j=0}^{K-1} w[c, j] x_{t-K+1+j}[c])

taps oldest first, inputs before the first token taken from the carried
state (zeros for a fresh sequence). The state carried between calls is the
last K - 1 inputs of every channel, oldest first (deltanet.rs keeps a ring of
K whose oldest entry never reaches another output; the blog post pads to K).
Decode follows the recurrence's slot rule: the entering state comes from slot
idx[b*S + n - 1] (n = accepted tokens, else the length) and the state after
valid token t goes to slot idx[b*S + t].
"""
import numpy as np

from .epilogue import silu


def split(y, Nk, Dk, Nv, Dv):
    """(B, S, C) -> q (B, Nk, S, Dk), k (B, Nk, S, Dk), v (B, Nv, S, Dv)."""
    B, S, _ = y.shape
    nq = Nk * Dk
    q = y[:, :, :nq].reshape(B, S, Nk, Dk).transpose(0, 2, 1, 3)
    k = y[:, :, nq:2 * nq].reshape(B, S, Nk, Dk).transpose(0, 2, 1, 3)
    v = y[:, :, 2 * nq:].reshape(B, S, Nv, Dv).transpose(0, 2, 1, 3)
    return q, k, v


def _step(win, x, w, bias):
    """One token for all channels: win (C, K-1) oldest first, x (C,). Returns
    (output (C,), new window)."""
    K = w.shape[1]
    acc = w[:, K - 1] * x + (bias if bias is not None else 0.0)
    for j in range(K - 1):
        acc = acc + w[:, j] * win[:, j]
    new = np.concatenate([win[:, 1:], x[:, None]], axis=1) if K > 1 else win
    return silu(acc), new


def prefill(x, w, bias, init, lens):
    """x (B, S, C); w (C, K); bias (C,) or None; init (B, C, K-1) or None;
    lens (B,) or None. Returns (y (B, S, C) with zero rows past each length,
    final state (B, C, K-1))."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    bias = None if bias is None else np.asarray(bias, dtype=np.float64)
    B, S, C = x.shape
    K = w.shape[1]
    y = np.zeros((B, S, C))
    fin = np.zeros((B, C, K - 1))
    for b in range(B):
        L = S if lens is None else min(max(int(lens[b]), 0), S)
        win = np.zeros((C, K - 1)) if init is None else np.asarray(init[b], dtype=np.float64).copy()
        for t in range(L):
            y[b, t], win = _step(win, x[b, t], w, bias)
        fin[b] = win
    return y, fin


def decode(x, w, bias, pool, lens, idx, n_acc):
    """x (B, S, C); pool (slots, C, K-1); lens (B,); idx (B*S,); n_acc (B,) or
    None. Returns (y (B, S, C), updated pool)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    bias = None if bias is None else np.asarray(bias, dtype=np.float64)
    pool = np.asarray(pool, dtype=np.float64).copy()
    B, S, C = x.shape
    slots = pool.shape[0]
    y = np.zeros((B, S, C))
    for b in range(B):
        L = min(max(int(lens[b]), 0), S)
        n = L if n_acc is None else int(n_acc[b])
        if L == 0 or n < 1 or n > S:
            continue
        r = int(idx[b * S + n - 1])
        if not 0 <= r < slots:
            continue
        win = pool[r].copy()
        for t in range(L):
            y[b, t], win = _step(win, x[b, t], w, bias)
            s = int(idx[b * S + t])
            if 0 <= s < slots:
                pool[s] = win
    return y, pool
