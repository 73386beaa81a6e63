"""NumPy model of the bf16 prefill kernel's arithmetic (test code).

It restates, in plain NumPy, where the matrix-core path rounds: operands of
every product are bf16 (round to nearest even), products accumulate in
float32, and float32 work happens where the kernel keeps float32. It is not
the oracle and is not used by the library; the tests use it on the CPU to
show that an algorithm's rounding stays inside the tolerance for inputs the
GPU tests cannot cover exhaustively (keys of a chunk that are nearly or
exactly equal). The quantity it models is the UT-transform inverse of the
chunked form (Gated DeltaNet blog post, torch_chunk_gated_delta_rule, the
forward-substitution step; lite_boost.ops.chunk_gated_delta_rule, formula
section): T = (I + A)^-1 with A = strict_lower(diag(beta) K K^T * exp(gamma_r - gamma_i)).
"""
import numpy as np

LOG2E = np.float32(1.4426950408889634)


def bf(x):
    """float32 -> nearest-even bf16 value, as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (((u >> 16) & 1) + 0x7FFF + u) >> 16
    return (r.astype(np.uint32) << 16).view(np.float32).reshape(x.shape)


def mm(a, b):
    """Matrix-core product: bf16 operands, float32 result."""
    return (bf(a).astype(np.float64) @ bf(b).astype(np.float64)).astype(np.float32)


def chunk_A(K, beta, g=None):
    """A of one chunk as the kernel forms it: the Gram K K^T from bf16 keys in
    float32, the decay ratio exp2 of a difference of log2 cumulative decays."""
    C = K.shape[0]
    G = mm(K, K.T)
    gam2 = np.zeros(C, np.float32) if g is None else (np.cumsum(np.asarray(g, np.float32)).astype(np.float32) * LOG2E)
    r = np.arange(C)
    below = r[:, None] > r[None, :]
    ex = np.exp2(np.where(below, gam2[:, None] - gam2[None, :], -np.inf)).astype(np.float32)
    return (np.asarray(beta, np.float32)[:, None] * ex * G).astype(np.float32)


def fsub16(A16):
    """(I + A)^-1 of a 16x16 strictly lower A by forward substitution in
    float32: row m, final at step m, is subtracted A[r, m] times from every
    row r (A[r, m] = 0 for r <= m)."""
    X = np.eye(16, dtype=np.float32)
    for m in range(15):
        X = (X - A16[:, m:m + 1] * X[m:m + 1, :]).astype(np.float32)
    return X


def merge(D0, D1, A10):
    """Inverse of [[I + ., 0], [A10, I + .]] from the inverses of its diagonal
    blocks: T_10 = -D1 A10 D0, on the matrix cores (bf16 operands)."""
    n = D0.shape[0]
    T = np.zeros((2 * n, 2 * n), np.float32)
    T[:n, :n], T[n:, n:] = D0, D1
    T[n:, :n] = -mm(D1, mm(A10, D0))
    return T


def t_blocked(A):
    """T = (I + A)^-1 of a 64-token chunk as the T kernel computes it: 16x16
    diagonal blocks by forward substitution, merged into 32-blocks, then into
    the chunk; the result stored in bf16."""
    D = [fsub16(A[16 * i:16 * i + 16, 16 * i:16 * i + 16]) for i in range(4)]
    T00 = merge(D[0], D[1], A[16:32, 0:16])
    T11 = merge(D[2], D[3], A[48:64, 32:48])
    return bf(merge(bf(T00), bf(T11), A[32:, :32]))


def t_power_series(A):
    """The product form (I - A)(I + A^2)(I + A^4)(I + A^8)(I + A^16) of each
    32x32 diagonal block (A is nilpotent there), every factor on the matrix
    cores, merged like t_blocked. Exact in exact arithmetic, but its powers
    grow far beyond T before they cancel when keys are alike; kept to show
    that the tests below tell the two solves apart."""
    def dinv(Ad):
        N = -Ad
        R = np.eye(32, dtype=np.float32) + N
        M = mm(N, N)
        for _ in range(4):
            R = (R + mm(M, R)).astype(np.float32)
            M = mm(M, M)
        return R
    T00, T11 = dinv(A[:32, :32]), dinv(A[32:, 32:])
    return bf(merge(bf(T00), bf(T11), A[32:, :32]))


def t_exact(A):
    return np.linalg.inv(np.eye(A.shape[0]) + A.astype(np.float64))


def prefill_model(q, k, v, beta, g, S0, scale, tsolve=t_blocked, C=64):
    """One sequence on one value head through the bf16 kernel's chunk step
    (float32 arrays holding bf16 values). Per chunk, with T from tsolve:
      W = T diag(beta e^gamma) K and U = T diag(beta) V, the first factor and
      W rounded to bf16; Vnew = U - W S0 with S0 as a bf16 operand;
      O = scale e^gamma Q S0 + P Vnew with P = scale (Q K^T * decay) and Vnew
      as bf16 operands, O stored in bf16;
      S = e^{gamma_C} S0 + K^T (decay Vnew) with float32 accumulation.
    Returns (out (L, Dv), final state (Dk, Dv)), both bf16 values."""
    L, Dk = k.shape
    Dv = v.shape[1]
    S = np.zeros((Dk, Dv), np.float32) if S0 is None else np.array(S0, np.float32)
    out = np.zeros((L, Dv), np.float32)
    r = np.arange(C)
    for c0 in range(0, L, C):
        n = min(C, L - c0)
        K = np.zeros((C, Dk), np.float32)
        Q = np.zeros_like(K)
        V = np.zeros((C, Dv), np.float32)
        b = np.zeros(C, np.float32)
        gg = np.zeros(C, np.float32)
        K[:n], Q[:n], V[:n], b[:n] = k[c0:c0 + n], q[c0:c0 + n], v[c0:c0 + n], beta[c0:c0 + n]
        if g is not None:
            gg[:n] = g[c0:c0 + n]
        gam2 = (np.cumsum(gg).astype(np.float32) * LOG2E).astype(np.float32)
        eg = np.exp2(gam2).astype(np.float32)
        T = tsolve(chunk_A(K, b, None if g is None else gg))
        W = bf(mm(bf(T * (b * eg)[None, :]), K))
        U = mm(bf(T * b[None, :]), V)
        vn = (U - mm(W, S)).astype(np.float32)
        vec = np.where(r < n, np.float32(scale) * eg, 0).astype(np.float32)
        decq = np.exp2(np.where(r[:, None] >= r[None, :], gam2[:, None] - gam2[None, :], -np.inf)).astype(np.float32)
        P = bf(np.float32(scale) * decq * mm(Q, K.T))
        o = (mm(Q, S) * vec[:, None] + mm(P, vn)).astype(np.float32)
        out[c0:c0 + n] = bf(o)[:n]
        d = np.exp2(gam2[-1] - gam2).astype(np.float32)
        S = (S * np.exp2(gam2[-1]) + mm(K.T, vn * d[:, None])).astype(np.float32)
    return out, bf(S)
