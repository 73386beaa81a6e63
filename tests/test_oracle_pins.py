"""Pins the float64 oracle to things other than itself.

Each test ties the token-loop oracle to a value printed on the pages, a closed
form, an independent algorithm (brute force, the chunked UT form) or an
invariant, chosen so that a dropped term, a wrong sign or index, or a
transposed operand in the oracle fails at least one of them.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import brute, chunk_form
from tests.conftest import read_golden


def _rand_unit(rng, n, d):
    x = rng.standard_normal((n, d))
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + 1e-6)


def _rand_seq(rng, L, Dk, Dv, gate=True, gk=False, s0=True):
    q = _rand_unit(rng, L, Dk)
    k = _rand_unit(rng, L, Dk)
    v = rng.standard_normal((L, Dv))
    beta = 1 / (1 + np.exp(-rng.standard_normal(L)))
    g = -np.exp(rng.uniform(-2, 1)) * np.log1p(np.exp(rng.standard_normal(L) + rng.uniform(-1, 1))) if gate else None
    gkv = rng.uniform(-0.5, -0.001, (L, Dk)) if gk else None
    S0 = rng.standard_normal((Dk, Dv)) * 0.3 if s0 else None
    return q, k, v, beta, g, gkv, S0


# --- values printed on the deltanet.rs page ---------------------------------

def test_hand_computed_step():
    f = read_golden("deltanet_rs_hand_step.txt")
    S0 = np.array(f["S0"]).reshape(2, 2)
    out, S = oracle.sequence(np.array([f["q"]]), np.array([f["k"]]), np.array([f["v"]]),
                             np.array(f["beta"]), g=np.array(f["g"]), state=S0,
                             scale=f["scale"][0])
    np.testing.assert_allclose(out[0], f["out"], atol=1e-12, rtol=0)
    np.testing.assert_allclose(S.reshape(-1), f["S"], atol=1e-12, rtol=0)


def test_decay_applies_before_read():
    f = read_golden("deltanet_rs_decay_first.txt")
    S0 = np.array(f["S0"]).reshape(2, 2)
    out, S = oracle.sequence(np.array([f["q"]]), np.array([f["k"]]), np.array([f["v"]]),
                             np.array(f["beta"]), g=np.array(f["g"]), state=S0,
                             scale=f["scale"][0])
    assert abs(out[0, 0] - f["out0"][0]) < 1e-12
    assert abs(S[0, 0] - f["S00"][0]) < 1e-12
    # A read before the decay would give kv = 2, delta = -1, S[0,0] = 0: a different answer.
    assert abs(S[0, 0]) > 0.5


def test_beta_one_is_pure_delta_rule_closed_form():
    f = read_golden("deltanet_rs_beta_one.txt")
    Dk, Dv = int(f["Dk"][0]), int(f["Dv"][0])
    S0 = np.array([((n * 37 % 11) - 5) * 0.1 for n in range(Dk * Dv)]).reshape(Dk, Dv)
    k = np.array(f["k_raw"])
    k = k / math.sqrt((k * k).sum() + 1e-6)
    v = np.array(f["v"])
    _, S = oracle.sequence(np.array([f["q"]]), k[None], v[None], np.array(f["beta"]),
                           g=np.array(f["g"]), state=S0, scale=1.0)
    expect = S0 - np.outer(k, k @ S0) + np.outer(k, v)
    np.testing.assert_allclose(S, expect, atol=1e-12, rtol=0)
    assert np.abs(S - expect).max() < f["tolerance_on_page"][0]


def test_retention_at_g_minus_one():
    # The decode operator page: g = -1 keeps about 37 % of the state per step.
    S0 = np.eye(3)
    _, S = oracle.sequence(np.zeros((1, 3)), np.zeros((1, 3)), np.zeros((1, 3)),
                           np.zeros(1), g=np.array([-1.0]), state=S0)
    assert abs(S[0, 0] - 0.36787944117144233) < 1e-15
    assert round(S[0, 0], 2) == 0.37


# --- (a) brute force: explicit transition-matrix products --------------------

@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("gk", [False, True])
def test_brute_force_unrolled(seed, gk):
    rng = np.random.default_rng(1000 + seed)
    L = int(rng.integers(1, 7))
    Dk = int(rng.integers(1, 5))
    Dv = int(rng.integers(1, 5))
    q, k, v, beta, g, gkv, S0 = _rand_seq(rng, L, Dk, Dv, gate=seed % 3 != 0, gk=gk, s0=seed % 2 == 0)
    scale = 0.7
    out, S = oracle.sequence(q, k, v, beta, g=g, gk=gkv, state=S0, scale=scale)
    out_b, states_b = brute.unrolled(q, k, v, beta, g, gkv, S0, scale)
    np.testing.assert_allclose(out, out_b, atol=1e-12, rtol=0)
    np.testing.assert_allclose(S, states_b[-1], atol=1e-12, rtol=0)


# --- (b) store then recall with orthonormal keys -----------------------------

@pytest.mark.parametrize("Dk,n,rewrite", [(8, 6, 2), (16, 16, 5), (5, 3, 3)])
def test_store_then_recall(Dk, n, rewrite):
    rng = np.random.default_rng(Dk * 100 + n)
    Dv = 7
    Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    keys = Qm.T[:n]                         # n orthonormal rows
    vals = rng.standard_normal((n, Dv))
    new_vals = rng.standard_normal((rewrite, Dv))
    # Tokens: write all n pairs (each query recalls a random earlier key), then rewrite
    # the first `rewrite` keys, then read every key once with beta = 0.
    ks, vs, bs, qs, want = [], [], [], [], []
    for t in range(n):
        j = int(rng.integers(0, t + 1))
        ks.append(keys[t]); vs.append(vals[t]); bs.append(1.0); qs.append(keys[j]); want.append(vals[j])
    cur = vals.copy()
    for i in range(rewrite):
        cur[i] = new_vals[i]
        ks.append(keys[i]); vs.append(new_vals[i]); bs.append(1.0); qs.append(keys[i]); want.append(new_vals[i])
    for j in range(n):
        ks.append(keys[j]); vs.append(np.zeros(Dv)); bs.append(0.0); qs.append(keys[j]); want.append(cur[j])
    out, S = oracle.sequence(np.array(qs), np.array(ks), np.array(vs), np.array(bs),
                             g=np.zeros(len(ks)), state=None, scale=1.0)
    np.testing.assert_allclose(out, np.array(want), atol=1e-12, rtol=0)
    np.testing.assert_allclose(S.T @ keys.T, cur.T, atol=1e-12, rtol=0)


# --- (c) chunked == recurrent ------------------------------------------------

@pytest.mark.parametrize("C", [1, 4, 16, 64])
@pytest.mark.parametrize("gate", [True, False])
def test_chunked_equals_recurrent(C, gate):
    rng = np.random.default_rng(C * 7 + gate)
    for L, Dk, Dv, s0 in [(150, 16, 12, True), (64, 8, 8, False), (37, 32, 16, True), (5, 4, 4, True)]:
        q, k, v, beta, g, _, S0 = _rand_seq(rng, L, Dk, Dv, gate=gate, s0=s0)
        out, S = oracle.sequence(q, k, v, beta, g=g, state=S0, scale=0.3)
        out_c, S_c = chunk_form.chunked(q, k, v, beta, g, S0, 0.3, chunk=C)
        tol_o = 1e-10 * max(1.0, np.abs(out).max())
        tol_s = 1e-10 * max(1.0, np.abs(S).max())
        assert np.abs(out - out_c).max() <= tol_o
        assert np.abs(S - S_c).max() <= tol_s


def test_chunked_equals_recurrent_strong_decay():
    # Large negative log decays (gamma over a chunk in the hundreds): log-space ratios.
    rng = np.random.default_rng(99)
    L, Dk, Dv = 130, 16, 16
    q, k, v, beta, _, _, S0 = _rand_seq(rng, L, Dk, Dv)
    g = -rng.uniform(0.0, 10.0, L)
    out, S = oracle.sequence(q, k, v, beta, g=g, state=S0, scale=1.0)
    out_c, S_c = chunk_form.chunked(q, k, v, beta, g, S0, 1.0, chunk=64)
    assert np.isfinite(out_c).all() and np.isfinite(S_c).all()
    assert np.abs(out - out_c).max() <= 1e-10 * max(1, np.abs(out).max())
    assert np.abs(S - S_c).max() <= 1e-10 * max(1, np.abs(S).max())


# --- (d) g absent == alpha 1 -------------------------------------------------

def test_g_absent_is_bitwise_g_zero():
    rng = np.random.default_rng(5)
    B, Nk, Nv, S, D = 2, 1, 2, 9, 8
    q = _rand_unit(rng, B * Nk * S, D).reshape(B, Nk, S, D)
    k = _rand_unit(rng, B * Nk * S, D).reshape(B, Nk, S, D)
    v = rng.standard_normal((B, Nv, S, D))
    beta = rng.uniform(0, 1, (B, Nv, S))
    init = rng.standard_normal((B, Nv, D, D))
    o1, f1 = oracle.prefill(q, k, v, beta, None, init, [9, 4], 0.5)
    o2, f2 = oracle.prefill(q, k, v, beta, np.zeros((B, Nv, S)), init, [9, 4], 0.5)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)
    # and with a nonzero g the results differ
    o3, _ = oracle.prefill(q, k, v, beta, np.full((B, Nv, S), -0.1), init, [9, 4], 0.5)
    assert not np.array_equal(o1, o3)


# --- closed forms and reductions ---------------------------------------------

def test_pure_decay_closed_form():
    rng = np.random.default_rng(11)
    L, Dk, Dv = 6, 5, 3
    q, k, v, _, g, gk, S0 = _rand_seq(rng, L, Dk, Dv, gk=True)
    _, S = oracle.sequence(q, k, v, np.zeros(L), g=g, gk=gk, state=S0)
    expect = math.exp(g.sum()) * np.exp(gk.sum(0))[:, None] * S0
    np.testing.assert_allclose(S, expect, atol=1e-13, rtol=0)


def test_orthogonal_keys_reduce_to_decayed_linear_attention():
    # With mutually orthogonal keys and a zero entering state the memory read is
    # always zero, so the recurrence is gated linear attention with keys beta_t k_t
    # (ssm_lab.py, linear_attention_parallel with per-step decays):
    #   O = scale * ((Q (beta K)^T) * M) V,  M[t,s] = prod_{s<j<=t} alpha_j (s <= t).
    rng = np.random.default_rng(12)
    Dk, Dv, L = 12, 5, 9
    Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    k = Qm.T[:L]
    q = _rand_unit(rng, L, Dk)
    v = rng.standard_normal((L, Dv))
    beta = rng.uniform(0.1, 1.0, L)
    g = -rng.uniform(0.01, 1.0, L)
    out, _ = oracle.sequence(q, k, v, beta, g=g, scale=0.6)
    logc = np.cumsum(g)
    M = np.zeros((L, L))
    for t in range(L):
        for s in range(t + 1):
            M[t, s] = math.exp(logc[t] - logc[s])
    expect = 0.6 * ((q @ (beta[:, None] * k).T) * M) @ v
    np.testing.assert_allclose(out, expect, atol=1e-12, rtol=0)


def test_axis_keys_with_per_key_gate_reduce_to_linear_attention():
    # Standard-basis keys stay orthogonal under the per-key decay, so the same
    # reduction holds with a decay per key coordinate.
    rng = np.random.default_rng(13)
    Dk, Dv, L = 6, 4, 6
    perm = rng.permutation(Dk)[:L]
    k = np.eye(Dk)[perm]
    q = _rand_unit(rng, L, Dk)
    v = rng.standard_normal((L, Dv))
    beta = rng.uniform(0.1, 1.0, L)
    g = -rng.uniform(0.01, 0.5, L)
    gk = -rng.uniform(0.001, 0.5, (L, Dk))
    out, _ = oracle.sequence(q, k, v, beta, g=g, gk=gk, scale=1.0)
    expect = np.zeros((L, Dv))
    for t in range(L):
        for s in range(t + 1):
            i = perm[s]
            dec = math.exp(sum(g[s + 1:t + 1]) + sum(gk[s + 1:t + 1, i]))
            expect[t] += q[t, i] * beta[s] * dec * v[s]
    np.testing.assert_allclose(out, expect, atol=1e-12, rtol=0)


def test_dk1_is_an_ema():
    rng = np.random.default_rng(14)
    L, Dv = 20, 3
    k = rng.choice([-1.0, 1.0], L)[:, None]
    q = rng.choice([-1.0, 1.0], L)[:, None]
    v = rng.standard_normal((L, Dv))
    beta = rng.uniform(0, 1, L)
    g = -rng.uniform(0, 1, L)
    s0 = rng.standard_normal((1, Dv))
    out, S = oracle.sequence(q, k, v, beta, g=g, state=s0, scale=1.0)
    # closed form: S_t = P_t s0 + sum_i (P_t / P_i) beta_i k_i v_i, P_t = prod_{j<=t} alpha_j (1 - beta_j)
    a = np.exp(g) * (1 - beta)
    for t in range(L):
        St = np.prod(a[:t + 1]) * s0[0]
        for i in range(t + 1):
            St = St + np.prod(a[i + 1:t + 1]) * beta[i] * k[i, 0] * v[i]
        np.testing.assert_allclose(out[t], q[t, 0] * St, atol=1e-12, rtol=0)
    np.testing.assert_allclose(S[0], St, atol=1e-12, rtol=0)


def test_per_step_write_identity():
    # After token t: S_t^T k_t = (1 - beta ||k||^2) (D_t S_{t-1})^T k_t + beta ||k||^2 v_t,
    # for any k (not only unit k). Checked step by step on bf16-rounded inputs.
    import synth
    c = synth.config(3, B=2, Nk=1, Nv=2, Dk=32, Dv=16, slots=4)
    q, k, v, beta, g, gk = (c.f64(n) for n in ("q", "k", "v", "beta", "g", "gk"))
    S = synth.widen(c.state, c.dtype)[c.idx[0], 0]
    for t in range(c.S):
        kt, bt = k[0, 0, t], beta[0, 0, t]
        DS = math.exp(g[0, 0, t]) * np.exp(gk[0, 0, t])[:, None] * S
        _, S = oracle.sequence(q[0, 0, t:t + 1], k[0, 0, t:t + 1], v[0, 0, t:t + 1],
                               beta[0, 0, t:t + 1], g=g[0, 0, t:t + 1], gk=gk[0, 0, t:t + 1],
                               state=S)
        nk2 = kt @ kt
        lhs = S.T @ kt
        rhs = (1 - bt * nk2) * (DS.T @ kt) + bt * nk2 * v[0, 0, t]
        np.testing.assert_allclose(lhs, rhs, atol=1e-12, rtol=0)


def test_contractive_under_decay_and_bounded_beta():
    # deltanet.rs stability test scenario: 200 random steps, Dk = Dv = 8, norm stays bounded.
    rng = np.random.default_rng(42)
    d = 8
    S = np.zeros((d, d))
    peak = 0.0
    for _ in range(200):
        u = lambda n: rng.uniform(-0.5, 0.5, n)
        q = _rand_unit(rng, 1, d)
        k = _rand_unit(rng, 1, d)
        v = u(d)[None]
        g = np.array([-math.log1p(math.exp(u(1)[0] * 4))])
        beta = np.array([1 / (1 + math.exp(-u(1)[0] * 4))])
        # the decay-and-erase part alone never grows the Frobenius norm
        _, Sz = oracle.sequence(q, k, np.zeros((1, d)), beta, g=g, state=S)
        assert np.linalg.norm(Sz) <= np.linalg.norm(S) + 1e-12
        _, S = oracle.sequence(q, k, v, beta, g=g, state=S)
        peak = max(peak, np.linalg.norm(S))
        assert np.isfinite(S).all()
    assert peak < 20.0


# --- fused gates (blog post layer code; deltanet.rs module header) ----------

def test_sigmoid_closed_forms():
    from oracle.gates import sigmoid
    assert sigmoid(np.array([0.0]))[0] == 0.5
    assert abs(sigmoid(np.array([math.log(3.0)]))[0] - 0.75) < 1e-15          # 1 / (1 + 1/3)
    assert abs(sigmoid(np.array([-math.log(3.0)]))[0] - 0.25) < 1e-15
    x = np.random.default_rng(5).uniform(-30, 30, 1000)
    assert np.abs(sigmoid(x) + sigmoid(-x) - 1.0).max() < 1e-15               # symmetry
    ext = sigmoid(np.array([-800.0, 800.0]))
    assert ext[0] == 0.0 and ext[1] == 1.0                                      # no overflow, no NaN
    assert np.all(np.diff(sigmoid(np.sort(x))) >= 0)


def test_softplus_closed_forms():
    from oracle.gates import softplus
    assert abs(softplus(np.array([0.0]))[0] - math.log(2.0)) < 1e-16
    assert abs(softplus(np.array([math.log(math.e - 1.0)]))[0] - 1.0) < 1e-15  # ln(1 + e - 1) = 1
    x = np.random.default_rng(6).uniform(-40, 40, 1000)
    assert np.abs(softplus(x) - softplus(-x) - x).max() < 1e-12                 # ln((1+e^x)/(1+e^-x)) = x
    assert abs(softplus(np.array([50.0]))[0] - (50.0 + math.exp(-50.0))) < 1e-12
    assert abs(softplus(np.array([-50.0]))[0] - math.exp(-50.0)) < 1e-30
    assert np.all(softplus(x) > 0)


def test_gate_closed_forms():
    from oracle.gates import gates
    Nv, S = 3, 4
    A_log = np.array([math.log(2.0), 0.0, -1.0])
    dt_bias = np.array([0.5, -0.25, 1.0])
    # a + dt_bias = ln(e - 1) everywhere: softplus = 1, so g = -exp(A_log)
    a = np.full((1, Nv, S), math.log(math.e - 1.0)) - dt_bias[None, :, None]
    b = np.zeros((1, Nv, S))
    beta, g = gates(b, a, A_log, dt_bias)
    assert beta.shape == g.shape == (1, Nv, S)
    assert np.all(beta == 0.5)
    assert np.abs(g - (-np.exp(A_log))[None, :, None]).max() < 1e-15
    assert abs(g[0, 0, 0] + 2.0) < 1e-15
    # g < 0, increasing toward 0 as a falls; per-head parameters act per head
    rng = np.random.default_rng(7)
    a = rng.standard_normal((2, Nv, 64)) * 3
    _, g = gates(rng.standard_normal((2, Nv, 64)), a, A_log, dt_bias)
    assert np.all(g < 0)
    order = np.argsort(a[0, 1])
    assert np.all(np.diff(g[0, 1][order]) <= 0)


def test_l2norm_closed_forms():
    from oracle.gates import l2norm
    e = 1e-6
    x = np.zeros((2, 5))
    x[0, 2] = 3.0
    y = l2norm(x)
    assert y[0, 2] == 3.0 / math.sqrt(9.0 + e) and np.all(np.delete(y[0], 2) == 0)
    assert np.all(y[1] == 0)                                                  # zero vector stays zero
    r = np.random.default_rng(8).standard_normal((64, 128)) * 5
    n = np.sqrt((r * r).sum(-1))
    ny = np.sqrt((l2norm(r) ** 2).sum(-1))
    assert np.abs(ny - n / np.sqrt(n * n + e)).max() < 1e-15                   # norm closed form
    assert np.abs(l2norm(r) * np.sqrt(n * n + e)[:, None] - r).max() < 1e-12  # direction kept


def test_silu_closed_forms():
    from oracle.epilogue import silu
    assert silu(np.array([0.0]))[0] == 0.0
    assert abs(silu(np.array([math.log(3.0)]))[0] - 0.75 * math.log(3.0)) < 1e-15   # x sigmoid(x), sigmoid = 3/4
    x = np.random.default_rng(6).uniform(-30, 30, 1000)
    assert np.abs(silu(x) - silu(-x) - x).max() < 1e-13            # x (sigmoid(x) + sigmoid(-x)) = x
    big = silu(np.array([-800.0, 800.0]))
    assert big[0] == 0.0 and big[1] == 800.0                       # no overflow, no NaN


def test_gated_rmsnorm_closed_forms():
    from oracle.epilogue import gated_rmsnorm, silu
    w = np.array([1.0, 2.0, 0.5, 1.5])
    z = np.array([0.3, -1.2, 2.0, 0.0])
    # A constant row c*1 with eps = 0 normalises to sign(c): the mean of the
    # squares is c^2 (with their sum, 4c^2, the result would be halved).
    for c in (3.0, -0.25):
        out = gated_rmsnorm(np.full(4, c), z, w, 0.0)
        assert np.abs(out - np.sign(c) * w * silu(z)).max() < 1e-15
    # eps inside the square root: o = (3, 4, 0, 0), mean(o^2) = 25/4; with
    # eps = 3/4 the factor is 1/sqrt(7).
    o = np.array([3.0, 4.0, 0.0, 0.0])
    out = gated_rmsnorm(o, z, w, 0.75)
    assert np.abs(out - o / math.sqrt(7.0) * w * silu(z)).max() < 1e-15
    # Scale invariance with eps = 0, and per-row independence over leading axes.
    rng = np.random.default_rng(7)
    rows = rng.standard_normal((3, 5, 16))
    zz, ww = rng.standard_normal((3, 5, 16)), rng.uniform(0.5, 1.5, 16)
    base = gated_rmsnorm(rows, zz, ww, 0.0)
    assert np.abs(gated_rmsnorm(7.5 * rows, zz, ww, 0.0) - base).max() < 1e-13
    assert np.abs(gated_rmsnorm(rows[1, 2], zz[1, 2], ww, 0.0) - base[1, 2]).max() < 1e-15
    # Zero gate, zero output; an all-zero row stays zero even with eps = 0.
    assert np.all(gated_rmsnorm(rows, np.zeros_like(zz), ww, 1e-6) == 0.0)
    assert np.all(gated_rmsnorm(np.zeros(8), np.ones(8), np.ones(8), 0.0) == 0.0)


def test_conv_closed_forms():
    from oracle import conv
    from oracle.epilogue import silu
    rng = np.random.default_rng(9)
    B, S, C, K = 2, 11, 6, 4
    x = rng.standard_normal((B, S, C))
    w = rng.standard_normal((C, K))
    bias = rng.standard_normal(C)
    # K = 1: a pointwise silu(w x + bias)
    y, fin = conv.prefill(x, w[:, :1], bias, None, None)
    assert np.abs(y - silu(x * w[:, 0] + bias)).max() < 1e-15 and fin.shape == (B, C, 0)
    # impulse response: taps oldest first, so output t0 + m sees w[K - 1 - m]
    imp = np.zeros((1, S, C))
    imp[0, 3, 2] = 1.0
    y, _ = conv.prefill(imp, w, None, None, None)
    for t in range(S):
        want = silu(np.array([w[2, K - 1 - (t - 3)] if 0 <= t - 3 < K else 0.0]))[0]
        assert abs(y[0, t, 2] - want) < 1e-15
    assert np.all(np.delete(y[0], 2, axis=1) == 0.0)
    # the carried state alone (zero inputs): y_t = silu(sum_j w[j] init[j + t])
    init = rng.standard_normal((1, C, K - 1))
    y, fin = conv.prefill(np.zeros((1, 5, C)), w, None, init, None)
    for t in range(5):
        pre = sum(w[:, j] * init[0, :, j + t] for j in range(K - 1 - t)) if t < K - 1 else np.zeros(C)
        assert np.abs(y[0, t] - silu(pre)).max() < 1e-14
    assert np.all(fin == 0.0)                                  # the last K-1 inputs were zeros
    # against numpy's full convolution (zero state): y_t = silu(bias + (x * w reversed)_t)
    y, _ = conv.prefill(x, w, bias, None, None)
    for c in range(C):
        ref = np.convolve(x[1, :, c], w[c, ::-1])[:S] + bias[c]
        assert np.abs(y[1, :, c] - silu(ref)).max() < 1e-13


def test_conv_state_handoff_decode_and_split():
    from oracle import conv
    rng = np.random.default_rng(10)
    B, S, C, K = 2, 13, 10, 4
    x = rng.standard_normal((B, S, C))
    w = rng.standard_normal((C, K))
    bias = rng.standard_normal(C)
    init = rng.standard_normal((B, C, K - 1))
    y, fin = conv.prefill(x, w, bias, init, None)
    # prefill of 5 then 8 tokens through the final state equals one call (bitwise)
    y1, f1 = conv.prefill(x[:, :5], w, bias, init, None)
    y2, f2 = conv.prefill(x[:, 5:], w, bias, f1, None)
    assert np.array_equal(np.concatenate([y1, y2], axis=1), y) and np.array_equal(f2, fin)
    # a length of 2 < K - 1: the final state mixes the initial state and the inputs
    _, f = conv.prefill(x[:1], w, bias, init[:1], [2])
    assert np.array_equal(f[0], np.concatenate([init[0, :, 2:], x[0, :2].T], axis=1))
    # one-token decode steps through a one-slot pool equal the prefill (bitwise)
    pool = init[1:2].copy()
    for t in range(S):
        yt, pool = conv.decode(x[1:2, t:t + 1], w, bias, pool, [1], [0], None)
        assert np.array_equal(yt[0, 0], y[1, t])
    assert np.array_equal(pool[0], fin[1])
    # split: channel c of the (q | k | v) concatenation lands at its head and offset
    Nk, Dk, Nv, Dv = 1, 2, 3, 2
    yy = np.arange(1 * 4 * (2 * Nk * Dk + Nv * Dv), dtype=float).reshape(1, 4, -1)
    q, k, v = conv.split(yy, Nk, Dk, Nv, Dv)
    assert q[0, 0, 3, 1] == yy[0, 3, 1] and k[0, 0, 2, 0] == yy[0, 2, 2] and v[0, 2, 1, 1] == yy[0, 1, 4 + 2 * 2 + 1]
