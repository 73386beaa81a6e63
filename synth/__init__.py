"""Seeded synthetic inputs for the Gated Delta Rule operators.

Shared by the tests, the benchmark and the smoke check; used to feed both the
GPU library and the float64 oracle. It holds none of the recurrence's
arithmetic: only random draws, the input recipes the Gated DeltaNet pages
apply upstream of the operators, and bf16 storage rounding.

Input recipes (Gated DeltaNet blog post, gate computation; inferencelayer
deltanet.rs, module header and l2norm):
  q, k  : standard normal per head vector, then x / sqrt(sum(x^2) + 1e-6)
          (in float32)
  v     : standard normal
  beta  : sigmoid(N(0, 1))                      write strength in (0, 1)
  g     : -exp(A_log[h]) * softplus(a + dt_bias[h]) with A_log ~ U(-2, 1),
          dt_bias ~ U(-1, 1) per value head and a ~ N(0, 1) per token
Storage: bf16 tensors are rounded from float32 to nearest-even; g and gk are
float32. Every draw comes from numpy's PCG64 generator seeded with
(base, tensor_id, b), so each batch slice can be produced on its own.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# tensor ids for seeding
T_ALOG, T_DTBIAS, T_Q, T_K, T_V, T_A, T_B, T_GK, T_STATE, T_LENS, T_NACC, T_IDX, T_Z, T_W, T_X, T_CW, T_CB, T_CS, T_KDIR = range(19)

BF16_NAN = np.uint16(0x7FC0)


def bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (NaN -> quiet NaN)."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    u = x32.view(np.uint32)
    # u + bias can wrap only for NaN bit patterns, which are replaced below
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= 16
    out = r.astype(np.uint16)
    nan = np.isnan(x32)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _rng(base, tid, b=None):
    return np.random.default_rng([base, tid] if b is None else [base, tid, b])


def _l2n(x):
    """x / sqrt(sum(x^2) + 1e-6) over the last axis, in place, float32."""
    n = np.sqrt(np.einsum("...d,...d->...", x, x)[..., None] + np.float32(1e-6))
    x /= n
    return x


def _softplus(x):
    return np.log1p(np.exp(x))


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _store(x, dtype):
    """float array -> storage array: float32, float16 (numpy rounds to nearest
    even), or uint16 bf16 bit patterns."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(np.asarray(x, dtype=np.float32).astype(np.float16))
    return bf16_bits(np.asarray(x, dtype=np.float32))


def widen(x, dtype) -> Optional[np.ndarray]:
    """storage array -> float64 (exact)."""
    if x is None:
        return None
    if x.dtype == np.uint16:
        return bf16_to_f64(x)
    return np.asarray(x, dtype=np.float64)


@dataclass
class Case:
    """One seeded operator input. Storage arrays are float32, float16, or uint16 (bf16 bits)."""
    kind: str                      # "decode" or "prefill"
    dtype: str                     # "f32", "bf16" or "f16": q/k/v/beta/state/out
    B: int
    Nk: int
    Nv: int
    S: int
    Dk: int
    Dv: int
    scale: float
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    beta: np.ndarray
    g: Optional[np.ndarray]        # float32 (B, Nv, S) or None
    lens: Optional[np.ndarray]     # int32 (B,) or None
    gk: Optional[np.ndarray] = None          # float32 (B, Nv, S, Dk), decode only
    state: Optional[np.ndarray] = None       # decode: pool; prefill: initial state or None
    n_acc: Optional[np.ndarray] = None       # decode only
    idx: Optional[np.ndarray] = None         # decode only, int32 (B*S,)
    chunk: int = 64
    meta: dict = field(default_factory=dict)

    @property
    def slots(self):
        return None if self.state is None or self.kind != "decode" else self.state.shape[0]

    def f64(self, name):
        return widen(getattr(self, name), self.dtype)

    def valid_lengths(self):
        if self.lens is None:
            return np.full(self.B, self.S, dtype=np.int64)
        return np.clip(self.lens.astype(np.int64), 0, self.S)


def _per_b(base, tid, B, fn, threads=8):
    """Runs fn(rng, b) for every batch slice (independent streams) into one array."""
    first = fn(_rng(base, tid, 0), 0)
    out = np.empty((B,) + first.shape, dtype=first.dtype)
    out[0] = first
    del first

    def one(b):
        out[b] = fn(_rng(base, tid, b), b)
    if B > 1:
        if threads <= 1:
            for b in range(1, B):
                one(b)
        else:
            with ThreadPoolExecutor(min(threads, B - 1)) as ex:
                list(ex.map(one, range(1, B)))
    return out


def _unit_vectors(base, tid, B, N, S, D, dtype):
    def fn(rng, b):
        return _store(_l2n(rng.standard_normal((N, S, D), dtype=np.float32)), dtype)
    return _per_b(base, tid, B, fn)


def _correlated_keys(base, B, N, S, D, dtype, mix):
    """Keys that resemble one another, as repeated or related tokens give after
    a short convolution. mix = m in [0, 1]: k_t = l2norm(m sqrt(D) c + (1 - m) n_t)
    with one unit direction c per (b, key head) and n_t ~ N(0, I); the mean
    cosine between two keys is about m^2 / (m^2 + (1 - m)^2), and m = 1 makes
    every key equal. mix = ("vocab", n): every key is one of n unit vectors
    per (b, key head), drawn at random per token (runs of repeated tokens)."""
    def fn(rng, b):
        if isinstance(mix, tuple) and mix[0] == "vocab":
            voc = _l2n(rng.standard_normal((N, mix[1], D), dtype=np.float32))
            pick = rng.integers(0, mix[1], (N, S))
            x = np.take_along_axis(voc, pick[:, :, None], axis=1)
        else:
            m = np.float32(mix)
            c = _l2n(rng.standard_normal((N, 1, D), dtype=np.float32)) * np.float32(math.sqrt(D))
            x = m * c + (np.float32(1) - m) * rng.standard_normal((N, S, D), dtype=np.float32)
        return _store(_l2n(np.ascontiguousarray(x, dtype=np.float32)), dtype)
    return _per_b(base, T_KDIR, B, fn)


def _normals(base, tid, B, shape, dtype, std=1.0):
    def fn(rng, b):
        x = rng.standard_normal(shape, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        return _store(x, dtype)
    return _per_b(base, tid, B, fn)


def _betas(base, B, Nv, S, dtype):
    return _per_b(base, T_B, B, lambda rng, b: _store(_sigmoid(rng.standard_normal((Nv, S))), dtype))


def _gates(base, B, Nv, S):
    """g = -exp(A_log) * softplus(a + dt_bias), computed in float64, stored float32."""
    a_log = _rng(base, T_ALOG).uniform(-2.0, 1.0, Nv)
    dt_bias = _rng(base, T_DTBIAS).uniform(-1.0, 1.0, Nv)

    def fn(rng, b):
        a = rng.standard_normal((Nv, S))
        g = -np.exp(a_log)[:, None] * _softplus(a + dt_bias[:, None])
        return g.astype(np.float32)
    return _per_b(base, T_A, B, fn)


def _uniform_gates(base, B, Nv, S, lo, hi):
    return _per_b(base, T_A, B, lambda rng, b: rng.uniform(lo, hi, (Nv, S)).astype(np.float32))


def gate_inputs(base, B, Nv, S, dtype):
    """Raw inputs of the fused gates, drawn from the same streams as the gate
    recipe above: beta logits b ~ N(0, 1) and a ~ N(0, 1) per token (stored in
    the I/O dtype), A_log ~ U(-2, 1) and dt_bias ~ U(-1, 1) per value head
    (float32). Returns (beta_logits, a, A_log, dt_bias)."""
    logits = _per_b(base, T_B, B, lambda rng, b: _store(rng.standard_normal((Nv, S)), dtype))
    a = _per_b(base, T_A, B, lambda rng, b: _store(rng.standard_normal((Nv, S)), dtype))
    a_log = _rng(base, T_ALOG).uniform(-2.0, 1.0, Nv).astype(np.float32)
    dt_bias = _rng(base, T_DTBIAS).uniform(-1.0, 1.0, Nv).astype(np.float32)
    return logits, a, a_log, dt_bias


def norm_inputs(base, B, Nv, S, Dv, dtype):
    """Inputs of the gated RMSNorm epilogue: the gate z ~ N(0, 1) per output
    element (stored in the I/O dtype) and the weight w ~ U(0.5, 1.5) per column
    (float32; a trained norm weight sits near 1). Returns (z, w)."""
    z = _per_b(base, T_Z, B, lambda rng, b: _store(rng.standard_normal((Nv, S, Dv)), dtype))
    w = _rng(base, T_W).uniform(0.5, 1.5, Dv).astype(np.float32)
    return z, w


def conv_inputs(base, B, S, C, K, dtype, slots=None):
    """Inputs of the depthwise conv1d ahead of the recurrence: the fused
    projection x ~ N(0, 1) per token and channel (the I/O dtype), weights
    w ~ U(-1, 1) / sqrt(K) per channel and tap and bias ~ N(0, 0.1) per channel
    (float32), and carried states ~ N(0, 1) in the I/O dtype: (B, C, K-1) per
    sequence, or (slots, C, K-1) for a pool. Returns (x, w, bias, state)."""
    x = _per_b(base, T_X, B, lambda rng, b: _store(rng.standard_normal((S, C)), dtype))
    w = (_rng(base, T_CW).uniform(-1.0, 1.0, (C, K)) / np.sqrt(K)).astype(np.float32)
    bias = (_rng(base, T_CB).standard_normal(C) * 0.1).astype(np.float32)
    n = B if slots is None else slots
    state = _store(_rng(base, T_CS).standard_normal((n, C, K - 1)), dtype)
    return x, w, bias, state


def _poison(case: Case):
    """Puts NaN into every input position past each sequence's valid length."""
    L = case.valid_lengths()
    nanv = BF16_NAN if case.dtype == "bf16" else (np.float16(np.nan) if case.dtype == "f16" else np.float32(np.nan))
    for b in range(case.B):
        t0 = int(L[b])
        if t0 >= case.S:
            continue
        case.q[b, :, t0:] = nanv
        case.k[b, :, t0:] = nanv
        case.v[b, :, t0:] = nanv
        case.beta[b, :, t0:] = nanv
        if case.g is not None:
            case.g[b, :, t0:] = np.nan
        if case.gk is not None:
            case.gk[b, :, t0:] = np.nan


def prefill_case(*, B, Nk, Nv, S, Dk, Dv, dtype="bf16", base=404, gate="gate",
                 init_std: Optional[float] = 0.02, lens=None, chunk=64, scale=None,
                 poison_pad=False, key_mix=None) -> Case:
    """Chunked-prefill inputs. gate: "gate" (the -exp(A_log)*softplus recipe),
    ("uniform", lo, hi), or None (g absent, alpha = 1). lens: None (all S),
    ("uniform", lo, hi) seeded draws, or an explicit int sequence. key_mix:
    None (independent keys) or correlated keys (see _correlated_keys)."""
    q = _unit_vectors(base, T_Q, B, Nk, S, Dk, dtype)
    if key_mix is None:
        k = _unit_vectors(base, T_K, B, Nk, S, Dk, dtype)
    else:
        k = _correlated_keys(base, B, Nk, S, Dk, dtype, key_mix)
    v = _normals(base, T_V, B, (Nv, S, Dv), dtype)
    beta = _betas(base, B, Nv, S, dtype)
    if gate is None:
        g = None
    elif gate == "gate":
        g = _gates(base, B, Nv, S)
    else:
        g = _uniform_gates(base, B, Nv, S, gate[1], gate[2])
    init = None if init_std is None else _normals(base, T_STATE, B, (Nv, Dk, Dv), dtype, init_std)
    if lens is None:
        L = None
    elif isinstance(lens, tuple) and lens[0] == "uniform":
        L = _rng(base, T_LENS).integers(lens[1], lens[2] + 1, B).astype(np.int32)
    else:
        L = np.asarray(lens, dtype=np.int32)
    c = Case("prefill", dtype, B, Nk, Nv, S, Dk, Dv,
             scale if scale is not None else 1.0 / math.sqrt(Dk),
             q, k, v, beta, g, L, state=init, chunk=chunk)
    if poison_pad:
        _poison(c)
    return c


def decode_case(*, B, Nk, Nv, S, Dk, Dv, slots, dtype="bf16", base=202, gate="gate",
                gk=None, pool_std=0.05, lens=None, n_acc="lens", idx="perm",
                scale=None, poison_pad=False) -> Case:
    """Recurrent-decode inputs with an indexed state pool.

    lens: None (all S), ("uniform", lo, hi) or explicit; n_acc: "lens" (equal to
    lens), None (omitted), ("uniform", lo, hi) or explicit; idx: "perm" (one
    slot per sequence: the first B of a seeded permutation of the slots,
    repeated over the sequence's S positions), "per_token" (B*S distinct slots
    from a seeded permutation), or explicit (B*S,) ints. gk: None or (lo, hi)
    for a U(lo, hi) per-key gate."""
    q = _unit_vectors(base, T_Q, B, Nk, S, Dk, dtype)
    k = _unit_vectors(base, T_K, B, Nk, S, Dk, dtype)
    v = _normals(base, T_V, B, (Nv, S, Dv), dtype)
    beta = _betas(base, B, Nv, S, dtype)
    if gate is None:
        g = None
    elif gate == "gate":
        g = _gates(base, B, Nv, S)
    else:
        g = _uniform_gates(base, B, Nv, S, gate[1], gate[2])
    gkt = None
    if gk is not None:
        gkt = _per_b(base, T_GK, B, lambda rng, b: rng.uniform(gk[0], gk[1], (Nv, S, Dk)).astype(np.float32))
    pool = _store(_rng(base, T_STATE).standard_normal((slots, Nv, Dk, Dv), dtype=np.float32)
                  * np.float32(pool_std), dtype)
    if lens is None:
        L = np.full(B, S, dtype=np.int32)
    elif isinstance(lens, tuple) and lens[0] == "uniform":
        L = _rng(base, T_LENS).integers(lens[1], lens[2] + 1, B).astype(np.int32)
    else:
        L = np.asarray(lens, dtype=np.int32)
    if isinstance(n_acc, str) and n_acc == "lens":
        na = L.copy()
    elif n_acc is None:
        na = None
    elif isinstance(n_acc, tuple) and n_acc[0] == "uniform":
        na = _rng(base, T_NACC).integers(n_acc[1], n_acc[2] + 1, B).astype(np.int32)
    else:
        na = np.asarray(n_acc, dtype=np.int32)
    if isinstance(idx, str) and idx == "perm":
        assert B <= slots
        p = _rng(base, T_IDX).permutation(slots)[:B].astype(np.int32)
        ix = np.repeat(p, S)
    elif isinstance(idx, str) and idx == "per_token":
        assert B * S <= slots
        ix = _rng(base, T_IDX).permutation(slots)[:B * S].astype(np.int32)
    else:
        ix = np.asarray(idx, dtype=np.int32).reshape(-1)
    c = Case("decode", dtype, B, Nk, Nv, S, Dk, Dv,
             scale if scale is not None else 1.0 / math.sqrt(Dk),
             q, k, v, beta, g, L, gk=gkt, state=pool, n_acc=na, idx=ix)
    if poison_pad:
        _poison(c)
    return c


# The five workloads: shapes, dtypes and distributions.
def config(cid: int, **over) -> Case:
    """Builds workload cid (1..5); keyword overrides shrink or vary it for tests."""
    base = 101 * cid
    if cid == 1:
        kw = dict(B=1, Nk=1, Nv=1, S=64, Dk=16, Dv=16, dtype="f32", base=base,
                  gate=("uniform", -1.0, -0.01), init_std=None, chunk=16, scale=0.25)
        kw.update(over)
        return prefill_case(**kw)
    if cid == 2:
        kw = dict(B=64, Nk=16, Nv=32, S=1, Dk=128, Dv=128, slots=64, dtype="bf16", base=base)
        kw.update(over)
        return decode_case(**kw)
    if cid == 3:
        kw = dict(B=128, Nk=16, Nv=32, S=4, Dk=128, Dv=128, slots=256, dtype="bf16", base=base,
                  gk=(-0.5, -0.001), lens=("uniform", 1, 4), n_acc=("uniform", 1, 4))
        kw.update(over)
        return decode_case(**kw)
    if cid == 4:
        kw = dict(B=4, Nk=16, Nv=32, S=4096, Dk=128, Dv=128, dtype="bf16", base=base,
                  init_std=0.02, chunk=64)
        kw.update(over)
        return prefill_case(**kw)
    if cid == 5:
        kw = dict(B=16, Nk=16, Nv=64, S=16384, Dk=128, Dv=128, dtype="bf16", base=base,
                  gate=None, init_std=None, lens=("uniform", 256, 16384), chunk=64)
        kw.update(over)
        return prefill_case(**kw)
    raise ValueError(f"unknown workload {cid}")


def decode_view_of_prefill(c: Case, t: int) -> Case:
    """Token t of a single-state prefill case as an S=1 decode call on a 1-slot-per-(b) pool
    (the chained-decode form of the tiny fp32 workload)."""
    sl = slice(t, t + 1)
    B = c.B
    return Case("decode", c.dtype, B, c.Nk, c.Nv, 1, c.Dk, c.Dv, c.scale,
                np.ascontiguousarray(c.q[:, :, sl]), np.ascontiguousarray(c.k[:, :, sl]),
                np.ascontiguousarray(c.v[:, :, sl]), np.ascontiguousarray(c.beta[:, :, sl]),
                None if c.g is None else np.ascontiguousarray(c.g[:, :, sl]),
                np.ones(B, dtype=np.int32), state=None, n_acc=np.ones(B, dtype=np.int32),
                idx=np.arange(B, dtype=np.int32))
