"""Float64 CPU oracle for the Gated Delta Rule — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. It shares no code with the GPU library and never imports
it. Every function here takes float64 NumPy arrays (the exact widening of the
tensors the GPU path receives) and returns float64 results, never rounded.

Contents:
  decode / prefill / sequence  the token-by-token recurrence (C, gdr_oracle.c),
                               following the operator pages
                               lite_boost.ops.recurrent_gated_delta_rule and
                               lite_boost.ops.chunk_gated_delta_rule.
  brute                        explicit transition-matrix products (tiny sizes).
  chunk_form                   the chunk-parallel (UT transform) form in float64.
  gates                        the fused gates beta = sigmoid(b) and
                               g = -exp(A_log) softplus(a + dt_bias) (blog post's
                               layer code; deltanet.rs module header).
  epilogue                     the gated RMSNorm o w silu(z) / sqrt(mean(o^2) + eps)
                               applied to the output rows (deltanet.rs).
  conv                         the depthwise causal conv1d + SiLU ahead of the
                               recurrence and its split into q, k, v (blog post's
                               layer code; deltanet.rs conv ring).

Pins (tests/test_oracle_*.py) tie these to the pages: the worked examples of
inferencelayer deltanet.rs's tests, brute force, store-then-recall with
orthonormal keys, chunked == recurrent, g absent == alpha 1, pure decay,
reduction to decayed linear attention, the per-step write identity, the Dk=1
EMA, and contractivity; the gate and epilogue functions against their closed
forms. Parity unpinned: the speculative-decode slot rule
(read slot idx[b*S + n_acc - 1], write slot idx[b*S + t]) beyond its special
cases S = 1 and all tokens of a sequence on one slot.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)


def load():
    """Loads libgdr_oracle.so, building it first only if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    lib.gdr_oracle_sequence.restype = ctypes.c_int
    lib.gdr_oracle_sequence.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int,
        _dp, ctypes.c_int64, _dp, ctypes.c_int64, _dp, ctypes.c_int64,
        _dp, _dp, _dp, ctypes.c_double, _dp, _dp, ctypes.c_int64]
    lib.gdr_oracle_prefill.restype = ctypes.c_int
    lib.gdr_oracle_prefill.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        _dp, _dp, _dp, _dp, _dp, _dp, _ip, ctypes.c_double, _dp, _dp, ctypes.c_int]
    lib.gdr_oracle_decode.restype = ctypes.c_int
    lib.gdr_oracle_decode.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, _dp, _dp, _dp, _dp, _dp, _dp, _ip, _ip, _ip, ctypes.c_double,
        _dp, _dp, _dp, ctypes.c_int]
    lib.gdr_oracle_num_threads.restype = ctypes.c_int
    lib.gdr_oracle_num_threads.argtypes = []
    _lib = lib
    return lib


def num_threads() -> int:
    return load().gdr_oracle_num_threads()


def _f64(x):
    if x is None:
        return None
    a = np.ascontiguousarray(x, dtype=np.float64)
    return a


def _i32(x):
    if x is None:
        return None
    return np.ascontiguousarray(x, dtype=np.int32)


def _p(a, ptype):
    return None if a is None else a.ctypes.data_as(ptype)


def sequence(q, k, v, beta, g=None, gk=None, state=None, scale=1.0):
    """One sequence on one value head.

    q, k: (L, Dk); v: (L, Dv); beta: (L,); g: (L,) or None (alpha = 1);
    gk: (L, Dk) or None; state: (Dk, Dv) entering state or None (zeros).
    Returns (out (L, Dv), final state (Dk, Dv)).
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    g, gk = _f64(g), _f64(gk)
    L, Dk = k.shape
    Dv = v.shape[1]
    assert q.shape == (L, Dk) and v.shape == (L, Dv) and beta.shape == (L,)
    S = np.zeros((Dk, Dv)) if state is None else np.array(state, dtype=np.float64, copy=True)
    out = np.zeros((L, Dv))
    rc = load().gdr_oracle_sequence(L, Dk, Dv, _p(q, _dp), Dk, _p(k, _dp), Dk, _p(v, _dp), Dv,
                                    _p(beta, _dp), _p(g, _dp), _p(gk, _dp), float(scale),
                                    _p(S, _dp), _p(out, _dp), Dv)
    if rc:
        raise RuntimeError("oracle sequence failed")
    return out, S


def prefill(q, k, v, beta, g=None, initial_state=None, lengths=None, scale=1.0, nthreads=0):
    """Chunked-prefill operator semantics, token by token.

    q, k: (B, Nk, S, Dk); v: (B, Nv, S, Dv); beta: (B, Nv, S); g: (B, Nv, S) or None;
    initial_state: (B, Nv, Dk, Dv) or None; lengths: (B,) int or None (all S).
    Returns (out (B, Nv, S, Dv), final_state (B, Nv, Dk, Dv)).
    """
    q, k, v, beta, g, init = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(g), _f64(initial_state)
    lens = _i32(lengths)
    B, Nk, S, Dk = k.shape
    Nv, Dv = v.shape[1], v.shape[3]
    out = np.empty((B, Nv, S, Dv))
    fin = np.empty((B, Nv, Dk, Dv))
    rc = load().gdr_oracle_prefill(B, Nk, Nv, S, Dk, Dv, _p(q, _dp), _p(k, _dp), _p(v, _dp),
                                   _p(beta, _dp), _p(g, _dp), _p(init, _dp), _p(lens, _ip),
                                   float(scale), _p(out, _dp), _p(fin, _dp), int(nthreads))
    if rc:
        raise RuntimeError(f"oracle prefill failed ({rc})")
    return out, fin


def decode(q, k, v, beta, g, gk, lengths, n_accepted, indices, pool, scale=1.0, nthreads=0):
    """Recurrent-decode operator semantics with the indexed state pool.

    q, k: (B, Nk, S, Dk); v: (B, Nv, S, Dv); beta, g: (B, Nv, S) (g may be None);
    gk: (B, Nv, S, Dk) or None; lengths: (B,); n_accepted: (B,) or None;
    indices: (B*S,); pool: (slots, Nv, Dk, Dv).
    Returns (out (B, Nv, S, Dv), pool after the call).
    """
    q, k, v, beta, g, gk = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(g), _f64(gk)
    lens, nacc, idx = _i32(lengths), _i32(n_accepted), _i32(indices)
    pool_in = _f64(pool)
    B, Nk, S, Dk = k.shape
    Nv, Dv = v.shape[1], v.shape[3]
    slots = pool_in.shape[0]
    assert idx.size == B * S
    out = np.empty((B, Nv, S, Dv))
    pool_out = pool_in.copy()
    rc = load().gdr_oracle_decode(B, Nk, Nv, S, Dk, Dv, slots, _p(q, _dp), _p(k, _dp),
                                  _p(v, _dp), _p(beta, _dp), _p(g, _dp), _p(gk, _dp),
                                  _p(lens, _ip), _p(nacc, _ip), _p(idx, _ip), float(scale),
                                  _p(pool_in, _dp), _p(pool_out, _dp), _p(out, _dp),
                                  int(nthreads))
    if rc:
        raise RuntimeError(f"oracle decode failed ({rc})")
    return out, pool_out
