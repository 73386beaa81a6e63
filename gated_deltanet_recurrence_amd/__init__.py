"""Python binding of libgdr.so, the gfx950 Gated Delta Rule library.

Argument marshalling only: every step of both operators runs in the HIP
kernels behind the C ABI declared in include/gdr.h. PyTorch supplies device
memory and the current stream. There is no CPU fallback: if the library has
not been built, importing the binding works but every call raises.

Calls (same names as the C entry points):
  gdr_decode(...)  recurrent decode over an indexed state pool
                   (lite_boost.ops.recurrent_gated_delta_rule)
  gdr_chunk(...)   chunked prefill over padded variable-length inputs
                   (lite_boost.ops.chunk_gated_delta_rule)
Errors follow the operator pages: shape problems raise ValueError; dtype,
device and launch problems raise RuntimeError.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdr.so")

GDR_OK, GDR_ERR_NULL, GDR_ERR_SHAPE, GDR_ERR_DTYPE, GDR_ERR_UNSUPPORTED, GDR_ERR_LAUNCH, GDR_ERR_SCRATCH_LIMIT = range(7)
GDR_NOALLOC_SCRATCH_BYTES = 48 << 20
GDR_F32, GDR_BF16, GDR_F16 = 0, 1, 2

_vp = ctypes.c_void_p


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("B", ctypes.c_int32), ("Nk", ctypes.c_int32),
        ("Nv", ctypes.c_int32), ("S", ctypes.c_int32), ("Dk", ctypes.c_int32),
        ("Dv", ctypes.c_int32), ("num_slots", ctypes.c_int32),
        ("num_state_indices", ctypes.c_int64),
        ("q", _vp), ("k", _vp), ("v", _vp), ("beta", _vp),
        ("g", _vp), ("gk", _vp), ("state_pool", _vp),
        ("actual_seq_lengths", _vp), ("ssm_state_indices", _vp), ("num_accepted_tokens", _vp),
        ("scale_value", ctypes.c_float), ("out", _vp),
        ("beta_logits", _vp), ("gate_a", _vp), ("A_log", _vp), ("dt_bias", _vp),
        ("use_qk_l2norm", ctypes.c_int32),
        ("norm_z", _vp), ("norm_w", _vp), ("norm_eps", ctypes.c_float),
    ]


class ChunkArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("B", ctypes.c_int32), ("Nk", ctypes.c_int32),
        ("Nv", ctypes.c_int32), ("S", ctypes.c_int32), ("Dk", ctypes.c_int32),
        ("Dv", ctypes.c_int32), ("chunk_size", ctypes.c_int32),
        ("q", _vp), ("k", _vp), ("v", _vp), ("beta", _vp), ("g", _vp),
        ("initial_state", _vp), ("actual_seq_lengths", _vp),
        ("scale_value", ctypes.c_float), ("out", _vp), ("final_state", _vp),
        ("workspace", _vp), ("workspace_bytes", ctypes.c_int64),
        ("beta_logits", _vp), ("gate_a", _vp), ("A_log", _vp), ("dt_bias", _vp),
        ("use_qk_l2norm", ctypes.c_int32),
        ("norm_z", _vp), ("norm_w", _vp), ("norm_eps", ctypes.c_float),
    ]


class ConvPrefillArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("B", ctypes.c_int32), ("S", ctypes.c_int32), ("Nk", ctypes.c_int32),
        ("Nv", ctypes.c_int32), ("Dk", ctypes.c_int32), ("Dv", ctypes.c_int32), ("K", ctypes.c_int32),
        ("x", _vp), ("weight", _vp), ("bias", _vp), ("initial_state", _vp), ("final_state", _vp),
        ("actual_seq_lengths", _vp), ("q", _vp), ("k", _vp), ("v", _vp),
    ]


class ConvDecodeArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("B", ctypes.c_int32), ("S", ctypes.c_int32), ("Nk", ctypes.c_int32),
        ("Nv", ctypes.c_int32), ("Dk", ctypes.c_int32), ("Dv", ctypes.c_int32), ("K", ctypes.c_int32),
        ("num_slots", ctypes.c_int32), ("num_state_indices", ctypes.c_int64),
        ("x", _vp), ("weight", _vp), ("bias", _vp), ("state_pool", _vp),
        ("actual_seq_lengths", _vp), ("ssm_state_indices", _vp), ("num_accepted_tokens", _vp),
        ("q", _vp), ("k", _vp), ("v", _vp),
    ]


_lib = None


def load_library(path: str = LIB_PATH):
    """Loads libgdr.so and declares its entry points. Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libgdr.so is not built ({path}); run gated_deltanet_recurrence_amd/build.py")
    lib = ctypes.CDLL(path)
    lib.gdr_decode.restype = ctypes.c_int
    lib.gdr_decode.argtypes = [ctypes.POINTER(DecodeArgs), _vp]
    lib.gdr_chunk.restype = ctypes.c_int
    lib.gdr_chunk.argtypes = [ctypes.POINTER(ChunkArgs), _vp]
    lib.gdr_chunk_noalloc.restype = ctypes.c_int
    lib.gdr_chunk_noalloc.argtypes = [ctypes.POINTER(ChunkArgs), _vp]
    lib.gdr_chunk_workspace_size.restype = ctypes.c_int64
    lib.gdr_chunk_workspace_size.argtypes = [ctypes.POINTER(ChunkArgs)]
    lib.gdr_status_string.restype = ctypes.c_char_p
    lib.gdr_status_string.argtypes = [ctypes.c_int]
    lib.gdr_abi_version.restype = ctypes.c_int32
    lib.gdr_abi_version.argtypes = []
    lib.gdr_conv_prefill.restype = ctypes.c_int
    lib.gdr_conv_prefill.argtypes = [ctypes.POINTER(ConvPrefillArgs), _vp]
    lib.gdr_conv_decode.restype = ctypes.c_int
    lib.gdr_conv_decode.argtypes = [ctypes.POINTER(ConvDecodeArgs), _vp]
    _lib = lib
    return lib


def _check(rc: int, what: str):
    if rc == GDR_OK:
        return
    msg = f"{what}: {load_library().gdr_status_string(rc).decode()} (status {rc})"
    if rc in (GDR_ERR_SHAPE, GDR_ERR_SCRATCH_LIMIT):
        raise ValueError(msg)
    raise RuntimeError(msg)


_DT = {torch.bfloat16: GDR_BF16, torch.float16: GDR_F16, torch.float32: GDR_F32}


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t, name, dtype, device, shape=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise RuntimeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise RuntimeError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise RuntimeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise RuntimeError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _gates(beta, g, gates, dt, dev, B, Nv, S):
    """Checks beta/g or the fused gates (beta_logits, a, A_log, dt_bias) and
    returns the four fused-gate pointers (None when unused)."""
    if gates is None:
        if beta is None:
            raise ValueError("beta is required unless fused gates are given")
        _need(beta, "beta", dt, dev, (B, Nv, S))
        _need(g, "g", torch.float32, dev, (B, Nv, S))
        return None, None, None, None
    if beta is not None or g is not None:
        raise ValueError("fused gates replace beta and g: pass beta=None, g=None")
    try:
        bl, ga, al, db = gates
    except (TypeError, ValueError):
        raise ValueError("gates must be (beta_logits, a, A_log, dt_bias)")
    _need(bl, "beta_logits", dt, dev, (B, Nv, S))
    _need(ga, "a", dt, dev, (B, Nv, S))
    _need(al, "A_log", torch.float32, dev, (Nv,))
    _need(db, "dt_bias", torch.float32, dev, (Nv,))
    if bl is None or ga is None or al is None or db is None:
        raise ValueError("fused gates need all of beta_logits, a, A_log, dt_bias")
    return _ptr(bl), _ptr(ga), _ptr(al), _ptr(db)


def _norm(norm, dt, dev, B, Nv, S, Dv):
    """Checks the gated RMSNorm epilogue's (z, w, eps) and returns its ABI
    fields (None, None, 0.0 when unused)."""
    if norm is None:
        return None, None, 0.0
    try:
        z, w, eps = norm
    except (TypeError, ValueError):
        raise ValueError("norm must be (z, w, eps)")
    if z is None or w is None:
        raise ValueError("the epilogue needs both z and w")
    _need(z, "norm z", dt, dev, (B, Nv, S, Dv))
    _need(w, "norm w", torch.float32, dev, (Dv,))
    return _ptr(z), _ptr(w), float(eps)


def gdr_decode(q, k, v, beta, state_pool, actual_seq_lengths, ssm_state_indices, g=None, gk=None,
               num_accepted_tokens=None, scale_value=1.0, out=None, gates=None, use_qk_l2norm=False,
               norm=None):
    """Recurrent decode; updates state_pool in place. Returns (out, state_pool).

    q, k (B, Nk, S, Dk); v (B, Nv, S, Dv); beta (B, Nv, S); state_pool
    (slots, Nv, Dk, Dv) — all of one dtype (bfloat16, float16 or float32); g (B, Nv, S)
    and gk (B, Nv, S, Dk) float32 or None; actual_seq_lengths (B,),
    ssm_state_indices (B*S,), num_accepted_tokens (B,) or None — int32.
    gates: None, or (beta_logits, a, A_log, dt_bias) — logits and a (B, Nv, S)
    in the dtype, A_log and dt_bias (Nv,) float32 — in place of beta and g
    (pass beta=None): the kernels form beta = sigmoid(beta_logits) and
    g = -exp(A_log) * softplus(a + dt_bias). use_qk_l2norm: the kernels
    normalise q and k (x / sqrt(sum(x^2) + 1e-6)) before use. norm: None, or
    (z, w, eps) — z (B, Nv, S, Dv) in the dtype, w (Dv,) float32 — for the
    gated RMSNorm epilogue o * w * silu(z) / sqrt(mean(o^2) + eps) on every
    valid output row.
    """
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D (B, N, S, D)")
    B, Nk, S, Dk = k.shape
    Nv, Dv = v.shape[1], v.shape[3]
    dt = q.dtype
    if dt not in _DT:
        raise RuntimeError(f"unsupported dtype {dt}")
    dev = q.device
    if dev.type != "cuda":
        raise RuntimeError("tensors must be on a GPU")
    _need(q, "query", dt, dev, (B, Nk, S, Dk))
    _need(k, "key", dt, dev)
    _need(v, "value", dt, dev, (B, Nv, S, Dv))
    fused = _gates(beta, g, gates, dt, dev, B, Nv, S)
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (Nv, Dk, Dv):
        raise ValueError(f"state has shape {tuple(state_pool.shape)}, expected (slots, {Nv}, {Dk}, {Dv})")
    _need(state_pool, "state", dt, dev)
    _need(gk, "gk", torch.float32, dev, (B, Nv, S, Dk))
    _need(actual_seq_lengths, "actual_seq_lengths", torch.int32, dev, (B,))
    _need(ssm_state_indices, "ssm_state_indices", torch.int32, dev)
    _need(num_accepted_tokens, "num_accepted_tokens", torch.int32, dev, (B,))
    if out is None:
        out = torch.empty((B, Nv, S, Dv), dtype=dt, device=dev)
    _need(out, "out", dt, dev, (B, Nv, S, Dv))
    a = DecodeArgs(_DT[dt], B, Nk, Nv, S, Dk, Dv, state_pool.shape[0], ssm_state_indices.numel(),
                   _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(gk), _ptr(state_pool),
                   _ptr(actual_seq_lengths), _ptr(ssm_state_indices), _ptr(num_accepted_tokens),
                   float(scale_value), _ptr(out), *fused, int(bool(use_qk_l2norm)),
                   *_norm(norm, dt, dev, B, Nv, S, Dv))
    _check(load_library().gdr_decode(ctypes.byref(a), _stream(dev)), "gdr_decode")
    return out, state_pool


def _chunk_args(q, k, v, beta, initial_state, actual_seq_lengths, g, scale_value, chunk_size, out,
                final_state, gates, use_qk_l2norm, norm):
    """Checks and marshals gdr_chunk's arguments; returns (ChunkArgs, out,
    final_state, device), the workspace fields left empty."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D (B, N, S, D)")
    B, Nk, S, Dk = k.shape
    Nv, Dv = v.shape[1], v.shape[3]
    dt = q.dtype
    if dt not in _DT:
        raise RuntimeError(f"unsupported dtype {dt}")
    dev = q.device
    if dev.type != "cuda":
        raise RuntimeError("tensors must be on a GPU")
    _need(q, "query", dt, dev, (B, Nk, S, Dk))
    _need(k, "key", dt, dev)
    _need(v, "value", dt, dev, (B, Nv, S, Dv))
    fused = _gates(beta, g, gates, dt, dev, B, Nv, S)
    _need(initial_state, "initial_state", dt, dev, (B, Nv, Dk, Dv))
    _need(actual_seq_lengths, "actual_seq_lengths", torch.int32, dev, (B,))
    if out is None:
        out = torch.empty((B, Nv, S, Dv), dtype=dt, device=dev)
    if final_state is None:
        final_state = torch.empty((B, Nv, Dk, Dv), dtype=dt, device=dev)
    _need(out, "out", dt, dev, (B, Nv, S, Dv))
    _need(final_state, "final_state", dt, dev, (B, Nv, Dk, Dv))
    a = ChunkArgs(_DT[dt], B, Nk, Nv, S, Dk, Dv, int(chunk_size),
                  _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(initial_state),
                  _ptr(actual_seq_lengths), float(scale_value), _ptr(out), _ptr(final_state),
                  None, 0, *fused, int(bool(use_qk_l2norm)), *_norm(norm, dt, dev, B, Nv, S, Dv))
    return a, out, final_state, dev


def gdr_chunk(q, k, v, beta, initial_state=None, actual_seq_lengths=None, g=None, scale_value=1.0,
              chunk_size=64, out=None, final_state=None, gates=None, use_qk_l2norm=False, norm=None):
    """Chunked prefill. Returns (out, final_state).

    q, k (B, Nk, S, Dk); v (B, Nv, S, Dv); beta (B, Nv, S); initial_state
    (B, Nv, Dk, Dv) or None — one dtype; g (B, Nv, S) float32 or None;
    actual_seq_lengths (B,) int32 or None. final_state may be initial_state
    itself (updated in place). gates, use_qk_l2norm, norm: as for gdr_decode.
    """
    a, out, final_state, dev = _chunk_args(q, k, v, beta, initial_state, actual_seq_lengths, g, scale_value,
                                           chunk_size, out, final_state, gates, use_qk_l2norm, norm)
    lib = load_library()
    ws = chunk_workspace(a, dev)
    _check(lib.gdr_chunk(ctypes.byref(a), _stream(dev)), "gdr_chunk")
    del ws   # stream-ordered reuse by the caching allocator is safe after the enqueue
    return out, final_state


def gdr_chunk_noalloc(q, k, v, beta, initial_state=None, actual_seq_lengths=None, g=None, scale_value=1.0,
                      chunk_size=64, out=None, final_state=None, gates=None, use_qk_l2norm=False, norm=None):
    """gdr_chunk through the allocation-free entry point: the library's fixed
    per-GPU scratch array replaces the workspace (GDR_NOALLOC_SCRATCH_BYTES;
    calls beyond it raise ValueError). Pass out and final_state to keep the
    call free of allocations; calls that overlap on one GPU race on the array."""
    a, out, final_state, dev = _chunk_args(q, k, v, beta, initial_state, actual_seq_lengths, g, scale_value,
                                           chunk_size, out, final_state, gates, use_qk_l2norm, norm)
    _check(load_library().gdr_chunk_noalloc(ctypes.byref(a), _stream(dev)), "gdr_chunk_noalloc")
    return out, final_state


def chunk_workspace(a, dev):
    """Allocates the workspace gdr_chunk needs for the arguments `a` (a
    ChunkArgs) on `dev`, stores it in `a` and returns the tensor, which must
    stay alive until the call has been enqueued."""
    n = int(load_library().gdr_chunk_workspace_size(ctypes.byref(a)))
    if n <= 0:
        a.workspace, a.workspace_bytes = None, 0
        return None
    ws = torch.empty(n, dtype=torch.uint8, device=dev)
    a.workspace, a.workspace_bytes = ws.data_ptr(), n
    return ws


def _conv_common(x, weight, bias, heads):
    if x.dim() != 3:
        raise ValueError("x must be (B, S, C)")
    try:
        Nk, Dk, Nv, Dv = (int(h) for h in heads)
    except (TypeError, ValueError):
        raise ValueError("heads must be (Nk, Dk, Nv, Dv)")
    B, S, C = x.shape
    if C != 2 * Nk * Dk + Nv * Dv:
        raise ValueError(f"x has {C} channels, expected 2*Nk*Dk + Nv*Dv = {2 * Nk * Dk + Nv * Dv}")
    dt = x.dtype
    if dt not in _DT:
        raise RuntimeError(f"unsupported dtype {dt}")
    dev = x.device
    if dev.type != "cuda":
        raise RuntimeError("tensors must be on a GPU")
    _need(x, "x", dt, dev)
    if weight is None or weight.dim() != 2 or weight.shape[0] != C:
        raise ValueError(f"weight must be ({C}, K)")
    _need(weight, "weight", torch.float32, dev)
    _need(bias, "bias", torch.float32, dev, (C,))
    K = weight.shape[1]
    q = torch.empty((B, Nk, S, Dk), dtype=dt, device=dev)
    k = torch.empty((B, Nk, S, Dk), dtype=dt, device=dev)
    v = torch.empty((B, Nv, S, Dv), dtype=dt, device=dev)
    return B, S, C, K, Nk, Dk, Nv, Dv, dt, dev, q, k, v


def gdr_conv_prefill(x, weight, heads, bias=None, initial_state=None, final_state=None, actual_seq_lengths=None):
    """Depthwise causal conv1d + SiLU over x (B, S, C), split into q, k, v.

    heads = (Nk, Dk, Nv, Dv) with C = 2*Nk*Dk + Nv*Dv; weight (C, K) and bias
    (C,) float32; initial_state (B, C, K-1) or None (zeros); final_state
    (B, C, K-1) or None (allocated; may be initial_state itself);
    actual_seq_lengths (B,) int32 or None. Returns (q, k, v, final_state):
    q, k (B, Nk, S, Dk) and v (B, Nv, S, Dv), zero past each length.
    """
    B, S, C, K, Nk, Dk, Nv, Dv, dt, dev, q, k, v = _conv_common(x, weight, bias, heads)
    _need(initial_state, "initial_state", dt, dev, (B, C, K - 1))
    if final_state is None:
        final_state = torch.empty((B, C, K - 1), dtype=dt, device=dev)
    _need(final_state, "final_state", dt, dev, (B, C, K - 1))
    _need(actual_seq_lengths, "actual_seq_lengths", torch.int32, dev, (B,))
    a = ConvPrefillArgs(_DT[dt], B, S, Nk, Nv, Dk, Dv, K, _ptr(x), _ptr(weight), _ptr(bias),
                        _ptr(initial_state), _ptr(final_state), _ptr(actual_seq_lengths), _ptr(q), _ptr(k), _ptr(v))
    _check(load_library().gdr_conv_prefill(ctypes.byref(a), _stream(dev)), "gdr_conv_prefill")
    return q, k, v, final_state


def gdr_conv_decode(x, weight, heads, state_pool, actual_seq_lengths, ssm_state_indices, bias=None,
                    num_accepted_tokens=None):
    """The conv1d + SiLU of up to 8 tokens per sequence over a pool of conv
    states (slots, C, K-1), updated in place with gdr_decode's slot rule.
    Returns (q, k, v, state_pool)."""
    B, S, C, K, Nk, Dk, Nv, Dv, dt, dev, q, k, v = _conv_common(x, weight, bias, heads)
    if state_pool.dim() != 3 or tuple(state_pool.shape[1:]) != (C, K - 1):
        raise ValueError(f"state_pool has shape {tuple(state_pool.shape)}, expected (slots, {C}, {K - 1})")
    _need(state_pool, "state_pool", dt, dev)
    _need(actual_seq_lengths, "actual_seq_lengths", torch.int32, dev, (B,))
    _need(ssm_state_indices, "ssm_state_indices", torch.int32, dev)
    _need(num_accepted_tokens, "num_accepted_tokens", torch.int32, dev, (B,))
    a = ConvDecodeArgs(_DT[dt], B, S, Nk, Nv, Dk, Dv, K, state_pool.shape[0], ssm_state_indices.numel(),
                       _ptr(x), _ptr(weight), _ptr(bias), _ptr(state_pool), _ptr(actual_seq_lengths),
                       _ptr(ssm_state_indices), _ptr(num_accepted_tokens), _ptr(q), _ptr(k), _ptr(v))
    _check(load_library().gdr_conv_decode(ctypes.byref(a), _stream(dev)), "gdr_conv_decode")
    return q, k, v, state_pool
