"""GPU parity of the fused preprocessing against the float64 oracle.

With fused gates the kernels form beta = sigmoid(b) and
g = -exp(A_log) softplus(a + dt_bias) themselves, and with use_qk_l2norm
they normalise q and k (the Gated DeltaNet blog post's layer code and its
use_qk_l2norm_in_kernel; inferencelayer deltanet.rs, module header and
l2norm). The reference is the same token-by-token oracle, fed with
oracle.gates and oracle.gates.l2norm of the same raw inputs in float64."""
import copy

import numpy as np
import pytest
import torch

import synth
from oracle.gates import gates as oracle_gates, l2norm as oracle_l2norm
from tests.gpu_util import say, to_dev
from tests.test_gpu_chunk import _check_full
from tests.test_gpu_decode import _check_decode
import gated_deltanet_recurrence_amd as gdr

pytestmark = pytest.mark.gpu


def _fused(c, base, poison=False):
    """(reference case with float64 beta and g from the oracle's gates, device gate tensors)."""
    bl, a, al, db = synth.gate_inputs(base, c.B, c.Nv, c.S, c.dtype)
    if poison:
        nanv = synth.BF16_NAN if c.dtype == "bf16" else np.float32(np.nan)
        for b, Lb in enumerate(c.valid_lengths()):
            bl[b, :, int(Lb):] = nanv
            a[b, :, int(Lb):] = nanv
    beta, g = oracle_gates(synth.widen(bl, c.dtype), synth.widen(a, c.dtype), al, db)
    ref = copy.copy(c)
    ref.beta, ref.g = beta, g
    return ref, (to_dev(bl), to_dev(a), to_dev(al), to_dev(db))


def _raw_qk(c, base):
    """Replaces q and k by unnormalised draws (3 N(0, 1), stored in the I/O
    dtype); the reference gets their float64 normalisation."""
    rng = np.random.default_rng([base, 99])
    ref = copy.copy(c)
    for name in ("q", "k"):
        raw = synth._store(rng.standard_normal(getattr(c, name).shape) * 3.0, c.dtype)
        setattr(c, name, raw)
        setattr(ref, name, oracle_l2norm(synth.widen(raw, c.dtype)))
    return ref


def _decode(c, base, gates=True, qk_norm=False):
    ref = _raw_qk(c, base) if qk_norm else copy.copy(c)
    g = None
    if gates:
        gref, g = _fused(c, base)
        ref.beta, ref.g = gref.beta, gref.g
    say(f"gdr_decode {c.dtype} B={c.B} S={c.S} Dk={c.Dk} gk={c.gk is not None} fused gates={gates} qk norm={qk_norm}")
    out, pool = gdr.gdr_decode(to_dev(c.q), to_dev(c.k), to_dev(c.v), None if gates else to_dev(c.beta),
                               to_dev(c.state), to_dev(c.lens), to_dev(c.idx), g=None if gates else to_dev(c.g),
                               gk=to_dev(c.gk), num_accepted_tokens=to_dev(c.n_acc), scale_value=c.scale,
                               gates=g, use_qk_l2norm=qk_norm)
    torch.cuda.synchronize()
    _check_decode(ref, out, pool)


@pytest.mark.parametrize("gk", [None, (-0.5, -0.001)])
def test_fused_gates_one_token(gk):
    _decode(synth.config(2, B=24, gk=gk, base=611), 611)


@pytest.mark.parametrize("gk", [None, (-0.5, -0.001)])
def test_fused_gates_multi_token(gk):
    _decode(synth.config(3, B=40, gk=gk, base=612), 612)


def test_fused_gates_decode_fp32_small_heads():
    c = synth.decode_case(B=5, Nk=2, Nv=4, S=3, Dk=32, Dv=64, slots=9, dtype="f32", base=613,
                          lens=[3, 1, 0, 2, 3])
    _decode(c, 613)


def _chunk(c, base, poison=False, gates=True, qk_norm=False):
    ref = _raw_qk(c, base) if qk_norm else copy.copy(c)
    g = None
    if gates:
        gref, g = _fused(c, base, poison)
        ref.beta, ref.g = gref.beta, gref.g
    say(f"gdr_chunk {c.dtype} B={c.B} S={c.S} Dk={c.Dk} C={c.chunk} fused gates={gates} qk norm={qk_norm}")
    out, fin = gdr.gdr_chunk(to_dev(c.q), to_dev(c.k), to_dev(c.v), None if gates else to_dev(c.beta),
                             initial_state=to_dev(c.state), actual_seq_lengths=to_dev(c.lens),
                             g=None if gates else to_dev(c.g), scale_value=c.scale, chunk_size=c.chunk,
                             gates=g, use_qk_l2norm=qk_norm)
    torch.cuda.synchronize()
    _check_full(ref, out, fin)


def test_fused_gates_prefill():
    # several chunks, ragged tails and an empty sequence; NaN gate inputs in the
    # padding must never be read
    c = synth.config(4, B=3, Nk=2, Nv=4, S=300, lens=[300, 129, 0], base=614, poison_pad=True)
    _chunk(c, 614, poison=True)


def test_fused_gates_prefill_fp32():
    c = synth.prefill_case(B=2, Nk=1, Nv=2, S=100, Dk=32, Dv=32, dtype="f32", base=615, lens=[100, 37],
                           chunk=32, scale=0.3, init_std=0.1)
    _chunk(c, 615)


# --- in-kernel q/k normalisation, alone and with the fused gates ------------

@pytest.mark.parametrize("gates,gk", [(False, None), (True, (-0.5, -0.001))])
def test_qk_norm_one_token(gates, gk):
    _decode(synth.config(2, B=24, gk=gk, base=621), 621, gates=gates, qk_norm=True)


@pytest.mark.parametrize("gates", [False, True])
def test_qk_norm_multi_token(gates):
    _decode(synth.config(3, B=40, base=622), 622, gates=gates, qk_norm=True)


def test_qk_norm_decode_fp32_small_heads():
    c = synth.decode_case(B=5, Nk=2, Nv=4, S=3, Dk=32, Dv=64, slots=9, dtype="f32", base=623,
                          lens=[3, 1, 0, 2, 3])
    _decode(c, 623, gates=False, qk_norm=True)


@pytest.mark.parametrize("gates", [False, True])
def test_qk_norm_prefill(gates):
    c = synth.config(4, B=3, Nk=2, Nv=4, S=300, lens=[300, 129, 0], base=624)
    _chunk(c, 624, gates=gates, qk_norm=True)


def test_qk_norm_prefill_fp32():
    c = synth.prefill_case(B=2, Nk=1, Nv=2, S=100, Dk=32, Dv=32, dtype="f32", base=625, lens=[100, 37],
                           chunk=32, scale=0.3, init_std=0.1)
    _chunk(c, 625, gates=False, qk_norm=True)


def test_qk_norm_prefill_no_decay():
    # g absent takes the kernel variant without decay factors; rows past each
    # length must still come out zero with normalised (zero) q rows there
    c = synth.config(5, B=3, Nk=2, Nv=4, S=300, lens=[300, 129, 1], base=626)
    _chunk(c, 626, gates=False, qk_norm=True)


def test_whole_heads_fused_gates_and_qk_norm():
    # 512 heads: one workgroup per whole head, which scales the staged V rows
    # by the gate's beta; NaN gate inputs in the padding must never be read
    c = synth.config(4, B=8, Nk=16, Nv=64, S=130, lens=[130, 64, 1, 0, 99, 130, 128, 65], base=627, poison_pad=True)
    _chunk(c, 627, poison=True, gates=True, qk_norm=True)
