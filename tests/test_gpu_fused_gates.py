"""GPU parity of the fused gates against the float64 oracle.

With fused gates the kernels form beta = sigmoid(b) and
g = -exp(A_log) softplus(a + dt_bias) themselves (the Gated DeltaNet blog
post's layer code; inferencelayer deltanet.rs, module header). The reference
is the same token-by-token oracle, fed with oracle.gates of the same raw
inputs in float64."""
import copy

import numpy as np
import pytest
import torch

import synth
from oracle.gates import gates as oracle_gates
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


def _decode(c, base):
    ref, gates = _fused(c, base)
    say(f"gdr_decode fused gates {c.dtype} B={c.B} S={c.S} Dk={c.Dk} gk={c.gk is not None}")
    out, pool = gdr.gdr_decode(to_dev(c.q), to_dev(c.k), to_dev(c.v), None, to_dev(c.state), to_dev(c.lens),
                               to_dev(c.idx), gk=to_dev(c.gk), num_accepted_tokens=to_dev(c.n_acc),
                               scale_value=c.scale, gates=gates)
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


def _chunk(c, base, poison=False):
    ref, gates = _fused(c, base, poison)
    say(f"gdr_chunk fused gates {c.dtype} B={c.B} S={c.S} Dk={c.Dk} C={c.chunk}")
    out, fin = gdr.gdr_chunk(to_dev(c.q), to_dev(c.k), to_dev(c.v), None, initial_state=to_dev(c.state),
                             actual_seq_lengths=to_dev(c.lens), scale_value=c.scale, chunk_size=c.chunk,
                             gates=gates)
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
