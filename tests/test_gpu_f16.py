"""fp16 I/O: GPU parity of every call with IEEE half inputs, outputs and
states, against the float64 oracle.

The prefill operator accepts bf16 and fp16 and returns the input's type
(lite_boost.ops.chunk_gated_delta_rule: the wrapper paragraph and the final
note). The kernels take fp16 through the same code as bf16, with the element
format as a template parameter: fp16 matrix-core operands, float32
accumulation and state, round-to-nearest-even stores. The bar is the bf16
one, 2e-2 max-abs (fp16 rounds 8x finer; the margins are printed)."""
import numpy as np
import pytest

import synth
from tests.gpu_util import check_all_units, run_chunk, run_decode
from tests.test_gpu_chunk import _check_full
from tests.test_gpu_decode import _check_decode
from tests import test_gpu_conv, test_gpu_fused_gates, test_gpu_norm

pytestmark = pytest.mark.gpu

F16 = dict(dtype="f16")


def test_f16_decode_step_workload():
    c = synth.config(2, **F16)
    out, pool = run_decode(c)
    _check_decode(c, out, pool)


def test_f16_speculative_decode_workload():
    c = synth.config(3, **F16)
    out, pool = run_decode(c)
    _check_decode(c, out, pool)


def test_f16_decode_per_token_slots_and_odd_heads():
    # the slot rule with one slot per token, and an odd head count (one-token
    # calls then run the multi-token kernel)
    c = synth.decode_case(B=32, Nk=16, Nv=32, S=4, Dk=128, Dv=128, slots=256, idx="per_token",
                          lens=("uniform", 1, 4), n_acc=("uniform", 1, 4), gk=(-0.5, -0.001), base=901, **F16)
    out, pool = run_decode(c)
    _check_decode(c, out, pool)
    c = synth.decode_case(B=3, Nk=1, Nv=3, S=1, Dk=128, Dv=128, slots=5, base=902, **F16)
    out, pool = run_decode(c)
    _check_decode(c, out, pool)


@pytest.mark.parametrize("Dk,Dv,S", [(64, 64, 3), (32, 128, 2), (128, 64, 1)])
def test_f16_decode_general_kernel(Dk, Dv, S):
    c = synth.decode_case(B=5, Nk=2, Nv=4, S=S, Dk=Dk, Dv=Dv, slots=9, base=903 + Dk, lens=("uniform", 0, S),
                          gk=(-0.5, -0.001), **F16)
    out, pool = run_decode(c)
    _check_decode(c, out, pool)


@pytest.mark.parametrize("cid,qk_norm", [(2, False), (2, True), (3, True)])
def test_f16_decode_fused_gates(cid, qk_norm):
    c = synth.config(cid, B=24, gk=(-0.5, -0.001), base=904, **F16)
    test_gpu_fused_gates._decode(c, 904, gates=True, qk_norm=qk_norm)


def test_f16_prefill_reduced():
    c = synth.config(4, B=2, Nk=2, Nv=4, S=300, lens=[300, 201], base=905, **F16)
    out, fin = run_chunk(c)
    _check_full(c, out, fin)


def test_f16_whole_heads():
    # 512 heads: one workgroup per whole head
    c = synth.config(4, B=8, Nk=16, Nv=64, S=200, lens=[200, 129, 64, 1, 0, 150, 77, 200], base=911, **F16)
    out, fin = run_chunk(c)
    _check_full(c, out, fin)


def test_f16_prefill_workload_full():
    c = synth.config(4, **F16)
    out, fin = run_chunk(c)
    check_all_units(c, out, fin, "chunked prefill workload, fp16")


def test_f16_varlen_workload_full():
    c = synth.config(5, **F16)
    out, fin = run_chunk(c, use_init=False)
    check_all_units(c, out, fin, "varlen prefill workload, fp16")


@pytest.mark.parametrize("mix,gate", [(1.0, None), (("vocab", 4), "gate"), (0.9, "gate")], ids=str)
def test_f16_correlated_keys(mix, gate):
    c = synth.prefill_case(B=2, Nk=1, Nv=2, S=300, Dk=128, Dv=128, base=906, gate=gate, key_mix=mix,
                           lens=[300, 213], init_std=0.02, **F16)
    out, fin = run_chunk(c)
    _check_full(c, out, fin)


@pytest.mark.parametrize("gates,qk_norm", [(True, False), (False, True), (True, True)])
def test_f16_prefill_fused_gates_and_qk_norm(gates, qk_norm):
    c = synth.config(4, B=3, Nk=2, Nv=4, S=300, lens=[300, 129, 0], base=907, poison_pad=True, **F16)
    test_gpu_fused_gates._chunk(c, 907, poison=gates, gates=gates, qk_norm=qk_norm)


def test_f16_epilogue():
    test_gpu_norm._decode(synth.config(2, B=24, base=908, **F16), 908)
    test_gpu_norm._decode(synth.config(3, B=40, gk=(-0.5, -0.001), base=909, **F16), 909)
    test_gpu_norm._chunk(synth.config(4, B=3, Nk=2, Nv=4, S=300, lens=[300, 129, 0], base=910, **F16), 910)


def test_f16_conv():
    test_gpu_conv._prefill(3, 300, (2, 128, 4, 128), 4, "f16", 911, lens=[300, 129, 0])
    rng = np.random.default_rng(912)
    lens = rng.integers(1, 5, 20)
    n_acc = np.minimum(rng.integers(1, 5, 20), lens)
    test_gpu_conv._decode(20, 4, (2, 128, 4, 128), 4, "f16", 912, slots=88, lens=lens, n_acc=n_acc,
                          idx_mode="per_token")
