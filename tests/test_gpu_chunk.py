"""GPU parity of gdr_chunk against the float64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import (TOL, assert_zero_rows, max_err, oracle_prefill, oracle_units, raw_bits,
                            run_chunk, run_decode, say, to_dev, to_f64)
import gated_deltanet_recurrence_amd as gdr

pytestmark = pytest.mark.gpu


def _check_full(c, out, fin):
    tol = TOL[c.dtype]
    o_ref, f_ref = oracle_prefill(c)
    o = to_f64(out)
    L = c.valid_lengths()
    for b in range(c.B):
        e = max_err(o[b, :, :L[b]], o_ref[b, :, :L[b]])
        assert e <= tol, f"output b={b} err {e}"
    assert_zero_rows(out, L)
    e = max_err(to_f64(fin), f_ref)
    assert e <= tol, f"final state err {e}"


def _check_units(c, out, fin, units):
    tol = TOL[c.dtype]
    ref = oracle_units(c, units)
    L = c.valid_lengths()
    for (b, h), (o_ref, f_ref) in ref.items():
        o = to_f64(out[b, h, :L[b]])
        assert max_err(o, o_ref) <= tol, f"output unit {(b, h)}"
        assert max_err(to_f64(fin[b, h]), f_ref) <= tol, f"final unit {(b, h)}"
    assert_zero_rows(out, L)


def test_tiny_fp32_chunked():
    c = synth.config(1)
    out, fin = run_chunk(c, use_init=False)
    _check_full(c, out, fin)


@pytest.mark.parametrize("D,C", [(16, 16), (16, 32), (16, 64), (32, 16), (32, 32), (32, 64), (64, 16), (64, 32)])
def test_fp32_head_and_chunk_sizes(D, C):
    c = synth.prefill_case(B=3, Nk=1, Nv=2, S=150, Dk=D, Dv=D, dtype="f32", base=D * 10 + C,
                           init_std=0.1, lens=[150, 77, 0], chunk=C, scale=0.3)
    out, fin = run_chunk(c)
    _check_full(c, out, fin)


def test_prefill_workload_reduced():
    # the prefill workload's distributions at a size the oracle runs in full:
    # several chunks, a ragged tail, two value heads per key head
    c = synth.config(4, B=2, Nk=2, Nv=4, S=300, lens=[300, 201], base=414)
    out, fin = run_chunk(c)
    _check_full(c, out, fin)


def test_prefill_workload_full_sampled():
    c = synth.config(4)
    out, fin = run_chunk(c)
    units = [(0, 0), (0, 1), (1, 7), (2, 16), (3, 31), (3, 30), (1, 22), (2, 9)]
    _check_units(c, out, fin, units)


def test_varlen_no_decay_reduced():
    c = synth.config(5, B=6, Nk=2, Nv=8, S=1000, lens=[0, 1, 64, 65, 999, 1000], base=515)
    out, fin = run_chunk(c, use_init=False)
    _check_full(c, out, fin)


def test_varlen_no_decay_full_sampled():
    c = synth.config(5)
    out, fin = run_chunk(c, use_init=False)
    L = c.valid_lengths()
    bmax, bmin = int(np.argmax(L)), int(np.argmin(L))
    units = [(bmax, 0), (bmax, 63), (bmin, 5), (bmin, 34), (3, 17), (11, 50)]
    _check_units(c, out, fin, units)


def test_nan_in_padding_is_never_read():
    c = synth.config(4, B=3, Nk=1, Nv=2, S=200, lens=[200, 130, 1], base=416, poison_pad=True)
    out, fin = run_chunk(c)
    assert bool(torch.isfinite(out.float()).all()) and bool(torch.isfinite(fin.float()).all())
    _check_full(c, out, fin)


def test_initial_state_none_equals_zeros():
    c = synth.config(5, B=2, Nk=1, Nv=2, S=130, lens=[130, 70], base=517)
    o1, f1 = run_chunk(c, use_init=False)
    zeros = torch.zeros(2, 2, 128, 128, dtype=torch.bfloat16, device="cuda")
    o2, f2 = run_chunk(c, init=zeros)
    assert torch.equal(raw_bits(o1), raw_bits(o2)) and torch.equal(raw_bits(f1), raw_bits(f2))


def test_final_state_may_alias_initial_state():
    c = synth.config(4, B=2, Nk=1, Nv=2, S=100, base=418)
    o1, f1 = run_chunk(c)
    st = to_dev(c.state)
    o2, f2 = run_chunk(c, init=st, final=st)
    assert f2.data_ptr() == st.data_ptr()
    assert torch.equal(raw_bits(o1), raw_bits(o2)) and torch.equal(raw_bits(f1), raw_bits(f2))


def test_empty_sequences_keep_the_initial_state():
    c = synth.config(4, B=2, Nk=1, Nv=2, S=70, lens=[0, 0], base=419)
    out, fin = run_chunk(c)
    assert torch.equal(raw_bits(fin), raw_bits(to_dev(c.state)))
    assert bool((raw_bits(out) == 0).all())


@pytest.mark.parametrize("S", [1, 63, 64, 65, 128])
def test_short_and_boundary_lengths(S):
    c = synth.config(4, B=1, Nk=1, Nv=2, S=S, base=420 + S)
    out, fin = run_chunk(c)
    _check_full(c, out, fin)


@pytest.mark.parametrize("gate", [("uniform", -30.0, -3.0), ("uniform", 0.0, 0.0), ("uniform", -1e-4, 0.0)])
def test_decay_extremes(gate):
    # decay strong enough that exp(gamma) underflows within a chunk, exactly
    # none (g = 0 given), and barely any
    c = synth.prefill_case(B=2, Nk=1, Nv=2, S=200, Dk=128, Dv=128, base=430, gate=gate, init_std=0.05,
                           lens=[200, 131])
    out, fin = run_chunk(c)
    _check_full(c, out, fin)


@pytest.mark.parametrize("Nk,Nv", [(3, 3), (1, 8)])
def test_head_grouping(Nk, Nv):
    # one value head per key head, and eight: the workgroup groups that share
    # q/k (and are kept on one XCD) are 2 and 16 units wide
    c = synth.config(4, B=5, Nk=Nk, Nv=Nv, S=200, lens=[200, 64, 1, 0, 133], base=440 + Nv)
    out, fin = run_chunk(c)
    _check_full(c, out, fin)


def test_resume_equals_one_shot():
    # prefill of 200 tokens, then 170 more from the returned state, against the
    # oracle's single 370-token pass (the intermediate state is stored in bf16)
    c = synth.config(4, B=2, Nk=1, Nv=2, S=370, base=421)
    o_ref, f_ref = oracle_prefill(c)
    first = synth.config(4, B=2, Nk=1, Nv=2, S=370, base=421, lens=[200, 200])
    o1, f1 = run_chunk(first)
    say("resume")
    sl = slice(200, 370)
    q, k, v, be, g = (to_dev(np.ascontiguousarray(getattr(c, n)[:, :, sl])) for n in ("q", "k", "v", "beta", "g"))
    o2, f2 = gdr.gdr_chunk(q, k, v, be, initial_state=f1, g=g, scale_value=c.scale)
    torch.cuda.synchronize()
    assert max_err(to_f64(o1)[:, :, :200], o_ref[:, :, :200]) <= 2e-2
    assert max_err(to_f64(o2), o_ref[:, :, 200:]) <= 2e-2
    assert max_err(to_f64(f2), f_ref) <= 2e-2


def test_prefill_then_decode():
    # a prefill's final state handed to the decode pool continues the sequence
    c = synth.config(4, B=2, Nk=2, Nv=4, S=129, base=422)
    o_ref, f_ref = oracle_prefill(c)
    pre = synth.config(4, B=2, Nk=2, Nv=4, S=129, base=422, lens=[128, 128])
    _, fin = run_chunk(pre)
    pool = fin.clone()                      # slot b holds sequence b
    sl = slice(128, 129)
    out, pool = gdr.gdr_decode(*(to_dev(np.ascontiguousarray(getattr(c, n)[:, :, sl])) for n in ("q", "k", "v", "beta")),
                               pool, to_dev(np.ones(2, np.int32)), to_dev(np.arange(2, dtype=np.int32)),
                               g=to_dev(np.ascontiguousarray(c.g[:, :, sl])), scale_value=c.scale)
    torch.cuda.synchronize()
    assert max_err(to_f64(out)[:, :, 0], o_ref[:, :, 128]) <= 2e-2
    assert max_err(to_f64(pool), f_ref) <= 2e-2


def test_zero_batch_is_noop():
    z = lambda *s: torch.zeros(*s, dtype=torch.bfloat16, device="cuda")
    out, fin = gdr.gdr_chunk(z(0, 1, 8, 128), z(0, 1, 8, 128), z(0, 1, 8, 128), z(0, 1, 8))
    torch.cuda.synchronize()
    assert out.numel() == 0 and fin.numel() == 0
