"""GPU parity of gdr_chunk against the float64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import (TOL, assert_zero_rows, check_all_units, max_err, oracle_prefill, raw_bits, run_chunk,
                            run_decode, say, to_dev, to_f64)
import gated_deltanet_recurrence_amd as gdr

pytestmark = pytest.mark.gpu


def _check_full(c, out, fin):
    tol = TOL[c.dtype]
    o_ref, f_ref = oracle_prefill(c)
    o = to_f64(out)
    L = c.valid_lengths()
    eo = 0.0
    for b in range(c.B):
        e = max_err(o[b, :, :L[b]], o_ref[b, :, :L[b]])
        eo = max(eo, e)
        assert e <= tol, f"output b={b} err {e}"
    assert_zero_rows(out, L)
    e = max_err(to_f64(fin), f_ref)
    say(f"margins: output max-abs err {eo:.3e}, final state {e:.3e}; bar {tol:g}")
    assert e <= tol, f"final state err {e}"


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


def test_prefill_workload_full():
    # the chunked prefill workload at full size, in the launch bench.py times:
    # every (b, h) unit against the oracle
    c = synth.config(4)
    out, fin = run_chunk(c)
    check_all_units(c, out, fin, "chunked prefill workload")


def test_varlen_no_decay_reduced():
    c = synth.config(5, B=6, Nk=2, Nv=8, S=1000, lens=[0, 1, 64, 65, 999, 1000], base=515)
    out, fin = run_chunk(c, use_init=False)
    _check_full(c, out, fin)


def test_varlen_no_decay_full():
    # the varlen prefill workload at full size: every one of its 1024 units
    c = synth.config(5)
    out, fin = run_chunk(c, use_init=False)
    check_all_units(c, out, fin, "varlen prefill workload")


# --- workgroups of whole heads ----------------------------------------------
# The launch takes a workgroup per half of a head's value columns while those
# fit one per CU (B * Nv <= 128 on a 256-CU MI355X), and one per whole head
# beyond; the workloads above cover B * Nv = 128 (halves) and 1024 (whole
# heads).

@pytest.mark.parametrize("gate", ["g", None], ids=["decay", "no-decay"])
def test_whole_heads(gate):
    # several chunks, ragged, one-token and empty sequences, an initial state;
    # NaN in every padded input position
    kw = dict(B=8, Nk=16, Nv=64, S=200, lens=[200, 129, 64, 1, 0, 150, 77, 200], poison_pad=True)
    c = synth.config(4, base=431, **kw) if gate else synth.config(5, base=432, init_std=0.02, **kw)
    assert c.B * c.Nv > 128
    out, fin = run_chunk(c)
    assert bool(torch.isfinite(out.float()).all()) and bool(torch.isfinite(fin.float()).all())
    _check_full(c, out, fin)


@pytest.mark.parametrize("gate", [None, "gate"])
@pytest.mark.parametrize("mix", [0.9, 1.0, ("vocab", 4)], ids=str)
def test_whole_heads_correlated_keys(mix, gate):
    c = synth.prefill_case(B=4, Nk=8, Nv=128, S=130, Dk=128, Dv=128, base=433, gate=gate, key_mix=mix,
                           lens=[130, 64, 1, 99], init_std=0.02)
    out, fin = run_chunk(c)
    _check_full(c, out, fin)


def test_whole_heads_agree_with_column_halves():
    # the same heads through both launches (a 128-head half of the batch takes
    # the column halves). They round differently in one place (diag(beta)
    # joins T or V before its bf16 rounding), so they agree to the parity bar,
    # and both are checked against the oracle.
    c = synth.config(4, B=4, Nk=16, Nv=64, S=130, lens=[130, 64, 1, 0], base=434)
    o_all, f_all = run_chunk(c)
    h = synth.config(4, B=2, Nk=16, Nv=64, S=130, lens=[130, 64], base=434)
    assert h.B * h.Nv <= 128 < c.B * c.Nv and np.array_equal(h.q, c.q[:2]) and np.array_equal(h.v, c.v[:2])
    o_half, f_half = run_chunk(h)
    _check_full(c, o_all, f_all)
    _check_full(h, o_half, f_half)
    eo = max_err(to_f64(o_all[:2]), to_f64(o_half))
    ef = max_err(to_f64(f_all[:2]), to_f64(f_half))
    say(f"whole heads vs column halves: output {eo:.3e}, final state {ef:.3e}")
    assert eo <= TOL[c.dtype] and ef <= TOL[c.dtype]
    assert_zero_rows(o_all, c.valid_lengths())


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("chunk", [16, 32])
def test_16_bit_chunk_sizes_16_and_32(chunk, dtype):
    # the 16-bit path takes chunk sizes 16 and 32 and computes in chunks of
    # 64: a blocking of the same recurrence, so the oracle's results hold
    c = synth.config(4, B=2, Nk=2, Nv=4, S=300, lens=[300, 201], base=420 + chunk, chunk=chunk, dtype=dtype)
    out, fin = run_chunk(c)
    _check_full(c, out, fin)


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


def _degenerate(c, zero_keys):
    """beta = 0 on even value heads (nothing written: the state only decays,
    A = 0 and T = I) and beta = 1 on odd ones, and all-zero keys on the tokens
    of zero_keys (their rows and columns of A vanish)."""
    one = synth.bf16_bits(np.float32(1.0)) if c.dtype == "bf16" else np.asarray(1.0, c.beta.dtype)
    c.beta = c.beta.copy()
    c.beta[:, 0::2] = 0
    c.beta[:, 1::2] = one
    c.k = c.k.copy()
    c.k[:, :, zero_keys] = 0
    return c


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("Nk,Nv", [(1, 2), (16, 160)])
def test_degenerate_betas_and_keys(Nk, Nv, dtype):
    # column halves (2 heads) and whole heads (320 heads); the zero keys span
    # the boundary between the first two chunks
    c = _degenerate(synth.prefill_case(B=2, Nk=Nk, Nv=Nv, S=150, Dk=128, Dv=128, dtype=dtype, base=460 + Nv,
                                       init_std=0.05, lens=[150, 97]), slice(40, 80))
    say(f"gdr_chunk {dtype} B=2 Nv={Nv} S=150: beta 0 / 1 by head, zero keys on tokens 40-79")
    out, fin = run_chunk(c)
    _check_full(c, out, fin)


@pytest.mark.parametrize("B,Nk,Nv", [(4, 40, 40), (3, 8, 64)])
def test_whole_heads_head_grouping(B, Nk, Nv):
    # whole-head workgroups (over 128 heads) with one value head per key head,
    # and eight: the groups kept on one XCD are 1 and 8 units wide
    c = synth.config(4, B=B, Nk=Nk, Nv=Nv, S=130, lens=[130, 64, 1, 0][:B], base=445 + Nv)
    assert c.B * c.Nv > 128
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


# Keys of one chunk that resemble one another (repeated or related tokens):
# the regime where a series form of (I + A)^-1 loses all accuracy. m is the
# mixing weight of a shared direction (m = 1: all keys equal); ("vocab", n)
# draws every key from n unit vectors.
@pytest.mark.parametrize("gate", [None, "gate"])
@pytest.mark.parametrize("mix", [0.5, 0.9, 1.0, ("vocab", 4), ("vocab", 1)], ids=str)
def test_correlated_keys(mix, gate):
    c = synth.prefill_case(B=2, Nk=1, Nv=2, S=300, Dk=128, Dv=128, base=450, gate=gate, key_mix=mix,
                           lens=[300, 213], init_std=0.02)
    out, fin = run_chunk(c)
    _check_full(c, out, fin)


@pytest.mark.parametrize("mix", [1.0, ("vocab", 4)], ids=str)
def test_correlated_keys_long_no_decay(mix):
    # no decay over 4096 tokens, as in the varlen workload: the state grows
    c = synth.prefill_case(B=1, Nk=1, Nv=2, S=4096, Dk=128, Dv=128, base=451, gate=None, key_mix=mix,
                           init_std=None)
    out, fin = run_chunk(c, use_init=False)
    _check_full(c, out, fin)


@pytest.mark.parametrize("mix", [0.9, 1.0, ("vocab", 2)], ids=str)
def test_correlated_keys_fp32(mix):
    c = synth.prefill_case(B=2, Nk=1, Nv=2, S=150, Dk=64, Dv=64, dtype="f32", base=452, gate=None,
                           key_mix=mix, lens=[150, 97], chunk=32, init_std=0.1)
    out, fin = run_chunk(c)
    _check_full(c, out, fin)
