"""GPU parity of the gated RMSNorm output epilogue against the float64 oracle.

With norm=(z, w, eps) every valid output row o becomes
o w silu(z) / sqrt(mean(o^2) + eps) (inferencelayer deltanet.rs: module header,
and the per-head gated RMSNorm of its step and chunk code and of DN_STEP /
DN_CHUNK). The one- and multi-token bf16 decode kernels apply it in-kernel;
the other paths (prefill, the general decode kernel) run it as a pass of its
own. The reference is the token-by-token oracle's float64 output passed
through oracle.epilogue.gated_rmsnorm; the states must be those of a call
without the epilogue.

Tolerance, derived from the arithmetic. If o carries an error e (the core
path's, within its own parity bar), the epilogue turns it into at most
e r (|w_j silu(z_j)| + |out_j|) on element j, r = 1 / sqrt(mean(o^2) + eps):
the division by the row's RMS amplifies it by r, and the RMS itself moves by
at most e. e is measured per row, from the same call without the epilogue.
On top of that, storing a value x in bf16 rounds it by up to 2^-8 |x| (half
an ulp of 8 significand bits is 2^-8 of the value's power of two, at most
2^-8 |x|), and the separate pass reads o already rounded (a second 2^-8 |x|);
so the bar per element is that term plus 2e-2 + 2^-7 |ref| for bf16 I/O, and
plus 1e-4 + 1e-5 |ref| for float32. The plain call's error e is asserted to
meet the core bar first, so a wrong recurrence cannot widen its own bound."""
import copy

import numpy as np
import pytest
import torch

import synth
from oracle.epilogue import gated_rmsnorm, silu
from tests.gpu_util import (TOL, assert_zero_rows, max_err, oracle_decode, oracle_prefill, oracle_units, raw_bits,
                             say, to_dev, to_f64)
from tests.test_gpu_fused_gates import _fused, _raw_qk
import gated_deltanet_recurrence_amd as gdr

pytestmark = pytest.mark.gpu

EPS = 1e-6
REL = {"bf16": 2.0 ** -7, "f16": 2.0 ** -10, "f32": 1e-5}


def _norm_inputs(c, base, poison=False):
    z, w = synth.norm_inputs(base, c.B, c.Nv, c.S, c.Dv, c.dtype)
    if poison:
        nanv = synth.BF16_NAN if c.dtype == "bf16" else np.float32(np.nan)
        for b, Lb in enumerate(c.valid_lengths()):
            z[b, :, int(Lb):] = nanv
    return z, w


def _check_rows(c, out, plain, o_ref, z, w, eps):
    """Valid rows against the oracle's rows through the epilogue; rows past the
    length exact zeros. plain: the output of the same call without it."""
    o = to_f64(out)
    e_row = np.abs(to_f64(plain) - o_ref).max(-1, keepdims=True)
    # the bound below leans on the plain call's error, which must itself meet its bar
    assert float(e_row.max()) <= TOL[c.dtype], f"plain output err {float(e_row.max())}"
    z64 = synth.widen(z, c.dtype)
    L = c.valid_lengths()
    for b in range(c.B):
        n = int(L[b])
        ob = o_ref[b, :, :n]
        ref = gated_rmsnorm(ob, z64[b, :, :n], w, eps)
        m = (ob * ob).mean(-1, keepdims=True) + eps
        r = np.where(m > 0, 1.0 / np.sqrt(np.where(m > 0, m, 1.0)), 0.0)
        gate = np.abs(w * silu(z64[b, :, :n]))
        err = np.abs(o[b, :, :n] - ref)
        bound = TOL[c.dtype] + REL[c.dtype] * np.abs(ref) + e_row[b, :, :n] * r * (gate + np.abs(ref))
        assert np.all(err <= bound), f"output b={b}: worst {float((err - bound).max()):.3e} over the bound"
    assert_zero_rows(out, L)


def _decode(c, base, gates=False, qk_norm=False, eps=EPS):
    ref = _raw_qk(c, base) if qk_norm else copy.copy(c)
    g = None
    if gates:
        gref, g = _fused(c, base)
        ref.beta, ref.g = gref.beta, gref.g
    z, w = _norm_inputs(c, base)
    say(f"gdr_decode {c.dtype} B={c.B} S={c.S} Dk={c.Dk} Dv={c.Dv} gk={c.gk is not None} gates={gates} "
        f"qk norm={qk_norm} epilogue eps={eps}")

    def call(norm):
        return gdr.gdr_decode(to_dev(c.q), to_dev(c.k), to_dev(c.v), None if gates else to_dev(c.beta),
                              to_dev(c.state), to_dev(c.lens), to_dev(c.idx), g=None if gates else to_dev(c.g),
                              gk=to_dev(c.gk), num_accepted_tokens=to_dev(c.n_acc), scale_value=c.scale,
                              gates=g, use_qk_l2norm=qk_norm, norm=norm)
    plain, _ = call(None)
    out, pool = call((to_dev(z), to_dev(w), eps))
    torch.cuda.synchronize()
    o_ref, p_ref = oracle_decode(ref)
    _check_rows(c, out, plain, o_ref, z, w, eps)
    # the states are those of the plain recurrence: written slots within
    # tolerance, every other slot bit-identical
    S, slots, L = c.S, c.state.shape[0], c.valid_lengths()
    written = set()
    for b in range(c.B):
        n = int(L[b]) if c.n_acc is None else int(c.n_acc[b])
        if L[b] == 0 or n < 1 or n > S or not 0 <= int(c.idx[b * S + n - 1]) < slots:
            continue
        written |= {int(c.idx[b * S + t]) for t in range(L[b]) if 0 <= c.idx[b * S + t] < slots}
    p = to_f64(pool)
    for s in sorted(written):
        assert max_err(p[s], p_ref[s]) <= TOL[c.dtype], f"slot {s}"
    untouched = [s for s in range(slots) if s not in written]
    if untouched:
        assert torch.equal(raw_bits(pool)[untouched], raw_bits(to_dev(c.state))[untouched])


def _chunk(c, base, gates=False, eps=EPS):
    ref = copy.copy(c)
    g = None
    if gates:
        gref, g = _fused(c, base)
        ref.beta, ref.g = gref.beta, gref.g
    z, w = _norm_inputs(c, base, poison=True)
    say(f"gdr_chunk {c.dtype} B={c.B} S={c.S} Dk={c.Dk} C={c.chunk} gates={gates} epilogue eps={eps}")

    def call(norm):
        return gdr.gdr_chunk(to_dev(c.q), to_dev(c.k), to_dev(c.v), None if gates else to_dev(c.beta),
                             initial_state=to_dev(c.state), actual_seq_lengths=to_dev(c.lens),
                             g=None if gates else to_dev(c.g), scale_value=c.scale, chunk_size=c.chunk,
                             gates=g, norm=norm)
    plain, _ = call(None)
    out, fin = call((to_dev(z), to_dev(w), eps))
    torch.cuda.synchronize()
    o_ref, f_ref = oracle_prefill(ref)
    _check_rows(c, out, plain, o_ref, z, w, eps)
    assert max_err(to_f64(fin), f_ref) <= TOL[c.dtype], "final state"


@pytest.mark.parametrize("gk", [None, (-0.5, -0.001)])
def test_epilogue_one_token(gk):
    # the single-token kernel, epilogue in-kernel
    _decode(synth.config(2, B=24, gk=gk, base=711), 711)


@pytest.mark.parametrize("gk", [None, (-0.5, -0.001)])
def test_epilogue_multi_token(gk):
    # the multi-token kernel with random lengths and accepted counts
    _decode(synth.config(3, B=40, gk=gk, base=712), 712)


def test_epilogue_with_fused_gates_and_qk_norm():
    _decode(synth.config(2, B=24, gk=(-0.5, -0.001), base=713), 713, gates=True, qk_norm=True)
    _decode(synth.config(3, B=24, base=714), 714, gates=True, qk_norm=True)


def test_epilogue_eps_zero():
    _decode(synth.config(2, B=16, base=715), 715, eps=0.0)


def test_epilogue_decode_general_kernels():
    # head sizes and dtypes outside the two bf16 128 x 128 kernels: the
    # epilogue runs as a separate pass
    c = synth.decode_case(B=5, Nk=2, Nv=4, S=3, Dk=32, Dv=64, slots=9, dtype="f32", base=716,
                          lens=[3, 1, 0, 2, 3])
    _decode(c, 716)
    c = synth.decode_case(B=6, Nk=2, Nv=4, S=2, Dk=64, Dv=64, slots=12, dtype="bf16", base=717,
                          lens=("uniform", 0, 2))
    _decode(c, 717)


def test_epilogue_prefill():
    # several chunks, ragged tails and an empty sequence; NaN in z past each
    # length must never be read
    c = synth.config(4, B=3, Nk=2, Nv=4, S=300, lens=[300, 129, 0], base=718)
    _chunk(c, 718)
    _chunk(synth.config(4, B=2, Nk=2, Nv=4, S=200, lens=[200, 77], base=719), 719, gates=True)


def test_epilogue_prefill_whole_heads():
    # 512 heads: the prefill takes whole-head workgroups before the epilogue
    c = synth.config(4, B=8, Nk=16, Nv=64, S=130, lens=[130, 64, 1, 0, 99, 130, 128, 65], base=721)
    _chunk(c, 721)


def test_epilogue_prefill_fp32():
    c = synth.prefill_case(B=2, Nk=1, Nv=2, S=100, Dk=32, Dv=32, dtype="f32", base=720, lens=[100, 37],
                           chunk=32, scale=0.3, init_std=0.1)
    _chunk(c, 720)


def test_epilogue_decode_step_workload_full():
    # the decode step workload at full size with bench.py's epilogue inputs
    _decode(synth.config(2), 202)


def test_epilogue_prefill_workload_full():
    # the chunked prefill workload at full size with bench.py's epilogue
    # inputs; every (b, h) unit against the oracle
    c = synth.config(4)
    z, w = synth.norm_inputs(404, c.B, c.Nv, c.S, c.Dv, c.dtype)
    say(f"gdr_chunk {c.dtype} B={c.B} S={c.S} Nv={c.Nv} epilogue, full size")

    def call(norm):
        return gdr.gdr_chunk(to_dev(c.q), to_dev(c.k), to_dev(c.v), to_dev(c.beta), initial_state=to_dev(c.state),
                             actual_seq_lengths=to_dev(c.lens), g=to_dev(c.g), scale_value=c.scale,
                             chunk_size=c.chunk, norm=norm)
    plain, _ = call(None)
    out, _ = call((to_dev(z), to_dev(w), EPS))
    torch.cuda.synchronize()
    units = [(b, h) for b in range(c.B) for h in range(c.Nv)]
    z64 = synth.widen(z, c.dtype)
    L = c.valid_lengths()
    worst_plain = worst_over = worst_err = 0.0
    for i in range(0, len(units), 64):
        for (b, h), (o_ref, _) in oracle_units(c, units[i:i + 64]).items():
            n = int(L[b])
            o = to_f64(out[b, h, :n])
            e_row = np.abs(to_f64(plain[b, h, :n]) - o_ref).max(-1, keepdims=True)
            assert float(e_row.max()) <= TOL[c.dtype], f"plain output unit {(b, h)}"
            ref = gated_rmsnorm(o_ref, z64[b, h, :n], w, EPS)
            r = 1.0 / np.sqrt((o_ref * o_ref).mean(-1, keepdims=True) + EPS)
            gate = np.abs(w * silu(z64[b, h, :n]))
            bound = TOL[c.dtype] + REL[c.dtype] * np.abs(ref) + e_row * r * (gate + np.abs(ref))
            err = np.abs(o - ref)
            worst_plain = max(worst_plain, float(e_row.max()))
            worst_over = max(worst_over, float((err / bound).max()))
            worst_err = max(worst_err, float(err.max()))
            assert np.all(err <= bound), f"unit {(b, h)}: worst {float((err - bound).max()):.3e} over the bound"
    say(f"epilogue, chunked prefill workload: {len(units)} units; plain output err {worst_plain:.3e}, "
        f"epilogue max-abs err {worst_err:.3e}, at most {worst_over:.3f} of its bound")
    assert_zero_rows(out, L)
