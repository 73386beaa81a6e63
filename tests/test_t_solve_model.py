"""The prefill kernel's UT-transform solve, modelled on the CPU (no GPU).

T = (I + A)^-1 of a chunk is bounded (|T| <= 1 on every key set below), but
keys of one chunk that are alike — repeated tokens give exactly equal keys —
make A far from nilpotent-small, and series forms of the inverse then build
powers far larger than T before they cancel. The kernel therefore solves by
blocked forward substitution (tests/kernel_model.t_blocked restates its
rounding). These tests pin that choice on the key sets the GPU tests draw,
and show that the bars tell a stable solve from an unstable one.

Sources: the Gated DeltaNet blog post, torch_chunk_gated_delta_rule (the
forward-substitution step); lite_boost.ops.chunk_gated_delta_rule, formula
section (the chunked form).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.kernel_model import chunk_A, prefill_model, t_blocked, t_exact, t_power_series

MIXES = [0.0, 0.3, 0.5, 0.7, 0.9, 1.0, ("vocab", 4), ("vocab", 1)]
# T entries are at most 1 here; bf16 storage alone moves them by up to 2^-9,
# and each merge product rounds its two operands to bf16 once more.
T_TOL = 1e-2


def _chunks(mix, gate, beta_one=False):
    c = synth.prefill_case(B=4, Nk=1, Nv=1, S=256, Dk=128, Dv=128, key_mix=mix, gate=gate, base=77)
    for b in range(c.B):
        for c0 in range(0, c.S, 64):
            K = c.f64("k")[b, 0, c0:c0 + 64].astype(np.float32)
            be = np.ones(64, np.float32) if beta_one else c.f64("beta")[b, 0, c0:c0 + 64].astype(np.float32)
            g = None if c.g is None else c.g[b, 0, c0:c0 + 64]
            yield chunk_A(K, be, g)


@pytest.mark.parametrize("gate", [None, "gate"])
@pytest.mark.parametrize("mix", MIXES, ids=str)
def test_blocked_solve_matches_the_inverse(mix, gate):
    for A in _chunks(mix, gate):
        Te = t_exact(A)
        assert np.abs(Te).max() <= 1.0 + 1e-6
        assert np.abs(t_blocked(A) - Te).max() <= T_TOL


@pytest.mark.parametrize("mix", [0.9, 1.0, ("vocab", 1)], ids=str)
def test_blocked_solve_with_beta_one(mix):
    # beta = 1 and equal keys: every token erases the previous one's write
    for A in _chunks(mix, None, beta_one=True):
        assert np.abs(t_blocked(A) - t_exact(A)).max() <= T_TOL


@pytest.mark.parametrize("mix", [0.7, 1.0], ids=str)
def test_power_series_fails_the_same_bar(mix):
    # the product (I - A)(I + A^2)...(I + A^16) on bf16 operands, no decay
    worst = max(np.abs(t_power_series(A) - t_exact(A)).max() for A in _chunks(mix, None))
    assert worst > 100 * T_TOL


def _sequence(mix, gate, L=256, s0=0.0):
    c = synth.prefill_case(B=1, Nk=1, Nv=1, S=L, Dk=128, Dv=128, key_mix=mix, gate=gate, base=78,
                           init_std=s0 or None)
    f = lambda n: c.f64(n)[0, 0]
    S0 = None if c.state is None else c.f64("state")[0, 0]
    g = None if c.g is None else c.g[0, 0]
    ref = oracle.sequence(f("q"), f("k"), f("v"), f("beta"), g=g, state=S0, scale=c.scale)
    args = (f("q").astype(np.float32), f("k").astype(np.float32), f("v").astype(np.float32),
            f("beta").astype(np.float32), g, S0, c.scale)
    return ref, args


@pytest.mark.parametrize("gate,s0", [(None, 0.0), ("gate", 0.02)])
@pytest.mark.parametrize("mix", [0.5, 1.0, ("vocab", 4)], ids=str)
def test_chunk_step_model_within_tolerance(mix, gate, s0):
    # the whole bf16 chunk step with the blocked solve meets the 2e-2 bar
    (o_ref, s_ref), args = _sequence(mix, gate, s0=s0)
    o, s = prefill_model(*args, tsolve=t_blocked)
    assert np.abs(o - o_ref).max() <= 2e-2
    assert np.abs(s - s_ref).max() <= 2e-2


def test_chunk_step_model_detects_the_unstable_solve():
    (o_ref, _), args = _sequence(1.0, None)
    o, _ = prefill_model(*args, tsolve=t_power_series)
    assert not np.abs(o - o_ref).max() <= 2e-2
