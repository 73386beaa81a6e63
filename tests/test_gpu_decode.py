"""GPU parity of gdr_decode against the float64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import (TOL, assert_zero_rows, max_err, oracle_decode, raw_bits, run_decode,
                            say, to_dev, to_f64)
import gated_deltanet_recurrence_amd as gdr

pytestmark = pytest.mark.gpu


def _check_decode(c, out, pool):
    """Outputs (valid rows within tolerance, padded rows exact zeros), written
    slots within tolerance, every other slot bit-identical."""
    tol = TOL[c.dtype]
    o_ref, p_ref = oracle_decode(c)
    o = to_f64(out)
    L = c.valid_lengths()
    for b in range(c.B):
        assert max_err(o[b, :, :L[b]], o_ref[b, :, :L[b]]) <= tol, f"output b={b}"
    assert_zero_rows(out, c.lens)
    # slots: written set from the integer rule
    S, slots = c.S, c.state.shape[0]
    written = set()
    for b in range(c.B):
        n = int(L[b]) if c.n_acc is None else int(c.n_acc[b])
        if L[b] == 0 or n < 1 or n > S:
            continue
        r = int(c.idx[b * S + n - 1])
        if not 0 <= r < slots:
            continue
        written |= {int(c.idx[b * S + t]) for t in range(L[b]) if 0 <= c.idx[b * S + t] < slots}
    p = to_f64(pool)
    for s in sorted(written):
        assert max_err(p[s], p_ref[s]) <= tol, f"slot {s}"
    untouched = [s for s in range(slots) if s not in written]
    if untouched:
        before = raw_bits(to_dev(c.state))[untouched]
        assert torch.equal(raw_bits(pool)[untouched], before)
    return o_ref, p_ref


def test_tiny_fp32_chained_decode():
    # 64 single-token calls through a one-slot pool equal the 64-token recurrence.
    c = synth.config(1)
    o_ref, fin_ref = oracle.prefill(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("beta"),
                                    c.g.astype(np.float64), None, None, c.scale)
    pool = torch.zeros(1, 1, 16, 16, dtype=torch.float32, device="cuda")
    outs = []
    for t in range(c.S):
        d = synth.decode_view_of_prefill(c, t)
        out, pool = gdr.gdr_decode(to_dev(d.q), to_dev(d.k), to_dev(d.v), to_dev(d.beta), pool,
                                   to_dev(d.lens), to_dev(d.idx), g=to_dev(d.g),
                                   num_accepted_tokens=to_dev(d.n_acc), scale_value=d.scale)
        outs.append(to_f64(out)[:, :, 0])
    assert max_err(np.stack(outs, 2), o_ref) <= 1e-4
    assert max_err(to_f64(pool)[0], fin_ref[0]) <= 1e-4


def test_decode_step_workload():
    c = synth.config(2)
    out, pool = run_decode(c)
    _check_decode(c, out, pool)


def test_speculative_decode_workload():
    c = synth.config(3)
    out, pool = run_decode(c)
    _check_decode(c, out, pool)


def test_speculative_per_token_slots():
    # Each token position owns a distinct slot; the entering state is read from
    # the slot of token n_acc - 1 and every valid token stores its state.
    c = synth.config(3, B=32, lens=("uniform", 1, 4), n_acc=("uniform", 1, 4), idx="per_token", base=333)
    out, pool = run_decode(c)
    _check_decode(c, out, pool)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Dk,Dv", [(16, 16), (32, 64), (64, 32), (128, 16), (16, 128), (64, 64), (128, 128)])
def test_decode_head_sizes(dtype, Dk, Dv):
    c = synth.decode_case(B=5, Nk=2, Nv=4, S=3, Dk=Dk, Dv=Dv, slots=24, dtype=dtype, base=Dk * 7 + Dv,
                          gk=(-0.5, -0.001), lens=("uniform", 0, 3), n_acc=("uniform", 1, 3), idx="per_token")
    out, pool = run_decode(c)
    _check_decode(c, out, pool)


def test_decode_nan_in_padding_is_never_read():
    c = synth.config(3, B=16, base=313, poison_pad=True)
    out, pool = run_decode(c)
    assert bool(torch.isfinite(out.float()).all())
    _check_decode(c, out, pool)


def test_decode_out_of_range_integers():
    S, slots = 3, 8
    c = synth.decode_case(B=6, Nk=1, Nv=2, S=S, Dk=128, Dv=128, slots=slots, base=31,
                          lens=[3, 5, -1, 3, 2, 3], n_acc=[0, 4, 1, 2, 1, 3],
                          idx=[0, 1, 2, 3, 3, 3, -1, 4, 4, 5, 5, 5, 6, 9, 9, 7, 7, -3])
    out, pool = run_decode(c)
    _check_decode(c, out, pool)


def test_decode_without_g_and_n_acc():
    c = synth.config(3, B=8, gate=None, n_acc=None, base=314)
    out, pool = run_decode(c)
    _check_decode(c, out, pool)


def test_decode_per_key_gate_without_g():
    c = synth.config(3, B=8, gate=None, base=315)
    out, pool = run_decode(c)
    _check_decode(c, out, pool)


def test_decode_zero_batch_is_noop():
    d = lambda *s, dt=torch.bfloat16: torch.zeros(*s, dtype=dt, device="cuda")
    pool = torch.randn(2, 1, 128, 128, device="cuda").to(torch.bfloat16)
    before = pool.clone()
    out, _ = gdr.gdr_decode(d(0, 1, 1, 128), d(0, 1, 1, 128), d(0, 1, 1, 128), d(0, 1, 1), pool,
                            d(0, dt=torch.int32), d(0, dt=torch.int32))
    torch.cuda.synchronize()
    assert out.numel() == 0 and torch.equal(pool, before)


def test_decode_repeated_calls_advance_the_state():
    # Two calls of S = 1 against one call of S = 2 on the same slot: the same
    # recurrence, within the bf16 storage rounding of the intermediate state.
    c2 = synth.decode_case(B=4, Nk=2, Nv=4, S=2, Dk=128, Dv=128, slots=4, base=71)
    o_ref, p_ref = oracle_decode(c2)
    pool = to_dev(c2.state)
    outs = []
    for t in range(2):
        sl = slice(t, t + 1)
        out, pool = gdr.gdr_decode(to_dev(np.ascontiguousarray(c2.q[:, :, sl])), to_dev(np.ascontiguousarray(c2.k[:, :, sl])),
                                   to_dev(np.ascontiguousarray(c2.v[:, :, sl])), to_dev(np.ascontiguousarray(c2.beta[:, :, sl])),
                                   pool, to_dev(np.ones(4, np.int32)), to_dev(c2.idx[::2].copy()),
                                   g=to_dev(np.ascontiguousarray(c2.g[:, :, sl])), scale_value=c2.scale)
        outs.append(to_f64(out)[:, :, 0])
    assert max_err(np.stack(outs, 2), o_ref) <= 2e-2
    assert max_err(to_f64(pool), p_ref) <= 2e-2


# One-token steps of bf16 128 x 128 heads take the workgroup-per-head kernel:
# 256 persistent workgroups walk the heads with the next head's loads in
# flight. These cases exercise the walk (fewer and many more heads than
# workgroups, ragged tails), skipped heads and both gate variants.
@pytest.mark.parametrize("gk", [None, (-0.5, -0.001)])
def test_single_token_skipped_tiles_and_gates(gk):
    # lengths 0/1 and accepted counts 0..2 (0 and 2 are out of range for S = 1);
    # some read slots out of range; NaN in every input of a sequence of length 0.
    B, slots = 40, 64
    rng = np.random.default_rng(4242)
    lens = rng.integers(0, 2, B).astype(np.int32)
    n_acc = rng.integers(0, 3, B).astype(np.int32)
    idx = rng.permutation(slots)[:B].astype(np.int32)
    idx[::7] = slots + 3
    idx[3::11] = -2
    c = synth.decode_case(B=B, Nk=4, Nv=16, S=1, Dk=128, Dv=128, slots=slots, gk=gk, lens=lens,
                          n_acc=n_acc, idx=idx, base=4242, poison_pad=True)
    say(f"single token: skipped {int((lens == 0).sum())} by length, gk={gk is not None}")
    out, pool = run_decode(c)
    assert bool(torch.isfinite(out.float()).all())
    _check_decode(c, out, pool)


@pytest.mark.parametrize("S", [1, 4])
def test_degenerate_betas_and_keys(S):
    # beta = 0 on even value heads (the state only decays) and 1 on odd ones,
    # and all-zero keys for every token of every third sequence; the one-token
    # kernel (S = 1) and the multi-token kernel (S = 4)
    B = 24
    c = synth.decode_case(B=B, Nk=4, Nv=16, S=S, Dk=128, Dv=128, slots=B * S + 5, base=4747 + S)
    one = synth.bf16_bits(np.float32(1.0))
    c.beta = c.beta.copy()
    c.beta[:, 0::2] = 0
    c.beta[:, 1::2] = one
    c.k = c.k.copy()
    c.k[0::3] = 0
    say(f"decode bf16 B={B} S={S}: beta 0 / 1 by head, zero keys for every third sequence")
    out, pool = run_decode(c)
    _check_decode(c, out, pool)


def test_single_token_many_heads_per_workgroup():
    # 97 * 32 = 3104 heads: twelve or thirteen per workgroup.
    c = synth.decode_case(B=97, Nk=8, Nv=32, S=1, Dk=128, Dv=128, slots=128, base=4343)
    out, pool = run_decode(c)
    _check_decode(c, out, pool)


def test_single_token_without_g_and_n_acc():
    c = synth.decode_case(B=12, Nk=2, Nv=8, S=1, Dk=128, Dv=128, slots=16, gate=None, n_acc=None, base=4444)
    out, pool = run_decode(c)
    _check_decode(c, out, pool)


def test_single_token_one_head():
    # One head: a single workgroup.
    c = synth.decode_case(B=1, Nk=1, Nv=1, S=1, Dk=128, Dv=128, slots=3, base=4545)
    out, pool = run_decode(c)
    _check_decode(c, out, pool)


@pytest.mark.parametrize("gk", [None, (-0.5, -0.001)])
def test_single_token_odd_head_count(gk):
    # 3 x 3 = 9 heads: an odd number of beta values. The one-token kernel reads
    # beta of two heads as one 32-bit word, which would run one element past
    # the tensor here; such calls run the multi-token kernel, which reads each
    # head's beta alone.
    c = synth.decode_case(B=3, Nk=1, Nv=3, S=1, Dk=128, Dv=128, slots=5, gk=gk, base=4646)
    out, pool = run_decode(c)
    _check_decode(c, out, pool)


@pytest.mark.parametrize("S,gk", [(2, (-0.5, -0.001)), (3, None), (4, (-0.3, -0.01))])
def test_multi_token_many_heads_and_skips(S, gk):
    # 41 * 16 = 656 heads; lengths 0..S+1 (clamped to S), accepted counts
    # 0..S+1 (0 and S+1 skip the sequence), NaN in every input past a
    # sequence's length.
    B, slots = 41, 48
    rng = np.random.default_rng(5000 + S)
    lens = rng.integers(0, S + 2, B).astype(np.int32)
    n_acc = rng.integers(0, S + 2, B).astype(np.int32)
    idx = np.repeat(rng.permutation(slots)[:B].astype(np.int32), S)
    c = synth.decode_case(B=B, Nk=4, Nv=16, S=S, Dk=128, Dv=128, slots=slots, gk=gk, lens=lens,
                          n_acc=n_acc, idx=idx, base=5100 + S, poison_pad=True)
    say(f"multi token S={S}: skipped {int((c.valid_lengths() == 0).sum())} by length, gk={gk is not None}")
    out, pool = run_decode(c)
    assert bool(torch.isfinite(out.float()).all())
    _check_decode(c, out, pool)


def test_multi_token_slot_patterns():
    # Slots repeated and alternating within a sequence: a token stores the
    # state unless the next token writes the same slot, so slot a of
    # [a, b, b, a] ends with the state after the last token, and b with the
    # state after the third.
    S = 4
    pats = [[0, 0, 0, 0], [1, 2, 2, 1], [3, 4, 5, 6], [7, 7, 8, 8], [9, 10, 10, 10], [11, 12, 11, 12]]
    B = len(pats)
    idx = np.asarray(pats, dtype=np.int32).reshape(-1)
    c = synth.decode_case(B=B, Nk=2, Nv=8, S=S, Dk=128, Dv=128, slots=13, gk=(-0.5, -0.001),
                          lens=np.full(B, S, np.int32), n_acc=np.array([1, 4, 2, 3, 1, 2], np.int32),
                          idx=idx, base=5200)
    out, pool = run_decode(c)
    _check_decode(c, out, pool)
