"""Operator-level semantics of the oracle: head grouping, lengths, padding and
the decode state-pool rules. Expected index sets are built here from the
seeded integer arrays, independently of the oracle."""
import numpy as np
import pytest

import oracle
import synth


def _seq_ref(c, b, h, L, S0):
    """Oracle.sequence on one (b, h) unit of a case (the pinned single-sequence core)."""
    rep = c.Nv // c.Nk
    kh = h // rep
    q, k, v, beta = c.f64("q"), c.f64("k"), c.f64("v"), c.f64("beta")
    g = None if c.g is None else c.g.astype(np.float64)[b, h, :L]
    gk = None if c.gk is None else c.gk.astype(np.float64)[b, h, :L]
    return oracle.sequence(q[b, kh, :L], k[b, kh, :L], v[b, h, :L], beta[b, h, :L], g=g, gk=gk,
                           state=S0, scale=c.scale)


def test_gqa_is_repeat_interleave():
    c = synth.prefill_case(B=2, Nk=2, Nv=6, S=11, Dk=8, Dv=4, base=7, init_std=0.1)
    init = c.f64("state")
    out, fin = oracle.prefill(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("beta"), c.g, init,
                              None, c.scale)
    for b in range(2):
        for h in range(6):
            o, S = _seq_ref(c, b, h, 11, init[b, h])
            np.testing.assert_allclose(out[b, h], o, atol=1e-13, rtol=0)
            np.testing.assert_allclose(fin[b, h], S, atol=1e-13, rtol=0)
    # the modulo grouping h % Nk would pick another key head for h = 1
    q, k = c.f64("q"), c.f64("k")
    assert not np.allclose(k[0, 1 // 3], k[0, 1 % 2])


@pytest.mark.parametrize("with_init", [True, False])
def test_prefill_lengths_clamp_and_zero_pads(with_init):
    S = 9
    lens = [0, 3, S, S + 5, -2]
    c = synth.prefill_case(B=5, Nk=1, Nv=2, S=S, Dk=4, Dv=3, base=8,
                           init_std=0.2 if with_init else None, lens=lens)
    init = c.f64("state")
    out, fin = oracle.prefill(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("beta"), c.g, init,
                              c.lens, c.scale)
    for b, raw in enumerate(lens):
        L = min(max(raw, 0), S)
        for h in range(2):
            S0 = None if init is None else init[b, h]
            o, Sf = _seq_ref(c, b, h, L, S0)
            np.testing.assert_allclose(out[b, h, :L], o, atol=1e-13, rtol=0)
            assert np.all(out[b, h, L:] == 0.0)
            np.testing.assert_allclose(fin[b, h], Sf, atol=1e-13, rtol=0)
            if L == 0:
                expect = np.zeros((4, 3)) if S0 is None else S0
                assert np.array_equal(fin[b, h], expect)


def _decode_run(c, pool=None):
    pool_in = c.f64("state") if pool is None else pool
    return oracle.decode(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("beta"),
                         None if c.g is None else c.g.astype(np.float64),
                         None if c.gk is None else c.gk.astype(np.float64),
                         c.lens, c.n_acc, c.idx, pool_in, c.scale), pool_in


def _expected_decode_sets(c):
    """(read slot or None, list of (t, write slot)) per batch entry, from the integer rule."""
    S, slots = c.S, c.state.shape[0]
    plans = []
    for b in range(c.B):
        L = min(max(int(c.lens[b]), 0), S)
        n = L if c.n_acc is None else int(c.n_acc[b])
        if L == 0 or n < 1 or n > S:
            plans.append((None, []))
            continue
        r = int(c.idx[b * S + n - 1])
        if r < 0 or r >= slots:
            plans.append((None, []))
            continue
        writes = [(t, int(c.idx[b * S + t])) for t in range(L) if 0 <= c.idx[b * S + t] < slots]
        plans.append((r, writes))
    return plans


@pytest.mark.parametrize("layout", ["per_token", "perm"])
def test_decode_slot_rules(layout):
    c = synth.decode_case(B=12, Nk=2, Nv=4, S=4, Dk=8, Dv=8, slots=64, base=9, gk=(-0.5, -0.001),
                          lens=("uniform", 0, 5), n_acc=("uniform", 0, 5), idx=layout)
    (out, pool_out), pool_in = _decode_run(c)
    plans = _expected_decode_sets(c)
    written = set()
    for b, (r, writes) in enumerate(plans):
        L = min(max(int(c.lens[b]), 0), c.S)
        if r is None:
            assert np.all(out[b] == 0.0)
            continue
        for h in range(c.Nv):
            o, _ = _seq_ref(c, b, h, L, pool_in[r, h])
            np.testing.assert_allclose(out[b, h, :L], o, atol=1e-13, rtol=0)
            assert np.all(out[b, h, L:] == 0.0)
        last = {}
        for t, w in writes:
            last[w] = t
        for w, t in last.items():
            written.add(w)
            for h in range(c.Nv):
                _, St = _seq_ref(c, b, h, t + 1, pool_in[r, h])
                np.testing.assert_allclose(pool_out[w, :][h], St, atol=1e-13, rtol=0)
    untouched = [s for s in range(pool_in.shape[0]) if s not in written]
    assert np.array_equal(pool_out[untouched], pool_in[untouched])
    assert len(written) > 0


def test_decode_out_of_range_integers_skip():
    S, slots = 3, 8
    c = synth.decode_case(B=6, Nk=1, Nv=1, S=S, Dk=4, Dv=4, slots=slots, base=10,
                          lens=[3, 3, 3, 3, 2, 3], n_acc=[0, 4, 1, 2, 1, 3],
                          idx=[0, 1, 2,  3, 3, 3,  -1, 4, 4,  5, 5, 5,  6, 9, 9,  7, 7, -3])
    (out, pool_out), pool_in = _decode_run(c)
    # b0: n_acc 0 -> skipped; b1: n_acc 4 > S -> skipped; b2: read slot -1 -> skipped
    for b in (0, 1, 2):
        assert np.all(out[b] == 0.0)
    assert np.array_equal(pool_out[[0, 1, 2, 3, 4]], pool_in[[0, 1, 2, 3, 4]])
    # b3: reads idx[1] = 5, writes slot 5 three times (last wins)
    _, St = _seq_ref(c, 3, 0, 3, pool_in[5, 0])
    np.testing.assert_allclose(pool_out[5, 0], St, atol=1e-13)
    # b4: L = 2, writes slot 6 at t = 0, slot 9 out of range at t = 1 (skipped)
    _, St = _seq_ref(c, 4, 0, 1, pool_in[6, 0])
    np.testing.assert_allclose(pool_out[6, 0], St, atol=1e-13)
    assert np.all(out[4, 0, 2:] == 0.0)
    # b5: reads idx[5*3 + 2] = -3 -> skipped entirely
    assert np.all(out[5] == 0.0)
    assert np.array_equal(pool_out[7], pool_in[7])


def test_decode_n_acc_absent_means_lengths():
    c = synth.decode_case(B=4, Nk=1, Nv=2, S=3, Dk=4, Dv=4, slots=12, base=11,
                          lens=("uniform", 1, 3), n_acc="lens", idx="per_token")
    (o1, p1), _ = _decode_run(c)
    c.n_acc = None
    (o2, p2), _ = _decode_run(c)
    assert np.array_equal(o1, o2) and np.array_equal(p1, p2)


def test_chained_decode_equals_prefill():
    # Tiny fp32 workload: 64 chained single-token decode calls through a 1-slot
    # pool equal one prefill call over the 64 tokens.
    c = synth.config(1)
    out_p, fin = oracle.prefill(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("beta"),
                                c.g.astype(np.float64), None, None, c.scale)
    pool = np.zeros((1, 1, 16, 16))
    outs = []
    for t in range(c.S):
        d = synth.decode_view_of_prefill(c, t)
        o, pool = oracle.decode(d.f64("q"), d.f64("k"), d.f64("v"), d.f64("beta"),
                                d.g.astype(np.float64), None, d.lens, d.n_acc, d.idx, pool, d.scale)
        outs.append(o[:, :, 0])
    np.testing.assert_allclose(np.stack(outs, 2), out_p, atol=1e-13, rtol=0)
    np.testing.assert_allclose(pool[0], fin[0], atol=1e-13, rtol=0)
