"""The hot path's stages composed as one layer core, through the C ABI, against
the float64 oracle's pipeline: depthwise conv1d + SiLU with the q/k/v split
(gdr_conv_*), then the recurrence with in-kernel q/k normalisation, fused gates
and the gated RMSNorm epilogue (gdr_decode / gdr_chunk). This is the order of
inferencelayer deltanet.rs's layer core (conv ring, l2norm, beta and g, the
recurrence, the gated norm) and of the blog post's layer code.

The oracle runs the same chain in float64 without intermediate rounding. The
GPU rounds q, k, v to bf16 between the two calls, so the bar is derived as in
tests/test_gpu_norm.py: the error e of the same call without the epilogue,
measured per row, amplified by the epilogue's 1 / RMS, plus bf16 storage.
Without the epilogue the outputs must meet the plain 2e-2 bar."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import conv as oracle_conv
from oracle.epilogue import gated_rmsnorm, silu
from oracle.gates import gates as oracle_gates, l2norm
from tests.gpu_util import TOL, to_dev, to_f64, say
import gated_deltanet_recurrence_amd as gdr

pytestmark = pytest.mark.gpu

HEADS = (2, 128, 4, 128)   # Nk, Dk, Nv, Dv
K = 4
EPS = 1e-6


def _bound(o_gpu_plain, o_ref, ref_norm, z64, w, eps):
    e_row = np.abs(o_gpu_plain - o_ref).max(-1, keepdims=True)
    m = (o_ref * o_ref).mean(-1, keepdims=True) + eps
    r = 1.0 / np.sqrt(m)
    return TOL["bf16"] + 2.0 ** -7 * np.abs(ref_norm) + e_row * r * (np.abs(w * silu(z64)) + np.abs(ref_norm))


def test_layer_core_decode():
    Nk, Dk, Nv, Dv = HEADS
    C = 2 * Nk * Dk + Nv * Dv
    B, S, slots, base = 12, 3, 40, 911
    rng = np.random.default_rng(base)
    x, w, bias, cpool = synth.conv_inputs(base, B, S, C, K, "bf16", slots=slots)
    lens = rng.integers(0, S + 1, B).astype(np.int32)
    idx = rng.permutation(slots)[:B * S].astype(np.int32)
    n_acc = np.maximum(1, np.minimum(rng.integers(1, S + 1, B), np.maximum(lens, 1))).astype(np.int32)
    bl, a, al, db = synth.gate_inputs(base, B, Nv, S, "bf16")
    z, nw = synth.norm_inputs(base, B, Nv, S, Dv, "bf16")
    rpool = synth._store(rng.standard_normal((slots, Nv, Dk, Dv)) * 0.05, "bf16")
    scale = 1.0 / np.sqrt(Dk)
    say(f"layer core decode B={B} S={S} slots={slots}")

    def run(norm):
        q, k, v, _ = gdr.gdr_conv_decode(to_dev(x), to_dev(w), HEADS, to_dev(cpool), to_dev(lens), to_dev(idx),
                                         bias=to_dev(bias), num_accepted_tokens=to_dev(n_acc))
        out, pool = gdr.gdr_decode(q, k, v, None, to_dev(rpool), to_dev(lens), to_dev(idx), num_accepted_tokens=to_dev(n_acc),
                                   scale_value=scale, gates=[to_dev(t) for t in (bl, a, al, db)], use_qk_l2norm=True,
                                   norm=norm)
        return out, pool
    plain, pool = run(None)
    out, _ = run((to_dev(z), to_dev(nw), EPS))
    torch.cuda.synchronize()
    # float64 pipeline
    y, _ = oracle_conv.decode(synth.widen(x, "bf16"), w, bias, synth.widen(cpool, "bf16"), lens, idx, n_acc)
    q64, k64, v64 = oracle_conv.split(y, *HEADS)
    beta, g = oracle_gates(synth.widen(bl, "bf16"), synth.widen(a, "bf16"), al, db)
    o_ref, p_ref = oracle.decode(l2norm(q64), l2norm(k64), v64, beta, g, None, lens, n_acc, idx,
                                 synth.widen(rpool, "bf16"), scale)
    z64 = synth.widen(z, "bf16")
    o_plain, o = to_f64(plain), to_f64(out)
    for b in range(B):
        L = int(lens[b])
        n = int(n_acc[b])
        if L == 0 or n > S or not 0 <= idx[b * S + n - 1] < slots:
            assert np.all(o[b] == 0.0)
            continue
        e = float(np.abs(o_plain[b, :, :L] - o_ref[b, :, :L]).max())
        assert e <= TOL["bf16"], f"plain output b={b} err {e}"
        ref = gated_rmsnorm(o_ref[b, :, :L], z64[b, :, :L], nw, EPS)
        bound = _bound(o_plain[b, :, :L], o_ref[b, :, :L], ref, z64[b, :, :L], nw, EPS)
        assert np.all(np.abs(o[b, :, :L] - ref) <= bound), f"epilogue b={b}"
        assert np.all(o[b, :, L:] == 0.0)
    # the recurrent states written by the plain call
    p = to_f64(pool)
    for b in range(B):
        L, n = int(lens[b]), int(n_acc[b])
        if L == 0 or n > S or not 0 <= idx[b * S + n - 1] < slots:
            continue
        for t in range(L):
            s = int(idx[b * S + t])
            assert float(np.abs(p[s] - p_ref[s]).max()) <= TOL["bf16"], f"slot {s}"


def test_layer_core_prefill():
    Nk, Dk, Nv, Dv = HEADS
    C = 2 * Nk * Dk + Nv * Dv
    B, S, base = 3, 200, 912
    lens = np.array([200, 77, 0], np.int32)
    x, w, bias, cst = synth.conv_inputs(base, B, S, C, K, "bf16")
    bl, a, al, db = synth.gate_inputs(base, B, Nv, S, "bf16")
    z, nw = synth.norm_inputs(base, B, Nv, S, Dv, "bf16")
    rng = np.random.default_rng(base)
    init = synth._store(rng.standard_normal((B, Nv, Dk, Dv)) * 0.02, "bf16")
    scale = 1.0 / np.sqrt(Dk)
    say(f"layer core prefill B={B} S={S} lens={list(lens)}")

    def run(norm):
        q, k, v, cfin = gdr.gdr_conv_prefill(to_dev(x), to_dev(w), HEADS, bias=to_dev(bias), initial_state=to_dev(cst),
                                             actual_seq_lengths=to_dev(lens))
        out, fin = gdr.gdr_chunk(q, k, v, None, initial_state=to_dev(init), actual_seq_lengths=to_dev(lens),
                                 scale_value=scale, gates=[to_dev(t) for t in (bl, a, al, db)], use_qk_l2norm=True,
                                 norm=norm)
        return out, fin, cfin
    plain, fin, cfin = run(None)
    out, _, _ = run((to_dev(z), to_dev(nw), EPS))
    torch.cuda.synchronize()
    y, cf_ref = oracle_conv.prefill(synth.widen(x, "bf16"), w, bias, synth.widen(cst, "bf16"), lens)
    q64, k64, v64 = oracle_conv.split(y, *HEADS)
    beta, g = oracle_gates(synth.widen(bl, "bf16"), synth.widen(a, "bf16"), al, db)
    o_ref, f_ref = oracle.prefill(l2norm(q64), l2norm(k64), v64, beta, g, synth.widen(init, "bf16"), lens, scale)
    assert np.array_equal(to_f64(cfin), cf_ref), "conv final state"
    assert float(np.abs(to_f64(fin) - f_ref).max()) <= TOL["bf16"], "recurrent final state"
    z64 = synth.widen(z, "bf16")
    o_plain, o = to_f64(plain), to_f64(out)
    for b in range(B):
        L = int(lens[b])
        if L:
            e = float(np.abs(o_plain[b, :, :L] - o_ref[b, :, :L]).max())
            assert e <= TOL["bf16"], f"plain output b={b} err {e}"
            ref = gated_rmsnorm(o_ref[b, :, :L], z64[b, :, :L], nw, EPS)
            bound = _bound(o_plain[b, :, :L], o_ref[b, :, :L], ref, z64[b, :, :L], nw, EPS)
            assert np.all(np.abs(o[b, :, :L] - ref) <= bound), f"epilogue b={b}"
        assert np.all(o[b, :, L:] == 0.0)
