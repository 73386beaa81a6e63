"""Helpers for the GPU parity tests: move seeded cases to the device, call the
library through its C ABI binding, and compare with the float64 oracle."""
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import gated_deltanet_recurrence_amd as gdr
import oracle
import synth

# max-abs bars: float32 and bf16 I/O as stated for the workloads; fp16 I/O
# (the prefill operator's other accepted dtype) takes the bf16 bar.
TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 2e-2}


def say(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def to_dev(a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def to_f64(t):
    if t.dtype == torch.bfloat16:
        return synth.bf16_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.double().cpu().numpy()


def raw_bits(t):
    if t.element_size() == 2:
        return t.contiguous().view(torch.int16)
    return t.contiguous().view(torch.int32)


def run_decode(c, pool=None):
    """Calls gdr_decode on case c; returns (out, pool) device tensors."""
    say(f"gdr_decode {c.dtype} B={c.B} Nk={c.Nk} Nv={c.Nv} S={c.S} Dk={c.Dk} Dv={c.Dv} slots={c.state.shape[0]}")
    pool = to_dev(c.state) if pool is None else pool
    out, pool = gdr.gdr_decode(to_dev(c.q), to_dev(c.k), to_dev(c.v), to_dev(c.beta), pool,
                               to_dev(c.lens), to_dev(c.idx), g=to_dev(c.g), gk=to_dev(c.gk),
                               num_accepted_tokens=to_dev(c.n_acc), scale_value=c.scale)
    torch.cuda.synchronize()
    return out, pool


def run_chunk(c, init=None, use_init=True, out=None, final=None):
    say(f"gdr_chunk {c.dtype} B={c.B} Nk={c.Nk} Nv={c.Nv} S={c.S} Dk={c.Dk} Dv={c.Dv} C={c.chunk}")
    if init is None and use_init:
        init = to_dev(c.state)
    o, f = gdr.gdr_chunk(to_dev(c.q), to_dev(c.k), to_dev(c.v), to_dev(c.beta), initial_state=init,
                         actual_seq_lengths=to_dev(c.lens), g=to_dev(c.g), scale_value=c.scale,
                         chunk_size=c.chunk, out=out, final_state=final)
    torch.cuda.synchronize()
    return o, f


def oracle_decode(c):
    return oracle.decode(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("beta"),
                         None if c.g is None else c.g.astype(np.float64),
                         None if c.gk is None else c.gk.astype(np.float64),
                         c.lens, c.n_acc, c.idx, c.f64("state"), c.scale)


def oracle_prefill(c):
    return oracle.prefill(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("beta"),
                          None if c.g is None else c.g.astype(np.float64), c.f64("state"),
                          c.lens, c.scale)


def oracle_units(c, units, threads=16):
    """Oracle on selected (b, h) units only, from per-unit slices (large cases).
    Returns {(b, h): (out (L, Dv), final (Dk, Dv))}."""
    L = c.valid_lengths()
    rep = c.Nv // c.Nk

    def one(bh):
        b, h = bh
        kh = h // rep
        Lb = int(L[b])
        q = synth.widen(c.q[b, kh, :Lb], c.dtype)
        k = synth.widen(c.k[b, kh, :Lb], c.dtype)
        v = synth.widen(c.v[b, h, :Lb], c.dtype)
        be = synth.widen(c.beta[b, h, :Lb], c.dtype)
        g = None if c.g is None else c.g[b, h, :Lb].astype(np.float64)
        S0 = None if c.state is None else synth.widen(c.state[b, h], c.dtype)
        return bh, oracle.sequence(q, k, v, be, g=g, state=S0, scale=c.scale)

    with ThreadPoolExecutor(threads) as ex:
        return dict(ex.map(one, units))


def check_all_units(c, out, fin, label, threads=16, batch=64):
    """Every (b, h) unit of a prefill call against the oracle, streamed in
    batches of units so that no whole-tensor float64 copy is held: outputs at
    t < L_b and final states within the tolerance, pads exact zeros. Prints
    and returns the margins: max-abs errors and max-abs / RMS of the reference."""
    tol = TOL[c.dtype]
    L = c.valid_lengths()
    units = [(b, h) for b in range(c.B) for h in range(c.Nv)]
    eo = ef = 0.0
    so = sf = 0.0
    no = nf = 0
    for i in range(0, len(units), batch):
        ref = oracle_units(c, units[i:i + batch], threads)
        for (b, h), (o_ref, f_ref) in ref.items():
            n = int(L[b])
            eo = max(eo, max_err(to_f64(out[b, h, :n]), o_ref))
            ef = max(ef, max_err(to_f64(fin[b, h]), f_ref))
            so += float((o_ref * o_ref).sum())
            no += o_ref.size
            sf += float((f_ref * f_ref).sum())
            nf += f_ref.size
    rms_o = (so / max(no, 1)) ** 0.5
    rms_f = (sf / max(nf, 1)) ** 0.5
    say(f"{label}: {len(units)} units; output max-abs err {eo:.3e} (rel {eo / max(rms_o, 1e-30):.3e}), "
        f"final state max-abs err {ef:.3e} (rel {ef / max(rms_f, 1e-30):.3e}); bar {tol:g}")
    assert eo <= tol, f"{label}: output err {eo}"
    assert ef <= tol, f"{label}: final state err {ef}"
    assert_zero_rows(out, L)
    return eo, ef


def max_err(a, b):
    return float(np.abs(np.asarray(a) - np.asarray(b)).max()) if np.asarray(a).size else 0.0


def assert_zero_rows(out_dev, lens):
    """Every output row at t >= L_b is bitwise +0."""
    bits = raw_bits(out_dev)
    S = out_dev.shape[2]
    for b, Lb in enumerate(lens):
        Lb = int(min(max(Lb, 0), S))
        if Lb < S:
            assert bool((bits[b, :, Lb:] == 0).all()), f"nonzero padding in batch entry {b}"
