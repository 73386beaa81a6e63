"""Benchmark of the Gated Delta Rule library on one MI355X.

Headline: decode tokens/s on the decode step workload (B=64, Nk=16, Nv=32,
S=1, Dk=Dv=128, bf16, 64-slot pool), with the state traffic as a fraction of
HBM peak. Secondary entries: speculative decode (B=128, S=4, per-key gate),
chunked prefill (B=4, S=4096, Nv=32) and varlen prefill without decay (B=16,
S<=16384, Nv=64), each with its roofline and an oracle CPU baseline, plus the
fused-gate, epilogue and conv1d variants.

A step is one call of the operator over one batch. Inputs sit in HBM before
the timed region; decode rotates over enough pool copies that the working set
exceeds the 256 MB last-level cache. Kernel time comes from HIP events
recorded on the stream the kernels are launched on. Prints one JSON line.
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gated_deltanet_recurrence_amd as gdr  # noqa: E402
import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
F16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 matrix peak
METRIC = "decode tok/s + state GB/s (%HBM); prefill tok/s + TFLOP/s (%MFMA), Dk=Dv=128"


def dev(a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def esize(dtype):
    return 4 if dtype == "f32" else 2


def dtype_code(dtype):
    return {"bf16": gdr.GDR_BF16, "f16": gdr.GDR_F16, "f32": gdr.GDR_F32}[dtype]


# ---------------------------------------------------------------------------
# measured HBM traffic (rocprofv3 FETCH_SIZE / WRITE_SIZE), from profiles/
# ---------------------------------------------------------------------------
CSRC = os.path.join(ROOT, "gated_deltanet_recurrence_amd", "csrc")
KERNEL_SOURCES = {
    "decode": ["gdr_decode.hip", "gdr_common.h"],
    "chunk": ["gdr_chunk.hip", "gdr_common.h"],
    "chunk+norm": ["gdr_chunk.hip", "gdr_norm.hip", "gdr_common.h"],
    "conv": ["gdr_conv.hip", "gdr_common.h"],
}


def source_hash(kind):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(profile, kind, entry=None):
    """HBM bytes per launch recorded in a profiles/ summary, or None when the
    summary is missing or was taken from a different kernel source. A summary
    covering several launches labels each figure, as
    "traffic bytes per launch [entry]: `N`", and records the hash of every
    kind of source it covers as "kernel source sha256 [kind]: `H`"."""
    path = os.path.join(ROOT, "profiles", profile)
    try:
        text = open(path).read()
    except OSError:
        return None
    tag = "" if entry is None else re.escape(f" [{entry}]")
    m_bytes = re.search(r"traffic bytes per launch" + tag + r": `(\d+)`", text)
    hashes = dict(re.findall(r"kernel source sha256 \[([\w+]+)\]: `([0-9a-f]{64})`", text))
    m_hash = re.search(r"kernel source sha256: `([0-9a-f]{64})`", text)
    h = hashes.get(kind, m_hash.group(1) if m_hash else None)
    if not m_bytes or h != source_hash(kind):
        return None
    return int(m_bytes.group(1))


FUSED_PROFILE = "fused_gates_decode_step_and_chunked_prefill.txt"
NORM_PROFILE = "epilogue_kernels_decode_step_and_chunked_prefill.txt"
CONV_PROFILE = "conv_kernels_prefill_and_decode_step.txt"
F16_PROFILE = "f16_decode_step_and_chunked_prefill.txt"


# ---------------------------------------------------------------------------
# algorithmic work per call
# ---------------------------------------------------------------------------
def gate_bytes(c, fused):
    """Gate bytes per token and value head: beta and g, or with fused gates
    the beta logits and a (A_log and dt_bias are per call)."""
    e = esize(c.dtype)
    return 2 * e if fused else e + (4 if c.g is not None else 0)


def decode_bytes(c, fused=False, norm=False):
    """State read once per active sequence and written once per distinct
    consecutive write slot, plus token inputs, outputs and integers (and with
    the gated RMSNorm epilogue its z of every valid token and its w)."""
    e = esize(c.dtype)
    L = c.valid_lengths()
    S, slots = c.S, c.state.shape[0]
    hs = c.Nv * c.Dk * c.Dv * e
    state = 0
    tok = 0
    for b in range(c.B):
        n = int(L[b]) if c.n_acc is None else int(c.n_acc[b])
        if L[b] == 0 or n < 1 or n > S or not 0 <= c.idx[b * S + n - 1] < slots:
            continue
        writes = 0
        for t in range(L[b]):
            w = c.idx[b * S + t]
            last = t == L[b] - 1 or c.idx[b * S + t + 1] != w
            writes += int(last and 0 <= w < slots)
        state += hs * (1 + writes)
        tok += int(L[b])
    per_tok = 2 * c.Nk * c.Dk * e + c.Nv * c.Dv * e + c.Nv * gate_bytes(c, fused) \
        + (4 * c.Nv * c.Dk if c.gk is not None else 0) + (c.Nv * c.Dv * e if norm else 0)
    out = c.B * c.S * c.Nv * c.Dv * e + (4 * c.Dv if norm else 0)
    ints = c.B * 4 * (2 if c.n_acc is not None else 1) + c.B * c.S * 4 + (8 * c.Nv if fused else 0)
    return state, state + tok * per_tok + out + ints, tok


def prefill_work(c, fused=False, norm=False):
    """(bytes, flops) per call. Flops per token and value head:
    C(3Dk + 2Dv) + C^2/3 + 6 Dk Dv (triangular products counted at half).
    The gated RMSNorm epilogue adds its z (and w) to the bytes; its flops are
    left out."""
    e = esize(c.dtype)
    L = c.valid_lengths()
    T = int(L.sum())
    per_tok = 2 * c.Nk * c.Dk * e + c.Nv * c.Dv * e + c.Nv * gate_bytes(c, fused) + (c.Nv * c.Dv * e if norm else 0)
    out = c.B * c.S * c.Nv * c.Dv * e + (8 * c.Nv if fused else 0) + (4 * c.Dv if norm else 0)
    states = c.B * c.Nv * c.Dk * c.Dv * e * ((1 if c.state is not None else 0) + 1)
    C = c.chunk
    f_tok = C * (3 * c.Dk + 2 * c.Dv) + C * C / 3 + 6 * c.Dk * c.Dv
    return T * per_tok + out + states, T * c.Nv * f_tok, T


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------
WARM_S = 0.3   # untimed warm-up of at least this long before every timed run


GRAPH_MIN_LAUNCHES = 64


def time_calls(calls, steps, warmup, use_graph):
    """Runs `warmup` then `steps` calls (cycling through `calls`), timed with
    HIP events on the current stream. Returns (ms per call by events, wall s).
    The warm-up continues, untimed, until it has lasted WARM_S seconds: the
    GPU's clock ramps up over a few milliseconds of sustained work, and a
    short call run after an idle phase would otherwise be timed partly at
    idle clock."""
    stream = torch.cuda.current_stream()
    n = len(calls)
    if use_graph:
        for i in range(n):
            calls[i]()                               # first launch outside capture
        torch.cuda.synchronize()
        # A graph holds at least GRAPH_MIN_LAUNCHES calls (the list repeated),
        # so that the host's cost of one replay stays below the GPU time it
        # launches, also for calls of a few microseconds.
        rounds = max(1, math.ceil(GRAPH_MIN_LAUNCHES / n))
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(rounds):
                for i in range(n):
                    calls[i]()
        n *= rounds
        reps_w = max(1, math.ceil(warmup / n))
        t_w = time.perf_counter()
        for _ in range(reps_w):
            graph.replay()
        torch.cuda.synchronize()
        while time.perf_counter() - t_w < WARM_S:
            for _ in range(reps_w):
                graph.replay()
            torch.cuda.synchronize()
        reps = max(1, math.ceil(steps / n))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(reps):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return e0.elapsed_time(e1) / (reps * n), wall, reps * n
    t_w = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - t_w < WARM_S:
        calls[i % n]()
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        calls[i % n]()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall, steps


def fused_gate_tensors(c, fused):
    """Device tensors of the fused gates (beta logits, a, A_log, dt_bias), or
    None; the plain beta and g are then left out of the call."""
    return None if fused is None else [dev(x) for x in fused]


def norm_fields(a, t, c, norm):
    """Puts the gated RMSNorm epilogue's (z, w) storage arrays (synth.norm_inputs)
    on the device and into the marshalled arguments a (eps 1e-6)."""
    if norm is None:
        return
    t["nz"], t["nw"] = dev(norm[0]), dev(norm[1])
    a.norm_z, a.norm_w, a.norm_eps = t["nz"].data_ptr(), t["nw"].data_ptr(), 1e-6


def decode_calls(c, copies, fused=None, norm=None):
    """Pre-marshalled gdr_decode calls, one per copy of the pool and inputs.
    fused: None, or the fused-gate storage arrays (synth.gate_inputs); norm:
    None, or the epilogue's (synth.norm_inputs)."""
    lib = gdr.load_library()
    calls, keep = [], []
    for _ in range(copies):
        t = dict(q=dev(c.q), k=dev(c.k), v=dev(c.v), beta=None if fused else dev(c.beta),
                 g=None if fused else dev(c.g), gk=dev(c.gk),
                 pool=dev(c.state), lens=dev(c.lens), idx=dev(c.idx), nacc=dev(c.n_acc))
        t["out"] = torch.empty((c.B, c.Nv, c.S, c.Dv), dtype=t["q"].dtype, device="cuda")
        t["gates"] = fused_gate_tensors(c, fused)
        p = lambda x: None if x is None else x.data_ptr()
        a = gdr.DecodeArgs(dtype_code(c.dtype), c.B, c.Nk, c.Nv, c.S,
                           c.Dk, c.Dv, c.state.shape[0], c.idx.size, p(t["q"]), p(t["k"]), p(t["v"]),
                           p(t["beta"]), p(t["g"]), p(t["gk"]), p(t["pool"]), p(t["lens"]), p(t["idx"]),
                           p(t["nacc"]), c.scale, p(t["out"]), *[p(x) for x in (t["gates"] or [None] * 4)])
        norm_fields(a, t, c, norm)
        keep.append((t, a))

        def call(a=a):
            rc = lib.gdr_decode(a, torch.cuda.current_stream().cuda_stream)
            if rc:
                raise RuntimeError(f"gdr_decode failed: {rc}")
        calls.append(call)
    return calls, keep


def chunk_calls(c, copies, fused=None, norm=None):
    lib = gdr.load_library()
    calls, keep = [], []
    for _ in range(copies):
        t = dict(q=dev(c.q), k=dev(c.k), v=dev(c.v), beta=None if fused else dev(c.beta),
                 g=None if fused else dev(c.g), init=dev(c.state), lens=dev(c.lens))
        t["out"] = torch.empty((c.B, c.Nv, c.S, c.Dv), dtype=t["q"].dtype, device="cuda")
        t["fin"] = torch.empty((c.B, c.Nv, c.Dk, c.Dv), dtype=t["q"].dtype, device="cuda")
        t["gates"] = fused_gate_tensors(c, fused)
        p = lambda x: None if x is None else x.data_ptr()
        a = gdr.ChunkArgs(dtype_code(c.dtype), c.B, c.Nk, c.Nv, c.S, c.Dk,
                          c.Dv, c.chunk, p(t["q"]), p(t["k"]), p(t["v"]), p(t["beta"]), p(t["g"]),
                          p(t["init"]), p(t["lens"]), c.scale, p(t["out"]), p(t["fin"]), None, 0,
                          *[p(x) for x in (t["gates"] or [None] * 4)])
        norm_fields(a, t, c, norm)
        t["ws"] = gdr.chunk_workspace(a, torch.device("cuda"))
        keep.append((t, a))

        def call(a=a):
            rc = lib.gdr_chunk(a, torch.cuda.current_stream().cuda_stream)
            if rc:
                raise RuntimeError(f"gdr_chunk failed: {rc}")
        calls.append(call)
    return calls, keep


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle on a bounded sample
# ---------------------------------------------------------------------------
def cpu_baseline_decode(c, budget_s):
    import oracle
    args = (c.f64("q"), c.f64("k"), c.f64("v"), c.f64("beta"),
            None if c.g is None else c.g.astype(np.float64),
            None if c.gk is None else c.gk.astype(np.float64), c.lens, c.n_acc, c.idx, c.f64("state"), c.scale)
    tokens = int(c.valid_lengths().sum())
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.decode(*args)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    res = {"value": tokens * reps / el, "unit": "tok/s", "cores": oracle.num_threads(), "kind": "oracle",
           "sample": f"the whole decode step workload ({c.B} sequences x {c.Nv} heads), {reps} calls, {el:.1f} s"}
    # the same on one thread
    reps1, t0 = 0, time.perf_counter()
    while True:
        oracle.decode(*args, nthreads=1)
        reps1 += 1
        el1 = time.perf_counter() - t0
        if el1 >= budget_s / 4:
            break
    res["single_thread"] = {"value": tokens * reps1 / el1, "unit": "tok/s", "cores": 1,
                            "sample": f"{reps1} calls, {el1:.1f} s"}
    return res


def cpu_baseline_prefill(c, units, name, whole):
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    rep = c.Nv // c.Nk
    L = c.valid_lengths()
    work = []
    for b, h in units:
        kh = h // rep
        Lb = int(L[b])
        work.append((synth.widen(c.q[b, kh, :Lb], c.dtype), synth.widen(c.k[b, kh, :Lb], c.dtype),
                     synth.widen(c.v[b, h, :Lb], c.dtype), synth.widen(c.beta[b, h, :Lb], c.dtype),
                     None if c.g is None else c.g[b, h, :Lb].astype(np.float64),
                     None if c.state is None else synth.widen(c.state[b, h], c.dtype)))
    nt = oracle.num_threads()
    t0 = time.perf_counter()
    with ThreadPoolExecutor(nt) as ex:
        list(ex.map(lambda w: oracle.sequence(w[0], w[1], w[2], w[3], g=w[4], state=w[5], scale=c.scale), work))
    el = time.perf_counter() - t0
    th = int(sum(L[b] for b, _ in units))
    # tok/s counts a token once for all Nv value heads, as the GPU figure does
    what = "all" if whole else f"{len(units)} of the {c.B * c.Nv}"
    return {"value": th / c.Nv / el, "unit": "tok/s", "cores": nt, "kind": "oracle",
            "token_heads_per_s": th / el,
            "sample": f"{what} (sequence, value head) units of the {name} workload: {th} token-heads "
                      f"({th / c.Nv:.0f} tokens of {c.Nv} heads), {el:.1f} s"}


# ---------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--launch", choices=["graph", "eager"], default="graph")
    ap.add_argument("--copies", type=int, default=8, help="decode pool copies rotated per step")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--only", choices=["decode", "spec", "prefill", "varlen", "fused", "norm", "conv", "f16"], default=None)
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="first run a plain device copy of this many MiB (byte-counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the library and this benchmark run on one GPU; --gpus must be 1"}))
        sys.exit(2)
    torch.cuda.init()
    gdr.load_library()
    use_graph = args.launch == "graph"
    if args.copy_probe_mb:
        n = args.copy_probe_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").random_()
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log = lambda m: print(f"[bench] {m}", file=sys.stderr, flush=True)

    result = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
              "data": "synthetic (seeded; distributions of the operator pages' workloads)"}
    secondary = []

    if args.only in (None, "decode"):
        log("decode step workload: generating inputs")
        c = synth.config(2)
        state_b, bytes_call, tok = decode_bytes(c)
        calls, keep = decode_calls(c, args.copies)
        log("decode step workload: timing")
        ms, wall, nsteps = time_calls(calls, args.steps, args.warmup, use_graph)
        gbs = bytes_call / (ms * 1e-3) / 1e9
        result.update({
            "value": tok / (ms * 1e-3), "unit": "tok/s", "ms_per_step": ms,
            "config": {"workload": "decode step: B=64 Nk=16 Nv=32 S=1 Dk=Dv=128 bf16, 64-slot bf16 pool, "
                                   "permuted slots, no gk", "global_batch": c.B, "seq_len": c.S,
                       "parallelism": "none (1 GPU)", "pool_copies_rotated": args.copies,
                       "launch": args.launch},
            "state_GBps": state_b / (ms * 1e-3) / 1e9,
            "state_frac_hbm": state_b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "roofline": {"kernel": "decode_s1_kernel (one-token bf16 128x128)", "bound": "hbm", "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                         "traffic": measured_traffic("decode_kernel_decode_step.txt", "decode"),
                         "algorithmic_bytes_per_launch": bytes_call},
            "wall_s_timed": wall,
        })
        del keep, calls
        if not args.no_cpu:
            log("decode step workload: oracle CPU baseline")
            result["cpu_baseline"] = cpu_baseline_decode(c, 10.0)
        torch.cuda.empty_cache()

    if args.only in (None, "spec"):
        log("speculative decode workload")
        c = synth.config(3)
        state_b, bytes_call, tok = decode_bytes(c)
        calls, keep = decode_calls(c, max(2, args.copies // 4))
        ms, wall, _ = time_calls(calls, args.steps, args.warmup, use_graph)
        gbs = bytes_call / (ms * 1e-3) / 1e9
        secondary.append({"workload": "speculative decode: B=128 S=4 Nk=16 Nv=32 Dk=Dv=128 bf16, gk, "
                                      "lengths and accepted counts U{1..4}, 256-slot pool",
                          "tok_per_s": tok / (ms * 1e-3), "ms_per_call": ms, "tokens_per_call": tok,
                          "state_GBps": state_b / (ms * 1e-3) / 1e9,
                          "roofline": {"kernel": "decode_mt_kernel (multi-token bf16 128x128)", "bound": "hbm", "achieved": gbs,
                                       "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                                       "traffic": measured_traffic("decode_kernel_speculative_decode.txt", "decode"),
                                       "algorithmic_bytes_per_launch": bytes_call}})
        del keep, calls
        torch.cuda.empty_cache()

    if args.only in (None, "fused"):
        # The decode step and chunked prefill workloads with fused gates: the
        # kernels form beta and g from the beta logits and a (bf16) and the
        # per-head A_log and dt_bias, in place of reading beta (bf16) and g (f32).
        log("decode step workload, fused gates")
        c = synth.config(2)
        state_b, bytes_call, tok = decode_bytes(c, fused=True)
        calls, keep = decode_calls(c, args.copies, fused=synth.gate_inputs(202, c.B, c.Nv, c.S, c.dtype))
        ms, wall, _ = time_calls(calls, args.steps, args.warmup, use_graph)
        gbs = bytes_call / (ms * 1e-3) / 1e9
        secondary.append({"workload": "decode step, fused gates: B=64 Nk=16 Nv=32 S=1 Dk=Dv=128 bf16, beta logits "
                                      "and a in bf16, A_log and dt_bias per head",
                          "tok_per_s": tok / (ms * 1e-3), "ms_per_call": ms, "tokens_per_call": tok,
                          "state_GBps": state_b / (ms * 1e-3) / 1e9,
                          "roofline": {"kernel": "decode_s1_kernel (fused gates)", "bound": "hbm", "achieved": gbs,
                                       "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                                       "traffic": measured_traffic(FUSED_PROFILE, "decode", "decode step"),
                                       "algorithmic_bytes_per_launch": bytes_call}})
        del keep, calls
        torch.cuda.empty_cache()
        log("chunked prefill workload, fused gates")
        c = synth.config(4)
        bytes_call, flops, tok = prefill_work(c, fused=True)
        calls, keep = chunk_calls(c, 2, fused=synth.gate_inputs(404, c.B, c.Nv, c.S, c.dtype))
        ms, wall, _ = time_calls(calls, max(10, args.steps // 8), max(2, args.warmup // 8), use_graph)
        tf = flops / (ms * 1e-3) / 1e12
        secondary.append({"workload": "chunked prefill, fused gates: B=4 S=4096 Nk=16 Nv=32 Dk=Dv=128 bf16, "
                                      "initial state, C=64, beta logits and a in bf16",
                          "tok_per_s": tok / (ms * 1e-3), "ms_per_call": ms, "tokens_per_call": tok,
                          "TFLOPs": tf, "GBps": bytes_call / (ms * 1e-3) / 1e9,
                          "roofline": {"kernel": "chunk_t_kernel + chunk_mfma_kernel (fused gates)", "bound": "mfma",
                                       "achieved": tf, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                       "frac": tf / BF16_MFMA_PEAK_TFLOPS,
                                       "traffic": measured_traffic(FUSED_PROFILE, "chunk", "chunked prefill"),
                                       "algorithmic_flops_per_launch": flops,
                                       "algorithmic_bytes_per_launch": bytes_call}})
        del keep, calls, c
        torch.cuda.empty_cache()

    if args.only in (None, "f16"):
        # The decode step and chunked prefill workloads with fp16 I/O (the
        # prefill operator's other accepted dtype): same shapes, distributions
        # and seeds, stored in IEEE half.
        log("decode step workload, fp16")
        c = synth.config(2, dtype="f16")
        state_b, bytes_call, tok = decode_bytes(c)
        calls, keep = decode_calls(c, args.copies)
        ms, wall, _ = time_calls(calls, args.steps, args.warmup, use_graph)
        gbs = bytes_call / (ms * 1e-3) / 1e9
        secondary.append({"workload": "decode step, fp16: B=64 Nk=16 Nv=32 S=1 Dk=Dv=128 fp16, 64-slot fp16 pool",
                          "dtype": "f16", "tok_per_s": tok / (ms * 1e-3), "ms_per_call": ms, "tokens_per_call": tok,
                          "state_GBps": state_b / (ms * 1e-3) / 1e9,
                          "roofline": {"kernel": "decode_s1_kernel (fp16)", "bound": "hbm", "achieved": gbs,
                                       "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                                       "traffic": measured_traffic(F16_PROFILE, "decode", "decode step"),
                                       "algorithmic_bytes_per_launch": bytes_call}})
        del keep, calls
        torch.cuda.empty_cache()
        log("chunked prefill workload, fp16")
        c = synth.config(4, dtype="f16")
        bytes_call, flops, tok = prefill_work(c)
        calls, keep = chunk_calls(c, 2)
        ms, wall, _ = time_calls(calls, max(10, args.steps // 8), max(2, args.warmup // 8), use_graph)
        tf = flops / (ms * 1e-3) / 1e12
        secondary.append({"workload": "chunked prefill, fp16: B=4 S=4096 Nk=16 Nv=32 Dk=Dv=128 fp16, g, initial "
                                      "state, C=64", "dtype": "f16",
                          "tok_per_s": tok / (ms * 1e-3), "ms_per_call": ms, "tokens_per_call": tok,
                          "TFLOPs": tf, "GBps": bytes_call / (ms * 1e-3) / 1e9,
                          "roofline": {"kernel": "chunk_t_kernel + chunk_mfma_kernel (fp16)", "bound": "mfma",
                                       "achieved": tf, "peak": F16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                       "frac": tf / F16_MFMA_PEAK_TFLOPS,
                                       "traffic": measured_traffic(F16_PROFILE, "chunk", "chunked prefill"),
                                       "algorithmic_flops_per_launch": flops,
                                       "algorithmic_bytes_per_launch": bytes_call}})
        del keep, calls, c
        torch.cuda.empty_cache()

    if args.only in (None, "norm"):
        # The decode step and chunked prefill workloads with the gated RMSNorm
        # output epilogue (z in bf16, w float32): in the decode kernel itself,
        # and as a pass of its own after the prefill kernels.
        log("decode step workload, gated RMSNorm epilogue")
        c = synth.config(2)
        state_b, bytes_call, tok = decode_bytes(c, norm=True)
        calls, keep = decode_calls(c, args.copies, norm=synth.norm_inputs(202, c.B, c.Nv, c.S, c.Dv, c.dtype))
        ms, wall, _ = time_calls(calls, args.steps, args.warmup, use_graph)
        gbs = bytes_call / (ms * 1e-3) / 1e9
        secondary.append({"workload": "decode step, gated RMSNorm epilogue: B=64 Nk=16 Nv=32 S=1 Dk=Dv=128 bf16, "
                                      "z in bf16, w float32",
                          "tok_per_s": tok / (ms * 1e-3), "ms_per_call": ms, "tokens_per_call": tok,
                          "state_GBps": state_b / (ms * 1e-3) / 1e9,
                          "roofline": {"kernel": "decode_s1_kernel (epilogue in the kernel)", "bound": "hbm",
                                       "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                                       "traffic": measured_traffic(NORM_PROFILE, "decode", "decode step"),
                                       "algorithmic_bytes_per_launch": bytes_call}})
        del keep, calls
        torch.cuda.empty_cache()
        log("chunked prefill workload, gated RMSNorm epilogue")
        c = synth.config(4)
        bytes_call, flops, tok = prefill_work(c, norm=True)
        calls, keep = chunk_calls(c, 2, norm=synth.norm_inputs(404, c.B, c.Nv, c.S, c.Dv, c.dtype))
        ms, wall, _ = time_calls(calls, max(10, args.steps // 8), max(2, args.warmup // 8), use_graph)
        tf = flops / (ms * 1e-3) / 1e12
        secondary.append({"workload": "chunked prefill, gated RMSNorm epilogue: B=4 S=4096 Nk=16 Nv=32 Dk=Dv=128 "
                                      "bf16, g, initial state, C=64, z in bf16, w float32",
                          "tok_per_s": tok / (ms * 1e-3), "ms_per_call": ms, "tokens_per_call": tok,
                          "TFLOPs": tf, "GBps": bytes_call / (ms * 1e-3) / 1e9,
                          "roofline": {"kernel": "chunk_t_kernel + chunk_mfma_kernel + norm_kernel", "bound": "mfma",
                                       "achieved": tf, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                       "frac": tf / BF16_MFMA_PEAK_TFLOPS,
                                       "traffic": measured_traffic(NORM_PROFILE, "chunk+norm", "chunked prefill"),
                                       "algorithmic_flops_per_launch": flops,
                                       "algorithmic_bytes_per_launch": bytes_call}})
        del keep, calls, c
        torch.cuda.empty_cache()

    if args.only in (None, "conv"):
        # The depthwise causal conv1d + SiLU ahead of the recurrence, at the
        # chunked prefill and decode step sizes: C = 2 Nk Dk + Nv Dv = 8192
        # channels, K = 4 taps, bf16. Bytes: x read and q, k, v written once,
        # the carried states read and written, the weights and bias.
        log("conv1d workloads")
        lib = gdr.load_library()
        K = 4
        for name, B, S, slots in (("conv1d prefill", 4, 4096, None), ("conv1d decode step", 64, 1, 64)):
            Nk, Dk, Nv, Dv = 16, 128, 32, 128
            C = 2 * Nk * Dk + Nv * Dv
            x, w, bias, st = synth.conv_inputs(505, B, S, C, K, "bf16", slots=slots)
            calls, keep = [], []
            for _ in range(2 if slots is None else args.copies):
                t = dict(x=dev(x), w=dev(w), bias=dev(bias), st=dev(st),
                         q=torch.empty((B, Nk, S, Dk), dtype=torch.bfloat16, device="cuda"),
                         k=torch.empty((B, Nk, S, Dk), dtype=torch.bfloat16, device="cuda"),
                         v=torch.empty((B, Nv, S, Dv), dtype=torch.bfloat16, device="cuda"))
                if slots is None:
                    t["fin"] = torch.empty_like(t["st"])
                    a = gdr.ConvPrefillArgs(gdr.GDR_BF16, B, S, Nk, Nv, Dk, Dv, K, t["x"].data_ptr(), t["w"].data_ptr(),
                                            t["bias"].data_ptr(), t["st"].data_ptr(), t["fin"].data_ptr(), None,
                                            t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr())
                    fn = lib.gdr_conv_prefill
                else:
                    t["lens"] = dev(np.ones(B, np.int32))
                    t["idx"] = dev(np.random.default_rng(505).permutation(slots)[:B].astype(np.int32))
                    a = gdr.ConvDecodeArgs(gdr.GDR_BF16, B, S, Nk, Nv, Dk, Dv, K, slots, B * S, t["x"].data_ptr(),
                                           t["w"].data_ptr(), t["bias"].data_ptr(), t["st"].data_ptr(),
                                           t["lens"].data_ptr(), t["idx"].data_ptr(), None,
                                           t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr())
                    fn = lib.gdr_conv_decode
                keep.append((t, a))

                def call(a=a, fn=fn):
                    rc = fn(ctypes.byref(a), torch.cuda.current_stream().cuda_stream)
                    if rc:
                        raise RuntimeError(f"conv call failed: {rc}")
                calls.append(call)
            ms, wall, _ = time_calls(calls, args.steps if slots else max(10, args.steps // 8),
                                     args.warmup if slots else max(2, args.warmup // 8), use_graph)
            bytes_call = 2 * B * S * C * 2 + 2 * B * C * (K - 1) * 2 + C * (K + 1) * 4
            gbs = bytes_call / (ms * 1e-3) / 1e9
            secondary.append({"workload": f"{name}: B={B} S={S} C={C} (Nk=16 Dk=128 Nv=32 Dv=128) K={K} bf16, "
                                          f"bias, carried state" + (f", {slots}-slot pool" if slots else ""),
                              "tok_per_s": B * S / (ms * 1e-3), "ms_per_call": ms, "tokens_per_call": B * S,
                              "roofline": {"kernel": "conv_prefill_kernel" if slots is None else "conv_decode_kernel",
                                           "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                           "frac": gbs / HBM_PEAK_GBS,
                                           "traffic": measured_traffic(CONV_PROFILE, "conv", name),
                                           "algorithmic_bytes_per_launch": bytes_call}})
            del keep, calls
            torch.cuda.empty_cache()

    # Oracle samples: the whole chunked prefill workload (128 units, about
    # 2.5 s on 16 cores); every 8th unit of the varlen one (128 of 1024,
    # about 1/8 of its token-heads).
    prefill_sets = []
    if args.only in (None, "prefill"):
        prefill_sets.append(("chunked prefill", 4, "B=4 S=4096 Nk=16 Nv=32 Dk=Dv=128 bf16, g, initial state, C=64",
                             [(b, h) for b in range(4) for h in range(32)], True,
                             "chunk_kernels_chunked_prefill.txt"))
    if args.only in (None, "varlen"):
        prefill_sets.append(("varlen prefill", 5, "B=16 S=16384 (lengths U{256..16384}) Nk=16 Nv=64 Dk=Dv=128 "
                             "bf16, no decay, zero initial state, C=64",
                             [(b, h) for b in range(16) for h in range(64)][::8], False,
                             "chunk_kernels_varlen_prefill.txt"))
    for name, cid, desc, units, whole, profile in prefill_sets:
        log(f"{name}: generating inputs")
        c = synth.config(cid)
        bytes_call, flops, tok = prefill_work(c)
        calls, keep = chunk_calls(c, 2 if cid == 4 else 1)
        log(f"{name}: timing")
        steps = max(10, args.steps // 8)
        ms, wall, _ = time_calls(calls, steps, max(2, args.warmup // 8), use_graph)
        tf = flops / (ms * 1e-3) / 1e12
        gbs = bytes_call / (ms * 1e-3) / 1e9
        entry = {"workload": f"{name}: {desc}", "tok_per_s": tok / (ms * 1e-3), "ms_per_call": ms,
                 "tokens_per_call": tok, "TFLOPs": tf, "frac_mfma_bf16": tf / BF16_MFMA_PEAK_TFLOPS,
                 "GBps": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
                 "roofline": {"kernel": "chunk_t_kernel + chunk_mfma_kernel (one call)", "bound": "mfma",
                              "achieved": tf,
                              "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tf / BF16_MFMA_PEAK_TFLOPS,
                              "traffic": measured_traffic(profile, "chunk"), "algorithmic_flops_per_launch": flops,
                              "algorithmic_bytes_per_launch": bytes_call}}
        del keep, calls
        torch.cuda.empty_cache()
        if not args.no_cpu:
            log(f"{name}: oracle CPU baseline")
            entry["cpu_baseline"] = cpu_baseline_prefill(c, units, name, whole)
        secondary.append(entry)
        del c

    if "value" not in result:
        # a secondary-only run reports its first entry as the value
        s0 = secondary[0]
        result.update({"value": s0["tok_per_s"], "unit": "tok/s", "ms_per_step": s0["ms_per_call"],
                       "config": {"workload": s0["workload"]}, "roofline": s0["roofline"]})
    result["secondary"] = secondary
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
