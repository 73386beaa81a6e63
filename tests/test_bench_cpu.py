"""Host logic of bench.py, on the CPU: the algorithmic byte and flop counts
that its roofline entries divide by, pinned to figures derived by hand; the
gate that only reports profiled HBM traffic for the kernel source it was
taken from; and the one-GPU guard."""
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_decode_step_bytes_by_hand():
    # B = 64 one-token sequences, Nk = 16, Nv = 32, Dk = Dv = 128, bf16, g, one
    # slot per sequence. State: 64 x 32 heads x 128 x 128 x 2 B, read and
    # written once. Per token: q, k (2 x 16 x 128 x 2 B), v (32 x 128 x 2 B),
    # beta (2 B) and g (4 B) per value head. Output 64 x 32 x 128 x 2 B.
    # Integers: lengths and accepted counts (2 x 64 x 4 B), slots (64 x 4 B).
    c = synth.config(2)
    state = 64 * 32 * 128 * 128 * 2 * 2
    tok = 64 * (2 * 16 * 128 * 2 + 32 * 128 * 2 + 32 * (2 + 4))
    out = 64 * 32 * 128 * 2
    ints = 2 * 64 * 4 + 64 * 4
    assert bench.decode_bytes(c) == (state, state + tok + out + ints, 64)
    assert state + tok + out + ints == 135_803_648
    # the epilogue adds z per token and value head, and w once
    _, with_norm, _ = bench.decode_bytes(c, norm=True)
    assert with_norm - (state + tok + out + ints) == 64 * 32 * 128 * 2 + 4 * 128


def test_decode_state_writes_follow_the_slot_rule():
    # A state is written once per run of consecutive tokens with the same
    # slot: one write for a sequence whose positions share one slot, one per
    # valid token when every position has its own slot; skipped sequences
    # (length 0) move no state.
    hs = 2 * 16 * 16 * 2   # one sequence's state, Nv x Dk x Dv x 2 B, for the case below
    kw = dict(B=3, Nk=1, Nv=2, S=4, Dk=16, Dv=16, slots=16, lens=[4, 2, 0], n_acc=[1, 2, 1])
    per_seq = synth.decode_case(idx=np.repeat([3, 7, 9], 4), **kw)
    assert bench.decode_bytes(per_seq)[0] == hs * ((1 + 1) + (1 + 1))
    per_tok = synth.decode_case(idx=np.arange(12), **kw)
    assert bench.decode_bytes(per_tok)[0] == hs * ((1 + 4) + (1 + 2))
    # an accepted count past S or a slot out of range skips the sequence
    bad = synth.decode_case(idx=np.repeat([3, 99, 9], 4), **dict(kw, lens=[4, 2, 1], n_acc=[5, 2, 1]))
    assert bench.decode_bytes(bad)[0] == hs * (1 + 1)


def test_prefill_work_by_hand():
    # B = 4, S = 4096, Nk = 16, Nv = 32, Dk = Dv = 128, C = 64, bf16, g and an
    # initial state. Flops per token and value head:
    # C(3 Dk + 2 Dv) + C^2 / 3 + 6 Dk Dv.
    c = synth.config(4)
    T = 4 * 4096
    f_tok = 64 * (3 * 128 + 2 * 128) + 64 * 64 / 3 + 6 * 128 * 128
    per_tok = 2 * 16 * 128 * 2 + 32 * 128 * 2 + 32 * (2 + 4)
    out = 4 * 4096 * 32 * 128 * 2
    states = 2 * 4 * 32 * 128 * 128 * 2
    b, f, t = bench.prefill_work(c)
    assert t == T and b == T * per_tok + out + states == 414_187_520
    assert f == pytest.approx(T * 32 * f_tok, rel=1e-15)


def test_traffic_is_reported_only_for_the_profiled_source(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    good = prof / "good.txt"
    good.write_text(f"kernel source sha256: `{bench.source_hash('decode')}`\ntraffic bytes per launch: `12345`\n")
    stale = prof / "stale.txt"
    stale.write_text("kernel source sha256: `" + "0" * 64 + "`\ntraffic bytes per launch: `12345`\n")
    (prof / "nohash.txt").write_text("traffic bytes per launch: `12345`\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("good.txt", "decode") == 12345
    assert bench.measured_traffic("good.txt", "chunk") is None      # another kernel's source
    assert bench.measured_traffic("stale.txt", "decode") is None
    assert bench.measured_traffic("nohash.txt", "decode") is None
    assert bench.measured_traffic("missing.txt", "decode") is None
    # a summary of several launches: one labelled figure each, one hash per source kind
    multi = prof / "multi.txt"
    multi.write_text(f"kernel source sha256 [decode]: `{bench.source_hash('decode')}`\n"
                     f"kernel source sha256 [chunk+norm]: `{'1' * 64}`\n"
                     "traffic bytes per launch [decode step]: `111`\n"
                     "traffic bytes per launch [chunked prefill]: `222`\n")
    assert bench.measured_traffic("multi.txt", "decode", "decode step") == 111
    assert bench.measured_traffic("multi.txt", "chunk+norm", "chunked prefill") is None   # stale hash
    assert bench.measured_traffic("multi.txt", "decode", "conv1d prefill") is None         # no such figure


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "--gpus must be 1" in r.stdout
