"""Plants plausible mistakes in copies of the oracle's C source and checks that
the pins catch every one. The planted copies are built in a temporary folder
and only ever run here, on the CPU; the oracle itself is untouched."""
import ctypes
import os
import subprocess

import pytest

import oracle
from oracle import build as obuild
from tests import test_oracle_pins as pins
from tests import test_oracle_semantics as sem

MUTANTS = {
    "dropped_beta": ("kv[j] = beta * (v[j] - kv[j]);", "kv[j] = (v[j] - kv[j]);"),
    "update_sign": ("S[(size_t)i * Dv + j] += k[i] * kv[j];", "S[(size_t)i * Dv + j] -= k[i] * kv[j];"),
    "output_reads_key": ("o[j] += S[(size_t)i * Dv + j] * q[i];", "o[j] += S[(size_t)i * Dv + j] * k[i];"),
    "no_decay": ("const double alpha = has_g ? exp(g) : 1.0;", "const double alpha = 1.0;"),
    "read_before_decay": ("kv[j] += S[(size_t)i * Dv + j] * k[i];",
                          "kv[j] += S[(size_t)i * Dv + j] * k[i] / (has_g ? exp(g) : 1.0);"),
    "per_key_gate_index": ("alpha * exp(gk[i])", "alpha * exp(gk[0])"),
    "scale_dropped": ("o[j] *= scale;", "o[j] *= 1.0;"),
    "output_before_update": (
        "for (int j = 0; j < Dv; ++j) kv[j] = beta * (v[j] - kv[j]); /* kv now holds delta */",
        "for (int j = 0; j < Dv; ++j) kv[j] = 0.0 * beta * (v[j] - kv[j]);"),
    "gqa_modulo": ("kh = h / rep", "kh = h % Nk"),
    "decode_read_slot": ("idx[(size_t)b * S + n - 1]", "idx[(size_t)b * S]"),
    "prefill_pads_not_zeroed": ("for (int t = L; t < S; ++t) memset(out + v_off",
                                "for (int t = L; t < 0; ++t) memset(out + v_off"),
    "decode_writes_only_last": ("if (w >= 0 && w < slots)", "if (w >= 0 && w < slots && t == L - 1)"),
}

# Every pin and semantics test, as (name, callable).
CHECKS = [
    ("hand_step", pins.test_hand_computed_step),
    ("decay_first", pins.test_decay_applies_before_read),
    ("beta_one", pins.test_beta_one_is_pure_delta_rule_closed_form),
    ("retention", pins.test_retention_at_g_minus_one),
    *[(f"brute{s}{gk}", (lambda s=s, gk=gk: pins.test_brute_force_unrolled(s, gk)))
      for s in range(6) for gk in (False, True)],
    ("store_recall", lambda: pins.test_store_then_recall(8, 6, 2)),
    ("chunked", lambda: pins.test_chunked_equals_recurrent(16, True)),
    ("g_absent", pins.test_g_absent_is_bitwise_g_zero),
    ("pure_decay", pins.test_pure_decay_closed_form),
    ("ortho_linear_attention", pins.test_orthogonal_keys_reduce_to_decayed_linear_attention),
    ("axis_keys_gk", pins.test_axis_keys_with_per_key_gate_reduce_to_linear_attention),
    ("dk1_ema", pins.test_dk1_is_an_ema),
    ("write_identity", pins.test_per_step_write_identity),
    ("contractive", pins.test_contractive_under_decay_and_bounded_beta),
    ("gqa", sem.test_gqa_is_repeat_interleave),
    ("prefill_lengths", lambda: sem.test_prefill_lengths_clamp_and_zero_pads(True)),
    ("decode_slots", lambda: sem.test_decode_slot_rules("per_token")),
    ("decode_oob", sem.test_decode_out_of_range_integers_skip),
]


def _build_mutant(tmpdir, name, old, new):
    src = open(obuild.SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found for {name}"
    path_c = os.path.join(tmpdir, f"{name}.c")
    path_so = os.path.join(tmpdir, f"lib{name}.so")
    with open(path_c, "w") as f:
        f.write(src.replace(old, new))
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", path_c, "-o",
                    path_so, "-lm"], check=True)
    return path_so


def _load_as_oracle(path_so):
    saved = oracle._lib
    oracle._lib = None
    real = oracle._build.LIB
    try:
        oracle._build.LIB = path_so
        lib = oracle.load()
    finally:
        oracle._build.LIB = real
    return lib, saved


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    so = _build_mutant(str(tmp_path), name, old, new)
    lib, saved = _load_as_oracle(so)
    caught = []
    try:
        for cname, fn in CHECKS:
            try:
                fn()
            except AssertionError:
                caught.append(cname)
    finally:
        oracle._lib = saved
    assert caught, f"no pin detects the planted mistake '{name}'"


def test_unmutated_copy_passes_every_check(tmp_path):
    so = _build_mutant(str(tmp_path), "identity", "#include <math.h>", "#include <math.h>")
    lib, saved = _load_as_oracle(so)
    try:
        for cname, fn in CHECKS:
            fn()
    finally:
        oracle._lib = saved
