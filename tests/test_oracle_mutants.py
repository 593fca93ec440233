"""The oracle's pins have teeth: each planted mistake in a copy of kda_oracle.c
(compiled to a temporary library on the CPU) must fail at least one pin.

The mistakes are the plausible slips in writing the recurrence of "Kimi K3:
Open Frontier Intelligence and Implementation Framework", section "Hybrid
Attention Mechanism" (delta rule with a channel-wise forget gate)."""

import os
import shutil
import subprocess

import pytest

from oracle import oracle
import tests.test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

# (name, original fragment, replacement)
MUTANTS = [
    ("decay_dropped", "const double a = exp(gt[c]);", "const double a = 1.0;"),
    ("decay_on_columns", "for (int64_t j = 0; j < V; ++j) S[c * V + j] *= a;",
     "for (int64_t j = 0; j < V; ++j) S[c * V + j] *= exp(gt[j % K]);"),
    ("decay_sign", "const double a = exp(gt[c]);", "const double a = exp(-gt[c]);"),
    ("correction_sign", "S[c * V + j] += bk * (vt[j] - w[j]);",
     "S[c * V + j] += bk * (vt[j] + w[j]);"),
    ("beta_dropped", "const double bk = bt * kt[c];", "const double bk = kt[c];"),
    ("error_from_raw_value", "S[c * V + j] += bk * (vt[j] - w[j]);",
     "S[c * V + j] += bk * vt[j];"),
    ("output_not_transposed", "ot[j] += qt[c] * S[c * V + j];",
     "ot[j] += qt[c] * S[(j % K) * V + (c % V)];"),
    ("initial_state_ignored",
     "memcpy(S, s0 + unit * K * V, (size_t)(K * V) * sizeof(double));",
     "memset(S, 0, (size_t)(K * V) * sizeof(double));"),
    ("wrong_head_stride", "const double *kt = k + (t * H + h) * K;",
     "const double *kt = k + (t * H + (H - 1 - h)) * K;"),
]

PINS = [
    lambda gd: pins.test_hand_example_two_steps(gd),
    lambda gd: pins.test_decay_only_golden(gd),
    lambda gd: pins.test_decay_only_closed_form(),
    lambda gd: pins.test_no_decay_is_textbook_delta_rule_and_retrieves_written_value(),
    lambda gd: pins.test_orthonormal_keys_retrieval(),
    lambda gd: pins.test_bruteforce_exact_rationals(),
    lambda gd: pins.test_q_equals_k_delta_invariant(),
    lambda gd: pins.test_state_passing_resume(),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"fragment for {name} not found exactly once"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / f"lib_{name}.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", str(path),
                    "-o", str(lib), "-lm"], check=True)
    return str(lib)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, golden_dir, name, old, new, monkeypatch):
    lib = oracle.load_library(_build_mutant(tmp_path, name, old, new))
    monkeypatch.setattr(oracle, "_lib", lib)
    caught = []
    for i, pin in enumerate(PINS):
        try:
            pin(golden_dir)
        except AssertionError:
            caught.append(i)
    assert caught, f"mutant {name} passed every pin"


def test_unmutated_source_passes_every_pin(golden_dir):
    for pin in PINS:
        pin(golden_dir)
