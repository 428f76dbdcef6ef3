"""The pins are strong enough: each plausible mistake planted in a copy of the
oracle (on the CPU, in a temporary build) makes at least one pin fail.

Each mutant is the oracle's source with one textual edit.  The pins run in a
child process so that a mutant that reads out of bounds cannot take the test
runner down with it.
"""
import os
import subprocess
import sys

import pytest

from oracle import build as oracle_build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

MUTANTS = {
    # gate applied before the recall (recall from g * S_{t-1})
    "gate_before_recall": ("r[i] = acc;", "r[i] = gt * acc;"),
    # write strength dropped
    "no_beta": ("const double c = bt * (vt[i] - r[i]);", "const double c = (vt[i] - r[i]);"),
    # wrong sign of the correction
    "plus_recall": ("const double c = bt * (vt[i] - r[i]);", "const double c = bt * (vt[i] + r[i]);"),
    # gate never applied
    "no_gate": ("S[i * dk + j] = gt * S[i * dk + j] + c * kt[j];", "S[i * dk + j] = S[i * dk + j] + c * kt[j];"),
    # recall through the transposed state
    "transposed_recall": ("for (int64_t j = 0; j < dk; ++j) acc += S[i * dk + j] * kt[j];",
                          "for (int64_t j = 0; j < dk; ++j) acc += S[(j % dv) * dk + (i % dk)] * kt[j];"),
    # read-out with the key instead of the query
    "readout_with_key": ("acc += S[i * dk + j] * qt[j];", "acc += S[i * dk + j] * kt[j];"),
    # recall with the query instead of the key
    "recall_with_query": ("for (int64_t j = 0; j < dk; ++j) acc += S[i * dk + j] * kt[j];",
                          "for (int64_t j = 0; j < dk; ++j) acc += S[i * dk + j] * qt[j];"),
    # outer product written along the query
    "write_along_query": ("+ c * kt[j];", "+ c * qt[j];"),
    # every sequence starts reading at token 0
    "bad_sequence_start": ("const int64_t t0 = J->cu ? J->cu[s] : 0;", "const int64_t t0 = 0;"),
    # last token of each sequence dropped
    "drop_last_token": ("for (int64_t t = t0; t < t1; ++t) {", "for (int64_t t = t0; t + 1 < t1; ++t) {"),
    # initial state ignored
    "ignore_initial_state": ("if (J->s_init) {", "if (0) {"),
    # state not reset between sequences of one head (carried from the previous one)
    "no_reset": ("memset(S, 0, (size_t)(dv * dk) * sizeof(double));",
                 "if (s > 0) memcpy(S, J->s_final + ((s - 1) * H + h) * dv * dk, (size_t)(dv * dk) * sizeof(double)); else memset(S, 0, (size_t)(dv * dk) * sizeof(double));"),
    # variants: the no-erase flag ignored (recall still subtracted)
    "variant_erase_kept": ("if (!(J->variant & 2))", "if (1)"),
    # variants: the no-gate flag ignored (g still applied)
    "variant_gate_kept": ("(J->variant & 1) ? 1.0 : J->g[t * H + h]", "J->g[t * H + h]"),
    # variants: the two flags swapped
    "variant_flags_swapped": ("if (!(J->variant & 2))", "if (!(J->variant & 1))"),
}

RUNNER = r"""
import sys, functools
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle, oracle_pins
run = functools.partial(oracle.run, lib_path={lib!r}, threads=1)
failed = []
for pin in oracle_pins.ALL_PINS:
    try:
        pin(run)
    except Exception as e:
        failed.append(pin.__name__)
print("FAILED:" + ",".join(failed))
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    src = open(os.path.join(ROOT, "oracle", "gdn_oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new, 1)
    csrc = tmp_path / "mutant.c"
    csrc.write_text(mutated)
    lib = str(tmp_path / "libmutant.so")
    oracle_build.build(str(csrc), lib)
    code = RUNNER.format(root=ROOT, tests=HERE, lib=lib)
    proc = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    if proc.returncode != 0:
        return  # the mutant crashed: caught
    line = [l for l in proc.stdout.splitlines() if l.startswith("FAILED:")][-1]
    failed = [x for x in line[len("FAILED:"):].split(",") if x]
    assert failed, f"mutant {name} passed every pin"
