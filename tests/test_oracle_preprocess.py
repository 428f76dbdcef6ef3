"""The pre-processing oracle against its pins, and planted mistakes that the
pins must catch (each mutant is built in a temporary directory)."""
import os
import subprocess
import sys

import pytest

import oracle
from oracle import build as oracle_build
from oracle_pre_pins import ALL_PRE_PINS

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def pre_lib():
    if not os.path.exists(oracle.PRE_LIB_PATH):
        oracle_build.build()
    return oracle.PRE_LIB_PATH


@pytest.mark.parametrize("pin", ALL_PRE_PINS, ids=lambda f: f.__name__)
def test_preprocess_pin(pre_lib, pin):
    pin(pre_lib)


# Each mutant: (text to replace, replacement), applied once to gdn_preprocess.c.
MUTANTS = {
    "taps_reversed": ("w[((tau * H + h) * d + c) * 4 + j]", "w[((tau * H + h) * d + c) * 4 + (3 - j)]"),
    "window_off_by_one": ("t - 3 + j, t0", "t - 4 + j, t0"),
    "state_tap_index": ("const int64_t i = 3 - (t0 - p);", "const int64_t i = 2 - (t0 - p) + (t0 - p == 3);"),
    "normalise_v_too": ("if (tau < 2) {", "if (tau < 3) {"),
    "no_bias": ("const double bh = bias ? bias[h] : 0.0;", "const double bh = 0.0;"),
    "g_sign": ("g[t * H + h] = exp(-softplus(", "g[t * H + h] = exp(softplus(-"),
    "silu_as_sigmoid": ("buf[c] = activation ? acc * sigmoid(acc) : acc;", "buf[c] = activation ? sigmoid(acc) : acc;"),
    "state_out_unshifted": ("t1 - 3 + i, t0", "t1 - 2 + i, t0"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_preprocess_mutant_is_caught(tmp_path, name):
    src = open(oracle_build.PRE_SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    csrc = tmp_path / "mut.c"
    csrc.write_text(src.replace(old, new, 1))
    lib = str(tmp_path / "libmut.so")
    oracle_build.build(str(csrc), lib, extra=("-Wno-unused-function", "-Wno-unused-parameter"))
    script = (
        "import sys\n"
        f"sys.path[:0] = [{os.path.dirname(HERE)!r}, {HERE!r}]\n"
        "from oracle_pre_pins import ALL_PRE_PINS\n"
        "failed = 0\n"
        "for pin in ALL_PRE_PINS:\n"
        "    try:\n"
        f"        pin({lib!r})\n"
        "    except Exception:\n"
        "        failed += 1\n"
        "print(failed)\n"
    )
    out = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    assert int(out.stdout.strip().splitlines()[-1]) >= 1, f"no pin caught mutant {name}"
