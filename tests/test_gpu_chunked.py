"""GPU parity of the chunkwise-parallel MFMA prefill (bf16 q/k/v, d = 128)
against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, gpu_prefill, oracle_prefill, say, to_dev
from linear_attention_recurrence_gated_amd import gdn
from linear_attention_recurrence_gated_amd import workloads as w
from parity import TOL_BF16, rel_max_err

pytestmark = pytest.mark.gpu


def check(inp, tol=TOL_BF16, chunk=gdn.CHUNK_64, what=""):
    o, s = gpu_prefill(inp, chunk=chunk)
    o_ref, s_ref = oracle_prefill(inp)
    eo, es = rel_max_err(o, o_ref), rel_max_err(s, s_ref)
    say(f"{what} errors o={eo:.2e} state={es:.2e}")
    assert eo <= tol, f"output error {eo}"
    assert es <= tol, f"state error {es}"
    return o, s


def test_algorithm_is_chunked():
    assert gdn.prefill_algorithm(gdn.GDN_BF16, 128, 128) == gdn.CHUNK_64


@pytest.mark.parametrize("T", [1, 17, 63, 64, 65, 128, 200, 517])
def test_single_sequence_lengths(oracle_lib, T):
    say("chunked single sequence T =", T)
    inp = w.make_prefill([T], H=3, d=128, seed=100 + T, gate_shift=-1.0, init_std=0.3, packed=False)
    check(inp, what=f"T={T}")


@pytest.mark.parametrize("name, shift", [("strong_decay", 2.0), ("mild_decay", -4.0), ("very_slow", -7.0)])
def test_gate_regimes(oracle_lib, name, shift):
    say("chunked gate regime", name)
    inp = w.make_prefill([700], H=4, d=128, seed=7, gate_shift=shift, init_std=0.5, packed=False)
    check(inp, what=name)


def test_no_write_pure_decay(oracle_lib):
    """beta = 0 with g close to 1: only the carried state decays."""
    inp = w.make_prefill([300], H=2, d=128, seed=8, gate_shift=-7.0, init_std=1.0, packed=False)
    inp.beta[:] = 0.0
    check(inp, what="beta=0")


def test_unit_gate_unit_strength(oracle_lib):
    """g = beta = 1: each write replaces the value stored under its key."""
    inp = w.make_prefill([260], H=2, d=128, seed=9, init_std=0.2, packed=False)
    inp.g[:] = 1.0
    inp.beta[:] = 1.0
    check(inp, what="g=beta=1")


def test_varlen_with_empty_sequences(oracle_lib):
    say("chunked varlen")
    inp = w.make_prefill([130, 0, 64, 1, 0, 333, 65], H=5, d=128, seed=11, gate_shift=0.0, init_std=0.1)
    o, s = check(inp, what="varlen")
    assert np.array_equal(s[1], inp.s_init[1]) and np.array_equal(s[4], inp.s_init[4])


def test_chunked_matches_serial_on_gpu():
    inp = w.make_prefill([450, 77], H=4, d=128, seed=12, gate_shift=-2.0, init_std=0.2)
    o1, s1 = gpu_prefill(inp, chunk=gdn.CHUNK_64)
    o2, s2 = gpu_prefill(inp, chunk=gdn.CHUNK_SERIAL)
    assert rel_max_err(o1, o2) <= TOL_BF16 and rel_max_err(s1, s2) <= TOL_BF16


def test_segmented_equals_one_shot():
    """Running a sequence in segments with the state carried equals one shot."""
    say("chunked segmented vs one-shot")
    inp = w.make_prefill([1000], H=3, d=128, seed=13, gate_shift=-3.0, init_std=0.2, packed=False)
    o_full, s_full = gpu_prefill(inp)
    d = to_dev(inp)
    state = d["s0"].clone()
    outs = []
    for a, b in [(0, 100), (100, 164), (164, 165), (165, 1000)]:
        o, _ = gdn.prefill(d["q"][a:b], d["k"][a:b], d["v"][a:b], d["g"][a:b], d["beta"][a:b],
                           initial_state=state, final_state=state, chunk=gdn.CHUNK_64)
        outs.append(o)
    torch.cuda.synchronize()
    o_seg = torch.cat(outs).cpu().numpy()
    assert rel_max_err(o_seg, o_full) <= 1e-3
    assert rel_max_err(state.cpu().numpy(), s_full) <= 1e-3


def test_in_place_and_deterministic():
    inp = w.make_prefill([300, 90], H=3, d=128, seed=14, init_std=0.3)
    d = to_dev(inp)
    runs = []
    for _ in range(2):
        st = d["s0"].clone()
        o, _ = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu"], initial_state=st,
                           final_state=st)
        torch.cuda.synchronize()
        runs.append((o.cpu().numpy(), st.cpu().numpy()))
    assert np.array_equal(runs[0][0], runs[1][0]) and np.array_equal(runs[0][1], runs[1][1])
    o2, s2 = gpu_prefill(inp)
    assert np.array_equal(o2, runs[0][0]) and np.array_equal(s2, runs[0][1])


def test_config2_full_size(oracle_lib):
    """B=1, H=48, T=4096, d=128, bf16, S0 = 0, chunk 64: the whole output and state."""
    say("config2 full size")
    inp = w.config2()
    check(inp, what="config2")


def test_config2_shape_slow_decay(oracle_lib):
    """Same shape with g ~ 0.98 and nonzero initial state: exercises the carry."""
    say("config2 shape, slow decay")
    inp = w.config2(gate_shift=-4.0)
    inp.s_init = (0.02 * np.random.default_rng(5).standard_normal((1, 48, 128, 128))).astype(np.float32)
    check(inp, what="config2 slow decay")
