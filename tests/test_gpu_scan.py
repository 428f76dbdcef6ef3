"""GPU parity of the chunk-level scan (GDN_CHUNK_64_SCAN: each sequence cut
into segments whose affine state maps are formed in parallel and combined in
order) against the CPU oracle, next to the one-chain form on the same inputs."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, say, to_dev
from linear_attention_recurrence_gated_amd import gdn
from linear_attention_recurrence_gated_amd import workloads as w
from parity import TOL_BF16, rel_max_err

pytestmark = pytest.mark.gpu


def run(inp, chunk, variant=0, in_place=False):
    d = to_dev(inp)
    kw = {}
    if in_place and d["s0"] is not None:
        kw["final_state"] = d["s0"]
    o, s = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu"], initial_state=d["s0"],
                       chunk=chunk, variant=variant, **kw)
    torch.cuda.synchronize()
    return o.cpu().numpy(), s.cpu().numpy()


def check(inp, what, variant=0, in_place=False):
    o_ref, s_ref = oracle.run(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, inp.s_init, variant=variant)
    for name, chunk in (("scan", gdn.CHUNK_64_SCAN), ("chain", gdn.CHUNK_64_CHAIN)):
        o, s = run(inp, chunk, variant, in_place)
        eo, es = rel_max_err(o, o_ref), rel_max_err(s, s_ref)
        say(f"  {what} {name}: errors o={eo:.2e} state={es:.2e}")
        assert eo <= TOL_BF16 and es <= TOL_BF16, f"{name}: o {eo} state {es}"


@pytest.mark.parametrize("T, H", [(128, 1), (200, 2), (1000, 4), (4096, 6), (2500, 10), (777, 33)])
def test_lengths_and_heads(oracle_lib, T, H):
    say("scan T =", T, "H =", H)
    inp = w.make_prefill([T], H=H, d=128, seed=300 + T + H, gate_shift=-1.0, init_std=0.3, packed=False)
    check(inp, f"T={T} H={H}")


def test_slow_decay_carries_far(oracle_lib):
    """g close to 1: the state crosses every segment boundary nearly intact."""
    say("scan slow decay")
    inp = w.make_prefill([3000], H=4, d=128, seed=310, gate_shift=-7.0, init_std=0.5, packed=False)
    check(inp, "g~0.999")


def test_in_place_state_and_offsets(oracle_lib):
    """One sequence given with cu_seqlens, the final state written over the initial one."""
    say("scan in place with cu_seqlens")
    inp = w.make_prefill([1500], H=3, d=128, seed=311, gate_shift=-2.0, init_std=0.4, packed=True)
    check(inp, "in place", in_place=True)


@pytest.mark.parametrize("variant", [gdn.GDN_VARIANT_NO_GATE, gdn.GDN_VARIANT_NO_ERASE])
def test_variants(oracle_lib, variant):
    say("scan variant", variant)
    inp = w.make_prefill([1100], H=2, d=128, seed=312, gate_shift=-1.0, init_std=0.2, packed=False)
    if variant & gdn.GDN_VARIANT_NO_ERASE:
        inp.beta[:] = inp.beta * np.float32(0.05)
    check(inp, f"variant {variant}", variant=variant)


def test_auto_choice(oracle_lib):
    """GDN_CHUNK_64 takes the scan for one sequence with few heads (and the
    chain with many); the scan asks for more workspace."""
    small = gdn.prefill_workspace_bytes(4096, 1, 6, 128, 128, gdn.GDN_BF16, gdn.CHUNK_64)
    chain = gdn.prefill_workspace_bytes(4096, 1, 6, 128, 128, gdn.GDN_BF16, gdn.CHUNK_64_CHAIN)
    big = gdn.prefill_workspace_bytes(4096, 1, 48, 128, 128, gdn.GDN_BF16, gdn.CHUNK_64)
    big_chain = gdn.prefill_workspace_bytes(4096, 1, 48, 128, 128, gdn.GDN_BF16, gdn.CHUNK_64_CHAIN)
    assert small > chain and big == big_chain
    inp = w.make_prefill([4096], H=6, d=128, seed=313, gate_shift=2.0, packed=False)
    o_auto, s_auto = run(inp, gdn.CHUNK_64)
    o_scan, s_scan = run(inp, gdn.CHUNK_64_SCAN)
    assert np.array_equal(o_auto, o_scan) and np.array_equal(s_auto, s_scan)


@pytest.mark.parametrize("lengths, H", [
    ([700, 1500], 3),
    ([64, 3000, 0, 700, 1], 3),       # an empty sequence, a one-token one, one of a single chunk
    ([2048, 2048, 2048, 2048], 2),
    ([130] * 12, 8),                  # more sequences than the segment budget of 8: one segment each
    ([0, 900, 0], 4),
])
def test_several_sequences(oracle_lib, lengths, H):
    say("scan sequences", lengths, "H =", H)
    inp = w.make_prefill(lengths, H=H, d=128, seed=320 + H + len(lengths), gate_shift=-1.0, init_std=0.3,
                         packed=True)
    check(inp, f"{len(lengths)} sequences H={H}")


def test_many_short_sequences_in_place(oracle_lib):
    """64 sequences (the most the scan takes), some empty, updated in place."""
    rng = np.random.default_rng(330)
    lengths = [int(x) for x in rng.integers(0, 400, 64)]
    lengths[5] = lengths[40] = 0
    say("scan 64 sequences in place,", sum(lengths), "tokens")
    inp = w.make_prefill(lengths, H=1, d=128, seed=331, gate_shift=-1.5, init_std=0.2, packed=True)
    check(inp, "64 sequences", in_place=True)


def test_auto_choice_several_sequences(oracle_lib):
    """Two sequences with six heads: GDN_CHUNK_64 takes the scan (the same plan
    as when asked for); eleven sequences exceed the segment budget and take
    the chain."""
    inp = w.make_prefill([4096, 3000], H=6, d=128, seed=332, gate_shift=2.0, init_std=0.1, packed=True)
    o_auto, s_auto = run(inp, gdn.CHUNK_64)
    o_scan, s_scan = run(inp, gdn.CHUNK_64_SCAN)
    assert np.array_equal(o_auto, o_scan) and np.array_equal(s_auto, s_scan)
    inp = w.make_prefill([300] * 11, H=6, d=128, seed=333, gate_shift=2.0, init_std=0.1, packed=True)
    o_auto, s_auto = run(inp, gdn.CHUNK_64)
    o_chain, s_chain = run(inp, gdn.CHUNK_64_CHAIN)
    assert np.array_equal(o_auto, o_chain) and np.array_equal(s_auto, s_chain)


@pytest.mark.parametrize("variant", [gdn.GDN_VARIANT_NO_GATE, gdn.GDN_VARIANT_NO_ERASE,
                                     gdn.GDN_VARIANT_NO_GATE | gdn.GDN_VARIANT_NO_ERASE])
def test_several_sequences_variants(oracle_lib, variant):
    say("scan sequences, variant", variant)
    inp = w.make_prefill([900, 0, 1300, 64], H=3, d=128, seed=340 + variant, gate_shift=-1.0, init_std=0.2,
                         packed=True)
    if variant & gdn.GDN_VARIANT_NO_ERASE:
        inp.beta[:] = inp.beta * np.float32(0.05)
    check(inp, f"sequences variant {variant}", variant=variant, in_place=True)
