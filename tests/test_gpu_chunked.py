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


def test_prefill_t4096_h48_full_size(oracle_lib):
    """B=1, H=48, T=4096, d=128, bf16, S0 = 0, chunk 64: the whole output and state."""
    say("prefill T=4096 H=48 full size")
    inp = w.prefill_t4096_h48()
    check(inp, what="T=4096 H=48")


def test_prefill_t4096_h48_slow_decay(oracle_lib):
    """Same shape with g ~ 0.98 and nonzero initial state: exercises the carry."""
    say("prefill T=4096 H=48, slow decay")
    inp = w.prefill_t4096_h48(gate_shift=-4.0)
    inp.s_init = (0.02 * np.random.default_rng(5).standard_normal((1, 48, 128, 128))).astype(np.float32)
    check(inp, what="T=4096 H=48 slow decay")


def test_many_pairs_use_the_two_workgroup_chain(oracle_lib):
    """More than 64 (sequence, head) pairs: the chain with two workgroups per
    pair (no column split), ragged lengths, nonzero initial states."""
    say("72 pairs, varlen")
    inp = w.make_prefill([300, 129, 64], H=24, d=128, seed=15, gate_shift=-1.0, init_std=0.2)
    check(inp, what="72 pairs")


def test_thousands_of_short_sequences(oracle_lib):
    """5,000 packed sequences of 0 to 9 tokens (more than the planner orders
    by length), each with its own initial state."""
    say("5000 short sequences")
    lengths = np.random.default_rng(16).integers(0, 10, size=5000).tolist()
    inp = w.make_prefill(lengths, H=2, d=128, seed=16, gate_shift=-1.0, init_std=0.2)
    check(inp, what="5000 sequences")


def test_sixty_four_heads_fill_the_column_split(oracle_lib):
    """64 (sequence, head) pairs: the largest count that still takes the
    column-split chain (four workgroups per pair, 256 in all)."""
    say("64 heads, one sequence")
    inp = w.make_prefill([700], H=64, d=128, seed=17, gate_shift=-1.0, init_std=0.2, packed=False)
    check(inp, what="H=64")


def _head_slice(inp, heads):
    """The same inputs restricted to some heads (for oracle runs on a sample)."""
    return w.PrefillInputs(np.ascontiguousarray(inp.q[:, heads]), np.ascontiguousarray(inp.k[:, heads]),
                           np.ascontiguousarray(inp.v[:, heads]), np.ascontiguousarray(inp.g[:, heads]),
                           np.ascontiguousarray(inp.beta[:, heads]), inp.cu_seqlens,
                           None if inp.s_init is None else np.ascontiguousarray(inp.s_init[:, heads]), inp.dtype)


def test_varlen_8_sequences_full_size(oracle_lib):
    """8 packed sequences, log-uniform lengths in [1024, 65536] (130,093 tokens),
    H=48, per-sequence initial states: oracle on four sampled heads, and the
    token-serial GPU path on every head."""
    say("varlen 8 sequences: generating")
    inp = w.varlen_batch()
    heads = [0, 17, 35, 47]
    say("varlen 8 sequences: chunked prefill,", len(inp.meta["lengths"]), "sequences,", inp.q.shape[0], "tokens")
    d = to_dev(inp)
    o, s = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu"], initial_state=d["s0"])
    say("varlen 8 sequences: token-serial prefill")
    o_ser, s_ser = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu"], initial_state=d["s0"],
                               chunk=gdn.CHUNK_SERIAL)
    torch.cuda.synchronize()
    rms_o = float(torch.sqrt(torch.mean(o_ser.double() ** 2)))
    rms_s = float(torch.sqrt(torch.mean(s_ser.double() ** 2)))
    e_o = float((o - o_ser).abs().max()) / rms_o
    e_s = float((s - s_ser).abs().max()) / rms_s
    say(f"varlen 8 sequences chunked vs token-serial (all heads): o={e_o:.2e} state={e_s:.2e}")
    assert e_o <= TOL_BF16 and e_s <= TOL_BF16
    o_h = o[:, heads].cpu().numpy()
    s_h = s[:, heads].cpu().numpy()
    del d, o, s, o_ser, s_ser
    say("varlen 8 sequences: oracle on heads", heads)
    o_ref, s_ref = oracle_prefill(_head_slice(inp, heads))
    eo, es = rel_max_err(o_h, o_ref), rel_max_err(s_h, s_ref)
    say(f"varlen 8 sequences vs oracle (sampled heads): o={eo:.2e} state={es:.2e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16


def test_long_context_segments_equal_one_shot(oracle_lib):
    """262,144 tokens, H=48, as 16 segments of 16,384 with the fp32 state
    carried, against one call over all tokens; the oracle (run segment by
    segment, which is exact) on two sampled heads."""
    heads = [5, 42]
    qs, ks, vs, gs, bs, host = [], [], [], [], [], []
    state = torch.zeros((1, 48, 128, 128), dtype=torch.float32, device=DEV)
    o_seg = []
    for seg in w.long_context_segments():
        i = seg.meta["segment"]
        if i % 4 == 0:
            say(f"long context: segment {i}")
        d = to_dev(seg)
        o, state = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=state, final_state=state)
        o_seg.append(o)
        qs.append(d["q"]); ks.append(d["k"]); vs.append(d["v"]); gs.append(d["g"]); bs.append(d["beta"])
        host.append(_head_slice(seg, heads))
    say("long context: one-shot call over 262,144 tokens")
    q, k, v, g, b = (torch.cat(x) for x in (qs, ks, vs, gs, bs))
    del qs, ks, vs, gs, bs
    o_one, s_one = gdn.prefill(q, k, v, g, b)
    torch.cuda.synchronize()
    o_all = torch.cat(o_seg)
    rms_o = float(torch.sqrt(torch.mean(o_one.double() ** 2)))
    e_o = float((o_all - o_one).abs().max()) / rms_o
    e_s = float((state - s_one).abs().max()) / float(torch.sqrt(torch.mean(s_one.double() ** 2)))
    say(f"long context segmented vs one-shot: o={e_o:.2e} state={e_s:.2e}")
    assert e_o <= TOL_BF16 and e_s <= TOL_BF16
    o_h = o_all[:, heads].cpu().numpy()
    s_h = state[:, heads].cpu().numpy()
    del q, k, v, g, b, o_one, o_all, o_seg
    say("long context: oracle on heads", heads, "segment by segment")
    import oracle
    s_ref = None
    err_o, sq, n = 0.0, 0.0, 0
    for i, seg in enumerate(host):
        o_ref, s_ref = oracle.run(seg.q, seg.k, seg.v, seg.g, seg.beta, None, s_ref)
        blk = o_h[i * 16384:(i + 1) * 16384]
        err_o = max(err_o, float(np.max(np.abs(blk - o_ref))))
        sq += float(np.sum(o_ref * o_ref))
        n += o_ref.size
    eo = err_o / np.sqrt(sq / n)
    es = rel_max_err(s_h, s_ref)
    say(f"long context vs oracle (sampled heads): o={eo:.2e} state={es:.2e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16


@pytest.mark.parametrize("chunk", [gdn.CHUNK_64, gdn.CHUNK_64_CHAIN, gdn.CHUNK_SERIAL])
def test_batch_without_tokens(oracle_lib, chunk):
    """Three empty sequences: no output rows, and every final state equals its
    initial state (zero-length sequences copy their state); the oracle agrees."""
    say("prefill with no tokens, chunk", chunk)
    inp = w.make_prefill([0, 0, 0], H=3, d=128, seed=13, init_std=0.2)
    o, s = gpu_prefill(inp, chunk=chunk)
    o_ref, s_ref = oracle_prefill(inp)
    assert o.shape == (0, 3, 128) and o_ref.shape[0] == 0
    assert np.array_equal(s, inp.s_init) and np.array_equal(s_ref, inp.s_init)


def test_scan_refuses_a_batch_without_tokens():
    inp = w.make_prefill([0, 0], H=2, d=128, seed=14, init_std=0.2)
    with pytest.raises(gdn.GdnError) as e:
        gpu_prefill(inp, chunk=gdn.CHUNK_64_SCAN)
    assert e.value.name == "GDN_ERR_UNSUPPORTED"


@pytest.mark.parametrize("chunk", [gdn.CHUNK_16, gdn.CHUNK_32])
def test_shorter_chunks_varlen(oracle_lib, chunk):
    """16- and 32-token chunks on a ragged batch with empty sequences and
    initial states: against the oracle, and against 64-token chunks (the
    chunk length changes nothing beyond rounding)."""
    say("chunk length", chunk, "varlen")
    inp = w.make_prefill([130, 0, 64, 1, 333, 65, 17, 15, 16, 33], H=5, d=128, seed=61, gate_shift=-1.0,
                         init_std=0.3)
    o, s = check(inp, chunk=chunk, what=f"C={chunk}")
    o64, s64 = gpu_prefill(inp, chunk=gdn.CHUNK_64)
    eo, es = rel_max_err(o, o64), rel_max_err(s, s64)
    say(f"  C={chunk} vs C=64: o={eo:.2e} state={es:.2e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16


@pytest.mark.parametrize("chunk", [gdn.CHUNK_16, gdn.CHUNK_32, gdn.CHUNK_64])
def test_chunk_lengths_full_size(oracle_lib, chunk):
    """The one-layer prefill shape (T = 4096, H = 48) with slow gates and an
    initial state, at every chunk length, against the oracle."""
    say("chunk length", chunk, "T=4096 H=48")
    inp = w.make_prefill([4096], H=48, d=128, seed=62, gate_shift=-4.0, init_std=0.3, packed=False)
    check(inp, chunk=chunk, what=f"C={chunk} T=4096")

