"""GPU parity of the fused layer call (gdn_layer_prefill: convolution,
activation, L2 norm of q and k, gate maps and the chunked prefill in one
call), through the C ABI.

Two bars.  Against the two separate calls (gdn_preprocess, then gdn_prefill
with the same chunk form) everything is bit-exact: the fused chunk
preparation forms each processed row with the pre-processing kernel's own
per-row arithmetic and the state chain is the same.  Against the oracle
(its pre-processing, q, k, v rounded to bf16 as the GPU hands them over, its
recurrence) the bf16 bar of the prefill holds, on sampled heads at the full
one-layer size.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, say
from linear_attention_recurrence_gated_amd import gdn
from linear_attention_recurrence_gated_amd import workloads as w
from parity import TOL_BF16, rel_max_err

pytestmark = pytest.mark.gpu


def dev_inputs(inp):
    t = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    td = lambda x: None if x is None else w.to_torch(x, inp.dtype, DEV)
    return dict(xq=td(inp.xq), xk=td(inp.xk), xv=td(inp.xv), conv_w=t(inp.w), a_logit=t(inp.a_logit),
                b_logit=t(inp.b_logit), gate_bias=t(inp.bias), conv_state_in=td(inp.state_in))


def initial_states(inp, H, seed, std=0.3):
    rng = np.random.default_rng(seed)
    return (std * rng.standard_normal((inp.n_seq, H, 128, 128))).astype(np.float32)


def two_calls(d, inp, s0, chunk, variant=gdn.GDN_VARIANT_GATED_DELTA):
    a = None if variant & gdn.GDN_VARIANT_NO_GATE else d["a_logit"]
    q, k, v, g, beta, st = gdn.preprocess(d["xq"], d["xk"], d["xv"], d["conv_w"], d["a_logit"], d["b_logit"],
                                          gate_bias=d["gate_bias"], cu_seqlens=inp.cu_seqlens,
                                          conv_state_in=d["conv_state_in"], activation=inp.activation)
    o, s = gdn.prefill(q, k, v, None if a is None else g, beta, cu_seqlens=inp.cu_seqlens,
                       initial_state=None if s0 is None else s0.clone(), chunk=chunk, variant=variant)
    torch.cuda.synchronize()
    return dict(o=o, s=s, st=st, q=q, k=k, v=v, g=g, beta=beta)


def fused(d, inp, s0, chunk, variant=gdn.GDN_VARIANT_GATED_DELTA, gates=True, in_place=False):
    N, H, _ = d["xk"].shape
    a = None if variant & gdn.GDN_VARIANT_NO_GATE else d["a_logit"]
    gb = (torch.full((N, H), float("nan"), device=DEV), torch.full((N, H), float("nan"), device=DEV)) if gates else None
    st_in = d["conv_state_in"]
    if in_place:
        st_in = None if st_in is None else st_in.clone()
        s0 = None if s0 is None else s0.clone()
    o, s, st, q, k, v = gdn.layer_prefill(d["xq"], d["xk"], d["xv"], d["conv_w"], a, d["b_logit"],
                                          gate_bias=d["gate_bias"], cu_seqlens=inp.cu_seqlens,
                                          conv_state_in=st_in, conv_state_out=st_in if in_place else None,
                                          activation=inp.activation, initial_state=s0,
                                          final_state=s0 if in_place else None, chunk=chunk, gates=gb,
                                          variant=variant)
    torch.cuda.synchronize()
    if in_place:
        assert (st_in is None or st.data_ptr() == st_in.data_ptr()) and (s0 is None or s.data_ptr() == s0.data_ptr())
    r = dict(o=o, s=s, st=st, q=q, k=k, v=v)
    if gates:
        r["g"], r["beta"] = gb
    return r


def assert_same(got, ref, keys, what):
    for key in keys:
        if key not in got:
            continue
        a, b = got[key], ref[key]
        assert a.shape == b.shape, (what, key, a.shape, b.shape)
        assert torch.equal(a, b), f"{what}: {key} differs ({(a.float() - b.float()).abs().max().item():.3e})"
    say(f"  {what}: {', '.join(k for k in keys if k in got)} bit-exact")


CASES = {
    # name: (lengths, H, activation, conv state, bias, initial states, seed)
    "ragged_packed": ([300, 129, 0, 1, 64, 65, 7], 4, "silu", True, True, True, 11),
    "single_no_state": ([200], 3, "none", False, False, False, 12),
    "short_sequences": ([1, 2, 3, 5, 70, 1, 40, 2], 2, "silu", True, True, False, 13),
    "exact_chunks": ([64, 128, 192], 5, "none", True, True, True, 14),
}


@pytest.mark.parametrize("name", list(CASES))
def test_layer_equals_preprocess_then_prefill(name):
    lengths, H, act, with_state, with_bias, with_s0, seed = CASES[name]
    say("layer vs two calls:", name, lengths, f"H={H}")
    inp = w.make_preprocess(lengths, H=H, d=128, dtype="bf16", seed=seed, with_state=with_state,
                            with_bias=with_bias, activation=act)
    d = dev_inputs(inp)
    s0 = torch.from_numpy(initial_states(inp, H, 5)).to(DEV) if with_s0 else None
    ref = two_calls(d, inp, s0, gdn.CHUNK_64)
    got = fused(d, inp, s0, gdn.CHUNK_64)
    assert_same(got, ref, ("o", "s", "st", "q", "k", "v", "g", "beta"), name)


@pytest.mark.parametrize("lengths", [[130, 0, 64, 1, 333], [1, 2, 3, 64, 17, 2]])
def test_layer_in_place_states_and_no_gate_outputs(lengths):
    """conv_state_out == conv_state_in and final_state == initial_state; g and
    beta not requested.  With an empty or a multi-chunk sequence the returned
    conv state is written after the chunk preparation (k_conv_state); with
    single-chunk sequences only, by the chunk preparation itself."""
    say("layer in place", lengths)
    inp = w.make_preprocess(lengths, H=3, d=128, dtype="bf16", seed=21, activation="silu")
    d = dev_inputs(inp)
    s0 = torch.from_numpy(initial_states(inp, 3, 6)).to(DEV)
    ref = two_calls(d, inp, s0, gdn.CHUNK_64)
    got = fused(d, inp, s0, gdn.CHUNK_64, gates=False, in_place=True)
    assert_same(got, ref, ("o", "s", "st", "q", "k", "v"), "in place")


@pytest.mark.parametrize("chunk", [gdn.CHUNK_64_CHAIN, gdn.CHUNK_64_SCAN, gdn.CHUNK_32, gdn.CHUNK_16])
def test_layer_chunk_forms(chunk):
    """The per-pair chain, the chunk-level scan (segments) and the shorter
    chunks behind the fused preparation."""
    say("layer chunk form", chunk)
    inp = w.make_preprocess([900, 77], H=2, d=128, dtype="bf16", seed=22, activation="silu")
    d = dev_inputs(inp)
    s0 = torch.from_numpy(initial_states(inp, 2, 7)).to(DEV)
    ref = two_calls(d, inp, s0, chunk)
    got = fused(d, inp, s0, chunk)
    assert_same(got, ref, ("o", "s", "st", "q", "k", "v", "g", "beta"), f"chunk={chunk}")


@pytest.mark.parametrize("variant", [gdn.GDN_VARIANT_NO_GATE, gdn.GDN_VARIANT_NO_ERASE])
def test_layer_variants(variant):
    say("layer variant", variant)
    inp = w.make_preprocess([150, 40], H=2, d=128, dtype="bf16", seed=23, activation="none")
    d = dev_inputs(inp)
    ref = two_calls(d, inp, None, gdn.CHUNK_64, variant=variant)
    got = fused(d, inp, None, gdn.CHUNK_64, variant=variant)
    keys = ("o", "s", "st", "q", "k", "v", "beta") + (() if variant & gdn.GDN_VARIANT_NO_GATE else ("g",))
    assert_same(got, ref, keys, f"variant={variant}")


def test_layer_batch_without_tokens():
    """Sequences with no tokens: the final states are the initial states and
    the conv state is returned unchanged."""
    say("layer with no tokens")
    inp = w.make_preprocess([0, 0], H=4, d=128, dtype="bf16", seed=24, activation="silu")
    d = dev_inputs(inp)
    s0 = torch.from_numpy(initial_states(inp, 4, 8)).to(DEV)
    got = fused(d, inp, s0, gdn.CHUNK_64, gates=False)
    assert got["o"].shape[0] == 0
    assert torch.equal(got["s"], s0) and torch.equal(got["st"], d["conv_state_in"])


def test_layer_full_size_against_oracle(oracle_lib):
    """The one-layer prefill shape: T = 4096, H = 48, d = 128, bf16, SiLU, with
    starting conv states: bit-exact against the two calls; against the
    oracle's pre-processing of every head and its recurrence on four sampled
    heads, to the bar for inputs that the two sides round to bf16 separately
    (parity.assert_through_bf16_inputs)."""
    import oracle
    from parity import assert_through_bf16_inputs, rounded_apart
    heads = [0, 13, 30, 47]
    say("layer full size T=4096 H=48 against the two calls and the oracle, heads", heads)
    inp = w.make_preprocess([4096], H=48, d=128, dtype="bf16", seed=25, activation="silu", packed=False)
    d = dev_inputs(inp)
    got = fused(d, inp, None, gdn.CHUNK_AUTO)
    assert_same(got, two_calls(d, inp, None, gdn.CHUNK_AUTO), ("o", "s", "st", "q", "k", "v", "g", "beta"), "T=4096")
    rq, rk, rv, rg, rbeta, rst = oracle.preprocess(inp.xq, inp.xk, inp.xv, inp.w, inp.a_logit, inp.b_logit,
                                                   bias=inp.bias, cu_seqlens=None, state_in=inp.state_in,
                                                   activation="silu")
    assert np.array_equal(got["st"].float().cpu().numpy().astype(np.float64), rst), "conv state differs"
    r16 = lambda x: w.bf16_round(np.ascontiguousarray(x[:, heads]).astype(np.float32))
    q16, k16, v16 = r16(rq), r16(rk), r16(rv)
    o_ref, s_ref = oracle.run(q16, k16, v16, np.ascontiguousarray(rg[:, heads]).astype(np.float32),
                              np.ascontiguousarray(rbeta[:, heads]).astype(np.float32), None, None)
    hd = lambda x: x[:, heads].float().cpu().numpy()
    apart = rounded_apart(((hd(got["q"]), q16), (hd(got["k"]), k16), (hd(got["v"]), v16)))
    assert_through_bf16_inputs(got["o"][:, heads].cpu().numpy(), o_ref, got["s"][:, heads].cpu().numpy(), s_ref,
                               apart, None, "layer T=4096", say)
