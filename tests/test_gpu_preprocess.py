"""GPU parity of the pre-processing call (convolution, activation, L2 norm of
q and k, gate maps, returned conv state) against the CPU oracle, through the
C ABI.

Bar: the kernel computes in fp32 from the same inputs the oracle widens to
double, then rounds q, k, v to the run dtype (nearest even).  For bf16 the
rounding contributes at most half a unit in the last place, 2^-8 |y|, so
|got - ref| <= 2^-8 |ref| + atol; for fp32 the bound is rtol 1e-5.  atol =
2e-5 rms(ref) covers fp32 rounding on values near zero after cancellation.
g and beta: rtol 1e-5.  The returned conv state is a copy: bit-exact.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, say
from linear_attention_recurrence_gated_amd import gdn
from linear_attention_recurrence_gated_amd import workloads as w

pytestmark = pytest.mark.gpu

RTOL = {"bf16": 2.0 ** -8 + 1e-6, "fp32": 1e-5}


def to_dev(inp):
    t = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    td = lambda x: None if x is None else w.to_torch(x, inp.dtype, DEV)
    return dict(xq=td(inp.xq), xk=td(inp.xk), xv=td(inp.xv), conv_w=t(inp.w), a_logit=t(inp.a_logit),
                b_logit=t(inp.b_logit), gate_bias=t(inp.bias), conv_state_in=td(inp.state_in))


def host(x):
    x = x.cpu()
    if x.dtype == torch.bfloat16:
        x = x.float()
    return x.numpy().astype(np.float64)


def run_gpu(inp, conv_state_in="inputs", conv_state_out=None):
    d = to_dev(inp)
    if conv_state_in != "inputs":
        d["conv_state_in"] = conv_state_in
    res = gdn.preprocess(d["xq"], d["xk"], d["xv"], d["conv_w"], d["a_logit"], d["b_logit"],
                         gate_bias=d["gate_bias"], cu_seqlens=inp.cu_seqlens, conv_state_in=d["conv_state_in"],
                         conv_state_out=conv_state_out, activation=inp.activation)
    torch.cuda.synchronize()
    return res


def run_oracle(inp, state_in="inputs"):
    import oracle
    st = inp.state_in if isinstance(state_in, str) else state_in
    return oracle.preprocess(inp.xq, inp.xk, inp.xv, inp.w, inp.a_logit, inp.b_logit, bias=inp.bias,
                             cu_seqlens=inp.cu_seqlens, state_in=st, activation=inp.activation)


def close(got, ref, rtol, what):
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return
    rms = float(np.sqrt(np.mean(ref * ref)))
    bound = rtol * np.abs(ref) + 2e-5 * rms
    excess = float(np.max(np.abs(got - ref) - bound))
    worst = float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30)))
    say(f"  {what}: worst relative error {worst:.2e}, margin {-excess:.2e}")
    assert excess <= 0.0, f"{what}: error exceeds the bound by {excess}"


def compare(inp, res, ref, what=""):
    q, k, v, g, beta, st = res
    rq, rk, rv, rg, rbeta, rst = ref
    for name, a, b in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        close(host(a), b, RTOL[inp.dtype], f"{what} {name}")
    close(host(g), rg, 1e-5, f"{what} g")
    close(host(beta), rbeta, 1e-5, f"{what} beta")
    assert np.array_equal(host(st), rst), f"{what}: conv state differs"
    # the rounding of the outputs is the run dtype's own
    if inp.dtype == "bf16":
        assert q.dtype == torch.bfloat16 and v.dtype == torch.bfloat16


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("act", ["none", "silu"])
def test_packed_ragged(oracle_lib, dtype, act):
    lengths = [1, 2, 3, 5, 64, 200, 0, 37]
    say("preprocess packed", dtype, act, lengths)
    inp = w.make_preprocess(lengths, H=5, d=128, dtype=dtype, seed=1, activation=act)
    compare(inp, run_gpu(inp), run_oracle(inp), f"{dtype}/{act}")


@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_head_dims(oracle_lib, d):
    say("preprocess d =", d)
    inp = w.make_preprocess([77, 3], H=3, d=d, dtype="fp32", seed=2, activation="silu")
    compare(inp, run_gpu(inp), run_oracle(inp), f"d={d}")


def test_no_state_no_bias(oracle_lib):
    say("preprocess zero conv state, no bias")
    inp = w.make_preprocess([50], H=4, d=64, dtype="bf16", seed=3, with_state=False, with_bias=False)
    compare(inp, run_gpu(inp), run_oracle(inp), "zeros")


def test_zero_rows_stay_zero(oracle_lib):
    """A (token, head) whose convolved q is zero is passed through as zero."""
    say("preprocess zero rows")
    inp = w.make_preprocess([12], H=2, d=32, dtype="bf16", seed=4, with_state=False)
    inp.xq[:, 1, :] = 0.0
    res = run_gpu(inp)
    compare(inp, res, run_oracle(inp), "zero rows")
    assert torch.count_nonzero(res[0][:, 1, :]).item() == 0


def test_state_updated_in_place(oracle_lib):
    say("preprocess in-place conv state")
    inp = w.make_preprocess([4, 1, 0, 9], H=3, d=128, dtype="bf16", seed=5, activation="silu")
    d = to_dev(inp)
    st = d["conv_state_in"]
    res = run_gpu(inp, conv_state_in=st, conv_state_out=st)
    assert res[5].data_ptr() == st.data_ptr()
    compare(inp, res, run_oracle(inp), "in place")


@pytest.mark.parametrize("in_place", [False, True])
def test_short_sequences_across_ranges(oracle_lib, in_place):
    """No empty sequence, short ones crossing 16-token range boundaries: the
    returned conv state is written by the pre-processing kernel itself (new
    buffer) or, in place, by the separate pass."""
    lengths = [1, 2, 70, 3, 1, 40, 2]  # 119 tokens: ranges of 16 (at least 16 per sequence on average)
    say("preprocess short sequences, in place" if in_place else "preprocess short sequences")
    inp = w.make_preprocess(lengths, H=3, d=64, dtype="bf16", seed=9, activation="silu")
    d = to_dev(inp)
    st = d["conv_state_in"]
    res = run_gpu(inp, conv_state_in=st, conv_state_out=st if in_place else None)
    compare(inp, res, run_oracle(inp), "in place" if in_place else "new buffer")


def test_parts_equal_one_shot(oracle_lib):
    """Feeding each part's returned conv state to the next part gives the
    one-shot result bit for bit (the same kernel arithmetic either way)."""
    say("preprocess parts vs one shot")
    inp = w.make_preprocess([70], H=4, d=128, dtype="bf16", seed=6, activation="silu", packed=False)
    full = run_gpu(inp)
    d = to_dev(inp)
    st = d["conv_state_in"]
    outs = []
    for lo, hi in ((0, 2), (2, 33), (33, 34), (34, 70)):
        sl = lambda x: x[lo:hi].contiguous()
        r = gdn.preprocess(sl(d["xq"]), sl(d["xk"]), sl(d["xv"]), d["conv_w"], sl(d["a_logit"]), sl(d["b_logit"]),
                           gate_bias=d["gate_bias"], conv_state_in=st, activation="silu")
        outs.append(r[:5])
        st = r[5]
    torch.cuda.synchronize()
    for i in range(5):
        assert torch.equal(torch.cat([o[i] for o in outs]), full[i])
    assert torch.equal(st, full[5])


def test_decode_steps_chain_the_state(oracle_lib):
    """B one-token sequences per step, the conv state carried in place across
    steps; each step against the oracle run on the same step."""
    B, H, d = 64, 8, 128
    st_ref = None
    st_dev = None
    for step in range(4):
        say("preprocess decode step", step)
        inp = w.make_preprocess([1] * B, H=H, d=d, dtype="bf16", seed=100 + step, activation="silu")
        if step == 0:
            st_ref = inp.state_in.astype(np.float64)
            st_dev = to_dev(inp)["conv_state_in"]
        ref = run_oracle(inp, state_in=st_ref)
        res = run_gpu(inp, conv_state_in=st_dev, conv_state_out=st_dev)
        compare(inp, res, ref, f"step {step}")
        st_ref = ref[5]


def test_full_layer_size(oracle_lib):
    """The one-layer prefill shape: T = 4096, H = 48, d = 128, bf16."""
    say("preprocess full size T=4096 H=48")
    inp = w.make_preprocess([4096], H=48, d=128, dtype="bf16", seed=7, activation="silu", packed=False)
    compare(inp, run_gpu(inp), run_oracle(inp), "T=4096")


def test_feeds_the_recurrence(oracle_lib):
    """Pre-processing then chunked prefill on the GPU, against the oracle's
    pre-processing (q, k, v rounded to bf16, the dtype the GPU hands over) and
    the oracle's recurrence, to the bar for inputs that the two sides round
    separately."""
    import oracle
    from parity import assert_through_bf16_inputs, rounded_apart
    say("preprocess -> prefill")
    inp = w.make_preprocess([300, 129], H=4, d=128, dtype="bf16", seed=8, activation="silu")
    q, k, v, g, beta, _ = run_gpu(inp)
    o, s = gdn.prefill(q, k, v, g, beta, cu_seqlens=inp.cu_seqlens)
    torch.cuda.synchronize()
    rq, rk, rv, rg, rbeta, _ = run_oracle(inp)
    r16 = lambda x: w.bf16_round(x.astype(np.float32))
    q16, k16, v16 = r16(rq), r16(rk), r16(rv)
    o_ref, s_ref = oracle.run(q16, k16, v16, rg.astype(np.float32), rbeta.astype(np.float32), inp.cu_seqlens, None)
    apart = rounded_apart(((host(q), q16), (host(k), k16), (host(v), v16)))
    assert_through_bf16_inputs(host(o), o_ref, host(s), s_ref, apart, inp.cu_seqlens, "preprocess -> prefill", say)


def test_batch_without_tokens(oracle_lib):
    """Two empty sequences: no rows to compute; the returned conv state is the
    starting state, bit for bit (the oracle's as well)."""
    say("preprocess with no tokens")
    inp = w.make_preprocess([0, 0], H=4, d=64, dtype="bf16", seed=95, activation="silu")
    res = run_gpu(inp)
    ref = run_oracle(inp)
    assert res[0].shape[0] == 0 and res[3].shape[0] == 0
    assert np.array_equal(host(res[5]), ref[5]) and np.array_equal(ref[5], inp.state_in.astype(np.float64))
