"""GPU parity of the token-at-a-time kernels (decode step, token-serial prefill)
against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, gpu_prefill, oracle_prefill, say
from linear_attention_recurrence_gated_amd import gdn
from linear_attention_recurrence_gated_amd import workloads as w
from parity import TOL_BF16, TOL_FP32, rel_max_err, tol_for

pytestmark = pytest.mark.gpu


def run_decode_gpu(dec, steps=None):
    steps = dec.q.shape[0] if steps is None else steps
    state = torch.from_numpy(dec.s_init).to(DEV)
    tq = w.to_torch(dec.q[:steps], dec.dtype, DEV)
    tk = w.to_torch(dec.k[:steps], dec.dtype, DEV)
    tv = w.to_torch(dec.v[:steps], dec.dtype, DEV)
    tg = torch.from_numpy(np.ascontiguousarray(dec.g[:steps])).to(DEV)
    tb = torch.from_numpy(np.ascontiguousarray(dec.beta[:steps])).to(DEV)
    outs = torch.empty(tv.shape, dtype=torch.float32, device=DEV)
    for t in range(steps):
        gdn.decode_step(tq[t], tk[t], tv[t], tg[t], tb[t], state, out=outs[t])
    torch.cuda.synchronize()
    return outs.cpu().numpy(), state.cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_decode_small(oracle_lib, dtype, d):
    say("decode small", dtype, d)
    dec = w.make_decode(steps=7, B=3, H=5, d=d, dtype=dtype, seed=7 + d, gate_shift=-1.0, init_std=0.3)
    o, s = run_decode_gpu(dec)
    o_ref, s_ref = oracle_lib.run_decode(dec.q, dec.k, dec.v, dec.g, dec.beta, dec.s_init)
    tol = tol_for(dtype)
    assert rel_max_err(o, o_ref) <= tol
    assert rel_max_err(s, s_ref) <= tol


def test_decode_full_size_sampled(oracle_lib):
    """B=64, H=48, d=128, 256 steps in place (the decode workload), checked on
    sampled sequences: the oracle replays those sequences' 256 tokens."""
    say("decode full size B=64 H=48 d=128 steps=256")
    dec = w.decode_b64_h48()
    o, s = run_decode_gpu(dec)
    pick = [0, 17, 63]
    o_ref, s_ref = oracle_lib.run_decode(dec.q[:, pick], dec.k[:, pick], dec.v[:, pick], dec.g[:, pick],
                                         dec.beta[:, pick], dec.s_init[pick])
    eo, es = rel_max_err(o[:, pick], o_ref), rel_max_err(s[pick], s_ref)
    say(f"decode sampled errors o={eo:.2e} state={es:.2e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16
    # the untouched sequences still moved (every state was updated in place)
    assert not np.allclose(s[5], dec.s_init[5])


def test_decode_is_deterministic():
    dec = w.make_decode(steps=3, B=4, H=6, d=128, seed=3)
    a = run_decode_gpu(dec)
    b = run_decode_gpu(dec)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_tiny_fp32_d16_serial(oracle_lib):
    say("fp32 d=16 T=64")
    inp = w.prefill_t64_d16_fp32()
    assert gdn.prefill_algorithm(gdn.GDN_FP32, 16, 16) == gdn.CHUNK_SERIAL
    o, s = gpu_prefill(inp)
    o_ref, s_ref = oracle_prefill(inp)
    assert rel_max_err(o, o_ref) <= 1e-4
    assert rel_max_err(s, s_ref) <= 1e-4


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_serial_varlen(oracle_lib, dtype, d):
    say("serial varlen", dtype, d)
    inp = w.make_prefill([37, 0, 1, 130], H=3, d=d, dtype=dtype, seed=40 + d, gate_shift=-3.0, init_std=0.5)
    o, s = gpu_prefill(inp, chunk=gdn.CHUNK_SERIAL)
    o_ref, s_ref = oracle_prefill(inp)
    tol = tol_for(dtype)
    assert rel_max_err(o, o_ref) <= tol
    assert rel_max_err(s, s_ref) <= tol
    assert np.array_equal(s[1], inp.s_init[1])  # zero-length sequence keeps its state


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_serial_lookahead_edges(oracle_lib, dtype):
    """The token-serial kernel keeps the inputs of the next 8 tokens in flight
    (its loop unrolled by 8): sequences of 1 to 17 tokens, on both sides of
    each multiple of 8, packed in one batch at d = 128 (8-row tiles)."""
    say("serial lookahead edges", dtype)
    inp = w.make_prefill([7, 8, 9, 1, 15, 16, 17, 2], H=2, d=128, dtype=dtype, seed=71, gate_shift=-2.0,
                         init_std=0.3)
    o, s = gpu_prefill(inp, chunk=gdn.CHUNK_SERIAL)
    o_ref, s_ref = oracle_prefill(inp)
    tol = tol_for(dtype)
    assert rel_max_err(o, o_ref) <= tol
    assert rel_max_err(s, s_ref) <= tol


def test_serial_in_place_state(oracle_lib):
    inp = w.make_prefill([50, 20], H=2, d=64, dtype="fp32", seed=5, init_std=0.2)
    d = {k: v for k, v in zip(["q", "k", "v"], [w.to_torch(x, "fp32", DEV) for x in (inp.q, inp.k, inp.v)])}
    st = torch.from_numpy(inp.s_init).to(DEV)
    o, s = gdn.prefill(d["q"], d["k"], d["v"], torch.from_numpy(inp.g).to(DEV), torch.from_numpy(inp.beta).to(DEV),
                       cu_seqlens=inp.cu_seqlens, initial_state=st, final_state=st, chunk=gdn.CHUNK_SERIAL)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_prefill(inp)
    assert rel_max_err(st.cpu().numpy(), s_ref) <= 1e-4
    assert rel_max_err(o.cpu().numpy(), o_ref) <= 1e-4


def test_decode_equals_serial_prefill():
    """T decode steps on one sequence equal a T-token prefill of it."""
    inp = w.make_prefill([40], H=4, d=128, dtype="bf16", seed=9, init_std=0.1, packed=False)
    o_p, s_p = gpu_prefill(inp, chunk=gdn.CHUNK_SERIAL)
    dec = w.DecodeInputs(inp.q[:, None], inp.k[:, None], inp.v[:, None], inp.g[:, None], inp.beta[:, None],
                         inp.s_init, "bf16")
    o_d, s_d = run_decode_gpu(dec)
    assert rel_max_err(o_d[:, 0], o_p) <= 1e-5
    assert rel_max_err(s_d, s_p) <= 1e-5


def test_state_init_and_reset():
    n, H, d = 5, 3, 32
    init = torch.randn(n, H, d, d, device=DEV)
    st = torch.full((n, H, d, d), 7.0, device=DEV)
    gdn.state_init(st, init)
    torch.cuda.synchronize()
    assert torch.equal(st, init)
    gdn.state_reset(st, torch.tensor([3, -1, 99, 0], dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    ref = init.clone()
    ref[3] = 0
    ref[0] = 0
    assert torch.equal(st, ref)
    gdn.state_init(st)
    torch.cuda.synchronize()
    assert torch.count_nonzero(st).item() == 0


def test_fp32_prefill_d128_long(oracle_lib):
    """fp32 q/k/v at d = 128 over 4096 tokens (the token-serial kernel), slow
    decay and a nonzero initial state, against the oracle at the fp32 bar."""
    say("fp32 prefill d=128 T=4096 H=4")
    inp = w.make_prefill([4096], H=4, d=128, dtype="fp32", seed=61, gate_shift=-3.0, init_std=0.1, packed=False)
    assert gdn.prefill_algorithm(gdn.GDN_FP32, 128, 128) == gdn.CHUNK_SERIAL
    o, s = gpu_prefill(inp)
    o_ref, s_ref = oracle_prefill(inp)
    eo, es = rel_max_err(o, o_ref), rel_max_err(s, s_ref)
    say(f"fp32 d=128 T=4096 errors o={eo:.2e} state={es:.2e}")
    assert eo <= TOL_FP32 and es <= TOL_FP32
