"""GPU parity of the variant flags (no gate: the delta rule; no erase term:
the linear-attention write; both) on every kernel family -- chunked prefill
(bf16, d = 128), token-serial prefill (fp32) and the decode step -- against the
CPU oracle run with the same flags."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, say, to_dev
from linear_attention_recurrence_gated_amd import gdn
from linear_attention_recurrence_gated_amd import workloads as w
from parity import TOL_BF16, TOL_FP32, rel_max_err

pytestmark = pytest.mark.gpu

VARIANTS = {"no_gate": gdn.GDN_VARIANT_NO_GATE, "no_erase": gdn.GDN_VARIANT_NO_ERASE,
            "linear_attention": gdn.GDN_VARIANT_NO_GATE | gdn.GDN_VARIANT_NO_ERASE}


def run_both(inp, variant, chunk, g_none, tol, what):
    d = to_dev(inp)
    g = None if g_none else d["g"]
    o, s = gdn.prefill(d["q"], d["k"], d["v"], g, d["beta"], cu_seqlens=d["cu"], initial_state=d["s0"],
                       chunk=chunk, variant=variant)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.run(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, inp.s_init, variant=variant)
    eo, es = rel_max_err(o.cpu().numpy(), o_ref), rel_max_err(s.cpu().numpy(), s_ref)
    say(f"  {what}: errors o={eo:.2e} state={es:.2e}")
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("name", sorted(VARIANTS))
def test_chunked(oracle_lib, name):
    """Packed, ragged, with initial states; for the no-erase variants beta is
    scaled down so the memory stays of order one over 300 tokens."""
    say("chunked variant", name)
    variant = VARIANTS[name]
    inp = w.make_prefill([300, 1, 129, 64], H=3, d=128, seed=71, gate_shift=-1.0, init_std=0.2)
    if variant & gdn.GDN_VARIANT_NO_ERASE:
        inp.beta[:] = inp.beta * np.float32(0.05)
    run_both(inp, variant, gdn.CHUNK_64, g_none=bool(variant & gdn.GDN_VARIANT_NO_GATE), tol=TOL_BF16,
             what=name)


@pytest.mark.parametrize("name", sorted(VARIANTS))
def test_serial_fp32(oracle_lib, name):
    say("serial variant", name)
    variant = VARIANTS[name]
    inp = w.make_prefill([70, 33], H=2, d=64, dtype="fp32", seed=72, gate_shift=0.0, init_std=0.3)
    if variant & gdn.GDN_VARIANT_NO_ERASE:
        inp.beta[:] = inp.beta * np.float32(0.1)
    run_both(inp, variant, gdn.CHUNK_SERIAL, g_none=False, tol=TOL_FP32, what=name)


def test_plain_linear_attention_closed_form(oracle_lib):
    """Both flags with beta = 1 and a zero initial state: o_t = sum_{i<=t}
    (k_i . q_t) v_i, checked on the GPU output directly (chunked path)."""
    say("plain linear attention closed form")
    inp = w.make_prefill([150], H=2, d=128, seed=73, packed=False)
    inp.beta[:] = 1.0
    d = to_dev(inp)
    o, s = gdn.prefill(d["q"], d["k"], d["v"], None, d["beta"], chunk=gdn.CHUNK_64,
                       variant=gdn.GDN_VARIANT_NO_GATE | gdn.GDN_VARIANT_NO_ERASE)
    torch.cuda.synchronize()
    q, k, v = (x.astype(np.float64) for x in (inp.q, inp.k, inp.v))
    mask = np.tril(np.ones((150, 150)))
    ref = np.einsum("ts,hts,shd->thd", mask, np.einsum("thd,shd->hts", q, k), v)
    e = rel_max_err(o.cpu().numpy(), ref)
    say(f"  error {e:.2e}")
    assert e <= TOL_BF16
    assert rel_max_err(s.cpu().numpy()[0], np.einsum("thd,the->hde", v, k)) <= TOL_BF16


@pytest.mark.parametrize("name", sorted(VARIANTS))
def test_decode(oracle_lib, name):
    say("decode variant", name)
    variant = VARIANTS[name]
    dec = w.make_decode(5, 6, 4, 128, seed=74, init_std=0.3)
    q, k, v = (w.to_torch(x, "bf16", DEV) for x in (dec.q, dec.k, dec.v))
    g = torch.from_numpy(dec.g).to(DEV)
    beta = torch.from_numpy(dec.beta).to(DEV)
    st = torch.from_numpy(dec.s_init).to(DEV)
    pool = torch.zeros((9, 4, 128, 128), dtype=torch.float32, device=DEV)
    slots = np.array([8, 0, 3, 5, 1, 6], np.int32)
    pool[torch.from_numpy(slots).long()] = st
    os_, ps_ = [], []
    for t in range(5):
        gt = None if variant & gdn.GDN_VARIANT_NO_GATE else g[t]
        os_.append(gdn.decode_step(q[t], k[t], v[t], gt, beta[t], st, variant=variant))
        ps_.append(gdn.decode_step_slots(q[t], k[t], v[t], gt, beta[t], pool, torch.from_numpy(slots).to(DEV),
                                         variant=variant))
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.run_decode(dec.q, dec.k, dec.v, dec.g, dec.beta, dec.s_init, variant=variant)
    o = torch.stack(os_).cpu().numpy()
    eo, es = rel_max_err(o, o_ref), rel_max_err(st.cpu().numpy(), s_ref)
    say(f"  {name}: errors o={eo:.2e} state={es:.2e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16
    assert torch.equal(torch.stack(ps_), torch.stack(os_))
    assert torch.equal(pool[torch.from_numpy(slots).long()], st)
