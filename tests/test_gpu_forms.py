"""Seeded random batches through GDN_CHUNK_64, whichever form the library picks
for each (the column-split chain, the two-workgroup chain or the chunk-level
scan), against the token-serial GPU path on every head and the CPU oracle on
two sampled heads.  The batch shapes straddle the choice's thresholds: few or
many heads, one long sequence among short ones, empty sequences."""
import numpy as np
import pytest
import torch

from gpu_helpers import say, to_dev
import oracle
from linear_attention_recurrence_gated_amd import gdn
from linear_attention_recurrence_gated_amd import workloads as w
from parity import TOL_BF16, rel_max_err

pytestmark = pytest.mark.gpu

CASES = 12


def _batch(i):
    rng = np.random.default_rng(5000 + i)
    n = int(rng.integers(1, 13))
    H = (1, 6, 33, 48, 2, 12, 20, 48, 3, 6, 48, 12)[i]
    lengths = [int(x) for x in rng.integers(0, 900, n)]
    if rng.random() < 0.5:
        lengths[int(rng.integers(0, n))] = int(rng.integers(1500, 4000))
    if sum(lengths) == 0:
        lengths[0] = 65
    return lengths, H


@pytest.mark.parametrize("i", range(CASES))
def test_random_batch(oracle_lib, i):
    lengths, H = _batch(i)
    say(f"random batch {i}: H={H} lengths={lengths}")
    inp = w.make_prefill(lengths, H=H, d=128, seed=5100 + i, gate_shift=-1.0, init_std=0.2, packed=True)
    d = to_dev(inp)
    o, s = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu"], initial_state=d["s0"],
                       chunk=gdn.CHUNK_64)
    o_ser, s_ser = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu"],
                               initial_state=d["s0"], chunk=gdn.CHUNK_SERIAL)
    torch.cuda.synchronize()
    eo = rel_max_err(o.cpu().numpy(), o_ser.cpu().numpy())
    es = rel_max_err(s.cpu().numpy(), s_ser.cpu().numpy())
    say(f"  chunked vs token-serial (all heads): o={eo:.2e} state={es:.2e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16
    heads = sorted({0, H - 1})
    sl = lambda x: None if x is None else np.ascontiguousarray(x[:, heads])
    o_ref, s_ref = oracle.run(sl(inp.q), sl(inp.k), sl(inp.v), sl(inp.g), sl(inp.beta), inp.cu_seqlens,
                              sl(inp.s_init))
    eo = rel_max_err(o.cpu().numpy()[:, heads], o_ref)
    es = rel_max_err(s.cpu().numpy()[:, heads], s_ref)
    say(f"  chunked vs oracle (heads {heads}): o={eo:.2e} state={es:.2e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16
