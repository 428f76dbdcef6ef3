"""The per-token cost of a decode step does not depend on the token's
position ("Layouts híbridos: três DeltaNet, uma attention", section Conceito:
the state is a fixed set of matrices edited in place, so a late token costs
what an early one costs).  On the batched decode shape (B = 64, H = 48,
d = 128), 256 steps with the state updated in place: the mean time of steps
1..32 and of steps 225..256 agree within 3%."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, say
from linear_attention_recurrence_gated_amd import gdn
from linear_attention_recurrence_gated_amd import workloads as w

pytestmark = pytest.mark.gpu


def test_decode_step_time_is_flat_over_256_steps():
    dec = w.decode_b64_h48()
    steps = dec.q.shape[0]
    q, k, v = (w.to_torch(x, "bf16", DEV) for x in (dec.q, dec.k, dec.v))
    g, beta = torch.from_numpy(dec.g).to(DEV), torch.from_numpy(dec.beta).to(DEV)
    s0 = torch.from_numpy(dec.s_init).to(DEV)
    state = torch.empty_like(s0)
    o = torch.empty((steps,) + tuple(q.shape[1:]), dtype=torch.float32, device=DEV)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]

    def one_pass():
        gdn.state_init(state, s0)
        ev[0].record()
        for t in range(steps):
            gdn.decode_step(q[t], k[t], v[t], g[t], beta[t], state, out=o[t])
            ev[t + 1].record()
        torch.cuda.synchronize()
        return np.array([ev[t].elapsed_time(ev[t + 1]) for t in range(steps)])

    for _ in range(3):  # clocks settle
        one_pass()
    passes = np.stack([one_pass() for _ in range(5)])
    per_step = np.median(passes, axis=0)
    early, late = float(per_step[:32].mean()), float(per_step[-32:].mean())
    say(f"decode step time: steps 1-32 {early * 1e3:.1f} us, steps 225-256 {late * 1e3:.1f} us")
    assert abs(late - early) <= 0.03 * early
