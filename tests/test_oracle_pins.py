"""The CPU oracle against its pins (closed forms, special cases, expansion, invariants)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(oracle_lib, pin):
    pin(oracle_lib.run)


def test_run_decode_equals_separate_runs(oracle_lib):
    """oracle.run_decode (steps x B single-token steps, packed into one batch of
    B sequences) equals B separate oracle.run calls over each sequence's
    tokens in step order, bit for bit; also for the variants."""
    import numpy as np
    rng = np.random.default_rng(31)
    steps, B, H, d = 7, 3, 2, 8
    q, k, v = (rng.standard_normal((steps, B, H, d)) for _ in range(3))
    g = rng.uniform(0.3, 1.0, (steps, B, H))
    beta = rng.uniform(0.0, 1.0, (steps, B, H))
    s0 = rng.standard_normal((B, H, d, d))
    for variant in (0, oracle_lib.NO_GATE, oracle_lib.NO_ERASE):
        o, s = oracle_lib.run_decode(q, k, v, g, beta, s0, variant=variant)
        assert o.shape == (steps, B, H, d) and s.shape == (B, H, d, d)
        for b in range(B):
            ob, sb = oracle_lib.run(q[:, b], k[:, b], v[:, b], g[:, b], beta[:, b], None, s0[b:b + 1],
                                    variant=variant)
            assert np.array_equal(o[:, b], ob) and np.array_equal(s[b], sb[0])
    # one step is one token: the state after step t feeds step t + 1
    o1, s1 = oracle_lib.run_decode(q[:1], k[:1], v[:1], g[:1], beta[:1], s0)
    o2, s2 = oracle_lib.run_decode(q[1:], k[1:], v[1:], g[1:], beta[1:], s1)
    o_all, s_all = oracle_lib.run_decode(q, k, v, g, beta, s0)
    assert np.array_equal(np.concatenate([o1, o2]), o_all) and np.array_equal(s2, s_all)
