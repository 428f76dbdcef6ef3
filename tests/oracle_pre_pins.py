"""Pins of the pre-processing oracle (oracle/gdn_preprocess.c).

Each pin checks the oracle against something other than itself: a library
routine (numpy's convolve and norm, scipy's expit), a closed form, or an
invariant.  Every pin takes the library path so that mutated builds can be
checked too.
"""
import numpy as np
from scipy.special import expit

import oracle


def _inputs(rng, N, H, d, scale=1.0):
    xq, xk, xv = (scale * rng.standard_normal((N, H, d)) for _ in range(3))
    w = rng.standard_normal((3, H, d, 4))
    a, b = rng.standard_normal((N, H)), rng.standard_normal((N, H))
    return xq, xk, xv, w, a, b


def pin_identity_taps_normalise_q_k(lib):
    """Taps (0, 0, 0, 1): v passes through, q and k are x / ||x|| per (token, head)."""
    rng = np.random.default_rng(1)
    xq, xk, xv, w, a, b = _inputs(rng, 9, 2, 5)
    w[:] = 0.0
    w[..., 3] = 1.0
    q, k, v, _, _, _ = oracle.preprocess(xq, xk, xv, w, a, b, lib_path=lib)
    assert np.array_equal(v, xv)
    for y, x in ((q, xq), (k, xk)):
        ref = x / np.linalg.norm(x, axis=-1, keepdims=True)
        assert np.max(np.abs(y - ref)) < 1e-15


def pin_convolution_matches_numpy(lib):
    """One sequence, zero conv state: each channel of v is numpy's full
    convolution with the taps reversed, truncated to the sequence (causal)."""
    rng = np.random.default_rng(2)
    xq, xk, xv, w, a, b = _inputs(rng, 23, 2, 3)
    _, _, v, _, _, _ = oracle.preprocess(xq, xk, xv, w, a, b, lib_path=lib)
    for h in range(2):
        for c in range(3):
            # y[t] = sum_j w[j] x[t - 3 + j]  ==  (x * w[::-1])[t]
            ref = np.convolve(xv[:, h, c], w[2, h, c, ::-1])[:23]
            assert np.max(np.abs(v[:, h, c] - ref)) < 1e-13


def pin_impulse_response(lib):
    """A unit impulse at token 5 of one channel of v gives the taps, newest
    first, on tokens 5..8 and zero elsewhere."""
    rng = np.random.default_rng(3)
    xq, xk, _, w, a, b = _inputs(rng, 12, 1, 4)
    xv = np.zeros((12, 1, 4))
    xv[5, 0, 2] = 1.0
    _, _, v, _, _, _ = oracle.preprocess(xq, xk, xv, w, a, b, lib_path=lib)
    expect = np.zeros(12)
    for m in range(4):
        expect[5 + m] = w[2, 0, 2, 3 - m]
    assert np.array_equal(v[:, 0, 2], expect)
    assert np.all(v[:, 0, [0, 1, 3]] == 0.0)


def pin_gates_closed_form(lib):
    """beta = expit(b) and g = exp(-softplus(a + bias)) = expit(-(a + bias))."""
    rng = np.random.default_rng(4)
    xq, xk, xv, w, a, b = _inputs(rng, 7, 3, 2)
    a *= 6.0
    bias = np.array([2.0, -1.0, 0.5])
    _, _, _, g, beta, _ = oracle.preprocess(xq, xk, xv, w, a, b, bias=bias, lib_path=lib)
    assert np.max(np.abs(beta - expit(b))) < 1e-15
    assert np.max(np.abs(g - expit(-(a + bias)))) < 1e-15


def pin_silu(lib):
    """Identity taps with SiLU: v = x * expit(x)."""
    rng = np.random.default_rng(5)
    xq, xk, xv, w, a, b = _inputs(rng, 6, 2, 3, scale=3.0)
    w[:] = 0.0
    w[..., 3] = 1.0
    _, _, v, _, _, _ = oracle.preprocess(xq, xk, xv, w, a, b, activation="silu", lib_path=lib)
    assert np.max(np.abs(v - xv * expit(xv))) < 1e-14


def pin_normalisation_is_scale_invariant(lib):
    """No activation: scaling the raw q and k by c > 0 leaves the outputs
    unchanged (up to rounding); a zero row stays zero."""
    rng = np.random.default_rng(6)
    xq, xk, xv, w, a, b = _inputs(rng, 10, 2, 6)
    q1, k1, _, _, _, _ = oracle.preprocess(xq, xk, xv, w, a, b, lib_path=lib)
    q2, k2, _, _, _, _ = oracle.preprocess(7.5 * xq, 0.01 * xk, xv, w, a, b, lib_path=lib)
    assert np.max(np.abs(q1 - q2)) < 1e-13 and np.max(np.abs(k1 - k2)) < 1e-13
    assert np.allclose(np.linalg.norm(q1, axis=-1), 1.0, atol=1e-14)
    z = np.zeros_like(xq)
    q0, _, _, _, _, _ = oracle.preprocess(z, xk, xv, w, a, b, lib_path=lib)
    assert np.all(q0 == 0.0)


def pin_parts_equal_one_shot(lib):
    """A sequence processed in three parts, each part's returned conv state
    fed to the next, equals one call over the whole sequence, bit for bit;
    the final states agree too.  Includes a part shorter than three tokens."""
    rng = np.random.default_rng(7)
    N, H, d = 17, 2, 3
    xq, xk, xv, w, a, b = _inputs(rng, N, H, d)
    st0 = rng.standard_normal((1, 3, 3, H, d))
    full = oracle.preprocess(xq, xk, xv, w, a, b, state_in=st0, activation="silu", lib_path=lib)
    st = st0
    outs = []
    for lo, hi in ((0, 9), (9, 11), (11, 17)):
        part = oracle.preprocess(xq[lo:hi], xk[lo:hi], xv[lo:hi], w, a[lo:hi], b[lo:hi], state_in=st,
                                 activation="silu", lib_path=lib)
        outs.append(part[:5])
        st = part[5]
    for i in range(5):
        assert np.array_equal(np.concatenate([o[i] for o in outs]), full[i])
    assert np.array_equal(st, full[5])


def pin_state_out_is_last_raw_inputs(lib):
    """The returned conv state holds the last three raw inputs; a one-token
    sequence shifts its starting state by one."""
    rng = np.random.default_rng(8)
    H, d = 2, 3
    xq, xk, xv, w, a, b = _inputs(rng, 6, H, d)
    st0 = rng.standard_normal((2, 3, 3, H, d))
    cu = np.array([0, 5, 6])
    *_, st = oracle.preprocess(xq, xk, xv, w, a, b, cu_seqlens=cu, state_in=st0, lib_path=lib)
    for tau, x in enumerate((xq, xk, xv)):
        assert np.array_equal(st[0, tau], x[2:5])
        assert np.array_equal(st[1, tau, 0:2], st0[1, tau, 1:3])
        assert np.array_equal(st[1, tau, 2], x[5])


def pin_packed_sequences_are_independent(lib):
    """Each packed sequence starts from its own conv state: packing equals
    separate calls."""
    rng = np.random.default_rng(9)
    H, d = 2, 4
    xq, xk, xv, w, a, b = _inputs(rng, 11, H, d)
    st0 = rng.standard_normal((3, 3, 3, H, d))
    cu = np.array([0, 4, 4, 11])
    packed = oracle.preprocess(xq, xk, xv, w, a, b, cu_seqlens=cu, state_in=st0, lib_path=lib)
    for s in range(3):
        lo, hi = cu[s], cu[s + 1]
        one = oracle.preprocess(xq[lo:hi], xk[lo:hi], xv[lo:hi], w, a[lo:hi], b[lo:hi], state_in=st0[s:s + 1],
                                lib_path=lib)
        for i in range(5):
            ref = packed[i][lo:hi]
            assert np.array_equal(one[i], ref)
        assert np.array_equal(one[5][0], packed[5][s])


ALL_PRE_PINS = [pin_identity_taps_normalise_q_k, pin_convolution_matches_numpy, pin_impulse_response,
                pin_gates_closed_form, pin_silu, pin_normalisation_is_scale_invariant, pin_parts_equal_one_shot,
                pin_state_out_is_last_raw_inputs, pin_packed_sequences_are_independent]
