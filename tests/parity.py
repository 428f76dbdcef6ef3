"""Error measures used by the GPU parity tests.

The bar: max|got - ref| / rms(ref) <= 1e-4 for fp32 q/k/v and <= 3e-3 for
bf16 q/k/v with fp32 gates and state, applied to the outputs o and to the
final states alike (the state measure uses the state's own rms).
"""
import numpy as np

TOL_FP32 = 1e-4
TOL_BF16 = 3e-3


def rel_max_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = float(np.max(np.abs(got - ref)))
    if rms == 0.0:
        return err
    return err / rms


def tol_for(dtype):
    return TOL_FP32 if dtype == "fp32" else TOL_BF16


def assert_through_bf16_inputs(o, o_ref, s, s_ref, apart, cu_seqlens=None, what="", say=print):
    """End-to-end bar for outputs of the recurrence whose bf16 inputs q, k, v
    the two sides form separately: the oracle rounds its double-precision
    pre-processing to bf16, the kernels their fp32 one.  A few elements in
    100,000 lie so close to a rounding midpoint that the two round them one
    bf16 unit apart, which moves the outputs of that token, and through the
    state those of the following ones, by up to a few 1e-2 of rms(o).

    o, o_ref: [N, H, d]; s, s_ref: final states; apart: [N, H] bool, the
    tokens whose q, k or v the two sides round apart.  The bar: the final
    states within TOL_BF16 (max|err| / rms); o within TOL_BF16 in norm
    (||err|| / ||ref||); every token's outputs within TOL_BF16 (max|err| /
    rms of the head's outputs) except on tokens that follow a disagreement
    of their own head and sequence by less than 64 tokens, and those at most
    1 % of the (token, head) pairs."""
    o = np.asarray(o, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    es = rel_max_err(s, s_ref)
    eo = float(np.linalg.norm(o - o_ref) / max(np.linalg.norm(o_ref), 1e-300))
    say(f"  {what}: state max/rms {es:.2e}, o norm-wise {eo:.2e}")
    assert es <= TOL_BF16, f"{what}: state error {es}"
    assert eo <= TOL_BF16, f"{what}: norm-wise output error {eo}"
    N, H = apart.shape
    seq = np.zeros(N, dtype=np.int64)
    if cu_seqlens is not None:
        seq = np.searchsorted(np.asarray(cu_seqlens)[1:], np.arange(N), side="right")
    n_over = 0
    for h in range(H):
        rms = float(np.sqrt(np.mean(o_ref[:, h] ** 2)))
        over = np.nonzero(np.max(np.abs(o[:, h] - o_ref[:, h]), axis=1) > TOL_BF16 * rms)[0]
        flips = np.nonzero(apart[:, h])[0]
        for t in over:
            near = flips[(flips <= t) & (flips > t - 64)]
            assert np.any(seq[near] == seq[t]), f"{what}: head {h} token {t} over the bar with no disagreement"
        n_over += over.size
    say(f"  {what}: {int(apart.sum())} (token, head) pairs rounded apart, {n_over} over the element-wise bar")
    assert n_over <= 0.01 * N * H, f"{what}: {n_over} (token, head) pairs over the element-wise bar"


def rounded_apart(pairs):
    """[N, H] bool: tokens where any of the (got, ref) [N, H, d] pairs differ."""
    out = None
    for a, b in pairs:
        x = np.any(np.asarray(a) != np.asarray(b), axis=2)
        out = x if out is None else out | x
    return out
