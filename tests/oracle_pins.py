"""Pins for the CPU oracle: facts fixed by the pages or by mathematics.

None of these retypes the oracle's token loop.  Each one checks the oracle's
output against something independent of it: a closed form, a special case that
reduces to a textbook result, an explicit expansion built from matrix products,
or an invariant.  Each pin takes the oracle's ``run`` callable so the same pins
can be pointed at deliberately broken builds of the oracle (see
test_oracle_mutants.py).

Sources cited below:
  [GDN]  "Qwen3.8-27B 架构深读" (feifeigd.github.io, 2026-08-17), section 三
         (Gated DeltaNet): the linear-attention memory and read-out formulas, the
         delta rule read as an online regression step ("erase along the key, then
         write"), and the gated delta-rule equation.
  [PROF] "Hybrid · kết hợp nhiều cơ chế..." (openarchlab.com), section 4
         (Profiling): running in segments with carried state must not change
         the result.
  [STATE] "attention and memory" (stethem.com), "Sources, assumptions & limits":
         the recurrent state exists before any token arrives.
"""
import numpy as np

RTOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _close(a, b, tol=RTOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"{what}: max|diff| {err:.3e} > {tol:.1e} * {scale:.3e}"


def _inputs(seed, T, H, dk, dv, unit_keys=True, gate=(0.2, 1.0), strength=(0.0, 1.0)):
    r = _rng(seed)
    q = r.standard_normal((T, H, dk))
    k = r.standard_normal((T, H, dk))
    if unit_keys:
        k = _unit(k)
    v = r.standard_normal((T, H, dv))
    g = r.uniform(gate[0], gate[1], (T, H))
    beta = r.uniform(strength[0], strength[1], (T, H))
    return q, k, v, g, beta


def _prefix_states(run, q, k, v, g, beta, s0):
    """Final states after 0..T tokens, from one packed call of T+1 prefixes."""
    T, H = g.shape
    seqs = [np.arange(p) for p in range(T + 1)]
    idx = np.concatenate(seqs).astype(np.int64)
    cu = np.cumsum([0] + [p for p in range(T + 1)])
    s_init = np.broadcast_to(s0, (T + 1,) + s0.shape).copy()
    _, s = run(q[idx], k[idx], v[idx], g[idx], beta[idx], cu, s_init)
    return s  # [T+1, H, dv, dk]


def pin_per_token_closed_form(run):
    """With |k_t| = 1, any g and beta: S_t k_t = (g_t - beta_t) S_{t-1} k_t + beta_t v_t.

    Follows from [GDN]'s gated delta-rule equation by multiplying it by k_t
    (k_t^T k_t = 1).  It fixes the recall-before-gate order, the orientation of
    S and the sign of the correction.
    """
    T, H, dk, dv = 9, 2, 6, 4
    q, k, v, g, beta = _inputs(11, T, H, dk, dv, gate=(0.05, 1.0), strength=(-0.5, 1.5))
    s0 = _rng(12).standard_normal((H, dv, dk))
    S = _prefix_states(run, q, k, v, g, beta, s0)
    for t in range(1, T + 1):
        for h in range(H):
            kt = k[t - 1, h]
            lhs = S[t, h] @ kt
            rhs = (g[t - 1, h] - beta[t - 1, h]) * (S[t - 1, h] @ kt) + beta[t - 1, h] * v[t - 1, h]
            _close(lhs, rhs, what=f"S_t k_t closed form at t={t}")


def pin_unit_write(run):
    """g = beta = 1 and |k_t| = 1: the write stores v_t exactly under k_t.

    [GDN]: the delta rule first erases what the key recalls, then writes the
    new value, so S_t k_t = v_t; with q_t = k_t the read-out is o_t = v_t.
    """
    T, H, dk, dv = 12, 3, 8, 5
    q, k, v, g, beta = _inputs(21, T, H, dk, dv)
    g[:] = 1.0
    beta[:] = 1.0
    s0 = _rng(22).standard_normal((1, H, dv, dk))
    S = _prefix_states(run, q, k, v, g, beta, s0[0])
    for t in range(1, T + 1):
        for h in range(H):
            _close(S[t, h] @ k[t - 1, h], v[t - 1, h], what=f"S_t k_t = v_t at t={t}")
    o, _ = run(k, k, v, g, beta, None, s0)
    _close(o, v, what="o_t = v_t when q_t = k_t")


def pin_pure_decay(run):
    """beta = 0: the state only decays, S_t = (prod_{s<=t} g_s) S_0 and
    o_t = (prod_{s<=t} g_s) S_0 q_t; with g = 1 as well the state is constant.

    [GDN]: g decides how much of the old memory is kept; with no write
    (beta = 0) nothing else changes the state.
    """
    T, H, dk, dv = 10, 2, 5, 7
    q, k, v, g, beta = _inputs(31, T, H, dk, dv, unit_keys=False, gate=(0.3, 1.0))
    beta[:] = 0.0
    s0 = _rng(32).standard_normal((1, H, dv, dk))
    o, s = run(q, k, v, g, beta, None, s0)
    cp = np.cumprod(g, axis=0)  # [T, H]
    for h in range(H):
        _close(s[0, h], cp[-1, h] * s0[0, h], what="decayed final state")
        for t in range(T):
            _close(o[t, h], cp[t, h] * (s0[0, h] @ q[t, h]), what=f"decayed read-out t={t}")
    g[:] = 1.0
    o, s = run(q, k, v, g, beta, None, s0)
    _close(s, s0, tol=0.0, what="g=1, beta=0 leaves the state unchanged")


def pin_orthonormal_linear_attention(run):
    """Orthonormal keys, g = beta = 1, S_0 = 0: the recurrence reduces to the
    plain linear-attention memory S_T = sum_i v_i k_i^T and the causal read-out
    o_t = sum_{i<=t} (k_i . q_t) v_i ([GDN], linear-attention formulas).
    Writes along orthogonal keys never disturb each other's recall.
    """
    H, d, dv = 2, 8, 6
    T = d
    r = _rng(41)
    k = np.empty((T, H, d))
    for h in range(H):
        Qm, _ = np.linalg.qr(r.standard_normal((d, d)))
        k[:, h, :] = Qm.T  # rows orthonormal
    q = r.standard_normal((T, H, d))
    v = r.standard_normal((T, H, dv))
    g = np.ones((T, H))
    beta = np.ones((T, H))
    o, s = run(q, k, v, g, beta)
    for h in range(H):
        _close(s[0, h], sum(np.outer(v[i, h], k[i, h]) for i in range(T)), what="sum v k^T")
        for t in range(T):
            ref = sum((k[i, h] @ q[t, h]) * v[i, h] for i in range(t + 1))
            _close(o[t, h], ref, what=f"causal linear attention t={t}")


def pin_scalar(run):
    """d_k = d_v = 1: s_t = (g_t - beta_t k_t^2) s_{t-1} + beta_t k_t v_t and
    o_t = s_t q_t -- the gated delta-rule equation of [GDN] with 1x1 matrices."""
    T, H = 15, 3
    q, k, v, g, beta = _inputs(51, T, H, 1, 1, unit_keys=False, strength=(-1.0, 2.0))
    s0 = _rng(52).standard_normal((1, H, 1, 1))
    o, s = run(q, k, v, g, beta, None, s0)
    for h in range(H):
        st = s0[0, h, 0, 0]
        for t in range(T):
            kt, vt, qt = k[t, h, 0], v[t, h, 0], q[t, h, 0]
            st = (g[t, h] - beta[t, h] * kt * kt) * st + beta[t, h] * kt * vt
            _close(o[t, h, 0], st * qt, what=f"scalar read-out t={t}")
        _close(s[0, h, 0, 0], st, what="scalar final state")


def _expand(q, k, v, g, beta, s0):
    """Explicit sum over the history with the transitions built as matrices:
    S_t = S_0 A_1...A_t + sum_{i<=t} beta_i v_i k_i^T A_{i+1}...A_t,
    A_s = g_s I - beta_s k_s k_s^T (d_k x d_k), acting on S from the right."""
    T, dk = k.shape
    A = [g[s] * np.eye(dk) - beta[s] * np.outer(k[s], k[s]) for s in range(T)]
    outs, S = [], None
    for t in range(T):
        P = np.eye(dk)
        for s in range(t + 1):
            P = P @ A[s]
        S = s0 @ P
        for i in range(t + 1):
            Pi = np.eye(dk)
            for s in range(i + 1, t + 1):
                Pi = Pi @ A[s]
            S = S + beta[i] * np.outer(v[i], k[i]) @ Pi
        outs.append(S @ q[t])
    return np.array(outs), S


def pin_brute_force_expansion(run):
    """Tiny inputs (T <= 8, d <= 6, unnormalised keys, out-of-range gates):
    the oracle equals the explicit history expansion of [GDN]'s recurrence."""
    for seed, (T, dk, dv) in enumerate([(8, 5, 4), (7, 3, 6), (1, 4, 4), (6, 6, 6)]):
        q, k, v, g, beta = _inputs(60 + seed, T, 1, dk, dv, unit_keys=False,
                                   gate=(0.1, 1.2), strength=(-0.5, 1.5))
        s0 = _rng(70 + seed).standard_normal((1, 1, dv, dk))
        o, s = run(q, k, v, g, beta, None, s0)
        o_ref, s_ref = _expand(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], s0[0, 0])
        _close(o[:, 0], o_ref, tol=1e-11, what=f"expansion read-out {T}x{dk}x{dv}")
        _close(s[0, 0], s_ref, tol=1e-11, what=f"expansion final state {T}x{dk}x{dv}")


def pin_superposition(run):
    """For fixed q, k, g, beta the recurrence is linear in (V, S_0) jointly:
    o(V1+V2, S1+S2) = o(V1, S1) + o(V2, S2), and likewise for the final state.
    (The transition A_t does not depend on v; my algebra on [GDN]'s equation.)"""
    T, H, dk, dv = 11, 2, 6, 5
    q, k, v1, g, beta = _inputs(81, T, H, dk, dv)
    v2 = _rng(82).standard_normal(v1.shape)
    s1 = _rng(83).standard_normal((1, H, dv, dk))
    s2 = _rng(84).standard_normal((1, H, dv, dk))
    oa, sa = run(q, k, v1, g, beta, None, s1)
    ob, sb = run(q, k, v2, g, beta, None, s2)
    oc, sc = run(q, k, v1 + v2, g, beta, None, s1 + s2)
    _close(oc, oa + ob, tol=1e-12, what="read-out superposition")
    _close(sc, sa + sb, tol=1e-12, what="state superposition")
    oz, sz = run(q, k, 0 * v1, g, beta, None, 0 * s1)
    _close(oz, np.zeros_like(oz), tol=0.0, what="zero values and zero state give zero")


def pin_row_permutation(run):
    """Permuting the d_v components of v and the rows of S_0 permutes o and the
    rows of the final state the same way: each state row evolves on its own."""
    T, H, dk, dv = 9, 2, 5, 7
    q, k, v, g, beta = _inputs(91, T, H, dk, dv)
    s0 = _rng(92).standard_normal((1, H, dv, dk))
    perm = _rng(93).permutation(dv)
    o, s = run(q, k, v, g, beta, None, s0)
    op, sp = run(q, k, v[:, :, perm], g, beta, None, s0[:, :, perm, :])
    _close(op, o[:, :, perm], tol=0.0, what="permuted read-out")
    _close(sp, s[:, :, perm, :], tol=0.0, what="permuted state rows")


def pin_segmented_equals_one_shot(run):
    """[PROF]: splitting a run into segments and carrying the state over must
    not change the result.  For the token-by-token oracle it is bit-exact."""
    T, H, dk, dv = 40, 3, 6, 5
    q, k, v, g, beta = _inputs(101, T, H, dk, dv)
    s0 = _rng(102).standard_normal((1, H, dv, dk))
    o_full, s_full = run(q, k, v, g, beta, None, s0)
    cuts = [0, 7, 8, 8, 23, 40]
    state = s0
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        o_seg, state = run(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], None, state)
        parts.append(o_seg)
    _close(np.concatenate(parts), o_full, tol=0.0, what="segmented read-out")
    _close(state, s_full, tol=0.0, what="segmented final state")


def pin_packed_sequences_are_independent(run):
    """A packed batch equals its sequences run one by one, each from its own
    initial state ([STATE]: the state exists before any token); a zero-length
    sequence returns its initial state and no outputs; absent initial state
    means zeros; heads never interact."""
    H, dk, dv = 3, 4, 5
    lens = [5, 0, 9, 1, 0, 7]
    T = sum(lens)
    q, k, v, g, beta = _inputs(111, T, H, dk, dv)
    s0 = _rng(112).standard_normal((len(lens), H, dv, dk))
    cu = np.cumsum([0] + lens)
    o, s = run(q, k, v, g, beta, cu, s0)
    for i, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        oi, si = run(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], None, s0[i:i + 1])
        _close(o[a:b], oi, tol=0.0, what=f"sequence {i} read-out")
        _close(s[i], si[0], tol=0.0, what=f"sequence {i} final state")
        if a == b:
            _close(s[i], s0[i], tol=0.0, what="zero-length sequence keeps its state")
    oz, sz = run(q, k, v, g, beta, cu, None)
    oz2, sz2 = run(q, k, v, g, beta, cu, np.zeros_like(s0))
    _close(oz, oz2, tol=0.0, what="no initial state means zeros")
    for h in range(H):
        oh, sh = run(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], g[:, h:h + 1],
                     beta[:, h:h + 1], cu, s0[:, h:h + 1])
        _close(o[:, h:h + 1], oh, tol=0.0, what=f"head {h} alone")
        _close(s[:, h:h + 1], sh, tol=0.0, what=f"head {h} state alone")


def pin_stability_bound(run):
    """|k| = 1, 0 <= beta <= 1, 0 < g <= 1: the transition has spectral norm
    max(g, |g - beta|) <= 1, so |S_t|_F <= |S_{t-1}|_F + beta_t |v_t| (my
    algebra on [GDN]'s equation).  Checked along a long run."""
    T, H, dk, dv = 64, 2, 8, 8
    q, k, v, g, beta = _inputs(121, T, H, dk, dv, gate=(0.9, 1.0), strength=(0.0, 1.0))
    s0 = 3.0 * _rng(122).standard_normal((H, dv, dk))
    S = _prefix_states(run, q, k, v, g, beta, s0)
    for t in range(1, T + 1):
        for h in range(H):
            lhs = np.linalg.norm(S[t, h])
            rhs = np.linalg.norm(S[t - 1, h]) + beta[t - 1, h] * np.linalg.norm(v[t - 1, h])
            assert lhs <= rhs * (1 + 1e-12), f"norm bound broken at t={t}: {lhs} > {rhs}"


# ---------------------------------------------------------------------------
# Variants ([GDN] section 三: the linear-attention memory, the delta rule and
# its gated form).  NO_GATE = 1 (g_t = 1), NO_ERASE = 2 (no recall term).

NO_GATE, NO_ERASE = 1, 2


def pin_variant_plain_linear_attention(run):
    """No gate and no erase term, beta = 1: the linear-attention memory
    S_t = S_0 + sum_{i<=t} v_i k_i^T and o_t = S_t q_t ([GDN], linear-attention
    formulas), whatever g holds; unnormalised, non-orthogonal keys."""
    T, H, dk, dv = 9, 2, 5, 4
    q, k, v, g, _ = _inputs(81, T, H, dk, dv, unit_keys=False)
    beta = np.ones((T, H))
    s0 = _rng(82).standard_normal((1, H, dv, dk))
    o, s = run(q, k, v, g, beta, None, s0, variant=NO_GATE | NO_ERASE)
    for h in range(H):
        mem = s0[0, h] + np.cumsum(np.einsum("ti,tj->tij", v[:, h], k[:, h]), axis=0)
        _close(s[0, h], mem[-1], what="linear-attention memory")
        _close(o[:, h], np.einsum("tij,tj->ti", mem, q[:, h]), what="linear-attention read-out")


def pin_variant_gated_linear_attention(run):
    """No erase term: S_t = (prod_{s<=t} g_s) S_0 + sum_{i<=t} (prod_{i<s<=t} g_s)
    beta_i v_i k_i^T, written as an explicit sum of decayed writes."""
    T, H, dk, dv = 8, 2, 4, 3
    q, k, v, g, beta = _inputs(83, T, H, dk, dv, unit_keys=False, strength=(-0.5, 1.5))
    s0 = _rng(84).standard_normal((1, H, dv, dk))
    o, s = run(q, k, v, g, beta, None, s0, variant=NO_ERASE)
    for h in range(H):
        for t in range(T):
            St = np.prod(g[:t + 1, h]) * s0[0, h]
            for i in range(t + 1):
                St = St + np.prod(g[i + 1:t + 1, h]) * beta[i, h] * np.outer(v[i, h], k[i, h])
            _close(o[t, h], St @ q[t, h], what=f"decayed linear attention t={t}")
        _close(s[0, h], St, what="decayed linear-attention memory")


def pin_variant_delta_rule(run):
    """No gate: the delta rule, equal to the explicit history expansion with
    transitions A_s = I - beta_s k_s k_s^T; the g passed in is ignored."""
    for seed, (T, dk, dv) in enumerate([(7, 4, 3), (5, 5, 5)]):
        q, k, v, g, beta = _inputs(85 + seed, T, 1, dk, dv, unit_keys=False, strength=(-0.5, 1.5))
        s0 = _rng(87 + seed).standard_normal((1, 1, dv, dk))
        o, s = run(q, k, v, g, beta, None, s0, variant=NO_GATE)
        o_ref, s_ref = _expand(q[:, 0], k[:, 0], v[:, 0], np.ones(T), beta[:, 0], s0[0, 0])
        _close(o[:, 0], o_ref, tol=1e-11, what=f"delta-rule read-out {T}x{dk}x{dv}")
        _close(s[0, 0], s_ref, tol=1e-11, what=f"delta-rule final state {T}x{dk}x{dv}")


def pin_variant_delta_rule_repeated_key(run):
    """No gate, one unit key written again and again: the recall along that key
    is an exponential moving average, r_t = (1 - beta_t) r_{t-1} + beta_t v_t
    (the delta rule as an online regression step, [GDN])."""
    T, dk, dv = 12, 6, 3
    r = _rng(89)
    key = _unit(r.standard_normal(dk))
    k = np.broadcast_to(key, (T, 1, dk)).copy()
    q = k.copy()
    v = r.standard_normal((T, 1, dv))
    beta = r.uniform(0.0, 1.0, (T, 1))
    g = r.uniform(0.2, 0.9, (T, 1))
    o, _ = run(q, k, v, g, beta, variant=NO_GATE)
    rt = np.zeros(dv)
    for t in range(T):
        rt = (1.0 - beta[t, 0]) * rt + beta[t, 0] * v[t, 0]
        _close(o[t, 0], rt, what=f"moving average t={t}")


ALL_PINS = [
    pin_per_token_closed_form,
    pin_unit_write,
    pin_pure_decay,
    pin_orthonormal_linear_attention,
    pin_scalar,
    pin_brute_force_expansion,
    pin_superposition,
    pin_row_permutation,
    pin_segmented_equals_one_shot,
    pin_packed_sequences_are_independent,
    pin_stability_bound,
    pin_variant_plain_linear_attention,
    pin_variant_gated_linear_attention,
    pin_variant_delta_rule,
    pin_variant_delta_rule_repeated_key,
]
