"""CPU oracle for the gated delta-rule recurrence -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The GPU library and its Python binding never
import, load or call it, and it shares no code with them.

``run`` wraps the double-precision token loop in ``gdn_oracle.c``:
per head, the d_v x d_k state follows the gated delta-rule equation of
"Qwen3.8-27B 架构深读" (feifeigd.github.io, 2026-08-17), section 三
(Gated DeltaNet), S_t = g_t S_{t-1} + beta_t (v_t - S_{t-1} k_t) k_t^T, and
the read-out is o_t = S_t q_t from the updated state.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdn_oracle.so")
PRE_LIB_PATH = os.path.join(HERE, "libgdn_preprocess.so")

_libs = {}


def load(path=LIB_PATH):
    """Load (once per path) an oracle shared library and declare its entry point."""
    lib = _libs.get(path)
    if lib is not None:
        return lib
    if not os.path.exists(path):
        raise RuntimeError(f"oracle library {path} is not built; run oracle/build.py")
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int64)
    lib.gdn_oracle_run.restype = ctypes.c_int
    lib.gdn_oracle_run.argtypes = [dp, dp, dp, dp, dp, ip, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                   dp, dp, dp, ctypes.c_int]
    lib.gdn_oracle_run_variant.restype = ctypes.c_int
    lib.gdn_oracle_run_variant.argtypes = lib.gdn_oracle_run.argtypes + [ctypes.c_int]
    _libs[path] = lib
    return lib


def default_threads():
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


NO_GATE, NO_ERASE = 1, 2


def run(q, k, v, g, beta, cu_seqlens=None, s_init=None, threads=None, lib_path=LIB_PATH, variant=0):
    """Run the recurrence over a packed batch.

    q, k: [N, H, dk]; v: [N, H, dv]; g, beta: [N, H]; any real dtype (converted
    exactly to float64).  cu_seqlens: [n_seq + 1] integer offsets, or None for a
    single sequence.  s_init: [n_seq, H, dv, dk] or None (zeros).
    variant: 0 (gated delta rule), or NO_GATE (g ignored; may be None) and/or
    NO_ERASE (no recall term: the linear-attention write).
    Returns (o [N, H, dv], s_final [n_seq, H, dv, dk]) as float64.
    """
    q, k, v, beta = (_f64(x) for x in (q, k, v, beta))
    g = None if (g is None and variant & NO_GATE) else _f64(g)
    N, H, dk = k.shape
    dv = v.shape[2]
    assert q.shape == (N, H, dk) and v.shape[:2] == (N, H), "q/k/v shapes disagree"
    assert (g is None or g.shape == (N, H)) and beta.shape == (N, H), "g/beta must be [N, H]"
    if cu_seqlens is None:
        cu = None
        n_seq = 1
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        n_seq = cu.shape[0] - 1
    s0 = None if s_init is None else _f64(s_init)
    if s0 is not None:
        assert s0.shape == (n_seq, H, dv, dk), "s_init must be [n_seq, H, dv, dk]"
    o = np.zeros((N, H, dv), dtype=np.float64)
    s_final = np.zeros((n_seq, H, dv, dk), dtype=np.float64)
    lib = load(lib_path)
    cu_ptr = None if cu is None else cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    rc = lib.gdn_oracle_run_variant(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), cu_ptr,
                                    n_seq, N, H, dk, dv, _ptr(s0), _ptr(o), _ptr(s_final),
                                    int(threads or default_threads()), int(variant))
    if rc != 0:
        raise ValueError(f"gdn_oracle_run rejected its arguments (code {rc})")
    return o, s_final


def run_decode(q, k, v, g, beta, s_init, threads=None, lib_path=LIB_PATH, variant=0):
    """Oracle for repeated single-token steps on a batch of states.

    q, k: [steps, B, H, dk]; v: [steps, B, H, dv]; g, beta: [steps, B, H];
    s_init: [B, H, dv, dk].  Step t of sequence b is token t of sequence b, so
    this is the packed-batch recurrence with each sequence's tokens made
    contiguous.  Returns (o [steps, B, H, dv], s_final [B, H, dv, dk]).
    """
    q, k, v = (np.asarray(x) for x in (q, k, v))
    beta = np.asarray(beta)
    g = beta if (g is None and variant & NO_GATE) else np.asarray(g)  # ignored then
    steps, B, H, dk = k.shape
    dv = v.shape[3]
    pack = lambda x: np.ascontiguousarray(np.swapaxes(x, 0, 1)).reshape((B * steps,) + x.shape[2:])
    cu = np.arange(B + 1, dtype=np.int64) * steps
    o, s = run(pack(q), pack(k), pack(v), pack(g), pack(beta), cu, s_init, threads, lib_path, variant)
    o = np.swapaxes(o.reshape(B, steps, H, dv), 0, 1)
    return o, s


def _load_pre(path=PRE_LIB_PATH):
    lib = _libs.get(path)
    if lib is not None:
        return lib
    if not os.path.exists(path):
        raise RuntimeError(f"oracle library {path} is not built; run oracle/build.py")
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int64)
    lib.gdn_oracle_preprocess.restype = ctypes.c_int
    lib.gdn_oracle_preprocess.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, ip, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_int64, ctypes.c_int, dp, dp, dp, dp, dp, dp]
    _libs[path] = lib
    return lib


def preprocess(xq, xk, xv, w, a_logit, b_logit, bias=None, cu_seqlens=None, state_in=None, activation="none",
               lib_path=PRE_LIB_PATH):
    """Pre-processing in front of the recurrence (gdn_preprocess.c): causal
    depthwise 4-tap convolution of q, k, v with a per-sequence conv state,
    optional SiLU, per-(token, head) L2 normalisation of q and k, and the gate
    maps beta = sigmoid(b), g = exp(-softplus(a + bias)).

    xq, xk, xv: [N, H, d]; w: [3, H, d, 4]; a_logit, b_logit: [N, H]; bias: [H]
    or None; cu_seqlens: [n_seq + 1] or None; state_in: [n_seq, 3, 3, H, d] or
    None (zeros).  Returns (q, k, v, g, beta, state_out) as float64.
    """
    xq, xk, xv, w, a, b = (_f64(x) for x in (xq, xk, xv, w, a_logit, b_logit))
    N, H, d = xq.shape
    assert xk.shape == xq.shape and xv.shape == xq.shape and w.shape == (3, H, d, 4)
    assert a.shape == (N, H) and b.shape == (N, H)
    if cu_seqlens is None:
        cu, n_seq = None, 1
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        n_seq = cu.shape[0] - 1
    bias64 = None if bias is None else _f64(bias)
    st = None if state_in is None else _f64(state_in)
    if st is not None:
        assert st.shape == (n_seq, 3, 3, H, d)
    act = {"none": 0, "silu": 1}[activation]
    yq, yk, yv = (np.zeros((N, H, d)) for _ in range(3))
    g = np.zeros((N, H))
    beta = np.zeros((N, H))
    st_out = np.zeros((n_seq, 3, 3, H, d))
    lib = _load_pre(lib_path)
    cu_ptr = None if cu is None else cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    rc = lib.gdn_oracle_preprocess(_ptr(xq), _ptr(xk), _ptr(xv), _ptr(w), _ptr(st), _ptr(a), _ptr(b), _ptr(bias64),
                                   cu_ptr, n_seq, N, H, d, act, _ptr(yq), _ptr(yk), _ptr(yv), _ptr(g), _ptr(beta),
                                   _ptr(st_out))
    if rc != 0:
        raise ValueError(f"gdn_oracle_preprocess rejected its arguments (code {rc})")
    return yq, yk, yv, g, beta, st_out
