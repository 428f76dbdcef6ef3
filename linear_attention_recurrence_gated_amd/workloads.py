"""Seeded synthetic inputs for the gated delta-rule recurrence.

This module only draws and rounds inputs; it holds none of the recurrence's
arithmetic.  The GPU tests, the benchmark and the CPU oracle all consume the
exact values it returns (the oracle widens them to double without rounding).

Workload shapes follow the pages: 48 heads with 128 x 128 fp32 states per layer
(the factorisation that reproduces the ~144 MiB of fp32 DeltaNet state for 48
layers in "Layouts híbridos: três DeltaNet, uma attention", section Conceito),
a 262,144-token context (same section), and 16,384-token segments (the
training/cache plan in "attention and memory", "Sources, assumptions & limits").

Recipe (every draw from numpy's PCG64 via ``default_rng``; the tokens of a
workload are drawn in blocks of BLOCK tokens, block b from child b of the
workload's SeedSequence, so large workloads are generated on several threads
with a result that does not depend on the thread count):
  q, k, v     standard normal, float32, shape [n, H, d] per block; q and k are
              then L2-normalised per (token, head) in float64
  beta        sigmoid of a standard normal logit
  g           exp(-softplus(x + shift)) of a standard normal logit x
              (shift 2 for the prefill/decode workloads, 0 for the single-head
              fp32 case, negative shifts for slow-decay stress inputs)
  s_init      normal with the given standard deviation, float32
  lengths     log-uniform in [lo, hi], rounded to integers, from a separate
              child stream (so the data stream does not depend on them)
q, k, v are rounded once to the run dtype: float64 -> float32 (round to
nearest even) -> bfloat16 (round to nearest even).  g and beta are rounded
once to float32.
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

SEED_BASE = 1000


def bf16_round(x):
    """Round finite float32 values to the nearest bfloat16 (ties to even); float32 out."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u >> 16) & 1          # no uint32 overflow for finite inputs (|bits| <= 0xFF7FFFFF)
    r += 0x7FFF
    r += u
    r &= 0xFFFF0000
    return r.view(np.float32)


def bf16_bits(x):
    """Raw bfloat16 bit patterns (uint16) of float32 values that are bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not bfloat16-exact; call bf16_round first")
    return (u >> 16).astype(np.uint16)


def _sigmoid(x):
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def _gate_from_logit(x, shift):
    # exp(-softplus(y)) with softplus(y) = log(1 + e^y), evaluated stably
    return np.exp(-np.logaddexp(0.0, x + shift))


def _normalise(x):
    """L2-normalise the last axis in float64; float32 result (round to nearest)."""
    out = np.empty(x.shape, dtype=np.float32)
    step = 512
    for i in range(0, x.shape[0], step):
        xb = x[i:i + step].astype(np.float64)
        n = np.sqrt(np.sum(xb * xb, axis=-1, keepdims=True))
        n[n == 0] = 1.0
        out[i:i + step] = xb / n
    return out


def _round_run_dtype(x64, dtype):
    x32 = np.asarray(x64, dtype=np.float32)
    if dtype == "bf16":
        return bf16_round(x32)
    if dtype == "fp32":
        return np.ascontiguousarray(x32)
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclass
class PrefillInputs:
    q: np.ndarray                      # [N, H, dk] float32 holding run-dtype values
    k: np.ndarray                      # [N, H, dk]
    v: np.ndarray                      # [N, H, dv]
    g: np.ndarray                      # [N, H] float32
    beta: np.ndarray                   # [N, H] float32
    cu_seqlens: Optional[np.ndarray]   # [n_seq + 1] int32, or None (one sequence)
    s_init: Optional[np.ndarray]       # [n_seq, H, dv, dk] float32, or None (zeros)
    dtype: str = "bf16"
    meta: dict = field(default_factory=dict)

    @property
    def n_seq(self):
        return 1 if self.cu_seqlens is None else len(self.cu_seqlens) - 1


BLOCK = 1024  # tokens per independent stream


def _draw_block(ss, n, H, dk, dv, dtype, gate_shift):
    rng = np.random.default_rng(ss)
    q = rng.standard_normal((n, H, dk), dtype=np.float32)
    k = rng.standard_normal((n, H, dk), dtype=np.float32)
    v = rng.standard_normal((n, H, dv), dtype=np.float32)
    b_logit = rng.standard_normal((n, H), dtype=np.float32).astype(np.float64)
    g_logit = rng.standard_normal((n, H), dtype=np.float32).astype(np.float64)
    q = _round_run_dtype(_normalise(q), dtype)
    k = _round_run_dtype(_normalise(k), dtype)
    v = _round_run_dtype(v, dtype)
    beta = _sigmoid(b_logit).astype(np.float32)
    g = _gate_from_logit(g_logit, gate_shift).astype(np.float32)
    return q, k, v, g, beta


def _threads():
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _draw_tokens(ss, N, H, dk, dv, dtype, gate_shift):
    """N tokens in blocks of BLOCK, block b from child b of SeedSequence ss."""
    import concurrent.futures
    nb = (N + BLOCK - 1) // BLOCK
    children = ss.spawn(nb)
    q = np.empty((N, H, dk), np.float32)
    k = np.empty((N, H, dk), np.float32)
    v = np.empty((N, H, dv), np.float32)
    g = np.empty((N, H), np.float32)
    beta = np.empty((N, H), np.float32)

    def one(b):
        a, e = b * BLOCK, min(N, (b + 1) * BLOCK)
        q[a:e], k[a:e], v[a:e], g[a:e], beta[a:e] = _draw_block(children[b], e - a, H, dk, dv, dtype, gate_shift)

    if nb <= 1:
        for b in range(nb):
            one(b)
    else:
        with concurrent.futures.ThreadPoolExecutor(min(nb, _threads())) as ex:
            list(ex.map(one, range(nb)))
    return q, k, v, g, beta


def log_uniform_lengths(rng, n, lo, hi):
    x = np.exp(rng.uniform(np.log(lo), np.log(hi), size=n))
    return np.clip(np.rint(x), lo, hi).astype(np.int64)


def make_prefill(lengths, H, d, dtype="bf16", seed=SEED_BASE, gate_shift=2.0,
                 init_std=None, dv=None, packed=None):
    """Packed prefill inputs for sequences of the given lengths.

    lengths: list of sequence lengths (zeros allowed).  With one sequence and
    packed=False the batch carries no cu_seqlens.  init_std: None for zero
    initial states, else the standard deviation of per-sequence initial states.
    """
    lengths = [int(x) for x in lengths]
    dv = d if dv is None else dv
    N = sum(lengths)
    tok_ss, state_ss = np.random.SeedSequence(seed).spawn(2)
    q, k, v, g, beta = _draw_tokens(tok_ss, N, H, d, dv, dtype, gate_shift)
    n = len(lengths)
    s_init = None
    if init_std is not None:
        rng = np.random.default_rng(state_ss)
        s_init = (init_std * rng.standard_normal((n, H, dv, d), dtype=np.float32)).astype(np.float32)
    if packed is None:
        packed = n != 1
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32) if packed else None
    return PrefillInputs(q, k, v, g, beta, cu, s_init, dtype,
                         meta=dict(lengths=lengths, H=H, d=d, dv=dv, seed=seed, gate_shift=gate_shift))


@dataclass
class DecodeInputs:
    q: np.ndarray       # [steps, B, H, dk]
    k: np.ndarray
    v: np.ndarray       # [steps, B, H, dv]
    g: np.ndarray       # [steps, B, H]
    beta: np.ndarray
    s_init: np.ndarray  # [B, H, dv, dk]
    dtype: str = "bf16"


def make_decode(steps, B, H, d, dtype="bf16", seed=SEED_BASE + 3, gate_shift=2.0, init_std=0.02):
    tok_ss, state_ss = np.random.SeedSequence(seed).spawn(2)
    q, k, v, g, beta = _draw_tokens(tok_ss, steps * B, H, d, d, dtype, gate_shift)
    s_init = (init_std * np.random.default_rng(state_ss).standard_normal((B, H, d, d), dtype=np.float32)).astype(np.float32)
    rs = lambda x: x.reshape((steps, B) + x.shape[1:])
    return DecodeInputs(rs(q), rs(k), rs(v), rs(g), rs(beta), s_init, dtype)


# ---------------------------------------------------------------------------
# The five workloads, numbered 1..5 for their seeds (SeedSequence(1000 + n)):
# a tiny fp32 prefill, the one-layer prefill at T = 4096, batched decode, the
# long context in segments, and a packed varlen batch.

def prefill_t64_d16_fp32():
    """Single head, fp32: B=1, H=1, T=64, d=16, g = exp(-softplus(x)), S_0 = 0."""
    return make_prefill([64], H=1, d=16, dtype="fp32", seed=SEED_BASE + 1, gate_shift=0.0)


def prefill_t4096_h48(T=4096, H=48, d=128, seed=SEED_BASE + 2, gate_shift=2.0):
    """One-layer prefill: B=1, H=48, T=4096, d=128, bf16, S_0 = 0, chunk 64."""
    return make_prefill([T], H=H, d=d, dtype="bf16", seed=seed, gate_shift=gate_shift)


def decode_b64_h48(steps=256, B=64, H=48, d=128):
    """Batched decode: B=64, H=48, d=128, 256 single-token steps, S_0 ~ N(0, 0.02^2)."""
    return make_decode(steps, B, H, d, dtype="bf16", seed=SEED_BASE + 3)


def long_context_segments(n_seg=16, seg_len=16384, H=48, d=128):
    """Long context: 262,144 tokens as 16 segments of 16,384 with the state
    carried; segment i is drawn from child stream i of SeedSequence(1004)."""
    children = np.random.SeedSequence(SEED_BASE + 4).spawn(n_seg)
    for i, ss in enumerate(children):
        q, k, v, g, beta = _draw_tokens(ss, seg_len, H, d, d, "bf16", 2.0)
        yield PrefillInputs(q, k, v, g, beta, None, None, "bf16",
                            meta=dict(segment=i, seg_len=seg_len, H=H, d=d))


def varlen_lengths(n=8, lo=1024, hi=65536):
    ss = np.random.SeedSequence(SEED_BASE + 5)
    len_ss, _ = ss.spawn(2)
    return [int(x) for x in log_uniform_lengths(np.random.default_rng(len_ss), n, lo, hi)]


def varlen_batch(H=48, d=128):
    """Variable-length packed prefill: 8 sequences, log-uniform lengths in
    [1024, 65536], per-sequence initial states ~ N(0, 0.02^2), reset between
    sequences, per-sequence final states."""
    lengths = varlen_lengths()
    _, data_ss = np.random.SeedSequence(SEED_BASE + 5).spawn(2)
    tok_ss, state_ss = data_ss.spawn(2)
    N = sum(lengths)
    q, k, v, g, beta = _draw_tokens(tok_ss, N, H, d, d, "bf16", 2.0)
    rng = np.random.default_rng(state_ss)
    s_init = (0.02 * rng.standard_normal((len(lengths), H, d, d), dtype=np.float32)).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return PrefillInputs(q, k, v, g, beta, cu, s_init, "bf16", meta=dict(lengths=lengths, H=H, d=d))


# ---------------------------------------------------------------------------
# Inputs of the pre-processing (convolution, norm and gate maps) in front of
# the recurrence.

@dataclass
class PreprocessInputs:
    xq: np.ndarray                     # [N, H, d] float32 holding run-dtype values
    xk: np.ndarray
    xv: np.ndarray
    w: np.ndarray                      # [3, H, d, 4] float32 conv taps
    a_logit: np.ndarray                # [N, H] float32
    b_logit: np.ndarray                # [N, H] float32
    bias: Optional[np.ndarray]         # [H] float32 or None
    cu_seqlens: Optional[np.ndarray]   # [n_seq + 1] int32, or None
    state_in: Optional[np.ndarray]     # [n_seq, 3, 3, H, d] float32 run-dtype values, or None
    dtype: str = "bf16"
    activation: str = "none"

    @property
    def n_seq(self):
        return 1 if self.cu_seqlens is None else len(self.cu_seqlens) - 1


def make_preprocess(lengths, H, d, dtype="bf16", seed=SEED_BASE + 6, with_state=True, with_bias=True,
                    activation="none", packed=None):
    """Raw projections x ~ N(0, 1) rounded to the run dtype; conv taps uniform
    in [-1/2, 1/2] (the default init bound 1/sqrt(fan_in) of a depthwise
    kernel of 4 taps); logits a, b ~ N(0, 1); per-head bias uniform in [0, 4];
    starting conv states ~ N(0, 1) rounded to the run dtype."""
    lengths = [int(x) for x in lengths]
    N, n = sum(lengths), len(lengths)
    rng = np.random.default_rng(np.random.SeedSequence(seed))
    x = [_round_run_dtype(rng.standard_normal((N, H, d), dtype=np.float32), dtype) for _ in range(3)]
    w = rng.uniform(-0.5, 0.5, size=(3, H, d, 4)).astype(np.float32)
    a = rng.standard_normal((N, H), dtype=np.float32)
    b = rng.standard_normal((N, H), dtype=np.float32)
    bias = rng.uniform(0.0, 4.0, size=H).astype(np.float32) if with_bias else None
    st = _round_run_dtype(rng.standard_normal((n, 3, 3, H, d), dtype=np.float32), dtype) if with_state else None
    if packed is None:
        packed = n != 1
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32) if packed else None
    return PreprocessInputs(x[0], x[1], x[2], w, a, b, bias, cu, st, dtype, activation)


# ---------------------------------------------------------------------------
# Device placement (torch is used for memory only).

def to_torch(x, dtype, device):
    """Move a float32 array holding run-dtype values to a torch tensor."""
    import torch
    if dtype == "bf16":
        bits = bf16_bits(x).view(np.int16)
        return torch.from_numpy(bits).to(device).view(torch.bfloat16)
    if dtype == "fp32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)
    raise ValueError(dtype)
