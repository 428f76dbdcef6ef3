#!/usr/bin/env python3
"""Benchmark of the gated delta-rule recurrence on one MI355X.

Metric: GDN prefill tokens/s/layer at T = 4096 (B = 1, H = 48, d = 128, bf16
q/k/v, fp32 gates/state/outputs, chunk 64), plus the decode step's state-update
bandwidth (B = 64, H = 48, d = 128, 256 in-place steps) as GB/s and % of the HBM
peak.  Inputs are seeded synthetic data already resident in HBM when timing
starts.

One timed step = one gdn_prefill call over the 4096-token batch from a zero
initial state (initial_state NULL: the kernels start from zeros), writing o
and the final state.  The decode half is timed as one pass of 256
gdn_decode_step calls.  Further entries time the pre-processing, the serving
form of the decode step and the chunk-level scan.  Timing uses HIP events recorded on the stream every kernel is launched
on (torch's current stream): the reported means time each series of calls as
one block (one event pair around back-to-back calls); percentiles come from a
second series with an event pair around each call; the prefill's per-kernel
times come from events the library records between its two kernels.  The CPU
oracle (test infrastructure) is timed on the host's cores as a reported
baseline.

Prints one JSON line.
"""
import argparse
import hashlib
import json
import os
import platform
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN prefill tokens/s/layer @T=4096 + decode state-update GB/s (% HBM peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD public specification
BF16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA, AMD public specification

T, H, D, C = 4096, 48, 128, 64
DEC_B, DEC_STEPS = 64, 256

# Algorithmic work (the method's own, per token and head, at C = 64, d = 128):
PREFILL_BYTES_PER_TOKEN_HEAD = 3 * D * 2 + 2 * 4 + D * 4        # q, k, v bf16 + g, beta + o fp32 = 1288
STATE_BYTES_PER_HEAD = D * D * 4                                  # 64 KiB
PREFILL_FLOP_PER_TOKEN_HEAD = 3 * (C - 1) * D + 2 * (C + 1) * D + 3 * 2 * D * D   # 139,136 (causal count)
PREFILL_FLOP_FULL_PER_TOKEN_HEAD = 5 * 2 * C * D + 3 * 2 * D * D                    # 180,224 (dense C x C tiles)
# split of the causal count between the two kernels
PREP_FLOP_PER_TOKEN_HEAD = (C - 1) * D + (C + 1) * D + 2 * (C - 1) * D             # K K^T, Q K^T, W, U~ = 32,512
CHAIN_FLOP_PER_TOKEN_HEAD = PREFILL_FLOP_PER_TOKEN_HEAD - PREP_FLOP_PER_TOKEN_HEAD  # 106,624
DECODE_BYTES_PER_HEAD_TOKEN = 2 * STATE_BYTES_PER_HEAD + 3 * D * 2 + 2 * 4 + D * 4  # 132,360
# pre-processing: raw q, k, v in (bf16) + two logits, q, k, v out (bf16) + g, beta
PRE_BYTES_PER_TOKEN_HEAD = 2 * (3 * D * 2 + 2 * 4)                                  # 1,552
PRE_BYTES_FIXED = 3 * H * D * 4 * 4 + 2 * 9 * H * D * 2                              # taps + conv state in/out
# the whole layer from the raw projections: raw q, k, v (bf16) + two logits in, o (fp32) out; the
# processed q, k, v the fused call also hands back (written once, read again by its chain) are extra
LAYER_BYTES_PER_TOKEN_HEAD = 3 * D * 2 + 2 * 4 + D * 4                              # 1,288
LAYER_QKV_ROUND_TRIP_PER_TOKEN_HEAD = 2 * 3 * D * 2                                 # 1,536


# Sources each measured kernel is built from: its HBM byte counts (profiles/traffic.json)
# stay valid while these files are unchanged.
KERNEL_SOURCES = {
    "k_chunk_prep": ("gdn_chunked.hip", "gdn_chunk_common.h", "gdn_mfma.h", "gdn_device.h", "gdn_conv.h"),
    "k_chunk_chain": ("gdn_chain.hip", "gdn_chunk_common.h", "gdn_mfma.h", "gdn_device.h", "../build.py"),
    "k_layer_prep": ("gdn_chunked.hip", "gdn_chunk_common.h", "gdn_mfma.h", "gdn_device.h", "gdn_conv.h"),
    "k_decode_step": ("gdn_rowstream.hip", "gdn_device.h"),
    "k_preprocess": ("gdn_preprocess.hip", "gdn_device.h", "gdn_conv.h"),
}


def source_hash(kernel):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_recurrence_gated_amd", "csrc")
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/), if the
    kernel's sources still match those the counters were taken on."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except ValueError:
        return None
    entry = data.get("kernels", {}).get(kernel)
    if entry is None or entry.get("source_hash") != source_hash(kernel):
        return None
    return entry.get("bytes_per_launch")


def run_conditions(torch):
    props = torch.cuda.get_device_properties(0)
    cond = {"gpu": props.name, "gcn_arch": getattr(props, "gcnArchName", ""),
            "compute_units": props.multi_processor_count, "torch": torch.__version__,
            "hip": torch.version.hip, "host": platform.node()}
    try:
        cond["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        pass
    return cond


def time_block(torch, fn, steps):
    """Mean ms per call of `steps` back-to-back calls fn(0) .. fn(steps - 1) on
    the current stream, bracketed by one pair of events with a synchronize on
    both sides (no event between the calls: an event record leaves the GPU
    idle for several microseconds).  Returns (ms per call, wall seconds)."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record()
    for i in range(steps):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps, time.perf_counter() - t0


# After an idle spell the GPU's clocks take tens of milliseconds of continuous
# work to settle: measured on the prefill, the first 10 ms of back-to-back
# calls ran at 197 us per call, the next at 181, then 172-173 from about 20 ms
# on.  Each measurement below is therefore preceded by SPIN_UP_S seconds of
# the same untimed calls (on top of the warm-up steps), so that it reports the
# steady state that a model running layer after layer sees.
SPIN_UP_S = 0.15


def spin_up(torch, fn, seconds=SPIN_UP_S):
    """Untimed calls fn(0), fn(1), ... in batches of 16 until `seconds` of
    wall time have passed; returns the number of calls."""
    torch.cuda.synchronize()
    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            fn(i)
            i += 1
        torch.cuda.synchronize()
    return i


def time_each(torch, fn, steps):
    """Sorted ms of `steps` calls fn(i), each bracketed by its own pair of
    events (for percentiles; includes the events' own idle time)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(ev):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in ev)


def bench_prefill(torch, gdn, w, steps, warmup, rotate):
    """Times `steps` prefill steps cycling over `rotate` resident copies of the
    inputs and outputs (rotate > 1 keeps the 256 MB last-level cache from
    serving one step's inputs to the next)."""
    inp = w.prefill_t4096_h48(T=T, H=H, d=D)
    dev = "cuda:0"
    q0 = w.to_torch(inp.q, "bf16", dev)
    k0 = w.to_torch(inp.k, "bf16", dev)
    v0 = w.to_torch(inp.v, "bf16", dev)
    g0 = torch.from_numpy(inp.g).to(dev)
    b0 = torch.from_numpy(inp.beta).to(dev)
    sets = []
    for r in range(rotate):
        sets.append({"q": q0.clone(), "k": k0.clone(), "v": v0.clone(), "g": g0.clone(), "beta": b0.clone(),
                     "o": torch.empty((T, H, D), dtype=torch.float32, device=dev),
                     "state": torch.empty((1, H, D, D), dtype=torch.float32, device=dev)})
    del q0, k0, v0, g0, b0
    ws = torch.empty(gdn.prefill_workspace_bytes(T, 1, H, D, D, gdn.GDN_BF16, gdn.CHUNK_64), dtype=torch.uint8,
                     device=dev)

    def call(x):  # S_0 = 0: no initial state (the kernels start from zeros)
        gdn.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], initial_state=None, final_state=x["state"],
                    out=x["o"], workspace=ws, chunk=gdn.CHUNK_64)

    def step(i):
        call(sets[i % rotate])

    spin_up(torch, step)
    for i in range(warmup):
        step(i)
    block_ms, wall = time_block(torch, step, steps)
    ms = time_each(torch, step, steps)
    # the prefill call alone, with events between its kernels (library marks):
    # [0] before the first kernel, [1] after the per-chunk preparation, [2] after the chain
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for m in marks:
        for e in m:
            e.record()  # creates the underlying hipEvent_t
    torch.cuda.synchronize()
    for i, m in enumerate(marks):
        gdn.prefill_set_marks(m)
        call(sets[i % rotate])
    torch.cuda.synchronize()
    ms_call = {"call": sorted(m[0].elapsed_time(m[2]) for m in marks),
               "k_chunk_prep": sorted(m[0].elapsed_time(m[1]) for m in marks),
               "k_chunk_chain": sorted(m[1].elapsed_time(m[2]) for m in marks)}
    return block_ms, ms, ms_call, wall


def bench_decode(torch, gdn, w, steps, rotate):
    """One pass of `steps` decode steps; step t updates state copy t % rotate
    (rotate > 1 stands for successive layers, each with its own state, so the
    192 MiB state is not served from the last-level cache)."""
    dec = w.decode_b64_h48(steps=steps, B=DEC_B, H=H, d=D)
    dev = "cuda:0"
    q = w.to_torch(dec.q, "bf16", dev)
    k = w.to_torch(dec.k, "bf16", dev)
    v = w.to_torch(dec.v, "bf16", dev)
    g = torch.from_numpy(dec.g).to(dev)
    beta = torch.from_numpy(dec.beta).to(dev)
    s0 = torch.from_numpy(dec.s_init).to(dev)
    states = [torch.empty_like(s0) for _ in range(rotate)]
    o = torch.empty((steps, DEC_B, H, D), dtype=torch.float32, device=dev)

    def init():
        for st in states:
            gdn.state_init(st, s0)

    def step(t):
        gdn.decode_step(q[t], k[t], v[t], g[t], beta[t], states[t % rotate], out=o[t])

    init()
    spin_up(torch, lambda t: step(t % steps))
    init()
    for t in range(steps):  # warm-up pass
        step(t)
    init()
    block_ms, _ = time_block(torch, step, steps)
    init()
    ms = time_each(torch, step, steps)
    return block_ms, ms


def bench_scan(torch, gdn, w, steps, warmup):
    """One sequence with few heads: the per-GPU share of the one-layer prefill
    when its 48 heads are split over 8 GPUs (H = 6, T = 4096), and the same at
    T = 16384; each timed with the one-chain form and with the chunk-level
    scan (back-to-back calls timed as a block, inputs resident).  Returns a dict."""
    import numpy as np
    dev = "cuda:0"
    out = {}
    for T_ in (T, 4 * T):
        inp = w.make_prefill([T_], H=6, d=D, seed=w.SEED_BASE + 7, packed=False)
        q, k, v = (w.to_torch(x, "bf16", dev) for x in (inp.q, inp.k, inp.v))
        g = torch.from_numpy(inp.g).to(dev)
        beta = torch.from_numpy(inp.beta).to(dev)
        row = {}
        for name, ch in (("chain", gdn.CHUNK_64_CHAIN), ("scan", gdn.CHUNK_64_SCAN)):
            o = torch.empty((T_, 6, D), dtype=torch.float32, device=dev)
            st = torch.empty((1, 6, D, D), dtype=torch.float32, device=dev)
            ws = torch.empty(gdn.prefill_workspace_bytes(T_, 1, 6, D, D, gdn.GDN_BF16, ch), dtype=torch.uint8,
                             device=dev)
            call = lambda: gdn.prefill(q, k, v, g, beta, chunk=ch, out=o, final_state=st, workspace=ws)
            spin_up(torch, lambda i: call())
            for _ in range(warmup):
                call()
            row[name + "_ms"], _ = time_block(torch, lambda i: call(), steps)
        row["speedup"] = row["chain_ms"] / row["scan_ms"]
        row["scan_tokens_per_s"] = T_ / (row["scan_ms"] / 1e3)
        out[f"H6_T{T_}"] = row
    return out


def bench_decode_slots(torch, gdn, w, steps, rotate):
    """Serving form of the decode step: the 64 rows of the batch take a fixed
    random permutation of 64 of the 128 slots of a state pool (one pool per
    layer, `rotate` layers), with no host-side slot check.  Timed eagerly, and
    as replays of one HIP graph that holds one step per pool (a decode
    iteration over `rotate` layers, as a server would capture it); returns
    (eager, graph), each (block ms per step, sorted per-call ms)."""
    import numpy as np
    dec = w.decode_b64_h48(steps=1, B=DEC_B, H=H, d=D)
    dev = "cuda:0"
    n_slots = 2 * DEC_B
    q = w.to_torch(dec.q[0], "bf16", dev)
    k = w.to_torch(dec.k[0], "bf16", dev)
    v = w.to_torch(dec.v[0], "bf16", dev)
    g = torch.from_numpy(dec.g[0]).to(dev)
    beta = torch.from_numpy(dec.beta[0]).to(dev)
    slots = torch.from_numpy(np.random.default_rng(7).permutation(n_slots)[:DEC_B].astype(np.int32)).to(dev)
    pools = [torch.zeros((n_slots, H, D, D), dtype=torch.float32, device=dev) for _ in range(rotate)]
    o = torch.empty((DEC_B, H, D), dtype=torch.float32, device=dev)

    def step(pool):
        gdn.decode_step_slots(q, k, v, g, beta, pool, slots, slots_host=None, out=o)

    def timed(fns):
        spin_up(torch, lambda t: fns[t % len(fns)]())
        fn = lambda t: fns[t % len(fns)]()
        return time_block(torch, fn, steps)[0], time_each(torch, fn, steps)

    eager = timed([lambda p=p: step(p) for p in pools])
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for pool in pools:
            step(pool)
    replays = max(1, steps // len(pools))
    spin_up(torch, lambda t: gr.replay())
    blk, _ = time_block(torch, lambda t: gr.replay(), replays)
    each = time_each(torch, lambda t: gr.replay(), replays)
    return eager, (blk / len(pools), [x / len(pools) for x in each])


def bench_preprocess(torch, gdn, w, steps, warmup, rotate):
    """gdn_preprocess over the one-layer prefill shape (T = 4096, H = 48,
    d = 128, bf16, SiLU, with conv state and gate bias); successive calls cycle
    over `rotate` resident copies of the inputs."""
    inp = w.make_preprocess([T], H=H, d=D, dtype="bf16", seed=w.SEED_BASE + 6, activation="silu", packed=False)
    dev = "cuda:0"
    f = lambda x: torch.from_numpy(x).to(dev)
    bf = lambda x: w.to_torch(x, "bf16", dev)
    sets = [dict(xq=bf(inp.xq), xk=bf(inp.xk), xv=bf(inp.xv), a=f(inp.a_logit), b=f(inp.b_logit),
                 st=bf(inp.state_in)) for _ in range(rotate)]
    wt, bias = f(inp.w), f(inp.bias)
    outs = [(torch.empty_like(s["xq"]), torch.empty_like(s["xk"]), torch.empty_like(s["xv"]),
             torch.empty((T, H), dtype=torch.float32, device=dev), torch.empty((T, H), dtype=torch.float32, device=dev))
            for s in sets]
    st_out = [torch.empty_like(s["st"]) for s in sets]

    def call(i):
        s = sets[i % rotate]
        gdn.preprocess(s["xq"], s["xk"], s["xv"], wt, s["a"], s["b"], gate_bias=bias, conv_state_in=s["st"],
                       conv_state_out=st_out[i % rotate], activation="silu", out=outs[i % rotate])

    spin_up(torch, call)
    for i in range(warmup):
        call(i)
    return time_block(torch, call, steps)[0], time_each(torch, call, steps)


def bench_layer(torch, gdn, w, steps, warmup, rotate):
    """gdn_layer_prefill over the one-layer prefill shape (T = 4096, H = 48,
    d = 128, bf16, SiLU, with conv state and gate bias, zero initial state),
    and the same work as two calls (gdn_preprocess, then gdn_prefill), each
    timed as a block over `rotate` resident copies of the raw inputs.  Returns
    (layer ms, two-call ms, per-kernel ms of the layer call from the library's
    marks)."""
    inp = w.make_preprocess([T], H=H, d=D, dtype="bf16", seed=w.SEED_BASE + 6, activation="silu", packed=False)
    dev = "cuda:0"
    f = lambda x: torch.from_numpy(x).to(dev)
    bf = lambda x: w.to_torch(x, "bf16", dev)
    sets = [dict(xq=bf(inp.xq), xk=bf(inp.xk), xv=bf(inp.xv), a=f(inp.a_logit), b=f(inp.b_logit),
                 st=bf(inp.state_in), o=torch.empty((T, H, D), dtype=torch.float32, device=dev),
                 s=torch.empty((1, H, D, D), dtype=torch.float32, device=dev)) for _ in range(rotate)]
    for x in sets:
        x["qkv"] = (torch.empty_like(x["xq"]), torch.empty_like(x["xk"]), torch.empty_like(x["xv"]))
        x["gb"] = (torch.empty((T, H), dtype=torch.float32, device=dev),
                   torch.empty((T, H), dtype=torch.float32, device=dev))
        x["st_out"] = torch.empty_like(x["st"])
    wt, bias = f(inp.w), f(inp.bias)
    ws = torch.empty(gdn.prefill_workspace_bytes(T, 1, H, D, D, gdn.GDN_BF16, gdn.CHUNK_64), dtype=torch.uint8,
                     device=dev)

    def layer(i):
        x = sets[i % rotate]
        gdn.layer_prefill(x["xq"], x["xk"], x["xv"], wt, x["a"], x["b"], gate_bias=bias, conv_state_in=x["st"],
                          conv_state_out=x["st_out"], activation="silu", out=x["o"], final_state=x["s"],
                          qkv=x["qkv"], workspace=ws, chunk=gdn.CHUNK_64)

    def two_calls(i):
        x = sets[i % rotate]
        q, k, v = x["qkv"]
        gdn.preprocess(x["xq"], x["xk"], x["xv"], wt, x["a"], x["b"], gate_bias=bias, conv_state_in=x["st"],
                       conv_state_out=x["st_out"], activation="silu", out=(q, k, v) + x["gb"])
        gdn.prefill(q, k, v, x["gb"][0], x["gb"][1], initial_state=None, final_state=x["s"], out=x["o"],
                    workspace=ws, chunk=gdn.CHUNK_64)

    res = []
    for fn in (layer, two_calls):
        spin_up(torch, fn)
        for i in range(warmup):
            fn(i)
        res.append(time_block(torch, fn, steps)[0])
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for m in marks:
        for e in m:
            e.record()
    torch.cuda.synchronize()
    for i, m in enumerate(marks):
        gdn.prefill_set_marks(m)
        layer(i)
    torch.cuda.synchronize()
    kern = {"k_layer_prep + k_conv_state": mean([m[0].elapsed_time(m[1]) for m in marks]),
            "k_chunk_chain": mean([m[1].elapsed_time(m[2]) for m in marks])}
    return res[0], res[1], kern


def layer_entry(layer_ms, two_ms, kern):
    """The whole layer from the raw projections at T = 4096, H = 48."""
    nbytes = LAYER_BYTES_PER_TOKEN_HEAD * T * H + PRE_BYTES_FIXED + STATE_BYTES_PER_HEAD * H
    design = nbytes + LAYER_QKV_ROUND_TRIP_PER_TOKEN_HEAD * T * H
    gbs = nbytes / (layer_ms / 1e3) / 1e9
    tl, tc = load_traffic("k_layer_prep"), load_traffic("k_chunk_chain")
    return {"workload": "gdn_layer_prefill: raw projections -> conv (4 taps) + SiLU + L2 norm + gate maps + "
                        "chunked prefill, T = 4096, H = 48, d = 128, bf16, conv state in/out, zero initial state",
            "mean_ms": layer_ms, "tokens_per_s_layer": T / (layer_ms / 1e3),
            "two_calls_mean_ms": two_ms, "two_calls_tokens_per_s_layer": T / (two_ms / 1e3),
            "kernels_ms": kern,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes": nbytes,
                         "bytes_with_qkv_round_trip": design,
                         "traffic": None if tl is None or tc is None else tl + tc}}


def bench_long_context(torch, gdn, w, runs):
    """Long-context prefill: 262,144 tokens (H = 48) as 16 segments of 16,384
    with the fp32 state carried from each call to the next, in place; inputs
    resident (all 16 segments).  Returns (sorted per-run ms, tokens)."""
    dev = "cuda:0"
    segs = []
    for seg in w.long_context_segments():
        segs.append((w.to_torch(seg.q, "bf16", dev), w.to_torch(seg.k, "bf16", dev), w.to_torch(seg.v, "bf16", dev),
                     torch.from_numpy(seg.g).to(dev), torch.from_numpy(seg.beta).to(dev)))
        del seg
    n = segs[0][0].shape[0]
    state = torch.zeros((1, H, D, D), dtype=torch.float32, device=dev)
    o = torch.empty((n, H, D), dtype=torch.float32, device=dev)
    ws = torch.empty(gdn.prefill_workspace_bytes(n, 1, H, D, D, gdn.GDN_BF16, gdn.CHUNK_64), dtype=torch.uint8,
                     device=dev)

    def one_run():
        state.zero_()
        for q, k, v, g, b in segs:
            gdn.prefill(q, k, v, g, b, initial_state=state, final_state=state, out=o, workspace=ws,
                        chunk=gdn.CHUNK_64)

    spin_up(torch, lambda i: one_run())
    times = []
    for _ in range(runs):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        one_run()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    # the same 262,144 tokens as one call (its workspace: the records of all 4,096 chunks per head)
    del ws, o
    cat = [torch.cat([sg[i] for sg in segs]) for i in range(5)]
    del segs
    N1 = cat[0].shape[0]
    o1 = torch.empty((N1, H, D), dtype=torch.float32, device=dev)
    ws1 = torch.empty(gdn.prefill_workspace_bytes(N1, 1, H, D, D, gdn.GDN_BF16, gdn.CHUNK_64), dtype=torch.uint8,
                      device=dev)
    one = lambda i: gdn.prefill(*cat, initial_state=None, final_state=state, out=o1, workspace=ws1,
                                chunk=gdn.CHUNK_64)
    one(0)
    one_shot = sorted(time_each(torch, one, 2))
    ws_bytes = ws1.numel()
    del cat, o1, ws1
    return sorted(times), N1, one_shot, ws_bytes


def bench_varlen(torch, gdn, w, steps, warmup):
    """Variable-length packed prefill: 8 sequences (130,093 tokens), H = 48,
    per-sequence initial states; back-to-back calls timed as a block."""
    inp = w.varlen_batch()
    dev = "cuda:0"
    q, k, v = (w.to_torch(x, inp.dtype, dev) for x in (inp.q, inp.k, inp.v))
    g, b = torch.from_numpy(inp.g).to(dev), torch.from_numpy(inp.beta).to(dev)
    s0 = torch.from_numpy(inp.s_init).to(dev)
    cu = inp.cu_seqlens
    cu_dev = torch.from_numpy(cu).to(dev)
    N, n_seq = q.shape[0], len(cu) - 1
    o = torch.empty((N, H, D), dtype=torch.float32, device=dev)
    s1 = torch.empty_like(s0)
    ws = torch.empty(gdn.prefill_workspace_bytes(N, n_seq, H, D, D, gdn.GDN_BF16, gdn.CHUNK_64), dtype=torch.uint8,
                     device=dev)
    call = lambda i: gdn.prefill(q, k, v, g, b, cu_seqlens=cu, cu_seqlens_device=cu_dev, initial_state=s0,
                                 final_state=s1, out=o, workspace=ws, chunk=gdn.CHUNK_64)
    spin_up(torch, call)
    for i in range(warmup):
        call(i)
    return time_block(torch, call, steps)[0], N, n_seq


def bench_fp32(torch, gdn, w, steps):
    """fp32 q/k/v at the one-layer shape (T = 4096, H = 48, d = 128): the
    token-serial kernel (the chunked kernels take bf16)."""
    inp = w.make_prefill([T], H=H, d=D, dtype="fp32", seed=w.SEED_BASE + 2, packed=False)
    dev = "cuda:0"
    q, k, v = (torch.from_numpy(x).to(dev) for x in (inp.q, inp.k, inp.v))
    g, b = torch.from_numpy(inp.g).to(dev), torch.from_numpy(inp.beta).to(dev)
    o = torch.empty((T, H, D), dtype=torch.float32, device=dev)
    st = torch.empty((1, H, D, D), dtype=torch.float32, device=dev)
    call = lambda i: gdn.prefill(q, k, v, g, b, out=o, final_state=st)
    assert gdn.prefill_algorithm(gdn.GDN_FP32, D, D) == gdn.CHUNK_SERIAL
    spin_up(torch, call)
    return time_block(torch, call, steps)[0]


def bench_plan(torch, gdn, w, reps):
    """Packed batches of 1,024 and 4,096 short sequences (H = 2): the planning
    kernel's cost shows in a kernel trace of this part."""
    import numpy as np
    dev = "cuda:0"
    out = {}
    for n_seq in (1024, 4096):
        lengths = np.random.default_rng(n_seq).integers(1, 200, size=n_seq).tolist()
        inp = w.make_prefill(lengths, H=2, d=D, seed=w.SEED_BASE + 9)
        q, k, v = (w.to_torch(x, "bf16", dev) for x in (inp.q, inp.k, inp.v))
        g, b = torch.from_numpy(inp.g).to(dev), torch.from_numpy(inp.beta).to(dev)
        cu_dev = torch.from_numpy(inp.cu_seqlens).to(dev)
        call = lambda i: gdn.prefill(q, k, v, g, b, cu_seqlens=inp.cu_seqlens, cu_seqlens_device=cu_dev,
                                     chunk=gdn.CHUNK_64)
        call(0)
        out[f"n_seq_{n_seq}_call_ms"] = time_block(torch, call, reps)[0]
    return out


def bench_copy(torch, gdn, mib, reps):
    """Calibration run for the HBM byte counters: gdn_state_init copying a
    state of about `mib` MiB (k_state_fill reads and writes each byte once)."""
    n = max(1, int(round(mib * 2 ** 20 / (H * D * D * 4))))
    src = torch.randn((n, H, D, D), dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        gdn.state_init(dst, src)
        b.record()
    torch.cuda.synchronize()
    if not torch.equal(dst, src):
        raise RuntimeError("copy calibration: state_init copy mismatch")
    ms = sum(a.elapsed_time(b) for a, b in evs) / reps
    nbytes = src.numel() * 4
    return {"only": "copy", "bytes_read": nbytes, "bytes_written": nbytes, "mean_ms": ms,
            "gbs": 2 * nbytes / (ms / 1e3) / 1e9}


def mean(xs):
    return sum(xs) / len(xs)


def pct(xs, p):
    i = min(len(xs) - 1, max(0, int(round(p / 100.0 * (len(xs) - 1)))))
    return xs[i]


def cpu_baseline(w, seconds):
    """The oracle as it stands on the host's cores, on the prefill workload
    (all 48 heads x 4096 tokens), repeated until `seconds` have elapsed."""
    import oracle
    from oracle import build as oracle_build
    if not os.path.exists(oracle.LIB_PATH):
        oracle_build.build()
    inp = w.prefill_t4096_h48(T=T, H=H, d=D)
    threads = oracle.default_threads()
    runs, t0 = 0, time.perf_counter()
    while True:
        oracle.run(inp.q, inp.k, inp.v, inp.g, inp.beta, None, None, threads=threads)
        runs += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next(line.split(":", 1)[1].strip() for line in f if line.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": runs * T / el, "unit": "tokens/s/layer", "cores": threads, "kind": "oracle",
            "sample": f"full prefill workload (B=1, H=48, T=4096, d=128) run {runs}x in double precision, "
                      f"{el:.1f} s wall on {threads} host threads",
            "gflops": runs * T * H * 6 * D * D / el / 1e9, "cpu_model": cpu_model}


def pre_entry(pre_block_ms, pre_ms):
    """Pre-processing (convolution, SiLU, norm, gate maps) at T = 4096, H = 48."""
    nbytes = PRE_BYTES_PER_TOKEN_HEAD * T * H + PRE_BYTES_FIXED
    ms = pre_block_ms
    gbs = nbytes / (ms / 1e3) / 1e9
    return {"mean_ms": ms, "p50_ms": pct(pre_ms, 50), "tokens_per_s_layer": T / (ms / 1e3),
            "roofline": {"kernel": "k_preprocess (one gdn_preprocess call; it returns the conv state itself)",
                         "bound": "hbm",
                         "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                         "algorithmic_bytes": nbytes, "traffic": load_traffic("k_preprocess")}}


def long_entry(run_ms, tokens, one_shot_ms=None, one_shot_ws=None):
    """The long-context prefill: 16 calls of 16,384 tokens, the state carried (read and written by each call)."""
    nbytes = PREFILL_BYTES_PER_TOKEN_HEAD * tokens * H + 16 * 2 * STATE_BYTES_PER_HEAD * H
    ms = mean(run_ms)
    gbs = nbytes / (ms / 1e3) / 1e9
    return {"workload": "262,144 tokens as 16 segments of 16,384, H = 48, d = 128, bf16, fp32 state carried "
                        "in place; 3 full runs", "run_ms": run_ms, "mean_ms": ms, "p50_ms": pct(run_ms, 50),
            "max_ms": max(run_ms), "one_call_ms": one_shot_ms, "one_call_workspace_bytes": one_shot_ws,
            "tokens_per_s_layer": tokens / (ms / 1e3), "hbm_floor_ms": nbytes / (HBM_PEAK_GBS * 1e9) * 1e3,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes": nbytes}}


def varlen_entry(ms, tokens, n_seq):
    """The varlen prefill: one call over the 8-sequence packed batch, initial and final states per sequence."""
    nbytes = PREFILL_BYTES_PER_TOKEN_HEAD * tokens * H + n_seq * 2 * STATE_BYTES_PER_HEAD * H
    gbs = nbytes / (ms / 1e3) / 1e9
    return {"workload": f"{n_seq} packed sequences, log-uniform lengths in [1024, 65536] ({tokens} tokens), H = 48, "
                        "d = 128, bf16, per-sequence initial states", "mean_ms": ms,
            "tokens_per_s_layer": tokens / (ms / 1e3), "hbm_floor_ms": nbytes / (HBM_PEAK_GBS * 1e9) * 1e3,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes": nbytes}}


def fp32_entry(ms):
    """fp32 q/k/v at T = 4096, H = 48: the token-serial kernel."""
    nbytes = (3 * D * 4 + 2 * 4 + D * 4) * T * H + 2 * STATE_BYTES_PER_HEAD * H
    gbs = nbytes / (ms / 1e3) / 1e9
    return {"workload": "B = 1, H = 48, T = 4096, d = 128, fp32 q/k/v (token-serial kernel)", "mean_ms": ms,
            "tokens_per_s_layer": T / (ms / 1e3), "achieved_gbs": gbs, "frac_hbm": gbs / HBM_PEAK_GBS}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=DEC_STEPS)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None,
                    help="comma list of parts to time alone (prefill, decode, decode_slots, preprocess, scan, long_context, "
                         "varlen, fp32, plan, layer, copy), one JSON line each, for profiling runs; 'copy' is the "
                         "byte-counter calibration copy")
    ap.add_argument("--warm", action="store_true",
                    help="also time one resident copy (inputs and state may then sit in the last-level cache)")
    ap.add_argument("--rotate", type=int, default=4,
                    help="resident copies of the inputs/states cycled through by successive steps")
    ap.add_argument("--copy-mib", type=float, default=1024.0, help="size of the calibration copy")
    ap.add_argument("--long-context-runs", type=int, default=3, help="full 16-segment runs of the long-context prefill")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the recurrence shards across heads and sequences with no "
              "exchange, so each GPU runs its own share independently (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    from linear_attention_recurrence_gated_amd import gdn
    from linear_attention_recurrence_gated_amd import workloads as w
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    gdn.lib()  # fail loudly if the HIP library is missing

    if args.only:
        parts = args.only.split(",")
        bad = [p for p in parts if p not in ("prefill", "decode", "decode_slots", "preprocess", "scan", "copy",
                                             "long_context", "varlen", "fp32", "plan", "layer")]
        if bad:
            ap.error(f"--only: unknown part(s) {bad}")
        for part in parts:
            if part == "prefill":
                block_ms, ms, ms_call, _ = bench_prefill(torch, gdn, w, args.steps, args.warmup, args.rotate)
                print(json.dumps({"only": "prefill", "ms_per_step": block_ms, "event_bracketed_mean_ms": mean(ms),
                                  **{k + "_mean_ms": mean(x) for k, x in ms_call.items()}}), flush=True)
            elif part == "decode":
                dec_block_ms, dec_ms = bench_decode(torch, gdn, w, args.decode_steps, args.rotate)
                print(json.dumps({"only": "decode", "ms_per_step": dec_block_ms,
                                  "event_bracketed_mean_ms": mean(dec_ms)}), flush=True)
            elif part == "decode_slots":
                (ds_block, ds_ms), (dg_block, dg_ms) = bench_decode_slots(torch, gdn, w, args.decode_steps,
                                                                          args.rotate)
                print(json.dumps({"only": "decode_slots", "ms_per_step": ds_block,
                                  "graph_replay_ms_per_step": dg_block}), flush=True)
            elif part == "scan":
                print(json.dumps({"only": "scan", **bench_scan(torch, gdn, w, args.steps, args.warmup)}), flush=True)
            elif part == "preprocess":
                pre_block, pre_ms = bench_preprocess(torch, gdn, w, args.steps, args.warmup, args.rotate)
                print(json.dumps({"only": "preprocess", "ms_per_call": pre_block,
                                  "event_bracketed_mean_ms": mean(pre_ms)}), flush=True)
            elif part == "long_context":
                lc_ms, lc_tok, lc_one, lc_ws = bench_long_context(torch, gdn, w, args.long_context_runs)
                print(json.dumps({"only": "long_context", "run_ms": lc_ms, "tokens": lc_tok, "one_call_ms": lc_one,
                                  "one_call_workspace_bytes": lc_ws}), flush=True)
            elif part == "varlen":
                vl_ms, vl_tok, _ = bench_varlen(torch, gdn, w, args.steps, args.warmup)
                print(json.dumps({"only": "varlen", "ms_per_call": vl_ms, "tokens": vl_tok}), flush=True)
            elif part == "fp32":
                print(json.dumps({"only": "fp32", "ms_per_call": bench_fp32(torch, gdn, w, max(3, args.steps // 10))}),
                      flush=True)
            elif part == "plan":
                print(json.dumps({"only": "plan", **bench_plan(torch, gdn, w, max(3, args.steps))}), flush=True)
            elif part == "layer":
                print(json.dumps({"only": "layer", **layer_entry(*bench_layer(torch, gdn, w, args.steps, args.warmup,
                                                                             args.rotate))}), flush=True)
            else:
                print(json.dumps(bench_copy(torch, gdn, args.copy_mib, max(1, args.steps))), flush=True)
        return
    block_ms, ms, ms_call, wall = bench_prefill(torch, gdn, w, args.steps, args.warmup, args.rotate)
    dec_block_ms, dec_ms = bench_decode(torch, gdn, w, args.decode_steps, args.rotate)
    pre_block, pre_ms = bench_preprocess(torch, gdn, w, args.steps, args.warmup, args.rotate)
    (ds_block, ds_ms), (dg_block, dg_ms) = bench_decode_slots(torch, gdn, w, args.decode_steps, args.rotate)
    scan = bench_scan(torch, gdn, w, min(args.steps, 20), args.warmup)
    lc_ms, lc_tok, lc_one, lc_ws = bench_long_context(torch, gdn, w, args.long_context_runs)
    vl_ms, vl_tok, vl_nseq = bench_varlen(torch, gdn, w, min(args.steps, 20), args.warmup)
    fp32_ms = bench_fp32(torch, gdn, w, 5)
    layer_ms, layer_two_ms, layer_kern = bench_layer(torch, gdn, w, args.steps, args.warmup, args.rotate)

    step_ms = block_ms
    tok_s = T / (step_ms / 1e3)
    prep_ms, chain_ms, call_ms = mean(ms_call["k_chunk_prep"]), mean(ms_call["k_chunk_chain"]), mean(ms_call["call"])
    prefill_bytes = PREFILL_BYTES_PER_TOKEN_HEAD * T * H + 2 * STATE_BYTES_PER_HEAD * H
    prefill_flop = PREFILL_FLOP_PER_TOKEN_HEAD * T * H
    kern_ms = prep_ms + chain_ms
    ach_gbs = prefill_bytes / (kern_ms / 1e3) / 1e9
    ach_tflops = prefill_flop / (call_ms / 1e3) / 1e12
    prep_tflops = PREP_FLOP_PER_TOKEN_HEAD * T * H / (prep_ms / 1e3) / 1e12
    chain_tflops = CHAIN_FLOP_PER_TOKEN_HEAD * T * H / (chain_ms / 1e3) / 1e12
    traffic = None
    tp, tc = load_traffic("k_chunk_prep"), load_traffic("k_chunk_chain")
    if tp is not None and tc is not None:
        traffic = tp + tc

    dec_step_ms = dec_block_ms
    dec_bytes = DECODE_BYTES_PER_HEAD_TOKEN * DEC_B * H
    dec_gbs = dec_bytes / (dec_step_ms / 1e3) / 1e9

    out = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "spin_up_s": SPIN_UP_S,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gated delta-rule prefill, 1 sequence x 4096 tokens, 48 heads, d_k=d_v=128, "
                               "bf16 q/k/v, fp32 g/beta/state/o, chunk 64; plus 256 decode steps on 64 "
                               "sequences x 48 heads; successive steps cycle over `rotate` resident copies",
                   "batch": 1, "seq_len": T, "heads": H, "head_dim": D, "chunk": C,
                   "decode_batch": DEC_B, "decode_steps": args.decode_steps, "state_dtype": "fp32"},
        "prefill": {"mean_ms": step_ms, "p50_ms": pct(ms, 50), "p95_ms": pct(ms, 95), "p99_ms": pct(ms, 99),
                    "event_bracketed_mean_ms": mean(ms),
                    "call_mean_ms": call_ms, "algorithmic_tflops": ach_tflops,
                    "mfma_frac": ach_tflops / BF16_MFMA_PEAK_TFLOPS,
                    "mfma_frac_full_tiles": PREFILL_FLOP_FULL_PER_TOKEN_HEAD * T * H / (call_ms / 1e3) / 1e12
                    / BF16_MFMA_PEAK_TFLOPS, "wall_s": wall,
                    "kernels": {
                        "k_chunk_prep": {"mean_ms": prep_ms, "p50_ms": pct(ms_call["k_chunk_prep"], 50),
                                         "algorithmic_tflops": prep_tflops,
                                         "mfma_frac": prep_tflops / BF16_MFMA_PEAK_TFLOPS,
                                         "traffic": tp},
                        "k_chunk_chain": {"mean_ms": chain_ms, "p50_ms": pct(ms_call["k_chunk_chain"], 50),
                                          "algorithmic_tflops": chain_tflops,
                                          "mfma_frac": chain_tflops / BF16_MFMA_PEAK_TFLOPS,
                                          "traffic": tc}}},
        "roofline": {"kernel": "k_chunk_prep + k_chunk_chain (the two launches of one gdn_prefill call, "
                               "timed live by library event marks)", "bound": "hbm",
                     "achieved": ach_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach_gbs / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes": prefill_bytes, "mean_ms": kern_ms},
        "decode": {"value": dec_gbs, "unit": "GB/s", "pct_hbm_peak": 100.0 * dec_gbs / HBM_PEAK_GBS,
                   "ms_per_step": dec_step_ms, "event_bracketed_mean_ms": mean(dec_ms),
                   "p50_ms": pct(dec_ms, 50), "p95_ms": pct(dec_ms, 95),
                   "p99_ms": pct(dec_ms, 99), "tokens_per_s_layer": DEC_B / (dec_step_ms / 1e3),
                   "roofline": {"kernel": "k_decode_step", "bound": "hbm", "achieved": dec_gbs,
                                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dec_gbs / HBM_PEAK_GBS,
                                "traffic": load_traffic("k_decode_step")}},
        "preprocess": pre_entry(pre_block, pre_ms),
        "scan": {"workload": "one sequence, H = 6 (48 heads over 8 GPUs), d = 128, bf16: one-chain form vs the "
                             "chunk-level scan", **scan},
        "decode_slots": {"ms_per_step": ds_block, "p50_ms": pct(ds_ms, 50), "p99_ms": pct(ds_ms, 99),
                         "value": dec_bytes / (ds_block / 1e3) / 1e9, "unit": "GB/s",
                         "frac_hbm_peak": dec_bytes / (ds_block / 1e3) / 1e9 / HBM_PEAK_GBS,
                         "graph_replay_ms_per_step": dg_block, "graph_replay_p50_ms": pct(dg_ms, 50),
                         "workload": "decode step at B = 64, H = 48, d = 128, 64 rows on a permutation of 64 of 128 pool slots; eager "
                                     "launches, and replays of one captured HIP graph holding one step per pool "
                                     "(per-step time = replay time / pools); each timed as a block"},
        "long_context": long_entry(lc_ms, lc_tok, lc_one, lc_ws),
        "varlen": varlen_entry(vl_ms, vl_tok, vl_nseq),
        "fp32_prefill": fp32_entry(fp32_ms),
        "layer": layer_entry(layer_ms, layer_two_ms, layer_kern),
        "rotate": args.rotate,
        "conditions": run_conditions(torch),
    }
    if args.warm:
        # the same with one resident copy (inputs and state may be served from the last-level cache)
        block_warm, _, ms_call_warm, _ = bench_prefill(torch, gdn, w, args.steps, args.warmup, 1)
        dec_block_warm, _ = bench_decode(torch, gdn, w, args.decode_steps, 1)
        out["warm_single_copy"] = {
            "prefill_ms_per_step": block_warm, "prefill_tokens_per_s_layer": T / (block_warm / 1e3),
            "k_chunk_prep_ms": mean(ms_call_warm["k_chunk_prep"]),
            "k_chunk_chain_ms": mean(ms_call_warm["k_chunk_chain"]),
            "decode_ms_per_step": dec_block_warm,
            "decode_gbs": dec_bytes / (dec_block_warm / 1e3) / 1e9}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
