#!/usr/bin/env python3
"""Benchmark of the gated delta-rule recurrence on one MI355X.

Metric: GDN prefill tokens/s/layer at T = 4096 (B = 1, H = 48, d = 128, bf16
q/k/v, fp32 gates/state/outputs, chunk 64), plus the decode step's state-update
bandwidth (B = 64, H = 48, d = 128, 256 in-place steps) as GB/s and % of the HBM
peak.  Inputs are seeded synthetic data already resident in HBM when timing
starts.

One timed step = gdn_state_init (zero the layer's state) + gdn_prefill over the
4096-token batch.  The decode half is timed as one pass of 256 gdn_decode_step
calls.  Timing uses HIP events recorded on the stream every kernel is launched
on (torch's current stream).  The CPU oracle (test infrastructure) is timed on
the host's cores as a reported baseline.

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
DECODE_BYTES_PER_HEAD_TOKEN = 2 * STATE_BYTES_PER_HEAD + 3 * D * 2 + 2 * 4 + D * 4  # 132,360


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_recurrence_gated_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/), if the
    kernel sources still match the build the counters were taken on."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except ValueError:
        return None
    if data.get("source_hash") != source_hash():
        return None
    entry = data.get("kernels", {}).get(kernel)
    return None if entry is None else entry.get("bytes_per_launch")


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


def bench_prefill(torch, gdn, w, steps, warmup):
    inp = w.config2(T=T, H=H, d=D)
    dev = "cuda:0"
    q = w.to_torch(inp.q, "bf16", dev)
    k = w.to_torch(inp.k, "bf16", dev)
    v = w.to_torch(inp.v, "bf16", dev)
    g = torch.from_numpy(inp.g).to(dev)
    beta = torch.from_numpy(inp.beta).to(dev)
    o = torch.empty((T, H, D), dtype=torch.float32, device=dev)
    state = torch.empty((1, H, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(gdn.prefill_workspace_bytes(T, 1, H, D, D, gdn.GDN_BF16, gdn.CHUNK_64), dtype=torch.uint8,
                     device=dev)

    def step():
        gdn.state_init(state)
        gdn.prefill(q, k, v, g, beta, initial_state=state, final_state=state, out=o, workspace=ws,
                    chunk=gdn.CHUNK_64)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for a, b in ev:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    # the prefill call alone (its kernels), for the roofline
    evp = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evp:
        a.record()
        gdn.prefill(q, k, v, g, beta, initial_state=state, final_state=state, out=o, workspace=ws,
                    chunk=gdn.CHUNK_64)
        b.record()
    torch.cuda.synchronize()
    ms_call = sorted(a.elapsed_time(b) for a, b in evp)
    return ms, ms_call, wall


def bench_decode(torch, gdn, w, steps):
    dec = w.config3(steps=steps, B=DEC_B, H=H, d=D)
    dev = "cuda:0"
    q = w.to_torch(dec.q, "bf16", dev)
    k = w.to_torch(dec.k, "bf16", dev)
    v = w.to_torch(dec.v, "bf16", dev)
    g = torch.from_numpy(dec.g).to(dev)
    beta = torch.from_numpy(dec.beta).to(dev)
    s0 = torch.from_numpy(dec.s_init).to(dev)
    state = torch.empty_like(s0)
    o = torch.empty((steps, DEC_B, H, D), dtype=torch.float32, device=dev)

    def one_pass(events=None):
        gdn.state_init(state, s0)
        for t in range(steps):
            if events is not None:
                events[t][0].record()
            gdn.decode_step(q[t], k[t], v[t], g[t], beta[t], state, out=o[t])
            if events is not None:
                events[t][1].record()

    one_pass()  # warm-up pass
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    one_pass(ev)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    return ms


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
    inp = w.config2(T=T, H=H, d=D)
    threads = oracle.default_threads()
    runs, t0 = 0, time.perf_counter()
    while True:
        oracle.run(inp.q, inp.k, inp.v, inp.g, inp.beta, None, None, threads=threads)
        runs += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": runs * T / el, "unit": "tokens/s/layer", "cores": threads, "kind": "oracle",
            "sample": f"full prefill workload (B=1, H=48, T=4096, d=128) run {runs}x in double precision, "
                      f"{el:.1f} s wall on {threads} host threads",
            "gflops": runs * T * H * 6 * D * D / el / 1e9}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=DEC_STEPS)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode"], default=None,
                    help="time one half only and print its numbers (for profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the recurrence shards across heads and sequences with no "
              "exchange, so multi-GPU runs are not part of this build (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    from linear_attention_recurrence_gated_amd import gdn
    from linear_attention_recurrence_gated_amd import workloads as w
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    gdn.lib()  # fail loudly if the HIP library is missing

    if args.only == "prefill":
        ms, ms_call, _ = bench_prefill(torch, gdn, w, args.steps, args.warmup)
        print(json.dumps({"only": "prefill", "ms_per_step": sum(ms) / len(ms),
                          "call_mean_ms": sum(ms_call) / len(ms_call)}), flush=True)
        return
    if args.only == "decode":
        dec_ms = bench_decode(torch, gdn, w, args.decode_steps)
        print(json.dumps({"only": "decode", "ms_per_step": sum(dec_ms) / len(dec_ms)}), flush=True)
        return
    ms, ms_call, wall = bench_prefill(torch, gdn, w, args.steps, args.warmup)
    dec_ms = bench_decode(torch, gdn, w, args.decode_steps)

    step_ms = sum(ms) / len(ms)
    tok_s = T / (step_ms / 1e3)
    call_ms = sum(ms_call) / len(ms_call)
    prefill_bytes = PREFILL_BYTES_PER_TOKEN_HEAD * T * H + 2 * STATE_BYTES_PER_HEAD * H
    prefill_flop = PREFILL_FLOP_PER_TOKEN_HEAD * T * H
    ach_gbs = prefill_bytes / (call_ms / 1e3) / 1e9
    ach_tflops = prefill_flop / (call_ms / 1e3) / 1e12

    dec_step_ms = sum(dec_ms) / len(dec_ms)
    dec_bytes = DECODE_BYTES_PER_HEAD_TOKEN * DEC_B * H
    dec_gbs = dec_bytes / (dec_step_ms / 1e3) / 1e9

    out = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gated delta-rule prefill, 1 sequence x 4096 tokens, 48 heads, d_k=d_v=128, "
                               "bf16 q/k/v, fp32 g/beta/state/o, chunk 64; plus 256 decode steps on 64 "
                               "sequences x 48 heads",
                   "batch": 1, "seq_len": T, "heads": H, "head_dim": D, "chunk": C,
                   "decode_batch": DEC_B, "decode_steps": args.decode_steps, "state_dtype": "fp32"},
        "prefill": {"p50_ms": pct(ms, 50), "p95_ms": pct(ms, 95), "p99_ms": pct(ms, 99), "mean_ms": step_ms,
                    "call_mean_ms": call_ms, "algorithmic_tflops": ach_tflops,
                    "mfma_frac": ach_tflops / BF16_MFMA_PEAK_TFLOPS, "wall_s": wall},
        "roofline": {"kernel": "gdn_prefill (k_chunk_prep + k_chunk_chain)", "bound": "hbm",
                     "achieved": ach_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach_gbs / HBM_PEAK_GBS,
                     "traffic": load_traffic("gdn_prefill")},
        "decode": {"value": dec_gbs, "unit": "GB/s", "pct_hbm_peak": 100.0 * dec_gbs / HBM_PEAK_GBS,
                   "ms_per_step": dec_step_ms, "p50_ms": pct(dec_ms, 50), "p95_ms": pct(dec_ms, 95),
                   "p99_ms": pct(dec_ms, 99), "tokens_per_s_layer": DEC_B / (dec_step_ms / 1e3),
                   "roofline": {"kernel": "k_decode_step", "bound": "hbm", "achieved": dec_gbs,
                                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dec_gbs / HBM_PEAK_GBS,
                                "traffic": load_traffic("k_decode_step")}},
        "conditions": run_conditions(torch),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
