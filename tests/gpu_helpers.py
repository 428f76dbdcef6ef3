"""Shared plumbing for the GPU parity tests: inputs to the device, oracle runs."""
import sys

import numpy as np
import torch

from linear_attention_recurrence_gated_amd import gdn
from linear_attention_recurrence_gated_amd import workloads as w

DEV = "cuda:0"


def say(*a):
    """Name the case being run on the GPU before running it (flushed)."""
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def to_dev(inp):
    """PrefillInputs -> dict of device tensors (the values the oracle also sees)."""
    d = dict(q=w.to_torch(inp.q, inp.dtype, DEV), k=w.to_torch(inp.k, inp.dtype, DEV),
             v=w.to_torch(inp.v, inp.dtype, DEV), g=torch.from_numpy(inp.g).to(DEV),
             beta=torch.from_numpy(inp.beta).to(DEV))
    d["s0"] = None if inp.s_init is None else torch.from_numpy(inp.s_init).to(DEV)
    d["cu"] = None if inp.cu_seqlens is None else inp.cu_seqlens
    return d


def gpu_prefill(inp, chunk=gdn.CHUNK_AUTO, initial_state="inputs"):
    d = to_dev(inp)
    s0 = d["s0"] if initial_state == "inputs" else initial_state
    o, s = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu"], initial_state=s0, chunk=chunk)
    torch.cuda.synchronize()
    return o.cpu().numpy(), s.cpu().numpy()


def oracle_prefill(inp, threads=None):
    import oracle
    return oracle.run(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, inp.s_init, threads=threads)
