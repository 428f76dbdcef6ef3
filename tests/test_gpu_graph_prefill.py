"""The chunked prefill captured once in a HIP graph and replayed: the library
plans on the host and launches kernels only (no allocation, no memset, no
synchronisation), so a capture with a preallocated workspace replays the
whole call.  Each replay, with new inputs copied into the captured buffers and
eager work on the stream between replays, equals an eager call on the same
inputs bit for bit, and the first matches the oracle."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, say, to_dev
import oracle
from linear_attention_recurrence_gated_amd import gdn
from linear_attention_recurrence_gated_amd import workloads as w
from parity import TOL_BF16, rel_max_err

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("lengths, H, chunk", [
    ([300, 0, 517], 4, gdn.CHUNK_64),          # varlen, the column-split chain
    ([2000], 2, gdn.CHUNK_64_SCAN),            # the chunk-level scan (segment plan written by a kernel)
    ([700, 900], 40, gdn.CHUNK_64),            # two-workgroup chain (many heads)
])
def test_prefill_graph_replays(oracle_lib, lengths, H, chunk):
    say("prefill graph capture:", lengths, "H =", H, "chunk", chunk)
    inps = [w.make_prefill(lengths, H=H, d=128, seed=600 + r + H, gate_shift=-1.0, init_std=0.2, packed=True)
            for r in range(3)]
    N, n = sum(lengths), len(lengths)
    cu_host = inps[0].cu_seqlens
    d0 = to_dev(inps[0])
    sq, sk, sv = d0["q"].clone(), d0["k"].clone(), d0["v"].clone()
    sg, sb, ss0 = d0["g"].clone(), d0["beta"].clone(), d0["s0"].clone()
    cu_dev = torch.from_numpy(cu_host).to(DEV)
    so = torch.empty((N, H, 128), dtype=torch.float32, device=DEV)
    sfin = torch.empty((n, H, 128, 128), dtype=torch.float32, device=DEV)
    ws = torch.empty(gdn.prefill_workspace_bytes(N, n, H, 128, 128, gdn.GDN_BF16, chunk), dtype=torch.uint8,
                     device=DEV)

    def call():
        gdn.prefill(sq, sk, sv, sg, sb, cu_seqlens=cu_host, cu_seqlens_device=cu_dev, initial_state=ss0,
                    out=so, final_state=sfin, workspace=ws, chunk=chunk)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()

    for r, inp in enumerate(inps):
        d = to_dev(inp)
        for dst, key in ((sq, "q"), (sk, "k"), (sv, "v"), (sg, "g"), (sb, "beta"), (ss0, "s0")):
            dst.copy_(d[key])
        so.fill_(float("nan"))
        sfin.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        o_e, s_e = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu_host,
                               initial_state=d["s0"], chunk=chunk)
        torch.cuda.synchronize()
        assert torch.equal(so, o_e) and torch.equal(sfin, s_e), f"replay {r} differs from the eager call"
        if r == 0:
            o_ref, s_ref = oracle.run(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, inp.s_init)
            eo, es = rel_max_err(so.cpu().numpy(), o_ref), rel_max_err(sfin.cpu().numpy(), s_ref)
            say(f"  replay 0 vs oracle: o={eo:.2e} state={es:.2e}")
            assert eo <= TOL_BF16 and es <= TOL_BF16
