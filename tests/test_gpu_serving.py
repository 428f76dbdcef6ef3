"""Serving-form decode on the GPU: per-row state slots in a pool, reset on
reassignment, padding rows, and the step captured in a HIP graph.  Parity
against the CPU oracle run on each request's own token sequence."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, say
from linear_attention_recurrence_gated_amd import gdn
from linear_attention_recurrence_gated_amd import workloads as w
from parity import TOL_BF16, rel_max_err

pytestmark = pytest.mark.gpu

H, D = 4, 128


def dev_bf16(x):
    return w.to_torch(np.ascontiguousarray(x), "bf16", DEV)


def dev_f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def test_slots_match_the_oracle_on_gathered_states(oracle_lib):
    import oracle
    say("decode_step_slots one step, pool of 10")
    n_slots, slots = 10, np.array([7, 2, -1, 9, 0, 4], np.int32)
    B = len(slots)
    dec = w.make_decode(1, B, H, D, seed=51, init_std=0.3)
    pool0 = (0.3 * np.random.default_rng(52).standard_normal((n_slots, H, D, D))).astype(np.float32)
    pool = dev_f32(pool0)
    o = gdn.decode_step_slots(dev_bf16(dec.q[0]), dev_bf16(dec.k[0]), dev_bf16(dec.v[0]), dev_f32(dec.g[0]),
                              dev_f32(dec.beta[0]), pool, torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    o, pool1 = o.cpu().numpy(), pool.cpu().numpy()
    live = np.flatnonzero(slots >= 0)
    o_ref, s_ref = oracle.run_decode(dec.q[:, live], dec.k[:, live], dec.v[:, live], dec.g[:, live],
                                     dec.beta[:, live], pool0[slots[live]])
    eo, es = rel_max_err(o[live], o_ref[0]), rel_max_err(pool1[slots[live]], s_ref)
    say(f"  errors o={eo:.2e} state={es:.2e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16
    assert np.all(o[slots < 0] == 0.0)
    untouched = sorted(set(range(n_slots)) - set(slots[live].tolist()))
    assert np.array_equal(pool1[untouched], pool0[untouched])


def schedule(n_req=14, max_rows=6, seed=53):
    """Requests (id, arrival step, length) and, per step, the rows of the batch
    as (request, position), with slots from a free list (lowest first) that are
    reset when handed to a new request."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(1, 24, size=n_req)
    arrivals = np.sort(rng.integers(0, 30, size=n_req))
    n_slots = 8
    free = list(range(n_slots))
    active = {}            # request -> [slot, position]
    steps = []
    t, pending = 0, list(range(n_req))
    while pending or active:
        resets = []
        while pending and arrivals[pending[0]] <= t and len(active) < max_rows and free:
            r = pending.pop(0)
            slot = free.pop(0)
            active[r] = [slot, 0]
            resets.append(slot)
        rows = [(r, sp[1], sp[0]) for r, sp in sorted(active.items())]
        steps.append((resets, rows))
        for r in list(active):
            active[r][1] += 1
            if active[r][1] == lengths[r]:
                free.append(active.pop(r)[0])
                free.sort()
        t += 1
    return lengths, n_slots, steps


def request_inputs(lengths):
    return [w.make_prefill([int(n)], H=H, d=D, seed=600 + r, gate_shift=-1.0, packed=False)
            for r, n in enumerate(lengths)]


def batch_arrays(reqs, rows, B):
    """Stack row (request, position) token inputs; pad to B rows with slot -1."""
    q = np.zeros((B, H, D), np.float32)
    k, v = np.zeros_like(q), np.zeros_like(q)
    g, beta = np.ones((B, H), np.float32), np.zeros((B, H), np.float32)
    slots = np.full(B, -1, np.int32)
    for i, (r, pos, slot) in enumerate(rows):
        inp = reqs[r]
        q[i], k[i], v[i], g[i], beta[i] = inp.q[pos], inp.k[pos], inp.v[pos], inp.g[pos], inp.beta[pos]
        slots[i] = slot
    return q, k, v, g, beta, slots


def check_requests(reqs, outs, finals):
    import oracle
    worst_o = worst_s = 0.0
    for r, inp in enumerate(reqs):
        o_ref, s_ref = oracle.run(inp.q, inp.k, inp.v, inp.g, inp.beta)
        worst_o = max(worst_o, rel_max_err(np.stack(outs[r]), o_ref))
        worst_s = max(worst_s, rel_max_err(finals[r], s_ref[0]))
    say(f"  worst request errors o={worst_o:.2e} state={worst_s:.2e}")
    assert worst_o <= TOL_BF16 and worst_s <= TOL_BF16


def test_serving_trace_with_slot_reuse(oracle_lib):
    """Requests arrive, decode token by token in a shared batch, finish, and
    hand their slots to later requests (reset first).  Each request's outputs
    and final state equal the oracle run over its own tokens from a zero state."""
    lengths, n_slots, steps = schedule()
    reqs = request_inputs(lengths)
    say("serving trace:", len(reqs), "requests,", len(steps), "steps")
    B = 6
    pool = dev_f32(np.full((n_slots, H, D, D), 7.0, np.float32))  # garbage until reset
    outs = {r: [] for r in range(len(reqs))}
    finals = {}
    for resets, rows in steps:
        if resets:
            gdn.state_reset(pool, slots=torch.tensor(resets, dtype=torch.int32, device=DEV))
        q, k, v, g, beta, slots = batch_arrays(reqs, rows, B)
        o = gdn.decode_step_slots(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_f32(g), dev_f32(beta), pool,
                                  torch.from_numpy(slots).to(DEV), slots_host=slots)
        o = o.cpu().numpy()
        assert np.all(o[len(rows):] == 0.0)
        for i, (r, pos, slot) in enumerate(rows):
            outs[r].append(o[i])
            if pos == lengths[r] - 1:
                finals[r] = pool[slot].cpu().numpy()
    check_requests(reqs, outs, finals)


def test_graph_capture_of_reset_and_step(oracle_lib):
    """gdn_state_reset + gdn_decode_step_slots captured once in a HIP graph and
    replayed for every step of the serving trace, with the step's inputs,
    slots and resets copied into the graph's static buffers between replays.
    Each replay's output equals the eager step's, and the requests match the
    oracle."""
    lengths, n_slots, steps = schedule(seed=54)
    reqs = request_inputs(lengths)
    B = 6
    say("graph capture:", len(steps), "replays")
    pool_g = dev_f32(np.full((n_slots, H, D, D), 7.0, np.float32))
    pool_e = pool_g.clone()
    sq = torch.zeros((B, H, D), dtype=torch.bfloat16, device=DEV)
    sk, sv = torch.zeros_like(sq), torch.zeros_like(sq)
    sg = torch.ones((B, H), dtype=torch.float32, device=DEV)
    sb = torch.zeros((B, H), dtype=torch.float32, device=DEV)
    sslots = torch.full((B,), -1, dtype=torch.int32, device=DEV)
    sresets = torch.full((B,), -1, dtype=torch.int32, device=DEV)
    so = torch.empty((B, H, D), dtype=torch.float32, device=DEV)

    def step():
        gdn.state_reset(pool_g, slots=sresets)
        gdn.decode_step_slots(sq, sk, sv, sg, sb, pool_g, sslots, slots_host=None, out=so)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up outside the graph (all slots -1: no state touched)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    outs = {r: [] for r in range(len(reqs))}
    finals = {}
    for n, (resets, rows) in enumerate(steps):
        q, k, v, g, beta, slots = batch_arrays(reqs, rows, B)
        rs = np.full(B, -1, np.int32)
        rs[:len(resets)] = resets
        sq.copy_(dev_bf16(q)); sk.copy_(dev_bf16(k)); sv.copy_(dev_bf16(v))
        sg.copy_(dev_f32(g)); sb.copy_(dev_f32(beta))
        sslots.copy_(torch.from_numpy(slots).to(DEV)); sresets.copy_(torch.from_numpy(rs).to(DEV))
        torch.cuda.synchronize()
        graph.replay()
        # the same step eagerly on the second pool
        if resets:
            gdn.state_reset(pool_e, slots=torch.tensor(resets, dtype=torch.int32, device=DEV))
        o_e = gdn.decode_step_slots(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_f32(g), dev_f32(beta), pool_e,
                                    torch.from_numpy(slots).to(DEV), slots_host=slots)
        torch.cuda.synchronize()
        assert torch.equal(so, o_e), f"replay {n}: output differs from the eager step"
        o = so.cpu().numpy()
        for i, (r, pos, slot) in enumerate(rows):
            outs[r].append(o[i])
            if pos == lengths[r] - 1:
                finals[r] = pool_g[slot].cpu().numpy()
    assert torch.equal(pool_g, pool_e)
    check_requests(reqs, outs, finals)


def test_full_decode_size_with_permuted_slots(oracle_lib):
    """The batched-decode shape (B = 64, H = 48, d = 128; the state streams
    with non-temporal accesses at this size) over a pool of 80 slots: rows take
    a random permutation of slots, four rows are padding."""
    import oracle
    say("decode_step_slots B=64 H=48, pool of 80")
    Hf, B, n_slots = 48, 64, 80
    rng = np.random.default_rng(55)
    slots = rng.permutation(n_slots)[:B].astype(np.int32)
    slots[[3, 17, 40, 63]] = -1
    dec = w.make_decode(1, B, Hf, D, seed=56, init_std=0.02)
    pool0 = (0.02 * rng.standard_normal((n_slots, Hf, D, D), dtype=np.float32)).astype(np.float32)
    pool = dev_f32(pool0)
    o = gdn.decode_step_slots(dev_bf16(dec.q[0]), dev_bf16(dec.k[0]), dev_bf16(dec.v[0]), dev_f32(dec.g[0]),
                              dev_f32(dec.beta[0]), pool, torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    o, pool1 = o.cpu().numpy(), pool.cpu().numpy()
    live = np.flatnonzero(slots >= 0)
    o_ref, s_ref = oracle.run_decode(dec.q[:, live], dec.k[:, live], dec.v[:, live], dec.g[:, live],
                                     dec.beta[:, live], pool0[slots[live]])
    eo, es = rel_max_err(o[live], o_ref[0]), rel_max_err(pool1[slots[live]], s_ref)
    say(f"  errors o={eo:.2e} state={es:.2e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16
    assert np.all(o[slots < 0] == 0.0)
    untouched = sorted(set(range(n_slots)) - set(slots[live].tolist()))
    assert np.array_equal(pool1[untouched], pool0[untouched])
