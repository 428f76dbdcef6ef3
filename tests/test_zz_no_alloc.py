"""gdn_prefill_noalloc (the library's fixed scratch array in place of a
workspace) against gdn_prefill with a caller workspace, through the C ABI:
two calls in a row, the second smaller, each equal bit for bit (the same
kernels run on the same inputs)."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, say, to_dev
from linear_attention_recurrence_gated_amd import gdn
from linear_attention_recurrence_gated_amd import workloads as w

pytestmark = pytest.mark.gpu


def _both(inp, chunk):
    d = to_dev(inp)
    o1, s1 = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu"], initial_state=d["s0"],
                         chunk=chunk)
    o2, s2 = gdn.prefill_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu"],
                                 initial_state=d["s0"], chunk=chunk)
    torch.cuda.synchronize()
    return (o1.cpu().numpy(), s1.cpu().numpy()), (o2.cpu().numpy(), s2.cpu().numpy())


@pytest.mark.parametrize("chunk", [gdn.CHUNK_64, gdn.CHUNK_64_SCAN])
def test_noalloc_equals_workspace_call_twice(chunk):
    # first call: one 4096-token sequence, 48 heads (the one-layer prefill shape; the scan form at 6 heads)
    H1 = 48 if chunk == gdn.CHUNK_64 else 6
    say("noalloc: 4096 tokens, H =", H1, "chunk", chunk)
    big = w.make_prefill([4096], H=H1, d=128, seed=401, gate_shift=-2.0, init_std=0.1, packed=False)
    (o1, s1), (o2, s2) = _both(big, chunk)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
    # second call, smaller: three packed sequences (one empty) with their own initial states
    say("noalloc: varlen [700, 0, 129], H = 8")
    small = w.make_prefill([700, 0, 129], H=8, d=128, seed=402, gate_shift=-1.0, init_std=0.2)
    (o1, s1), (o2, s2) = _both(small, chunk)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
    assert np.array_equal(s2[1], small.s_init[1])


def test_noalloc_refuses_sizes_beyond_the_scratch():
    inp = w.make_prefill([64], H=2, d=128, seed=403)
    d = to_dev(inp)
    limit = gdn.lib().gdn_prefill_workspace_bytes
    n = 7000  # 7000 tokens at H = 48 need more than the 128 MiB array
    assert limit(n, 1, 48, 128, 128, gdn.GDN_BF16, gdn.CHUNK_64) > 128 << 20
    q = torch.zeros((n, 48, 128), dtype=torch.bfloat16, device=DEV)
    gb = torch.full((n, 48), 0.5, dtype=torch.float32, device=DEV)
    with pytest.raises(gdn.GdnError) as e:
        gdn.prefill_noalloc(q, q, q, gb, gb, chunk=gdn.CHUNK_64)
    assert e.value.name == "GDN_ERR_WORKSPACE"
    # the library still works after the refusal
    (o1, s1), (o2, s2) = _both(inp, gdn.CHUNK_64)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
