"""The C ABI without a GPU: symbols, sizes and host-side validation.

Every call here fails validation on the host, so nothing is ever enqueued
(the pointers passed are never dereferenced).
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from linear_attention_recurrence_gated_amd import gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")
FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ["gdn_prefill", "gdn_decode_step", "gdn_state_init", "gdn_state_reset",
                 "gdn_state_bytes", "gdn_prefill_workspace_bytes", "gdn_status_string", "gdn_last_error",
                 "gdn_prefill_algorithm"]:
        assert want in names
    assert set(names) == set(gdn.SIGNATURES), "binding signatures and header disagree"


def test_library_exports_every_declared_symbol():
    L = gdn.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", gdn.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (gdn_\w+)", out))
    assert set(declared_functions()) <= exported


def test_state_bytes_reproduces_the_pages_144_mib():
    vals = {}
    for line in open(os.path.join(ROOT, "tests", "golden", "state_memory.txt")):
        line = line.split("#")[0].strip()
        if line:
            k, v = (x.strip() for x in line.split("="))
            vals[k] = int(v)
    per_layer = gdn.state_bytes(1, vals["heads"], vals["dk"], vals["dv"])
    assert per_layer * vals["layers"] == vals["total_bytes"] == 144 * 2 ** 20
    # no length argument at all: the state does not grow with context
    assert gdn.state_bytes(64, 48, 128, 128) == 64 * per_layer
    assert gdn.state_bytes(-1, 48, 128, 128) == 0 and gdn.state_bytes(1, 0, 128, 128) == 0


def test_status_strings():
    L = gdn.lib()
    for code, name in gdn.STATUS.items():
        assert L.gdn_status_string(code)
    assert L.gdn_status_string(12345) == b"unknown status"


def test_algorithm_choice():
    A = gdn.prefill_algorithm
    assert A(gdn.GDN_FP32, 16, 16, 0) == gdn.CHUNK_SERIAL
    assert A(gdn.GDN_FP32, 128, 128, gdn.CHUNK_64) == 0
    assert A(gdn.GDN_BF16, 100, 100, 0) == 0
    assert A(gdn.GDN_BF16, 128, 64, 0) == 0
    assert A(7, 128, 128, 0) == 0
    assert A(gdn.GDN_BF16, 128, 128, 17) == 0
    assert A(gdn.GDN_BF16, 128, 128, gdn.CHUNK_SERIAL) == gdn.CHUNK_SERIAL
    assert A(gdn.GDN_BF16, 128, 128, gdn.CHUNK_16) == gdn.CHUNK_16
    assert A(gdn.GDN_BF16, 128, 128, gdn.CHUNK_32) == gdn.CHUNK_32
    assert A(gdn.GDN_FP32, 128, 128, gdn.CHUNK_32) == 0
    assert A(gdn.GDN_BF16, 64, 64, gdn.CHUNK_16) == 0


def test_shorter_chunks_take_more_records():
    """The workspace holds one record per chunk: 16-token chunks need about
    four times the records of 64-token ones, and no scan area."""
    W = lambda c: gdn.prefill_workspace_bytes(4096, 1, 48, 128, 128, gdn.GDN_BF16, c)
    assert W(gdn.CHUNK_32) > 1.9 * W(gdn.CHUNK_64_CHAIN) and W(gdn.CHUNK_16) > 3.8 * W(gdn.CHUNK_64_CHAIN)


def _prefill(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=gdn.GDN_BF16, g=FAKE, beta=FAKE, cu=None, cu_host=None, n_seq=1,
             N=64, H=2, dk=16, dv=16, s0=None, o=FAKE * 64, s1=FAKE * 128, chunk=gdn.CHUNK_SERIAL, ws=None,
             ws_bytes=0)
    a.update(kw)
    L = gdn.lib()
    st = L.gdn_prefill(a["q"], a["k"], a["v"], a["dtype"], a["g"], a["beta"], a["cu"], a["cu_host"], a["n_seq"],
                       a["N"], a["H"], a["dk"], a["dv"], a["s0"], a["o"], a["s1"], a["chunk"], a["ws"],
                       a["ws_bytes"], a.get("variant", 0), None)
    return st, L.gdn_last_error().decode()


def _host(arr):
    return arr.ctypes.data_as(ctypes.c_void_p).value


@pytest.mark.parametrize("kw, code", [
    (dict(dtype=5), 3),
    (dict(H=0), 2),
    (dict(N=-1), 2),
    (dict(dk=100, dv=100), 7),
    (dict(dk=16, dv=32), 7),
    (dict(chunk=3), 7),
    (dict(q=None), 1),
    (dict(beta=None), 1),
    (dict(s1=None), 1),
    (dict(q=FAKE + 8), 4),
    (dict(g=FAKE + 2), 4),
    (dict(n_seq=2), 5),                      # no cu_seqlens but more than one sequence
    (dict(o=FAKE), 8),                       # o on top of q
    (dict(s1=FAKE), 8),                      # final state on top of q
    (dict(variant=4), 7),                    # unknown variant bit
    (dict(g=None, variant=2), 1),            # g is needed unless the gate is off
    (dict(g=None, variant=1, q=None), 1),    # without the gate g may be NULL, q may not
])
def test_prefill_validation(kw, code):
    st, msg = _prefill(**kw)
    assert st == code, (st, msg)
    assert msg


def test_prefill_seqlens_validation():
    bad = [np.array([0, 10, 5, 64], np.int32), np.array([1, 10, 20, 64], np.int32),
           np.array([0, 10, 20, 63], np.int32)]
    for cu in bad:
        st, msg = _prefill(cu=FAKE * 512, cu_host=_host(cu), n_seq=3)
        assert st == 5, msg
    good = np.array([0, 10, 20, 64], np.int32)
    st, msg = _prefill(cu=FAKE * 512, cu_host=None, n_seq=3)
    assert st == 1  # device offsets without the host copy
    st, msg = _prefill(cu=FAKE * 512, cu_host=_host(good), n_seq=3, q=None)
    assert st == 1


def test_decode_validation():
    L = gdn.lib()

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=gdn.GDN_BF16, g=FAKE, beta=FAKE, s=FAKE * 64, o=FAKE * 128, B=4,
                 H=2, dk=128, dv=128)
        a.update(kw)
        return L.gdn_decode_step(a["q"], a["k"], a["v"], a["dtype"], a["g"], a["beta"], a["s"], a["o"], a["B"],
                                 a["H"], a["dk"], a["dv"], a.get("variant", 0), None)

    assert call(dtype=9) == 3
    assert call(B=-1) == 2
    assert call(dk=96, dv=96) == 7
    assert call(s=None) == 1
    assert call(o=FAKE + 4) == 4
    assert call(o=FAKE) == 8
    assert call(s=FAKE) == 8
    assert call(B=0) == 0  # nothing to do, nothing enqueued
    assert call(variant=8) == 7
    assert call(g=None) == 1
    assert call(g=None, variant=1, o=FAKE) == 8  # g may be NULL without the gate; o on q still caught


def test_state_calls_validation():
    L = gdn.lib()
    assert L.gdn_state_init(None, 2, 4, 128, 128, None, None) == 1
    assert L.gdn_state_init(FAKE + 4, 2, 4, 128, 128, None, None) == 4
    assert L.gdn_state_init(FAKE, 2, 4, 128, 64, None, None) == 7
    assert L.gdn_state_init(FAKE, 2, 4, 128, 128, FAKE + 64, None) == 8
    assert L.gdn_state_init(FAKE, 0, 4, 128, 128, None, None) == 0
    assert L.gdn_state_reset(FAKE, 2, 4, 128, 128, FAKE, -1, None) == 2
    assert L.gdn_state_reset(None, 2, 4, 128, 128, None, 0, None) == 1


def test_workspace_sizes():
    assert gdn.prefill_workspace_bytes(4096, 1, 48, 128, 128, gdn.GDN_FP32, 0) == 0
    assert gdn.prefill_workspace_bytes(4096, 1, 48, 128, 128, gdn.GDN_BF16, gdn.CHUNK_SERIAL) == 0


def test_prefill_set_marks_validation():
    L = gdn.lib()
    arr = (ctypes.c_void_p * 4)()
    assert L.gdn_prefill_set_marks(arr, 4) == 2
    assert L.gdn_prefill_set_marks(arr, -1) == 2
    assert L.gdn_prefill_set_marks(None, 2) == 1
    assert L.gdn_prefill_set_marks(arr, 3) == 0  # all NULL: armed with nothing
    assert L.gdn_prefill_set_marks(None, 0) == 0


def _preprocess(**kw):
    # N=64 tokens, H=2, d=16 bf16: every tensor is 4 KiB, so the regions below are disjoint.
    a = dict(xq=FAKE, xk=FAKE * 2, xv=FAKE * 3, dtype=gdn.GDN_BF16, w=FAKE * 4, sin=None, sout=FAKE * 5,
             a=FAKE * 6, b=FAKE * 7, bias=None, cu=None, cu_host=None, n_seq=1, N=64, H=2, d=16, act=0,
             q=FAKE * 8, k=FAKE * 9, v=FAKE * 10, g=FAKE * 11, beta=FAKE * 12)
    a.update(kw)
    L = gdn.lib()
    st = L.gdn_preprocess(a["xq"], a["xk"], a["xv"], a["dtype"], a["w"], a["sin"], a["sout"], a["a"], a["b"],
                          a["bias"], a["cu"], a["cu_host"], a["n_seq"], a["N"], a["H"], a["d"], a["act"], a["q"],
                          a["k"], a["v"], a["g"], a["beta"], None)
    return st, L.gdn_last_error().decode()


@pytest.mark.parametrize("kw, code", [
    (dict(dtype=7), 3),
    (dict(H=0), 2),
    (dict(N=-3), 2),
    (dict(d=48), 7),
    (dict(act=2), 7),
    (dict(sout=None), 1),
    (dict(xk=None), 1),
    (dict(beta=None), 1),
    (dict(n_seq=2), 5),
    (dict(xq=FAKE + 8), 4),
    (dict(sin=FAKE * 13 + 4), 4),
    (dict(g=FAKE * 11 + 2), 4),
    (dict(q=FAKE), 8),                      # output q on top of input xq
    (dict(g=FAKE * 6), 8),                  # gate on top of its logit
    (dict(k=FAKE * 8), 8),                  # two outputs on one buffer
    (dict(sout=FAKE * 9), 8),               # conv state on top of output k
    (dict(sout=FAKE * 3), 8),               # conv state on top of input xv
    (dict(sin=FAKE * 5 + 16), 8),           # starting state partly overlapping the returned one
])
def test_preprocess_validation(kw, code):
    st, msg = _preprocess(**kw)
    assert st == code, (st, msg)
    assert msg


def test_preprocess_seqlens_validation():
    for cu in (np.array([0, 30, 20, 64], np.int32), np.array([0, 30, 40, 60], np.int32)):
        st, msg = _preprocess(cu=FAKE * 64, cu_host=_host(cu), n_seq=3)
        assert st == 5, msg
    st, _ = _preprocess(cu=FAKE * 64, cu_host=None, n_seq=3)
    assert st == 1
    empty = np.array([0], np.int32)
    st, _ = _preprocess(cu=FAKE * 64, cu_host=_host(empty), n_seq=0, N=0)
    assert st == 0  # nothing to do, nothing enqueued


def _decode_slots(**kw):
    # B = 4 rows, H = 2, d = 16, bf16: q, k, v 256 B each; the pool is 8 slots x 2 KiB
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, dtype=gdn.GDN_BF16, g=FAKE * 4, beta=FAKE * 5, pool=FAKE * 64,
             n_slots=8, slots=FAKE * 6, slots_host=None, o=FAKE * 7, B=4, H=2, dk=16, dv=16)
    a.update(kw)
    L = gdn.lib()
    st = L.gdn_decode_step_slots(a["q"], a["k"], a["v"], a["dtype"], a["g"], a["beta"], a["pool"], a["n_slots"],
                                 a["slots"], a["slots_host"], a["o"], a["B"], a["H"], a["dk"], a["dv"],
                                 a.get("variant", 0), None)
    return st, L.gdn_last_error().decode()


@pytest.mark.parametrize("kw, code", [
    (dict(dtype=4), 3),
    (dict(B=-1), 2),
    (dict(n_slots=-2), 2),
    (dict(dk=16, dv=32), 7),
    (dict(slots=None), 1),
    (dict(pool=None), 1),
    (dict(slots=FAKE * 6 + 2), 4),
    (dict(o=FAKE * 7 + 8), 4),
    (dict(o=FAKE * 6), 8),                   # o on top of slots
    (dict(pool=FAKE * 2), 8),                # pool on top of k
    (dict(variant=16), 7),
    (dict(g=None), 1),
])
def test_decode_slots_validation(kw, code):
    st, msg = _decode_slots(**kw)
    assert st == code, (st, msg)
    assert msg


def test_decode_slots_host_checks():
    for bad in ([0, 8, 1, 2], [0, -2, 1, 2], [3, 1, 3, -1]):   # out of range, below -1, a slot twice
        host = np.array(bad, np.int32)
        st, msg = _decode_slots(slots_host=_host(host))
        assert st == 10, msg
        assert gdn.lib().gdn_status_string(10).decode() == "invalid state slots"
    st, _ = _decode_slots(B=0)
    assert st == 0  # nothing to do, nothing enqueued


def test_scan_mode_validation():
    # the scan takes 1 to 64 sequences and at least one token
    cu = np.arange(66, dtype=np.int32) * 10
    st, msg = _prefill(chunk=gdn.CHUNK_64_SCAN, dtype=gdn.GDN_BF16, dk=128, dv=128, cu=FAKE * 512,
                       cu_host=_host(cu), n_seq=65, N=650)
    assert st == 7, msg
    st, msg = _prefill(chunk=gdn.CHUNK_64_SCAN, dtype=gdn.GDN_BF16, dk=128, dv=128, N=0)
    assert st == 7, msg
    # two sequences pass that check and stop at the missing workspace (nothing is launched)
    cu = np.array([0, 100, 300], np.int32)
    st, msg = _prefill(chunk=gdn.CHUNK_64_SCAN, dtype=gdn.GDN_BF16, dk=128, dv=128, cu=FAKE * 512,
                       cu_host=_host(cu), n_seq=2, N=300)
    assert st == 6, msg
    assert gdn.prefill_algorithm(gdn.GDN_BF16, 128, 128, gdn.CHUNK_64_SCAN) == gdn.CHUNK_64_SCAN
    assert gdn.prefill_algorithm(gdn.GDN_FP32, 128, 128, gdn.CHUNK_64_SCAN) == 0
    # room for the scan's states: asked for, or possibly chosen (few heads, no more
    # sequences than the segment budget 256 / (4 H))
    ws = lambda n_seq, H, chunk: gdn.prefill_workspace_bytes(4096, n_seq, H, 128, 128, gdn.GDN_BF16, chunk)
    state = 128 * 128 * 4
    assert ws(1, 4, gdn.CHUNK_64_SCAN) >= ws(1, 4, gdn.CHUNK_64_CHAIN) + 3 * 16 * 4 * state
    assert ws(2, 6, gdn.CHUNK_64) >= ws(2, 6, gdn.CHUNK_64_CHAIN) + 3 * 10 * 6 * state
    assert ws(11, 6, gdn.CHUNK_64) == ws(11, 6, gdn.CHUNK_64_CHAIN)   # more sequences than the budget of 10
    assert ws(11, 6, gdn.CHUNK_64_SCAN) >= ws(11, 6, gdn.CHUNK_64_CHAIN) + 3 * 11 * 6 * state
    assert ws(1, 17, gdn.CHUNK_64) == ws(1, 17, gdn.CHUNK_64_CHAIN)   # a budget below 4 segments
    assert ws(1, 16, gdn.CHUNK_64) > ws(1, 16, gdn.CHUNK_64_CHAIN)
    assert ws(65, 1, gdn.CHUNK_64) == ws(65, 1, gdn.CHUNK_64_CHAIN)
    assert ws(1, 4, gdn.CHUNK_64_SCAN) > \
        gdn.prefill_workspace_bytes(4096, 1, 4, 128, 128, gdn.GDN_BF16, gdn.CHUNK_64_CHAIN)


def test_launch_size_limits():
    """A call whose kernels would exceed 2^32 - 1 work-items in one launch is
    rejected (GDN_ERR_SHAPE) before anything is enqueued; one size below each
    limit passes the check (and fails later on the fake pointers instead)."""
    # chunked prefill: 4 column-split workgroups of 512 per (sequence, head), in groups of 8 pairs
    kw = dict(dk=128, dv=128, chunk=gdn.CHUNK_64, N=40000)
    st, msg = _prefill(n_seq=2097152 // 64 + 1, H=64, **kw)
    assert st == 2 and "exceed one launch" in msg, (st, msg)
    st, msg = _prefill(n_seq=2097144 // 8, H=8, **kw)
    assert st == 5, (st, msg)  # past the size check: no cu_seqlens for several sequences
    # token-serial prefill at d = 128: 16 workgroups of 64 per (sequence, head)
    kw = dict(dk=128, dv=128, dtype=gdn.GDN_FP32, chunk=gdn.CHUNK_SERIAL, N=64)
    st, msg = _prefill(n_seq=(1 << 22) // 16, H=16, **kw)
    assert st == 2 and "exceed one launch" in msg, (st, msg)
    st, msg = _prefill(n_seq=(1 << 22) // 16 - 1, H=16, **kw)
    assert st == 5, (st, msg)

    L = gdn.lib()

    def decode(B, H):
        L.gdn_last_error()
        return L.gdn_decode_step(FAKE, FAKE, FAKE, gdn.GDN_BF16, FAKE, FAKE, FAKE * 64, FAKE * 128, B, H, 128, 128,
                                 0, None)

    # d = 128: four workgroups of 256 work-items per head
    assert decode(1 << 21, 2) == 2       # 2^22 heads of 1,024 work-items
    assert decode((1 << 21) - 1, 2) == 8  # past the size check: o overlaps q
    # pre-processing, d = 128 bf16: 3 tensors x ceil(H/16) head groups x ceil(N/16) ranges, 256 work-items each
    st, msg = _preprocess(N=16 * ((1 << 24) // 3 + 1), H=16, d=128)
    assert st == 2 and "exceed one launch" in msg, (st, msg)
    st, msg = _preprocess(N=16 * ((1 << 24) // 3), H=16, d=128)
    assert st != 2, (st, msg)


def test_noalloc_refuses_sizes_beyond_its_scratch():
    """gdn_prefill_noalloc checks the workspace its sizes need against the
    fixed scratch array before any device call."""
    L = gdn.lib()
    limit = 128 << 20
    assert L.gdn_prefill_workspace_bytes(6912, 1, 48, 128, 128, gdn.GDN_BF16, gdn.CHUNK_64) <= limit
    assert L.gdn_prefill_workspace_bytes(6913, 1, 48, 128, 128, gdn.GDN_BF16, gdn.CHUNK_64) > limit
    st = L.gdn_prefill_noalloc(FAKE, FAKE, FAKE, gdn.GDN_BF16, FAKE, FAKE, None, None, 1, 6913, 48, 128, 128,
                               None, FAKE * 4096, FAKE * 8192, gdn.CHUNK_64, 0, None)
    assert gdn.STATUS[st] == "GDN_ERR_WORKSPACE"
    assert b"scratch" in L.gdn_last_error()


def test_layer_prefill_refuses_what_it_does_not_build():
    """The fused layer runs the chunked bf16 path with d = 128 only; other
    dtypes and head sizes are refused before any device call."""
    L = gdn.lib()
    cu = (ctypes.c_int32 * 2)(0, 64)
    args = lambda dtype, d, chunk: (FAKE, FAKE, FAKE, dtype, FAKE, None, FAKE * 2, gdn.GDN_ACT_SILU, FAKE, FAKE,
                                    None, FAKE * 3, cu, 1, 64, 4, d, None, FAKE * 4, FAKE * 5, FAKE * 6, FAKE * 7,
                                    FAKE * 8, None, None, chunk, None, 0, 0, None)
    for dtype, d, chunk in ((gdn.GDN_FP32, 128, gdn.CHUNK_AUTO), (gdn.GDN_BF16, 64, gdn.CHUNK_AUTO),
                            (gdn.GDN_BF16, 128, gdn.CHUNK_SERIAL)):
        st = L.gdn_layer_prefill(*args(dtype, d, chunk))
        assert gdn.STATUS[st] == "GDN_ERR_UNSUPPORTED", (dtype, d, chunk, gdn.STATUS[st])
        assert b"gdn_preprocess" in L.gdn_last_error()
