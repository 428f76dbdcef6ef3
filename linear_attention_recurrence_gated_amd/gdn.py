"""Python binding of libgdn.so (argument marshalling only).

Every computation runs in the library's HIP kernels.  PyTorch only provides
device memory and the current stream.  There is no fallback: if libgdn.so is
missing or fails to load, every call raises.

Names mirror include/gdn.h:
    prefill(q, k, v, g, beta, cu_seqlens=None, initial_state=None, chunk=0) -> (o, final_state)
    prefill_noalloc(...)                               (the same with the library's fixed scratch)
    decode_step(q, k, v, g, beta, state) -> o          (state updated in place)
    decode_step_slots(q, k, v, g, beta, pool, slots) -> o   (slot b of the pool per row)
    state_init(state, init=None), state_reset(state, slots=None)
    preprocess(xq, xk, xv, conv_w, a_logit, b_logit, ...) -> (q, k, v, g, beta, conv_state)
    layer_prefill(xq, xk, xv, conv_w, a_logit, b_logit, ...) -> (o, final_state, conv_state, q, k, v)
    prefill_set_marks([ev0, ev1, ev2])                 (profiling hook)
    state_bytes(...), prefill_workspace_bytes(...), prefill_algorithm(...)
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdn.so")

GDN_BF16, GDN_FP32 = 0, 1
GDN_ACT_NONE, GDN_ACT_SILU = 0, 1
# variants (flags): the gated delta rule, no gate (g = 1), no erase term (linear-attention write)
GDN_VARIANT_GATED_DELTA, GDN_VARIANT_NO_GATE, GDN_VARIANT_NO_ERASE = 0, 1, 2
CHUNK_AUTO, CHUNK_SERIAL, CHUNK_64, CHUNK_64_CHAIN, CHUNK_64_SCAN = 0, 1, 64, 65, 66
CHUNK_16, CHUNK_32 = 16, 32

STATUS = {0: "GDN_OK", 1: "GDN_ERR_NULL", 2: "GDN_ERR_SHAPE", 3: "GDN_ERR_DTYPE", 4: "GDN_ERR_ALIGN",
          5: "GDN_ERR_SEQLENS", 6: "GDN_ERR_WORKSPACE", 7: "GDN_ERR_UNSUPPORTED", 8: "GDN_ERR_ALIAS",
          9: "GDN_ERR_HIP", 10: "GDN_ERR_SLOTS"}

# Every symbol include/gdn.h declares, with (restype, argtypes).
_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "gdn_state_bytes": (_sz, [_i64, _i32, _i32, _i32]),
    "gdn_prefill_algorithm": (_i32, [_i32, _i32, _i32, _i32]),
    "gdn_state_init": (_i32, [_vp, _i64, _i32, _i32, _i32, _vp, _vp]),
    "gdn_state_reset": (_i32, [_vp, _i64, _i32, _i32, _i32, _vp, _i32, _vp]),
    "gdn_prefill_workspace_bytes": (_sz, [_i64, _i64, _i32, _i32, _i32, _i32, _i32]),
    "gdn_prefill": (_i32, [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _i32,
                           _vp, _vp, _vp, _i32, _vp, _sz, _i32, _vp]),
    "gdn_decode_step": (_i32, [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _vp]),
    "gdn_decode_step_slots": (_i32, [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _i64, _i32, _i32,
                                     _i32, _i32, _vp]),
    "gdn_prefill_noalloc": (_i32, [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _i32,
                                   _vp, _vp, _vp, _i32, _i32, _vp]),
    "gdn_layer_prefill": (_i32, [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _i64, _i64,
                                 _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _sz, _i32, _vp]),
    "gdn_prefill_set_marks": (_i32, [ctypes.POINTER(_vp), _i32]),
    "gdn_preprocess": (_i32, [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i32, _i32,
                              _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "gdn_status_string": (ctypes.c_char_p, [_i32]),
    "gdn_last_error": (ctypes.c_char_p, []),
}


class GdnError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        self.name = STATUS.get(status, str(status))
        self.detail = detail
        super().__init__(f"{self.name}: {detail}")


_lib = None


def lib():
    """The loaded libgdn.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m linear_attention_recurrence_gated_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        L = lib()
        raise GdnError(status, L.gdn_last_error().decode(errors="replace"))


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_FP32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _dev_ptr(t, name, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(device, stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def state_bytes(n_seq, H, dk, dv):
    return int(lib().gdn_state_bytes(n_seq, H, dk, dv))


def prefill_algorithm(dtype_code, dk, dv, chunk=CHUNK_AUTO):
    return int(lib().gdn_prefill_algorithm(dtype_code, dk, dv, chunk))


def prefill_workspace_bytes(total_tokens, n_seq, H, dk, dv, dtype_code=GDN_BF16, chunk=CHUNK_AUTO):
    return int(lib().gdn_prefill_workspace_bytes(total_tokens, n_seq, H, dk, dv, dtype_code, chunk))


def state_init(state, init=None, stream=None):
    """Set state [n, H, dv, dk] (fp32) to a copy of `init`, or to zeros."""
    import torch
    n, H, dv, dk = state.shape
    _check(lib().gdn_state_init(_dev_ptr(state, "state", torch.float32), n, H, dk, dv,
                                _dev_ptr(init, "init", torch.float32), _stream(state.device, stream)))
    return state


def state_reset(state, slots=None, stream=None):
    """Zero the states of the sequences listed in `slots` (device int32), or all."""
    import torch
    n, H, dv, dk = state.shape
    n_slots = 0 if slots is None else slots.numel()
    _check(lib().gdn_state_reset(_dev_ptr(state, "state", torch.float32), n, H, dk, dv,
                                 _dev_ptr(slots, "slots", torch.int32), n_slots, _stream(state.device, stream)))
    return state


def prefill(q, k, v, g, beta, cu_seqlens=None, initial_state=None, chunk=CHUNK_AUTO,
            cu_seqlens_device=None, out=None, final_state=None, workspace=None, stream=None,
            variant=GDN_VARIANT_GATED_DELTA):
    """Chunkwise (or token-serial) prefill of a packed batch.

    q, k: [N, H, dk]; v: [N, H, dv] (bf16 or fp32, device); g, beta: [N, H] fp32.
    cu_seqlens: host offsets (list, numpy or CPU tensor) of the packed sequences,
    or None for one sequence; cu_seqlens_device: optional device int32 copy.
    initial_state: [n_seq, H, dv, dk] fp32 or None (zeros); it may be the same
    tensor as final_state.  variant: GDN_VARIANT_* flags (g may be None with
    GDN_VARIANT_NO_GATE).  Returns (o [N, H, dv] fp32, final_state).
    """
    import torch
    N, H, dk = k.shape
    dv = v.shape[2]
    dev = k.device
    if cu_seqlens is None:
        n_seq, cu_host, cu_dev = 1, None, None
    else:
        cu_host = np.ascontiguousarray(np.asarray(cu_seqlens.cpu() if torch.is_tensor(cu_seqlens) else cu_seqlens,
                                                  dtype=np.int32))
        n_seq = cu_host.shape[0] - 1
        cu_dev = cu_seqlens_device
        if cu_dev is None:
            cu_dev = torch.from_numpy(cu_host).to(dev)
    if out is None:
        out = torch.empty((N, H, dv), dtype=torch.float32, device=dev)
    if final_state is None:
        final_state = torch.empty((n_seq, H, dv, dk), dtype=torch.float32, device=dev)
    code = _dtype_code(k)
    for name, t in (("q", q), ("v", v)):
        if t.dtype != k.dtype:
            raise TypeError(f"{name} dtype {t.dtype} differs from k dtype {k.dtype}")
    ws_bytes = prefill_workspace_bytes(N, n_seq, H, dk, dv, code, chunk)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_ptr = _dev_ptr(workspace, "workspace") if ws_bytes else None
    ws_len = workspace.numel() * workspace.element_size() if (ws_bytes and workspace is not None) else 0
    cu_host_ptr = None if cu_host is None else cu_host.ctypes.data_as(ctypes.c_void_p)
    _check(lib().gdn_prefill(
        _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), code,
        _dev_ptr(g, "g", torch.float32), _dev_ptr(beta, "beta", torch.float32),
        _dev_ptr(cu_dev, "cu_seqlens_device", torch.int32), cu_host_ptr, n_seq, N, H, dk, dv,
        _dev_ptr(initial_state, "initial_state", torch.float32),
        _dev_ptr(out, "out", torch.float32), _dev_ptr(final_state, "final_state", torch.float32),
        chunk, ws_ptr, ws_len, variant, _stream(dev, stream)))
    return out, final_state


def prefill_noalloc(q, k, v, g, beta, cu_seqlens=None, initial_state=None, chunk=CHUNK_AUTO,
                    cu_seqlens_device=None, out=None, final_state=None, stream=None,
                    variant=GDN_VARIANT_GATED_DELTA):
    """prefill() through gdn_prefill_noalloc: the library's fixed per-device
    scratch array stands in for the workspace (no device allocation inside;
    pass out, final_state and cu_seqlens_device to allocate nothing here
    either).  Returns (o, final_state)."""
    import torch
    N, H, dk = k.shape
    dv = v.shape[2]
    dev = k.device
    n_seq, cu_host, cu_dev = _cu_pair(cu_seqlens, cu_seqlens_device, dev)
    if out is None:
        out = torch.empty((N, H, dv), dtype=torch.float32, device=dev)
    if final_state is None:
        final_state = torch.empty((n_seq, H, dv, dk), dtype=torch.float32, device=dev)
    code = _dtype_code(k)
    for name, t in (("q", q), ("v", v)):
        if t.dtype != k.dtype:
            raise TypeError(f"{name} dtype {t.dtype} differs from k dtype {k.dtype}")
    cu_host_ptr = None if cu_host is None else cu_host.ctypes.data_as(ctypes.c_void_p)
    _check(lib().gdn_prefill_noalloc(
        _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), code,
        _dev_ptr(g, "g", torch.float32), _dev_ptr(beta, "beta", torch.float32),
        _dev_ptr(cu_dev, "cu_seqlens_device", torch.int32), cu_host_ptr, n_seq, N, H, dk, dv,
        _dev_ptr(initial_state, "initial_state", torch.float32),
        _dev_ptr(out, "out", torch.float32), _dev_ptr(final_state, "final_state", torch.float32),
        chunk, variant, _stream(dev, stream)))
    return out, final_state


def prefill_set_marks(events):
    """Arm up to three torch.cuda.Event objects for the next prefill() on this
    thread: recorded before its first kernel, after the per-chunk kernels and
    after the state chain.  Each event must have been recorded once already
    (torch creates the underlying hipEvent_t lazily)."""
    for e in events:
        if e is not None and not e.cuda_event:
            e.record()
    handles = (_vp * max(3, len(events)))(*[e.cuda_event if e is not None else None for e in events])
    _check(lib().gdn_prefill_set_marks(handles, len(events)))


def decode_step(q, k, v, g, beta, state, out=None, stream=None, variant=GDN_VARIANT_GATED_DELTA):
    """One token per sequence: q, k [B, H, dk], v [B, H, dv], g, beta [B, H];
    state [B, H, dv, dk] fp32 updated in place.  variant: GDN_VARIANT_* flags.
    Returns o [B, H, dv] fp32."""
    import torch
    B, H, dk = k.shape
    dv = v.shape[2]
    if out is None:
        out = torch.empty((B, H, dv), dtype=torch.float32, device=k.device)
    _check(lib().gdn_decode_step(
        _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dtype_code(k),
        _dev_ptr(g, "g", torch.float32), _dev_ptr(beta, "beta", torch.float32),
        _dev_ptr(state, "state", torch.float32), _dev_ptr(out, "out", torch.float32),
        B, H, dk, dv, variant, _stream(k.device, stream)))
    return out


def _cu_pair(cu_seqlens, cu_seqlens_device, dev):
    import torch
    if cu_seqlens is None:
        return 1, None, None
    cu_host = np.ascontiguousarray(np.asarray(cu_seqlens.cpu() if torch.is_tensor(cu_seqlens) else cu_seqlens,
                                              dtype=np.int32))
    cu_dev = cu_seqlens_device if cu_seqlens_device is not None else torch.from_numpy(cu_host).to(dev)
    return cu_host.shape[0] - 1, cu_host, cu_dev


def preprocess(xq, xk, xv, conv_w, a_logit, b_logit, gate_bias=None, cu_seqlens=None, conv_state_in=None,
               conv_state_out=None, activation=GDN_ACT_NONE, cu_seqlens_device=None, out=None, stream=None):
    """Convolution (4 taps, causal, depthwise), optional SiLU, L2 norm of q and
    k, and the gate maps, in front of prefill() or decode_step().

    xq, xk, xv: [N, H, d] (bf16 or fp32, device); conv_w: [3, H, d, 4] fp32;
    a_logit, b_logit: [N, H] fp32; gate_bias: [H] fp32 or None.
    conv_state_in / conv_state_out: [n_seq, 3, 3, H, d] in the dtype of xq
    (None in: zeros; they may be the same tensor).  activation: GDN_ACT_NONE,
    GDN_ACT_SILU or "none" / "silu".  out: optional (q, k, v, g, beta).
    Returns (q, k, v, g, beta, conv_state_out).
    """
    import torch
    N, H, d = xk.shape
    dev = xk.device
    if isinstance(activation, str):
        activation = {"none": GDN_ACT_NONE, "silu": GDN_ACT_SILU}[activation]
    n_seq, cu_host, cu_dev = _cu_pair(cu_seqlens, cu_seqlens_device, dev)
    code = _dtype_code(xk)
    for name, t in (("xq", xq), ("xv", xv)):
        if t.dtype != xk.dtype:
            raise TypeError(f"{name} dtype {t.dtype} differs from xk dtype {xk.dtype}")
    if out is None:
        out = (torch.empty_like(xq), torch.empty_like(xk), torch.empty_like(xv),
               torch.empty((N, H), dtype=torch.float32, device=dev), torch.empty((N, H), dtype=torch.float32, device=dev))
    q, k, v, g, beta = out
    if conv_state_out is None:
        conv_state_out = torch.empty((n_seq, 3, 3, H, d), dtype=xk.dtype, device=dev)
    cu_host_ptr = None if cu_host is None else cu_host.ctypes.data_as(ctypes.c_void_p)
    _check(lib().gdn_preprocess(
        _dev_ptr(xq, "xq"), _dev_ptr(xk, "xk"), _dev_ptr(xv, "xv"), code,
        _dev_ptr(conv_w, "conv_w", torch.float32), _dev_ptr(conv_state_in, "conv_state_in", xk.dtype),
        _dev_ptr(conv_state_out, "conv_state_out", xk.dtype), _dev_ptr(a_logit, "a_logit", torch.float32),
        _dev_ptr(b_logit, "b_logit", torch.float32), _dev_ptr(gate_bias, "gate_bias", torch.float32),
        _dev_ptr(cu_dev, "cu_seqlens_device", torch.int32), cu_host_ptr, n_seq, N, H, d, activation,
        _dev_ptr(q, "q", xk.dtype), _dev_ptr(k, "k", xk.dtype), _dev_ptr(v, "v", xk.dtype),
        _dev_ptr(g, "g", torch.float32), _dev_ptr(beta, "beta", torch.float32), _stream(dev, stream)))
    return q, k, v, g, beta, conv_state_out


def layer_prefill(xq, xk, xv, conv_w, a_logit, b_logit, gate_bias=None, cu_seqlens=None, conv_state_in=None,
                  conv_state_out=None, activation=GDN_ACT_NONE, initial_state=None, chunk=CHUNK_AUTO,
                  cu_seqlens_device=None, out=None, final_state=None, qkv=None, gates=None, workspace=None,
                  stream=None, variant=GDN_VARIANT_GATED_DELTA):
    """gdn_layer_prefill: the pre-processing and the chunked prefill in one
    call from the raw projections (bf16, d = 128).

    Arguments as for preprocess() and prefill(); qkv: optional (q, k, v)
    output buffers for the processed inputs; gates: optional (g, beta) outputs
    (not formed when None).  Returns (o, final_state, conv_state_out, q, k, v).
    """
    import torch
    N, H, d = xk.shape
    dev = xk.device
    if isinstance(activation, str):
        activation = {"none": GDN_ACT_NONE, "silu": GDN_ACT_SILU}[activation]
    n_seq, cu_host, cu_dev = _cu_pair(cu_seqlens, cu_seqlens_device, dev)
    code = _dtype_code(xk)
    for name, t in (("xq", xq), ("xv", xv)):
        if t.dtype != xk.dtype:
            raise TypeError(f"{name} dtype {t.dtype} differs from xk dtype {xk.dtype}")
    if out is None:
        out = torch.empty((N, H, d), dtype=torch.float32, device=dev)
    if final_state is None:
        final_state = torch.empty((n_seq, H, d, d), dtype=torch.float32, device=dev)
    if conv_state_out is None:
        conv_state_out = torch.empty((n_seq, 3, 3, H, d), dtype=xk.dtype, device=dev)
    if qkv is None:
        qkv = (torch.empty_like(xq), torch.empty_like(xk), torch.empty_like(xv))
    q, k, v = qkv
    g, beta = (None, None) if gates is None else gates
    ws_bytes = prefill_workspace_bytes(N, n_seq, H, d, d, code, chunk)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_ptr = _dev_ptr(workspace, "workspace") if ws_bytes else None
    ws_len = workspace.numel() * workspace.element_size() if (ws_bytes and workspace is not None) else 0
    cu_host_ptr = None if cu_host is None else cu_host.ctypes.data_as(ctypes.c_void_p)
    _check(lib().gdn_layer_prefill(
        _dev_ptr(xq, "xq"), _dev_ptr(xk, "xk"), _dev_ptr(xv, "xv"), code,
        _dev_ptr(conv_w, "conv_w", torch.float32), _dev_ptr(conv_state_in, "conv_state_in", xk.dtype),
        _dev_ptr(conv_state_out, "conv_state_out", xk.dtype), activation,
        _dev_ptr(a_logit, "a_logit", torch.float32), _dev_ptr(b_logit, "b_logit", torch.float32),
        _dev_ptr(gate_bias, "gate_bias", torch.float32),
        _dev_ptr(cu_dev, "cu_seqlens_device", torch.int32), cu_host_ptr, n_seq, N, H, d,
        _dev_ptr(initial_state, "initial_state", torch.float32), _dev_ptr(out, "out", torch.float32),
        _dev_ptr(final_state, "final_state", torch.float32),
        _dev_ptr(q, "q", xk.dtype), _dev_ptr(k, "k", xk.dtype), _dev_ptr(v, "v", xk.dtype),
        _dev_ptr(g, "g", torch.float32), _dev_ptr(beta, "beta", torch.float32),
        chunk, ws_ptr, ws_len, variant, _stream(dev, stream)))
    return out, final_state, conv_state_out, q, k, v


def decode_step_slots(q, k, v, g, beta, state_pool, slots, slots_host="auto", out=None, stream=None,
                      variant=GDN_VARIANT_GATED_DELTA):
    """One token for each of B requests; row b updates state_pool[slots[b]]
    ([n_slots, H, dv, dk] fp32) in place; slots[b] = -1 marks a padding row
    (o row zeroed).  slots: device int32 [B].  slots_host: "auto" copies slots
    to the host for validation (a synchronising copy), None skips it (for graph
    capture), or a host array given by the caller.  Returns o [B, H, dv] fp32."""
    import torch
    B, H, dk = k.shape
    dv = v.shape[2]
    n_slots = state_pool.shape[0]
    if out is None:
        out = torch.empty((B, H, dv), dtype=torch.float32, device=k.device)
    if isinstance(slots_host, str):
        slots_host = slots.cpu().numpy()
    host = None
    if slots_host is not None:
        host = np.ascontiguousarray(np.asarray(slots_host, dtype=np.int32))
        if host.shape != (B,):
            raise ValueError(f"slots_host must have shape ({B},)")
    _check(lib().gdn_decode_step_slots(
        _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dtype_code(k),
        _dev_ptr(g, "g", torch.float32), _dev_ptr(beta, "beta", torch.float32),
        _dev_ptr(state_pool, "state_pool", torch.float32), n_slots, _dev_ptr(slots, "slots", torch.int32),
        None if host is None else host.ctypes.data_as(ctypes.c_void_p),
        _dev_ptr(out, "out", torch.float32), B, H, dk, dv, variant, _stream(k.device, stream)))
    return out
