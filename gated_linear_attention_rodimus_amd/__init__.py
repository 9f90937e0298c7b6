"""MI355X (gfx950) DDTS gated linear-attention recurrence of Rodimus.

Thin Python binding over the C ABI of ``librodimus_ddts.so`` (declared in
``include/rodimus_ddts.h``).  This module only marshals arguments: it checks
tensor shapes/dtypes/devices, allocates the outputs and the workspace with
torch, and passes raw device pointers and the current HIP stream.  Every step
of the computation runs in the library's HIP kernels; there is no fallback.

    o, S = chunk_fwd(q, k, v, g, tau, beta_hat, initial_state=None,
                     output_final_state=False, chunk=0)
    o = decode_step(q, k, v, g, tau, beta_hat, state)       # state updated in place
    grads = chunk_bwd(q, k, v, g, tau, beta_hat, d_out, initial_state=None,
                      d_final_state=None)                     # dict of fp32 gradients

Per head:  alpha = exp(-g*tau), alpha_hat = g**tau (over dk),
S_t = diag(alpha_t) S_{t-1} + (alpha_hat_t*k_t)(beta_hat_t*v_t)^T, o_t = S_t^T q_t
(gate formulas: Rodimus* digest page, "Method"; selection along n only:
Rodimus* rebuttal page, "Efficient Parallelization").
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["chunk_fwd", "chunk_fwd_fused", "chunk_fwd_no_alloc", "chunk_bwd", "decode_step",
           "decode_step_fused", "swska_fwd", "workspace_bytes", "fused_workspace_bytes",
           "trace_forward_events",
           "bwd_workspace_bytes", "chunk_fwd_plan", "STATIC_SCRATCH_BYTES",
           "lib", "RodimusError", "LIB_PATH", "abi_version"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librodimus_ddts.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
STATIC_SCRATCH_BYTES = 32 << 20     # RODIMUS_STATIC_SCRATCH_BYTES
DTYPE_F32, DTYPE_BF16 = 0, 1

_lib = None


class RodimusError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded C-ABI library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m gated_linear_attention_rodimus_amd.build` (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.rodimus_abi_version.restype = i
        L.rodimus_abi_version.argtypes = []
        L.rodimus_status_string.restype = ctypes.c_char_p
        L.rodimus_status_string.argtypes = [i]
        L.rodimus_ddts_chunk_fwd_workspace_bytes.restype = sz
        L.rodimus_ddts_chunk_fwd_workspace_bytes.argtypes = [i] * 6
        L.rodimus_ddts_chunk_fwd_ex_workspace_bytes.restype = sz
        L.rodimus_ddts_chunk_fwd_ex_workspace_bytes.argtypes = [i] * 7
        L.rodimus_ddts_chunk_fwd_plan.restype = i
        L.rodimus_ddts_chunk_fwd_plan.argtypes = [i] * 8 + [ctypes.POINTER(_ChunkPlan)]
        L.rodimus_ddts_chunk_fwd.restype = i
        L.rodimus_ddts_chunk_fwd.argtypes = [i] * 7 + [vp] * 9 + [vp, sz, vp]
        L.rodimus_ddts_chunk_fwd_ex.restype = i
        L.rodimus_ddts_chunk_fwd_ex.argtypes = [i] * 8 + [vp] * 9 + [vp, sz, vp]
        L.rodimus_ddts_chunk_fwd_static_scratch.restype = i
        L.rodimus_ddts_chunk_fwd_static_scratch.argtypes = [i] * 8 + [vp] * 9 + [vp]
        L.rodimus_ddts_chunk_fwd_fused.restype = i
        L.rodimus_ddts_chunk_fwd_fused.argtypes = ([i] * 8 + [vp] * 6 + [ctypes.POINTER(_Fused)]
                                                   + [vp] * 4 + [sz, vp])
        L.rodimus_ddts_chunk_fwd_fused_workspace_bytes.restype = sz
        L.rodimus_ddts_chunk_fwd_fused_workspace_bytes.argtypes = [i] * 7
        L.rodimus_ddts_decode_step_fused.restype = i
        L.rodimus_ddts_decode_step_fused.argtypes = ([i] * 5 + [vp] * 6 + [ctypes.POINTER(_Fused)]
                                                     + [vp] * 3)
        L.rodimus_swska_fwd.restype = i
        L.rodimus_swska_fwd.argtypes = [i] * 6 + [ctypes.c_float, i] + [vp] * 4 + [vp]
        L.rodimus_trace_forward_events.restype = i
        L.rodimus_trace_forward_events.argtypes = [vp, i]
        L.rodimus_ddts_decode_step.restype = i
        L.rodimus_ddts_decode_step.argtypes = [i] * 5 + [vp] * 8 + [vp]
        L.rodimus_ddts_chunk_bwd_workspace_bytes.restype = sz
        L.rodimus_ddts_chunk_bwd_workspace_bytes.argtypes = [i] * 5
        L.rodimus_ddts_chunk_bwd.restype = i
        L.rodimus_ddts_chunk_bwd.argtypes = [i] * 6 + [vp] * 16 + [vp, sz, vp]
        _lib = L
    return _lib


def _status_string(status: int) -> str:
    try:
        return lib().rodimus_status_string(status).decode()
    except Exception:
        return "unknown"


def abi_version() -> int:
    return lib().rodimus_abi_version()


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError(f"per-token inputs must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_tensor(name, t, shape, dtype, device):
    if t.shape != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _check_workspace(workspace, need, device):
    """A caller-supplied workspace: a contiguous tensor on ``device`` holding at
    least ``need`` bytes (any dtype; its size is numel * element_size).
    Returns its size in bytes (0 for None).  Raises before any library call."""
    if workspace is None:
        return 0
    torch = _torch()
    if not isinstance(workspace, torch.Tensor):
        raise TypeError(f"workspace: expected a torch tensor, got {type(workspace).__name__}")
    if workspace.device != device:
        raise ValueError(f"workspace: expected device {device}, got {workspace.device}")
    if not workspace.is_contiguous():
        raise ValueError("workspace: must be contiguous")
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < need:
        raise ValueError(f"workspace: {nbytes} bytes, the call needs {need}")
    return nbytes


def bwd_workspace_bytes(B, T, H, dk, dv) -> int:
    return int(lib().rodimus_ddts_chunk_bwd_workspace_bytes(B, T, H, dk, dv))


def workspace_bytes(B, T, H, dk, dv, chunk=0, segments=0) -> int:
    return int(lib().rodimus_ddts_chunk_fwd_ex_workspace_bytes(B, T, H, dk, dv, chunk, segments))


class _Fused(ctypes.Structure):
    """rodimus_fused: the steps fused around the recurrence."""
    _fields_ = [("u", ctypes.c_void_p), ("w", ctypes.c_void_p), ("rank", ctypes.c_int),
                ("d", ctypes.c_void_p), ("conv_width", ctypes.c_int),
                ("conv_q", ctypes.c_void_p), ("conv_k", ctypes.c_void_p),
                ("conv_v", ctypes.c_void_p)]


def fused_workspace_bytes(B, T, H, dk, dv, chunk=0, segments=0) -> int:
    return int(lib().rodimus_ddts_chunk_fwd_fused_workspace_bytes(B, T, H, dk, dv, chunk, segments))


def _fused_desc(u, w, d, conv, H, dk, dv, dt, dev, lead):
    """Check the fused-step tensors and build the rodimus_fused descriptor.
    ``lead``: the leading shape of u ((B, T) or (N,))."""
    torch = _torch()
    f = _Fused()
    if u is not None:
        if w is None:
            raise ValueError("u needs w")
        rank = u.shape[-1]
        _check_tensor("u", u, tuple(lead) + (H, rank), dt, dev)
        _check_tensor("w", w, (H, rank, dv), dt, dev)
        f.u, f.w, f.rank = u.data_ptr(), w.data_ptr(), rank
    if d is not None:
        _check_tensor("d", d, (H, dv), torch.float32, dev)
        f.d = d.data_ptr()
    f.conv_width = 1
    if conv is not None:
        cq, ck, cv = conv
        W = cq.shape[-1]
        for name, t, n in (("conv_q", cq, dk), ("conv_k", ck, dk), ("conv_v", cv, dv)):
            _check_tensor(name, t, (H, n, W), torch.float32, dev)
        f.conv_width = W
        f.conv_q, f.conv_k, f.conv_v = cq.data_ptr(), ck.data_ptr(), cv.data_ptr()
    return f


def chunk_fwd_fused(q, k, v, g, tau, beta_hat=None, u=None, w=None, d=None, conv=None,
                    initial_state=None, output_final_state=False, chunk=0, segments=0,
                    out=None, final_state=None, workspace=None):
    """Chunk forward with the fused steps (rodimus_ddts_chunk_fwd_fused):
    beta_hat = sigmoid(u w) when u ([B, T, H, r]) and w ([H, r, dv]) are given
    (beta_hat then unused), o += d * v when d ([H, dv] fp32) is given, and a
    ShortConv of q, k, v when conv = (c_q, c_k, c_v) ([H, D, W] fp32) is given,
    in which case q, k, v are [B, T + W - 1, H, D] with the W - 1 history rows
    first.  g, tau: [B, T, H, dk].  Returns (o, final state or None)."""
    torch = _torch()
    W = 1 if conv is None else conv[0].shape[-1]
    B, Tx, H, dk = q.shape
    T = Tx - (W - 1)
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("chunk_fwd_fused runs on the GPU only; inputs must be on a cuda device")
    dt = q.dtype
    code = _dtype_code(q)
    for name, t, shp in (("q", q, (B, Tx, H, dk)), ("k", k, (B, Tx, H, dk)), ("v", v, (B, Tx, H, dv)),
                         ("g", g, (B, T, H, dk)), ("tau", tau, (B, T, H, dk))):
        _check_tensor(name, t, shp, dt, dev)
    if u is None:
        if beta_hat is None:
            raise ValueError("beta_hat or (u, w) is needed")
        _check_tensor("beta_hat", beta_hat, (B, T, H, dv), dt, dev)
    f = _fused_desc(u, w, d, conv, H, dk, dv, dt, dev, (B, T))
    if initial_state is not None:
        _check_tensor("initial_state", initial_state, (B, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    else:
        _check_tensor("out", out, (B, T, H, dv), torch.float32, dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _check_tensor("final_state", final_state, (B, H, dk, dv), torch.float32, dev)
    wsb = fused_workspace_bytes(B, T, H, dk, dv, chunk, segments)
    if wsb and workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    ws_bytes = _check_workspace(workspace, wsb, dev)
    st = lib().rodimus_ddts_chunk_fwd_fused(
        B, T, H, dk, dv, int(chunk), int(segments), code,
        _ptr(q), _ptr(k), _ptr(g), _ptr(tau), _ptr(v), _ptr(beta_hat), ctypes.byref(f),
        _ptr(initial_state), _ptr(out), _ptr(final_state),
        _ptr(workspace), ws_bytes, _stream(dev))
    if st != OK:
        raise RodimusError(st, "rodimus_ddts_chunk_fwd_fused")
    return out, final_state


def decode_step_fused(q, k, v, g, tau, state, beta_hat=None, u=None, w=None, d=None, conv=None,
                      out=None):
    """One decode step with the fused steps (rodimus_ddts_decode_step_fused).
    Without conv, q, k [N, H, dk] and v [N, H, dv]; with conv (W taps), the
    windows of their last W raw tokens, [N, W, H, D], oldest first.  g, tau
    [N, H, dk]; u [N, H, r]; state updated in place.  Returns o [N, H, dv]."""
    torch = _torch()
    W = 1 if conv is None else conv[0].shape[-1]
    N, H, dk = g.shape
    dv = state.shape[-1]
    dev = g.device
    if dev.type != "cuda":
        raise ValueError("decode_step_fused runs on the GPU only; inputs must be on a cuda device")
    dt = g.dtype
    code = _dtype_code(g)
    win = (N, W, H) if conv is not None else (N, H)
    for name, t, shp in (("q", q, win + (dk,)), ("k", k, win + (dk,)), ("v", v, win + (dv,)),
                         ("g", g, (N, H, dk)), ("tau", tau, (N, H, dk))):
        _check_tensor(name, t, shp, dt, dev)
    if u is None:
        if beta_hat is None:
            raise ValueError("beta_hat or (u, w) is needed")
        _check_tensor("beta_hat", beta_hat, (N, H, dv), dt, dev)
    f = _fused_desc(u, w, d, conv, H, dk, dv, dt, dev, (N,))
    _check_tensor("state", state, (N, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((N, H, dv), dtype=torch.float32, device=dev)
    else:
        _check_tensor("out", out, (N, H, dv), torch.float32, dev)
    st = lib().rodimus_ddts_decode_step_fused(
        N, H, dk, dv, code, _ptr(q), _ptr(k), _ptr(g), _ptr(tau), _ptr(v), _ptr(beta_hat),
        ctypes.byref(f), _ptr(state), _ptr(out), _stream(dev))
    if st != OK:
        raise RodimusError(st, "rodimus_ddts_decode_step_fused")
    return out


class _ChunkPlan(ctypes.Structure):
    _fields_ = [("chunk", ctypes.c_int), ("dv_tile", ctypes.c_int), ("segments", ctypes.c_int),
                ("transfer_pieces", ctypes.c_int), ("workspace_bytes", ctypes.c_size_t)]


def chunk_fwd_plan(B, T, H, dk, dv, chunk=0, segments=0, dtype="bf16") -> dict:
    """How the chunk forward runs for these sizes (rodimus_ddts_chunk_fwd_plan):
    chunk, dv_tile, segments, transfer_pieces, workspace_bytes.  Host only."""
    code = {"bf16": DTYPE_BF16, "f32": DTYPE_F32}[dtype]
    p = _ChunkPlan()
    st = lib().rodimus_ddts_chunk_fwd_plan(B, T, H, dk, dv, chunk, segments, code, ctypes.byref(p))
    if st != OK:
        raise RodimusError(st, "rodimus_ddts_chunk_fwd_plan")
    return {n: int(getattr(p, n)) for n, _ in _ChunkPlan._fields_}


def chunk_fwd(q, k, v, g, tau, beta_hat, initial_state=None, output_final_state=False,
              chunk=0, segments=0, out=None, final_state=None, workspace=None):
    """Chunkwise-parallel forward.  q, k, g, tau: [B, T, H, dk]; v, beta_hat:
    [B, T, H, dv]; all six bf16 or all six fp32, contiguous, on one GPU.
    initial_state: [B, H, dk, dv] fp32 or None.  Returns (o fp32 [B, T, H, dv],
    final state fp32 [B, H, dk, dv] or None).  ``final_state`` may be passed
    (also as the same tensor as ``initial_state``, for in-place carry-over)."""
    torch = _torch()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("chunk_fwd runs on the GPU only; inputs must be on a cuda device")
    dt = q.dtype
    code = _dtype_code(q)
    for name, t, d in (("q", q, dk), ("k", k, dk), ("g", g, dk), ("tau", tau, dk),
                       ("v", v, dv), ("beta_hat", beta_hat, dv)):
        _check_tensor(name, t, (B, T, H, d), dt, dev)
    if initial_state is not None:
        _check_tensor("initial_state", initial_state, (B, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    else:
        _check_tensor("out", out, (B, T, H, dv), torch.float32, dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _check_tensor("final_state", final_state, (B, H, dk, dv), torch.float32, dev)
    wsb = workspace_bytes(B, T, H, dk, dv, chunk, segments)
    if wsb and workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    ws_bytes = _check_workspace(workspace, wsb, dev)
    st = lib().rodimus_ddts_chunk_fwd_ex(
        B, T, H, dk, dv, int(chunk), int(segments), code,
        _ptr(q), _ptr(k), _ptr(g), _ptr(tau), _ptr(v), _ptr(beta_hat),
        _ptr(initial_state), _ptr(out), _ptr(final_state),
        _ptr(workspace), ws_bytes, _stream(dev))
    if st != OK:
        raise RodimusError(st, "rodimus_ddts_chunk_fwd")
    return out, final_state


def chunk_fwd_no_alloc(q, k, v, g, tau, beta_hat, out, initial_state=None, final_state=None,
                       chunk=0, segments=0):
    """``chunk_fwd`` for callers that cannot allocate: ``out`` (and
    ``final_state`` if wanted) are passed in, and the segmented path's scratch
    is the library's fixed per-GPU buffer (rodimus_ddts_chunk_fwd_static_scratch;
    at most STATIC_SCRATCH_BYTES of workspace, calls on one GPU must not
    overlap).  Nothing is allocated here or in the library."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("chunk_fwd_no_alloc runs on the GPU only; inputs must be on a cuda device")
    torch = _torch()
    dt = q.dtype
    code = _dtype_code(q)
    for name, t, d in (("q", q, dk), ("k", k, dk), ("g", g, dk), ("tau", tau, dk),
                       ("v", v, dv), ("beta_hat", beta_hat, dv)):
        _check_tensor(name, t, (B, T, H, d), dt, dev)
    _check_tensor("out", out, (B, T, H, dv), torch.float32, dev)
    for name, t in (("initial_state", initial_state), ("final_state", final_state)):
        if t is not None:
            _check_tensor(name, t, (B, H, dk, dv), torch.float32, dev)
    st = lib().rodimus_ddts_chunk_fwd_static_scratch(
        B, T, H, dk, dv, int(chunk), int(segments), code,
        _ptr(q), _ptr(k), _ptr(g), _ptr(tau), _ptr(v), _ptr(beta_hat),
        _ptr(initial_state), _ptr(out), _ptr(final_state), _stream(dev))
    if st != OK:
        raise RodimusError(st, "rodimus_ddts_chunk_fwd_static_scratch")
    return out, final_state


def trace_forward_events(events):
    """Record the given 4 torch.cuda.Events around the launches of this host
    thread's following forward calls (rodimus_trace_forward_events); None
    stops.  One sweep: events 0 and 1 bracket the kernel; segmented: 0 | transfer
    | 1 | combine | 2 | output | 3."""
    if events is None:
        st = lib().rodimus_trace_forward_events(None, 0)
    else:
        if len(events) != 4:
            raise ValueError("trace_forward_events needs 4 events")
        handles = (ctypes.c_void_p * 4)(*[e.cuda_event for e in events])
        trace_forward_events._keep = handles
        st = lib().rodimus_trace_forward_events(handles, 4)
    if st != OK:
        raise RodimusError(st, "rodimus_trace_forward_events")


def swska_fwd(q, k, v, window, scale=0.0, out=None):
    """Sliding-window shared-key attention (rodimus_swska_fwd): q [B, T, H, dk],
    k [B, T, dk] (one key for all heads), v [B, T, H, dv], bf16, contiguous,
    on one GPU; each token attends to the ``window`` most recent tokens
    (itself included); scale 0 = 1/sqrt(dk).  Returns o fp32 [B, T, H, dv]."""
    torch = _torch()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("swska_fwd runs on the GPU only; inputs must be on a cuda device")
    code = _dtype_code(q)
    _check_tensor("q", q, (B, T, H, dk), q.dtype, dev)
    _check_tensor("k", k, (B, T, dk), q.dtype, dev)
    _check_tensor("v", v, (B, T, H, dv), q.dtype, dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    else:
        _check_tensor("out", out, (B, T, H, dv), torch.float32, dev)
    st = lib().rodimus_swska_fwd(B, T, H, dk, dv, int(window), float(scale), code, _ptr(q),
                                 _ptr(k), _ptr(v), _ptr(out), _stream(dev))
    if st != OK:
        raise RodimusError(st, "rodimus_swska_fwd")
    return out


def decode_step(q, k, v, g, tau, beta_hat, state, out=None):
    """One recurrent step for N sequences.  q, k, g, tau: [N, H, dk]; v,
    beta_hat: [N, H, dv]; state: [N, H, dk, dv] fp32, updated in place.
    Returns o fp32 [N, H, dv]."""
    torch = _torch()
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("decode_step runs on the GPU only; inputs must be on a cuda device")
    dt = q.dtype
    code = _dtype_code(q)
    for name, t, d in (("q", q, dk), ("k", k, dk), ("g", g, dk), ("tau", tau, dk),
                       ("v", v, dv), ("beta_hat", beta_hat, dv)):
        _check_tensor(name, t, (N, H, d), dt, dev)
    _check_tensor("state", state, (N, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((N, H, dv), dtype=torch.float32, device=dev)
    else:
        _check_tensor("out", out, (N, H, dv), torch.float32, dev)
    st = lib().rodimus_ddts_decode_step(
        N, H, dk, dv, code, _ptr(q), _ptr(k), _ptr(g), _ptr(tau), _ptr(v), _ptr(beta_hat),
        _ptr(state), _ptr(out), _stream(dev))
    if st != OK:
        raise RodimusError(st, "rodimus_ddts_decode_step")
    return out


def chunk_bwd(q, k, v, g, tau, beta_hat, d_out, initial_state=None, d_final_state=None,
              workspace=None):
    """Gradients of the chunk forward.  Inputs as ``chunk_fwd`` (bf16 or fp32,
    contiguous, one GPU); d_out [B, T, H, dv] fp32; d_final_state [B, H, dk, dv]
    fp32 or None.  Returns a dict of fp32 tensors: dq, dk, dg, dtau
    ([B, T, H, dk]), dv, dbeta_hat ([B, T, H, dv]), d_initial_state
    ([B, H, dk, dv])."""
    torch = _torch()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("chunk_bwd runs on the GPU only; inputs must be on a cuda device")
    dt = q.dtype
    _dtype_code(q)
    for n, t in (("q", q), ("k", k), ("g", g), ("tau", tau)):
        _check_tensor(n, t, (B, T, H, dk), dt, dev)
    for n, t in (("v", v), ("beta_hat", beta_hat)):
        _check_tensor(n, t, (B, T, H, dv), dt, dev)
    _check_tensor("d_out", d_out, (B, T, H, dv), torch.float32, dev)
    for n, t in (("initial_state", initial_state), ("d_final_state", d_final_state)):
        if t is not None:
            _check_tensor(n, t, (B, H, dk, dv), torch.float32, dev)
    grads = {n: torch.empty(B, T, H, dk, device=dev) for n in ("dq", "dk", "dg", "dtau")}
    grads.update({n: torch.empty(B, T, H, dv, device=dev) for n in ("dv", "dbeta_hat")})
    grads["d_initial_state"] = torch.empty(B, H, dk, dv, device=dev)
    wsb = bwd_workspace_bytes(B, T, H, dk, dv)
    if wsb and workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    ws_bytes = _check_workspace(workspace, wsb, dev)
    st = lib().rodimus_ddts_chunk_bwd(
        B, T, H, dk, dv, _dtype_code(q), _ptr(q), _ptr(k), _ptr(g), _ptr(tau), _ptr(v),
        _ptr(beta_hat), _ptr(initial_state), _ptr(d_out), _ptr(d_final_state),
        _ptr(grads["dq"]), _ptr(grads["dk"]), _ptr(grads["dg"]), _ptr(grads["dtau"]),
        _ptr(grads["dv"]), _ptr(grads["dbeta_hat"]), _ptr(grads["d_initial_state"]),
        _ptr(workspace), ctypes.c_size_t(ws_bytes), _stream(dev))
    if st != OK:
        raise RodimusError(st, "rodimus_ddts_chunk_bwd")
    return grads
