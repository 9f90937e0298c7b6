"""fp64 CPU oracle for the DDTS recurrence of Rodimus (TEST INFRASTRUCTURE).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package.  The product path (the HIP library and its Python binding)
never imports it, and it imports nothing from the product path.

``fwd`` and ``decode`` wrap the C implementation in ``ddts_oracle.c``: the
plain token-by-token recurrence

    alpha_t = exp(-g_t * tau_t),  alpha_hat_t = g_t ** tau_t      (over dk)
    S_t = diag(alpha_t) S_{t-1} + (alpha_hat_t * k_t)(beta_hat_t * v_t)^T
    o_t = S_t^T q_t

in float64.  The gate formulas follow the Rodimus* digest page
(digest.lyk-ai.com), section "Method"; the placement of alpha and alpha_hat on
the dk rows follows the authors' rebuttal page (paperhub.cn), the
"Efficient Parallelization" bullet (selection only along n).

``bwd`` is the reverse mode of ``fwd`` written out from the same recurrence
(the adjoint of the state walked from the last token to the first); at g = 0,
where g^tau has no derivative, its g^tau terms are taken as 0.

Every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` against a brute-force quadratic form, library
matmuls in the special cases tau = 0 and constant gates, a division-based
closed form for dk = dv = 1, the g = 0 invariant, linearity and bitwise
carry-over; ``bwd`` by ``tests/test_oracle_bwd.py`` against central finite
differences of ``fwd``, the matmul gradients of the tau = 0 case, dg = 0 at
tau = 0 and the T = 0 case.

``lowrank_beta``, ``short_conv``, ``fwd_fused`` and ``decode_fused`` are the
steps the library can fuse around the recurrence (beta_hat from low-rank
factors, a short causal convolution of q, k and v, the feedthrough d), in
plain fp64 numpy composed with ``fwd`` / ``decode``; they are pinned by
``tests/test_oracle_fused.py`` (hand-computed values, an impulse response,
saturation limits, carry-over of the convolution window and of the state,
and planted mistakes that the pins must catch).

Inputs may be any numpy floating dtype (bf16 inputs arrive as their exact
float32 upcast); they are converted to float64 exactly before the C call.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ddts_oracle.c")
_LIB = os.path.join(_HERE, "libddts_oracle.so")
_CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-pthread"]

_lib = None


def build() -> str:
    """Compile the oracle with gcc (IEEE, no fast-math).  Returns the .so path."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.ddts_oracle_fwd.restype = ctypes.c_int
        lib.ddts_oracle_fwd.argtypes = [ctypes.c_int] * 5 + [dp] * 9 + [ctypes.c_int]
        lib.ddts_oracle_decode.restype = ctypes.c_int
        lib.ddts_oracle_decode.argtypes = [ctypes.c_int] * 4 + [dp] * 8
        lib.ddts_oracle_bwd.restype = ctypes.c_int
        lib.ddts_oracle_bwd.argtypes = [ctypes.c_int] * 5 + [dp] * 16 + [ctypes.c_int]
        _lib = lib
    return _lib


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def fwd(q, k, v, g, tau, beta_hat, initial_state=None, return_final_state=True,
        nthreads=0):
    """Token-by-token fp64 forward over whole sequences.

    q, k, g, tau: [B, T, H, dk]; v, beta_hat: [B, T, H, dv];
    initial_state: [B, H, dk, dv] or None (zeros).
    Returns (o [B, T, H, dv], S_T [B, H, dk, dv] or None), both float64.
    The number of threads actually used is stored in ``fwd.last_threads``.
    """
    q, k, g, tau, v, beta_hat = map(_f64, (q, k, g, tau, v, beta_hat))
    B, T, H, dk = q.shape
    dv = v.shape[3]
    for a in (k, g, tau):
        assert a.shape == (B, T, H, dk)
    for a in (beta_hat,):
        assert a.shape == (B, T, H, dv)
    s0 = None if initial_state is None else _f64(initial_state)
    if s0 is not None:
        assert s0.shape == (B, H, dk, dv)
    out = np.empty((B, T, H, dv), np.float64)
    sf = np.empty((B, H, dk, dv), np.float64) if return_final_state else None
    rc = _load().ddts_oracle_fwd(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(g), _ptr(tau),
                                 _ptr(v), _ptr(beta_hat), _ptr(s0), _ptr(out), _ptr(sf),
                                 int(nthreads))
    if rc < 0:
        raise RuntimeError("ddts_oracle_fwd failed")
    fwd.last_threads = rc
    return out, sf


fwd.last_threads = 0


def decode(q, k, v, g, tau, beta_hat, state):
    """One fp64 recurrent step for N sequences.

    q, k, g, tau: [N, H, dk]; v, beta_hat: [N, H, dv]; state: [N, H, dk, dv].
    Returns (o [N, H, dv], new_state [N, H, dk, dv]); the input is not modified.
    """
    q, k, g, tau, v, beta_hat = map(_f64, (q, k, g, tau, v, beta_hat))
    N, H, dk = q.shape
    dv = v.shape[2]
    st = np.array(state, dtype=np.float64, order="C", copy=True)
    assert st.shape == (N, H, dk, dv)
    out = np.empty((N, H, dv), np.float64)
    rc = _load().ddts_oracle_decode(N, H, dk, dv, _ptr(q), _ptr(k), _ptr(g), _ptr(tau),
                                    _ptr(v), _ptr(beta_hat), _ptr(st), _ptr(out))
    if rc < 0:
        raise RuntimeError("ddts_oracle_decode failed")
    return out, st


def bwd(q, k, v, g, tau, beta_hat, d_out, initial_state=None, d_final_state=None,
        nthreads=0):
    """fp64 reverse mode of ``fwd``: gradients of a loss L given dL/do
    ([B, T, H, dv]) and optionally dL/dS_T ([B, H, dk, dv]).

    Returns a dict with dq, dk, dg, dtau ([B, T, H, dk]), dv, dbeta_hat
    ([B, T, H, dv]) and d_initial_state ([B, H, dk, dv]), all float64.  At
    g = 0 the g^tau terms of dg and dtau are taken as 0.
    """
    q, k, g, tau, v, beta_hat, d_out = map(_f64, (q, k, g, tau, v, beta_hat, d_out))
    B, T, H, dk = q.shape
    dv = v.shape[3]
    for a in (k, g, tau):
        assert a.shape == (B, T, H, dk)
    for a in (beta_hat, d_out):
        assert a.shape == (B, T, H, dv)
    s0 = None if initial_state is None else _f64(initial_state)
    dsf = None if d_final_state is None else _f64(d_final_state)
    for a in (s0, dsf):
        assert a is None or a.shape == (B, H, dk, dv)
    out = {n: np.empty((B, T, H, dk), np.float64) for n in ("dq", "dk", "dg", "dtau")}
    out.update({n: np.empty((B, T, H, dv), np.float64) for n in ("dv", "dbeta_hat")})
    out["d_initial_state"] = np.empty((B, H, dk, dv), np.float64)
    rc = _load().ddts_oracle_bwd(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(g), _ptr(tau),
                                 _ptr(v), _ptr(beta_hat), _ptr(s0), _ptr(d_out), _ptr(dsf),
                                 _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dg"]),
                                 _ptr(out["dtau"]), _ptr(out["dv"]), _ptr(out["dbeta_hat"]),
                                 _ptr(out["d_initial_state"]), int(nthreads))
    if rc < 0:
        raise RuntimeError("ddts_oracle_bwd failed")
    return out


def rel_to_rms_error(x_hat, x) -> float:
    """max_i |x_hat_i - x_i| / sqrt(mean_i x_i^2): the parity metric."""
    x = np.asarray(x, np.float64)
    x_hat = np.asarray(x_hat, np.float64)
    rms = float(np.sqrt(np.mean(x * x)))
    if rms == 0.0:
        return float(np.max(np.abs(x_hat - x))) if x.size else 0.0
    return float(np.max(np.abs(x_hat - x))) / rms


# ---------------------------------------------------------------- fused steps
# The steps on either side of the recurrence that the library can fuse into
# its kernels, written out plainly in fp64.  The pages name them without
# giving their equations, so each follows a stated reading:
#  - beta_hat from low-rank factors (digest page, "Method", low-rank bullet):
#    beta_hat_t = sigmoid(u_t W), u_t of rank r per token and head, W [r, dv]
#    per head, no scaling;
#  - ShortConv (digest page, "Method", ShortConv + GLU bullet): a causal
#    depthwise convolution along time of q, k and v, one filter of W taps per
#    head and channel, no bias, no activation; the W - 1 raw rows before the
#    first token come with the input (zeros at a sequence start);
#  - the feedthrough d (rebuttal page, answer to "How significant is d_t in
#    Eq. (11)?": the SSM feedthrough matrix): o_t += d * v_t, d a per-head
#    vector over dv constant in t, v_t the value entering the recurrence
#    (after the convolution, before beta_hat).


def lowrank_beta(u, w):
    """beta_hat = sigmoid(u W) in fp64: u [..., H, r], w [H, r, dv] -> [..., H, dv]."""
    u = _f64(u)
    w = _f64(w)
    z = np.einsum("...hr,hrj->...hj", u, w)
    return 1.0 / (1.0 + np.exp(-z))


def short_conv(x, c):
    """Causal depthwise convolution over time in fp64.

    x: [B, T + W - 1, H, D], the W - 1 raw rows before token 0 first;
    c: [H, D, W], tap j multiplying the input j tokens back.
    Returns y [B, T, H, D] with y[:, t] = sum_j c[..., j] * x[:, t + W - 1 - j].
    """
    x = _f64(x)
    c = _f64(c)
    W = c.shape[-1]
    T = x.shape[1] - (W - 1)
    assert T >= 0 and c.shape == (x.shape[2], x.shape[3], W)
    y = np.zeros((x.shape[0], T) + x.shape[2:])
    for j in range(W):
        y += c[None, None, :, :, j] * x[:, W - 1 - j:W - 1 - j + T]
    return y


def fwd_fused(q, k, v, g, tau, beta_hat=None, u=None, w=None, d=None, conv=None,
              initial_state=None, nthreads=0):
    """The recurrence with its fused steps, in fp64: ShortConv of q, k, v (conv
    = (c_q, c_k, c_v), each [H, D, W]; q, k, v then carry W - 1 history rows,
    [B, T + W - 1, H, D]), beta_hat = sigmoid(u w) when u is given (u
    [B, T, H, r], w [H, r, dv]), then ``fwd``, then o += d * v (d [H, dv]).
    Returns (o [B, T, H, dv], S_T)."""
    if conv is not None:
        cq, ck, cv = conv
        q, k, v = short_conv(q, cq), short_conv(k, ck), short_conv(v, cv)
    if u is not None:
        beta_hat = lowrank_beta(u, w)
    o, sf = fwd(q, k, v, g, tau, beta_hat, initial_state, nthreads=nthreads)
    if d is not None:
        o = o + _f64(d)[None, None] * _f64(v)
    return o, sf


def decode_fused(q, k, v, g, tau, state, beta_hat=None, u=None, w=None, d=None, conv=None):
    """One recurrent step with the fused steps, in fp64.  Without conv, q, k
    [N, H, dk] and v [N, H, dv]; with conv, each is the window of its last W
    raw tokens, oldest first ([N, W, H, D]).  u [N, H, r].  Returns (o [N, H,
    dv], new state)."""
    if conv is not None:
        cq, ck, cv = conv
        q, k, v = (short_conv(x, c)[:, 0] for x, c in ((q, cq), (k, ck), (v, cv)))
    if u is not None:
        beta_hat = lowrank_beta(u, w)
    o, st = decode(q, k, v, g, tau, beta_hat, state)
    if d is not None:
        o = o + _f64(d)[None] * _f64(v)
    return o, st


# ---------------------------------------------------------------- SW-SKA
# Rodimus+'s second token mixer: sliding-window attention whose keys are
# shared by all heads (summary page, "Approach"; digest page, "Method",
# Rodimus+ bullets; the rebuttal counts its projections as multi-head,
# multi-query and output, so q and v have a head each and k one for all).
# Readings: token t attends to the `window` most recent tokens s with
# t - window < s <= t (itself included); scores are q . k scaled by
# 1 / sqrt(dk) unless a scale is given; softmax over those tokens.


def swska_fwd(q, k, v, window, scale=None):
    """Sliding-window shared-key attention in fp64.

    q [B, T, H, dk], k [B, T, dk] (one key per token, shared by the heads),
    v [B, T, H, dv] -> o [B, T, H, dv]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H, dk = q.shape
    dv = v.shape[3]
    assert k.shape == (B, T, dk) and v.shape[:3] == (B, T, H) and window >= 1
    sc = 1.0 / np.sqrt(dk) if scale is None else float(scale)
    o = np.empty((B, T, H, dv))
    for b in range(B):
        for t in range(T):
            s0 = max(0, t - window + 1)
            z = (q[b, t] @ k[b, s0:t + 1].T) * sc                 # [H, L]
            z -= z.max(axis=1, keepdims=True)
            p = np.exp(z)
            p /= p.sum(axis=1, keepdims=True)
            o[b, t] = np.einsum("hl,lhd->hd", p, v[b, s0:t + 1])
    return o
