"""Seeded synthetic inputs for the DDTS recurrence (shared by tests, bench, smoke).

This module only draws and encodes inputs; it holds none of the recurrence's
arithmetic, so the fp64 oracle and the HIP path can both be fed from it
without sharing any computation.

Every tensor is drawn with ``numpy.random.Generator(PCG64(seed))`` in float32,
``seed = 1000 * workload_id + tensor_id``, and for bf16 workloads rounded once
to bfloat16 (round to nearest even) on the host.  The same bytes go to the
GPU and, upcast exactly, to the oracle.

The pages give no kernel-level input distributions (the model configuration
table they reference is not on them); the workloads below are shaped like
the 130M and 1.6B models and the 24K-token prefill that the pages discuss,
with gate distributions chosen as sigmoids of normals so that g and tau lie
in (0, 1).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# tensor ids inside one workload's seed space
_Q, _K, _V, _G, _TAU, _BETA, _S0, _BU, _BW = range(9)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int            # seed namespace
    B: int
    T: int
    H: int
    dk: int
    dv: int
    chunk: int          # 0 = let the library choose
    dtype: str          # "f32" or "bf16"
    g_mean: float       # g = sigmoid(N(g_mean, 1))
    beta: str           # "iid" -> sigmoid(N(0,1)); "rank16" -> sigmoid(U @ W)
    s0_std: float       # 0 -> no initial state
    final_state: bool   # the caller asks for S_T
    steps: int = 0      # decode workloads: number of recurrent steps


WORKLOADS = {
    # tiny recurrence, fp32, parity only
    "tiny": Workload("tiny", 1, 1, 64, 2, 16, 16, 16, "f32", 0.0, "iid", 0.0, False),
    # one layer of a 130M-scale model: 8 x 2048 tokens, 12 heads of 64 x 128
    "layer130m": Workload("layer130m", 2, 8, 2048, 12, 64, 128, 0, "bf16", 1.0, "rank16",
                          0.0, False),
    # one layer of a 1.6B-scale model: 4 x 4096 tokens, 16 heads, returns S_T
    "layer1p6b": Workload("layer1p6b", 3, 4, 4096, 16, 64, 128, 0, "bf16", 0.0, "iid",
                          0.0, True),
    # long-context prefill: 65536 tokens, 16 heads, nonzero initial state
    "long_prefill": Workload("long_prefill", 4, 1, 65536, 16, 64, 128, 0, "bf16", 2.0,
                             "iid", 0.1, False),
    # batched decode: 256 sequences x 16 heads, resident fp32 states, 1000 steps
    "decode_batch": Workload("decode_batch", 5, 256, 1, 16, 64, 128, 0, "bf16", 0.0, "iid",
                             0.1, True, steps=1000),
}

DECODE_POOL = 16   # distinct input sets cycled over decode steps


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    t = u >> 16
    t &= 1
    t += 0x7FFF
    t += u                       # no overflow for finite inputs (|x| <= FLT_MAX)
    t >>= 16
    r = t.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> exact float32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _sigmoid32(x):
    """1 / (1 + exp(-x)) in float32, computed in place (x is consumed)."""
    x = np.asarray(x, dtype=np.float32)
    np.negative(x, out=x)
    np.exp(x, out=x)
    x += np.float32(1.0)
    np.reciprocal(x, out=x)
    return x


@dataclasses.dataclass
class Inputs:
    """One batch of per-token inputs in their storage encoding.

    For dtype "bf16" the six per-token tensors hold uint16 bf16 bit patterns,
    for "f32" float32 values.  ``initial_state`` is float32 or None.
    Layout: q, k, g, tau [B, T, H, dk]; v, beta_hat [B, T, H, dv];
    initial_state [B, H, dk, dv].
    """
    wl: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    tau: np.ndarray
    beta_hat: np.ndarray
    initial_state: np.ndarray | None

    def f32(self, name: str) -> np.ndarray:
        """Exact float32 values of a tensor (upcast of the bf16 bits)."""
        a = getattr(self, name)
        if a is None:
            return None
        return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a

    def torch(self, name: str, device="cuda"):
        """The tensor as a torch tensor (bfloat16 or float32) on ``device``."""
        import torch
        a = getattr(self, name)
        if a is None:
            return None
        if a.dtype == np.uint16:
            t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(a)
        return t.to(device)


def _encode(x32: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_round_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, np.float32)


def _rng(wid: int, tid: int, sub: int = 0):
    seed = 1000 * wid + tid
    if sub:
        seed = np.random.SeedSequence([seed, sub])
    return np.random.Generator(np.random.PCG64(seed))


def make(name: str, sub: int = 0, **overrides) -> Inputs:
    """Draw one batch of a workload.  ``overrides`` replace Workload fields
    (e.g. a smaller T for CPU-checkable parity); ``sub`` selects an
    independent draw in the same workload (decode steps use it)."""
    wl = dataclasses.replace(WORKLOADS[name], **overrides)
    B, T, H, dk, dv = wl.B, wl.T, wl.H, wl.dk, wl.dv
    sk, sv = (B, T, H, dk), (B, T, H, dv)
    inv = np.float32(1.0 / math.sqrt(dk))

    def normal(tid, shape, mean=0.0, std=1.0):
        x = _rng(wl.wid, tid, sub).standard_normal(shape, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        if mean != 0.0:
            x += np.float32(mean)
        return x

    def scaled(tid, shape):
        x = normal(tid, shape)
        x *= inv
        return x

    q = _encode(scaled(_Q, sk), wl.dtype)
    k = _encode(scaled(_K, sk), wl.dtype)
    v = _encode(scaled(_V, sv), wl.dtype)
    g = _encode(_sigmoid32(normal(_G, sk, mean=wl.g_mean)), wl.dtype)
    tau = _encode(_sigmoid32(normal(_TAU, sk)), wl.dtype)
    if wl.beta == "rank16":
        U = normal(_BU, (B, T, H, 16))
        W = normal(_BW, (H, 16, dv))
        z = np.einsum("bthr,hrj->bthj", U, W, optimize=True).astype(np.float32)
        beta = _encode(_sigmoid32(z), wl.dtype)
    else:
        beta = _encode(_sigmoid32(normal(_BETA, sv)), wl.dtype)
    s0 = None
    if wl.s0_std > 0.0:
        s0 = normal(_S0, (B, H, dk, dv), std=wl.s0_std)
    return Inputs(wl, q, k, v, g, tau, beta, s0)


def make_decode_pool(name: str = "decode_batch", pool: int = DECODE_POOL, **overrides):
    """Inputs for recurrent decode: ``pool`` independent one-token input sets
    (step s uses set s mod pool) and one resident initial state.

    Returns (list of Inputs with T == 1, initial_state [N, H, dk, dv] float32).
    The per-step tensors keep the [N, 1, H, D] shape; callers index [:, 0].
    """
    sets = [make(name, sub=p + 1, **overrides) for p in range(pool)]
    state = make(name, sub=0, **overrides).initial_state
    return sets, state


# tensor ids of the fused-step inputs (their own seed space per workload)
_QX, _KX, _VX, _UF, _WF, _DF, _CQ, _CK, _CV = range(20, 29)


@dataclasses.dataclass
class FusedInputs:
    """Inputs of the recurrence with its fused steps.

    ``base`` holds g, tau (and beta_hat, unused when u is given) as in
    ``make``; q, k, v here carry ``conv_width - 1`` history rows before token
    0 ([B, T + W - 1, H, D], storage encoding like ``base``).  u [B, T, H, r]
    and w [H, r, dv] are in the workload's storage encoding; d [H, dv] and the
    taps conv_q / conv_k [H, dk, W], conv_v [H, dv, W] are float32.
    """
    base: Inputs
    conv_width: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    u: np.ndarray
    w: np.ndarray
    d: np.ndarray
    conv_q: np.ndarray
    conv_k: np.ndarray
    conv_v: np.ndarray

    def f32(self, name: str) -> np.ndarray:
        a = getattr(self, name) if name in ("q", "k", "v", "u", "w") else None
        if a is None:
            return self.base.f32(name)
        return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a

    def torch(self, name: str, device="cuda"):
        import torch
        if name in ("q", "k", "v", "u", "w"):
            a = getattr(self, name)
            t = (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16
                 else torch.from_numpy(a))
            return t.to(device)
        if name in ("d", "conv_q", "conv_k", "conv_v"):
            return torch.from_numpy(getattr(self, name)).to(device)
        return self.base.torch(name, device)


def make_fused(name: str, conv_width: int = 4, rank: int = 16, sub: int = 0,
               history: bool = True, **overrides) -> FusedInputs:
    """A workload's inputs for the fused path: the base draw of ``make``, plus
    q, k, v with ``conv_width - 1`` history rows (drawn like the tokens, or
    zeros when ``history`` is False: a sequence start), low-rank factors u,
    w ~ N(0, 1) (rank ``rank``), d ~ N(0, 1) and ShortConv taps ~ N(0, 1/W)."""
    base = make(name, sub=sub, **overrides)
    wl = base.wl
    B, T, H, dk, dv = wl.B, wl.T, wl.H, wl.dk, wl.dv
    W = max(1, conv_width)
    inv = np.float32(1.0 / math.sqrt(dk))

    def draw(tid, shape, scale=None):
        x = _rng(wl.wid, tid, sub).standard_normal(shape, dtype=np.float32)
        if scale is not None:
            x *= np.float32(scale)
        return x

    def with_history(tid, d):
        x = draw(tid, (B, T + W - 1, H, d), inv)
        if not history:
            x[:, :W - 1] = 0.0
        return _encode(x, wl.dtype)

    return FusedInputs(
        base, W,
        with_history(_QX, dk), with_history(_KX, dk), with_history(_VX, dv),
        _encode(draw(_UF, (B, T, H, rank)), wl.dtype),
        _encode(draw(_WF, (H, rank, dv)), wl.dtype),
        draw(_DF, (H, dv)),
        draw(_CQ, (H, dk, W), 1.0 / math.sqrt(W)),
        draw(_CK, (H, dk, W), 1.0 / math.sqrt(W)),
        draw(_CV, (H, dv, W), 1.0 / math.sqrt(W)))


# ---------------------------------------------------------------- SW-SKA inputs
@dataclasses.dataclass(frozen=True)
class SwskaWorkload:
    name: str
    wid: int
    B: int
    T: int
    H: int
    dk: int
    dv: int
    window: int
    dtype: str


SWSKA_WORKLOADS = {
    # the sliding-window shared-key attention of a 1.6B-scale Rodimus+ layer:
    # 4 sequences x 4096 tokens, 16 query/value heads of 128, one shared key
    # of 128, a 512-token window
    "swska_1p6b": SwskaWorkload("swska_1p6b", 6, 4, 4096, 16, 128, 128, 512, "bf16"),
}


@dataclasses.dataclass
class SwskaInputs:
    """q [B, T, H, dk], k [B, T, dk] (shared by the heads), v [B, T, H, dv],
    all N(0, 1), in the storage encoding."""
    wl: SwskaWorkload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray

    def f32(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a

    def torch(self, name: str, device="cuda"):
        import torch
        a = getattr(self, name)
        t = (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16
             else torch.from_numpy(a))
        return t.to(device)


def make_swska(name: str = "swska_1p6b", sub: int = 0, **overrides) -> SwskaInputs:
    wl = dataclasses.replace(SWSKA_WORKLOADS[name], **overrides)
    B, T, H = wl.B, wl.T, wl.H

    def draw(tid, shape):
        return _encode(_rng(wl.wid, tid, sub).standard_normal(shape, dtype=np.float32), wl.dtype)

    return SwskaInputs(wl, draw(_Q, (B, T, H, wl.dk)), draw(_K, (B, T, wl.dk)),
                       draw(_V, (B, T, H, wl.dv)))
