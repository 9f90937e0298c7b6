"""Pins for the fp64 oracle, written as functions of an oracle ``fwd`` callable.

Each check ties the oracle to something other than itself: a brute-force
quadratic form built from products of the forget gate (no recurrence), a
library matmul in special cases that reduce to plain causal linear attention,
a division-based closed form of the scalar recurrence, hand-checkable gate
values, and invariants (g = 0, linearity, carry-over).  They are shared by
tests/test_oracle_pins.py (the real oracle) and tests/test_oracle_mutants.py
(deliberately broken copies, which must fail at least one pin).

Gate definitions used as ground truth (Rodimus* digest page, section
"Method"): alpha = exp(-g * tau) and alpha_hat = g ** tau, both along dk; the
value-side gate beta_hat multiplies v (same section, low-rank bullet).
"""
import math

import numpy as np

RTOL = 1e-12


def relerr(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    rms = math.sqrt(float(np.mean(b * b))) or 1.0
    return float(np.max(np.abs(a - b))) / rms


def rand_inputs(rng, B, T, H, dk, dv, s0=True, gate_lo=0.0, gate_hi=1.0):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    g = rng.uniform(gate_lo, gate_hi, (B, T, H, dk))
    tau = rng.uniform(gate_lo, gate_hi, (B, T, H, dk))
    beta = rng.uniform(0.0, 1.0, (B, T, H, dv))
    S0 = rng.standard_normal((B, H, dk, dv)) if s0 else None
    return q, k, v, g, tau, beta, S0


def brute_force(q, k, v, g, tau, beta, S0):
    """o_t[j] = sum_{s<=t} sum_i q_t[i] (prod_{r=s+1..t} alpha_r[i]) k'_s[i] v'_s[j]
              + sum_i q_t[i] (prod_{r<=t} alpha_r[i]) S0[i, j]
    materialised per (b, h); products of alpha, never a recurrence."""
    B, T, H, dk = q.shape
    dv = v.shape[3]
    out = np.zeros((B, T, H, dv))
    alpha = np.exp(-g * tau)
    kp = np.power(g, tau) * k
    vp = beta * v
    for b in range(B):
        for h in range(H):
            for t in range(T):
                acc = np.zeros(dv)
                for s in range(t + 1):
                    decay = np.ones(dk)
                    for r in range(s + 1, t + 1):
                        decay = decay * alpha[b, r, h]
                    w = np.sum(q[b, t, h] * decay * kp[b, s, h])
                    acc = acc + w * vp[b, s, h]
                if S0 is not None:
                    decay = np.ones(dk)
                    for r in range(0, t + 1):
                        decay = decay * alpha[b, r, h]
                    acc = acc + (q[b, t, h] * decay) @ S0[b, h]
                out[b, t, h] = acc
    return out


# ---------------------------------------------------------------- the pins


def pin_bruteforce(fwd, seed=0):
    rng = np.random.default_rng(seed)
    worst = 0.0
    for (B, T, H, dk, dv) in [(1, 9, 1, 1, 1), (1, 13, 2, 3, 5), (2, 7, 1, 5, 3),
                              (1, 20, 1, 16, 3), (1, 6, 3, 4, 16)]:
        ins = rand_inputs(rng, B, T, H, dk, dv)
        o, _ = fwd(*ins)
        worst = max(worst, relerr(o, brute_force(*ins)))
    return worst <= RTOL, worst


def pin_attention_tau0(fwd, seed=1):
    """tau = 0: alpha = 1 and alpha_hat = g**0 = 1; with beta_hat = 1 the op is
    causal linear attention, o = tril(Q K^T) V + Q S0 (numpy matmul)."""
    rng = np.random.default_rng(seed)
    B, T, H, dk, dv = 2, 17, 2, 6, 5
    q, k, v, g, tau, beta, S0 = rand_inputs(rng, B, T, H, dk, dv)
    tau = np.zeros_like(tau)
    beta = np.ones_like(beta)
    o, sf = fwd(q, k, v, g, tau, beta, S0)
    ref = np.empty_like(o)
    sref = np.empty_like(S0)
    for b in range(B):
        for h in range(H):
            Q, K, V = q[b, :, h], k[b, :, h], v[b, :, h]
            ref[b, :, h] = np.tril(Q @ K.T) @ V + Q @ S0[b, h]
            sref[b, h] = S0[b, h] + K.T @ V
    err = max(relerr(o, ref), relerr(sf, sref))
    return err <= RTOL, err


def pin_g_zero(fwd, seed=2):
    """g = 0: alpha = 1 and alpha_hat = 0**tau = 0 (tau > 0): nothing is
    written and nothing forgotten, so S stays S0 and o_t = S0^T q_t."""
    rng = np.random.default_rng(seed)
    B, T, H, dk, dv = 1, 11, 2, 4, 7
    q, k, v, g, tau, beta, S0 = rand_inputs(rng, B, T, H, dk, dv, gate_lo=0.1)
    g = np.zeros_like(g)
    o, sf = fwd(q, k, v, g, tau, beta, S0)
    ref = np.einsum("bthi,bhij->bthj", q, S0)
    err = max(relerr(o, ref), float(np.max(np.abs(sf - S0))))
    return err <= RTOL, err


def pin_constant_gates(fwd, seed=3):
    """g, tau constant: alpha = gamma = exp(-g tau) and alpha_hat = c = g**tau
    for every token, so o = (tril(Q K^T) * D) (c beta_hat * V) + diag(gamma^t) Q S0
    with D[t, s] = gamma^(t - s)."""
    rng = np.random.default_rng(seed)
    B, T, H, dk, dv = 1, 15, 1, 5, 4
    q, k, v, g, tau, beta, S0 = rand_inputs(rng, B, T, H, dk, dv)
    gv, tv = 0.7, 0.45
    g = np.full_like(g, gv)
    tau = np.full_like(tau, tv)
    gamma, c = math.exp(-gv * tv), gv ** tv
    o, _ = fwd(q, k, v, g, tau, beta, S0)
    t_idx = np.arange(T)
    D = np.tril(gamma ** (t_idx[:, None] - t_idx[None, :]).clip(min=0))
    Q, K, V, Bt = q[0, :, 0], k[0, :, 0], v[0, :, 0], beta[0, :, 0]
    ref = (np.tril(Q @ K.T) * D) @ (c * Bt * V) + (gamma ** (t_idx + 1))[:, None] * (Q @ S0[0, 0])
    err = relerr(o[0, :, 0], ref)
    return err <= RTOL, err


def pin_scalar_division_form(fwd, seed=4):
    """dk = dv = 1: s_t = a_t s_{t-1} + x_t solves to s_t = P_t (s_0 + sum_{r<=t} x_r / P_r)
    with P_t = prod_{r<=t} a_r; o_t = q_t s_t."""
    rng = np.random.default_rng(seed)
    T = 40
    q, k, v, g, tau, beta, S0 = rand_inputs(rng, 1, T, 1, 1, 1, gate_lo=0.05, gate_hi=0.6)
    o, sf = fwd(q, k, v, g, tau, beta, S0)
    a = np.exp(-g[0, :, 0, 0] * tau[0, :, 0, 0])
    x = (g[0, :, 0, 0] ** tau[0, :, 0, 0]) * k[0, :, 0, 0] * beta[0, :, 0, 0] * v[0, :, 0, 0]
    P = np.cumprod(a)
    s = P * (S0[0, 0, 0, 0] + np.cumsum(x / P))
    err = max(relerr(o[0, :, 0, 0], q[0, :, 0, 0] * s), abs(sf[0, 0, 0, 0] - s[-1]) / abs(s[-1]))
    return err <= 1e-10, err


def pin_gate_values(fwd):
    """Hand-checkable gate values, dk = dv = 1, q = k = v = beta_hat = 1, S0 = 0:
    token 1 with g = 1/4, tau = 1/2 writes alpha_hat = 1/2, so o_1 = 1/2;
    token 2 with g = 1/2, tau = 2 ln 2 forgets with alpha = exp(-ln 2) = 1/2 and
    writes alpha_hat = (1/2)^(2 ln 2), so o_2 = 1/4 + 2^(-2 ln 2);
    token 3 with g = 0, tau = 0 forgets nothing (alpha = 1) and writes 0^0 = 1."""
    one = np.ones((1, 3, 1, 1))
    g = np.array([0.25, 0.5, 0.0]).reshape(1, 3, 1, 1)
    tau = np.array([0.5, 2.0 * math.log(2.0), 0.0]).reshape(1, 3, 1, 1)
    o, _ = fwd(one, one, one, g, tau, one, None)
    o2 = 0.25 + 2.0 ** (-2.0 * math.log(2.0))
    want = np.array([0.5, o2, o2 + 1.0])
    err = float(np.max(np.abs(o[0, :, 0, 0] - want)))
    return err <= 1e-15, err


def pin_linearity(fwd, seed=5):
    """o is linear in (v, S0) jointly and homogeneous in q; heads are independent."""
    rng = np.random.default_rng(seed)
    B, T, H, dk, dv = 1, 12, 3, 4, 6
    q, k, v, g, tau, beta, S0 = rand_inputs(rng, B, T, H, dk, dv)
    o, _ = fwd(q, k, v, g, tau, beta, S0)
    o_v, _ = fwd(q, k, v, g, tau, beta, np.zeros_like(S0))
    o_s, _ = fwd(q, k, np.zeros_like(v), g, tau, beta, S0)
    e1 = relerr(o, o_v + o_s)
    o2, _ = fwd(2.0 * q, k, v, g, tau, beta, S0)
    e2 = float(np.max(np.abs(o2 - 2.0 * o)))
    perm = [2, 0, 1]
    op, _ = fwd(q[:, :, perm], k[:, :, perm], v[:, :, perm], g[:, :, perm],
                tau[:, :, perm], beta[:, :, perm], S0[:, perm])
    e3 = float(np.max(np.abs(op - o[:, :, perm])))
    ok = e1 <= RTOL and e2 == 0.0 and e3 == 0.0
    return ok, max(e1, e2, e3)


def pin_carry_over(fwd, seed=6):
    """Running T tokens at once equals running T1 tokens, carrying S_T1 as the
    next call's initial state, then the remaining tokens: bitwise in fp64."""
    rng = np.random.default_rng(seed)
    B, T, H, dk, dv = 2, 23, 2, 5, 3
    q, k, v, g, tau, beta, S0 = rand_inputs(rng, B, T, H, dk, dv)
    o, sf = fwd(q, k, v, g, tau, beta, S0)
    T1 = 9
    sl = lambda a, s: np.ascontiguousarray(a[:, s])
    a_, s1 = fwd(*(sl(x, slice(0, T1)) for x in (q, k, v, g, tau, beta)), S0)
    b_, s2 = fwd(*(sl(x, slice(T1, T)) for x in (q, k, v, g, tau, beta)), s1)
    ok = np.array_equal(np.concatenate([a_, b_], 1), o) and np.array_equal(s2, sf)
    return ok, 0.0 if ok else 1.0


ALL_PINS = [pin_bruteforce, pin_attention_tau0, pin_g_zero, pin_constant_gates,
            pin_scalar_division_form, pin_gate_values, pin_linearity, pin_carry_over]
