"""CPU pins of the fp64 reverse-mode oracle (``oracle.bwd``).

The backward oracle is written out from the recurrence (adjoint state walked
from t = T down to 1).  It is pinned here by things that do not share its
derivation: central finite differences of the forward oracle, the closed-form
gradients of the tau = 0 case (plain causal linear attention, by numpy
matmuls), and two exact identities (dg = 0 wherever tau = 0; with no tokens
the initial-state gradient is the final-state gradient).
"""
import numpy as np
import pytest

import oracle_pins as P

NAMES = ("q", "k", "v", "g", "tau", "beta_hat")


def loss_and_weights(rng, B, T, H, dk, dv):
    W = rng.standard_normal((B, T, H, dv))
    V = rng.standard_normal((B, H, dk, dv))
    return W, V


def rand_case(seed, B=2, T=7, H=2, dk=3, dv=2):
    rng = np.random.default_rng(seed)
    q, k, v, g, tau, beta, S0 = P.rand_inputs(rng, B, T, H, dk, dv)
    g = 0.2 + 0.7 * rng.random(g.shape)          # away from g = 0 for finite differences
    tau = 0.1 + 0.8 * rng.random(tau.shape)
    W, V = loss_and_weights(rng, B, T, H, dk, dv)
    return dict(q=q, k=k, v=v, g=g, tau=tau, beta_hat=beta), S0, W, V


def L(oracle_mod, ins, S0, W, V):
    o, s = oracle_mod.fwd(*(ins[n] for n in NAMES), S0)
    return float(np.sum(W * o) + np.sum(V * s))


def test_bwd_matches_finite_differences(oracle_mod):
    ins, S0, W, V = rand_case(11)
    gr = oracle_mod.bwd(*(ins[n] for n in NAMES), W, S0, V)
    h = 1e-6
    names = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "tau": "dtau", "beta_hat": "dbeta_hat"}
    for n, dn in names.items():
        x = ins[n]
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + h
            lp = L(oracle_mod, ins, S0, W, V)
            x[idx] = keep - h
            lm = L(oracle_mod, ins, S0, W, V)
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(fd - gr[dn])) / np.sqrt(np.mean(fd * fd))
        assert err < 1e-6, (n, err)
    fd = np.empty_like(S0)
    for idx in np.ndindex(S0.shape):
        keep = S0[idx]
        S0[idx] = keep + h
        lp = L(oracle_mod, ins, S0, W, V)
        S0[idx] = keep - h
        lm = L(oracle_mod, ins, S0, W, V)
        S0[idx] = keep
        fd[idx] = (lp - lm) / (2 * h)
    err = np.max(np.abs(fd - gr["d_initial_state"])) / np.sqrt(np.mean(fd * fd))
    assert err < 1e-6, ("S0", err)


def test_bwd_tau0_is_linear_attention(oracle_mod):
    """tau = 0: alpha = alpha_hat = 1, o = tril(Q K^T) V' + Q S0 and
    S_T = S0 + K^T V'; gradients by numpy matmuls."""
    ins, S0, W, V = rand_case(12, B=1, T=9, H=1, dk=4, dv=3)
    ins["tau"][:] = 0.0
    gr = oracle_mod.bwd(*(ins[n] for n in NAMES), W, S0, V)
    Q, K = ins["q"][0, :, 0], ins["k"][0, :, 0]
    Vp = ins["beta_hat"][0, :, 0] * ins["v"][0, :, 0]
    dO, S, dS = W[0, :, 0], S0[0, 0], V[0, 0]
    M = np.tril(dO @ Vp.T)                      # M[t, s] = dO_t . v'_s, s <= t
    dQ = M @ K + dO @ S.T
    dK = M.T @ Q + Vp @ dS.T
    dVp = np.tril(Q @ K.T).T @ dO + K @ dS
    dS0 = Q.T @ dO + dS
    chk = lambda a, b: np.max(np.abs(a - b)) / np.sqrt(np.mean(b * b))
    assert chk(gr["dq"][0, :, 0], dQ) < 1e-12
    assert chk(gr["dk"][0, :, 0], dK) < 1e-12
    assert chk(gr["dv"][0, :, 0], ins["beta_hat"][0, :, 0] * dVp) < 1e-12
    assert chk(gr["dbeta_hat"][0, :, 0], ins["v"][0, :, 0] * dVp) < 1e-12
    assert chk(gr["d_initial_state"][0, 0], dS0) < 1e-12
    assert np.all(gr["dg"] == 0.0)


def test_bwd_no_tokens(oracle_mod):
    ins, S0, W, V = rand_case(13, T=0)
    gr = oracle_mod.bwd(*(ins[n] for n in NAMES), W, S0, V)
    assert np.array_equal(gr["d_initial_state"], V)


def test_bwd_thread_invariance(oracle_mod):
    ins, S0, W, V = rand_case(14, B=3, T=70, H=2, dk=5, dv=4)
    g1 = oracle_mod.bwd(*(ins[n] for n in NAMES), W, S0, V, nthreads=1)
    g6 = oracle_mod.bwd(*(ins[n] for n in NAMES), W, S0, V, nthreads=6)
    for n in g1:
        assert np.array_equal(g1[n], g6[n])
