"""CPU tests of the chunk form the HIP kernel implements, against the fp64 oracle.

``chunk_form`` below is a plain numpy transcription of the chunkwise identity the
chunk kernel evaluates (for the recurrence of the Rodimus* digest page, section
"Method"; alpha and alpha_hat on the dk rows as on the authors' rebuttal page,
"Efficient Parallelization"): inside a chunk with cumulative log-decay b_u,

    O   = tril(Qt Kt^T) V' + Qt S'
    S_o = diag(exp(b_L)) S_in + diag(exp(b_L - b_m)) Kt^T V'

with Qt = q exp(b_u - b_m), Kt = g^tau k exp(b_m - b_s), V' = beta_hat v,
S' = diag(exp(b_m)) S_in and b_m the cumulative sum at the chunk's middle token.
It shares no code with the kernel.  In fp64 it must equal the token-by-token
oracle to rounding, which pins the derivation; with its matrix-product operands
rounded to bf16 it shows why the kernel splits every operand into two bf16
terms: one term misses the bf16 tolerance (1e-2 max error over RMS), two terms
(three products) meet it by two orders of magnitude.  ``chunk_form_bwd`` does the
same for the backward kernel's identity (its decay gradient is a reverse
cumulative sum, not the token-level adjoint the reverse-mode oracle walks).
"""
import numpy as np
import pytest

import ddts_inputs as D

LOG2E = 1.4426950408889634


def bf16(x):
    """Round to the nearest bf16 (ties to even), returned as float64."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def product(a, b, ns):
    """a @ b with each operand split into ns bf16 terms, keeping the term
    products of total order < ns (ns = 0: exact fp64)."""
    if ns == 0:
        return a @ b
    ta, tb, ra, rb = [], [], a, b
    for _ in range(ns):
        ha, hb = bf16(ra), bf16(rb)
        ta.append(ha)
        tb.append(hb)
        ra, rb = ra - ha, rb - hb
    return sum(ta[i] @ tb[j] for i in range(ns) for j in range(ns) if i + j < ns)


def chunk_form(q, k, v, g, tau, beta, S0, C, ns):
    """One head: q, k, g, tau [T, dk]; v, beta [T, dv]; S0 [dk, dv]."""
    T, dk = q.shape
    dv = v.shape[1]
    S = S0.copy()
    O = np.zeros((T, dv))
    for c0 in range(0, T, C):
        n = min(C, T - c0)
        pad = lambda x: np.concatenate([x[c0:c0 + n], np.zeros((C - n, x.shape[1]))])
        qq, kk, gg, tt, vv, bb = (pad(x) for x in (q, k, g, tau, v, beta))
        b = -LOG2E * np.cumsum(gg * tt, axis=0)              # log2 units
        bm, bL = b[C // 2 - 1], b[C - 1]
        with np.errstate(divide="ignore", invalid="ignore"):
            la = np.where(tt == 0, 0.0, tt * np.log2(gg))    # log2(g ** tau)
        Qt = qq * 2.0 ** (b - bm)
        Kt = kk * 2.0 ** (la - (b - bm))
        Vp = bb * vv
        Sp = (2.0 ** bm)[:, None] * S
        A = np.triu(product(Kt, Qt.T, ns))                   # A[s, u], s <= u
        O[c0:c0 + n] = (product(Qt, Sp, ns) + product(A.T, Vp, ns))[:n]
        S = (2.0 ** bL)[:, None] * S + (2.0 ** (bL - bm))[:, None] * product(Kt.T, Vp, ns)
    return O, S


def run(x, heads, ns, C=64, T=None):
    ins = {n: x.f32(n).astype(np.float64) for n in ("q", "k", "v", "g", "tau", "beta_hat")}
    T = T or x.wl.T
    O = np.zeros((1, T, len(heads), x.wl.dv))
    S = np.zeros((1, len(heads), x.wl.dk, x.wl.dv))
    for j, h in enumerate(heads):
        s0 = np.zeros((x.wl.dk, x.wl.dv)) if x.initial_state is None else x.initial_state[0, h].astype(np.float64)
        O[0, :, j], S[0, j] = chunk_form(*(ins[n][0, :T, h] for n in ("q", "k", "v", "g", "tau", "beta_hat")),
                                         s0, C, ns)
    return O, S


def oracle_heads(oracle_mod, x, heads, T=None):
    T = T or x.wl.T
    sl = lambda n: np.ascontiguousarray(x.f32(n)[:1, :T][:, :, heads])
    s0 = None if x.initial_state is None else np.ascontiguousarray(x.initial_state[:1, heads])
    return oracle_mod.fwd(*(sl(n) for n in ("q", "k", "v", "g", "tau", "beta_hat")), s0)


@pytest.mark.parametrize("wl,C,T", [("tiny", 16, 64), ("layer130m", 64, 200), ("long_prefill", 64, 300)])
def test_chunk_form_equals_recurrence(oracle_mod, wl, C, T):
    """fp64 chunk form == token-by-token oracle (ragged last chunk, initial state);
    the workloads' value distributions at a CPU-sized length."""
    x = D.make(wl, B=1, T=T)
    heads = list(range(min(2, x.wl.H)))
    o, s = run(x, heads, 0, C=C, T=T)
    ro, rs = oracle_heads(oracle_mod, x, heads, T=T)
    assert oracle_mod.rel_to_rms_error(o, ro) < 1e-11
    assert oracle_mod.rel_to_rms_error(s, rs) < 1e-11


def test_bf16_operand_terms(oracle_mod):
    """130M-layer heads: one bf16 term per operand misses the 1e-2 bar, two meet it."""
    x = D.make("layer130m", B=1)
    heads = [0, 1, 2, 3]
    ro, rs = oracle_heads(oracle_mod, x, heads)
    o1, _ = run(x, heads, 1)
    o2, s2 = run(x, heads, 2)
    assert oracle_mod.rel_to_rms_error(o1, ro) > 1e-2
    assert oracle_mod.rel_to_rms_error(o2, ro) < 1e-3
    assert oracle_mod.rel_to_rms_error(s2, rs) < 1e-3


def chunk_form_bwd(q, k, v, g, tau, beta, S0, dO, dSf, C):
    """The backward of the chunk identity as the backward kernel evaluates it
    (one head, fp64): per chunk, from the last to the first, with D = dL/dS_out,
      dA = tril(dO V'^T),  A = tril(Qt Kt^T)
      dQt = diag-cols(e^{b_m}) dO S_in^T + dA Kt
      dKt = diag-cols(e^{b_L - b_m}) V' D^T + dA^T Qt
      dV' = A^T dO + Kt diag(e^{b_L - b_m}) D
      D  <- diag(e^{b_L}) D + diag(e^{b_m}) Qt^T dO
      dlambda_r = sum_{u >= r} (q dq - k' dk')_u + rowsum(S_out * D_out)
    then the elementwise chain rule (g^tau terms 0 at g = 0)."""
    T, dk = q.shape
    dv = v.shape[1]
    # forward states at every chunk start
    states, S = [], S0.copy()
    for c0 in range(0, T, C):
        states.append(S.copy())
        n = min(C, T - c0)
        gt = g[c0:c0 + n] * tau[c0:c0 + n]
        lam = np.cumsum(-gt, axis=0)
        with np.errstate(divide="ignore", invalid="ignore"):
            ah = np.where(tau[c0:c0 + n] == 0, 1.0, g[c0:c0 + n] ** tau[c0:c0 + n])
        kp = ah * k[c0:c0 + n]
        vp = beta[c0:c0 + n] * v[c0:c0 + n]
        S = np.exp(lam[-1])[:, None] * S + (np.exp(lam[-1] - lam) * kp).T @ vp
    out = {n_: np.zeros_like(x) for n_, x in (("dq", q), ("dk", k), ("dg", g), ("dtau", tau),
                                               ("dv", v), ("dbeta_hat", beta))}
    D = dSf.copy()
    S_out = S
    for ci in range(len(states) - 1, -1, -1):
        c0 = ci * C
        n = min(C, T - c0)
        sl = slice(c0, c0 + n)
        gg, tt, qq, kk, vv, bb, do = g[sl], tau[sl], q[sl], k[sl], v[sl], beta[sl], dO[sl]
        b = np.cumsum(-gg * tt, axis=0)
        m = min(C // 2 - 1, n - 1)           # the reference token (any choice gives the same)
        bm, bL = b[m], b[-1]
        with np.errstate(divide="ignore", invalid="ignore"):
            ah = np.where(tt == 0, 1.0, gg ** tt)
        kp, Vp = ah * kk, bb * vv
        Qt, Kt = qq * np.exp(b - bm), kp * np.exp(bm - b)
        S_in = states[ci]
        A = np.tril(Qt @ Kt.T)
        dA = np.tril(do @ Vp.T)
        f = np.exp(bL - bm)
        dQt = np.exp(bm)[None, :] * (do @ S_in.T) + dA @ Kt
        dKt = f[None, :] * (Vp @ D.T) + dA.T @ Qt
        dVp = A.T @ do + (Kt * f[None, :]) @ D
        rs = np.sum(S_out * D, axis=1)
        D = np.exp(bL)[:, None] * D + np.exp(bm)[:, None] * (Qt.T @ do)
        dq = np.exp(b - bm) * dQt
        dkp = np.exp(bm - b) * dKt
        dlam = np.cumsum((qq * dq - kp * dkp)[::-1], axis=0)[::-1] + rs[None, :]
        dah = kk * dkp
        with np.errstate(divide="ignore", invalid="ignore"):
            pos = gg > 0
            dg_ah = np.where(pos, tt * ah / np.where(pos, gg, 1.0), 0.0)
            dt_ah = np.where(pos, ah * np.log(np.where(pos, gg, 1.0)), 0.0)
        out["dq"][sl], out["dk"][sl] = dq, ah * dkp
        out["dv"][sl], out["dbeta_hat"][sl] = bb * dVp, vv * dVp
        out["dg"][sl] = -tt * dlam + dg_ah * dah
        out["dtau"][sl] = -gg * dlam + dt_ah * dah
        S_out = S_in
    out["d_initial_state"] = D
    return out


@pytest.mark.parametrize("wl,T,C", [("tiny", 37, 16), ("layer130m", 100, 16), ("long_prefill", 70, 32)])
def test_chunk_form_backward_equals_reverse_mode(oracle_mod, wl, T, C):
    """fp64 backward chunk identity (with the reverse-cumulative-sum decay
    gradient) == the token-level reverse-mode oracle."""
    x = D.make(wl, B=1, T=T)
    rng = np.random.default_rng(21)
    H = min(2, x.wl.H)
    dO = rng.standard_normal((1, T, x.wl.H, x.wl.dv))
    dSf = rng.standard_normal((1, x.wl.H, x.wl.dk, x.wl.dv))
    S0 = (np.zeros((1, x.wl.H, x.wl.dk, x.wl.dv)) if x.initial_state is None
          else x.initial_state.astype(np.float64))
    ins = {n: x.f32(n).astype(np.float64) for n in ("q", "k", "v", "g", "tau", "beta_hat")}
    ins["g"][0, :5, 0, :3] = 0.0                      # g = 0 edge
    ins["tau"][0, 5:9, 0, 3:6] = 0.0                  # tau = 0 edge
    ref = oracle_mod.bwd(*(ins[n] for n in ("q", "k", "v", "g", "tau", "beta_hat")), dO, S0, dSf)
    for h in range(H):
        got = chunk_form_bwd(*(ins[n][0, :, h] for n in ("q", "k", "v", "g", "tau", "beta_hat")),
                             S0[0, h], dO[0, :, h], dSf[0, h], C)
        for n in ("dq", "dk", "dv", "dbeta_hat", "dg", "dtau"):
            assert oracle_mod.rel_to_rms_error(got[n], ref[n][0, :, h]) < 1e-10, (n, h)
        assert oracle_mod.rel_to_rms_error(got["d_initial_state"], ref["d_initial_state"][0, h]) < 1e-10
