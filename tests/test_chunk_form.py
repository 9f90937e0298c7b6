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
(three products) meet it by two orders of magnitude.
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
