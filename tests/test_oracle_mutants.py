"""CPU test: the oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of oracle/ddts_oracle.c (a dropped
term, a wrong sign, a swapped operand, a wrong index, a readout before the
update), compiles it with gcc into a temporary directory and runs every pin
from oracle_pins.py against it.  At least one pin must fail for every mutant.
The real oracle is never modified.
"""
import ctypes
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle_pins as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ddts_oracle.c")

UPDATE_MARK = "        /* S <- diag(alpha) S + k' v'^T */\n"
READ_MARK = "        /* o_t = S_t^T q_t, summed over i in ascending order */\n"
READ_END = "            o[j] = acc;\n        }\n"


def _readout_first(src):
    a = src.index(UPDATE_MARK)
    b = src.index(READ_MARK)
    c = src.index(READ_END, b) + len(READ_END)
    return src[:a] + src[b:c] + src[a:b] + src[c:]


MUTANTS = {
    "forget_sign": [("a[i] = exp(-gi * ti);", "a[i] = exp(gi * ti);")],
    "forget_no_tau": [("a[i] = exp(-gi * ti);", "a[i] = exp(-gi);")],
    "forget_missing": [("Si[j] = a[i] * Si[j] + kk[i] * vv[j];",
                        "Si[j] = Si[j] + kk[i] * vv[j];")],
    "forget_on_input_too": [("Si[j] = a[i] * Si[j] + kk[i] * vv[j];",
                             "Si[j] = a[i] * (Si[j] + kk[i] * vv[j]);")],
    "input_gate_swapped": [("pow(gi, ti)", "pow(ti, gi)")],
    "input_gate_missing": [("kk[i] = pow(gi, ti) * J->k[rk + i];", "kk[i] = J->k[rk + i];")],
    "input_gate_on_q": [("kk[i] = pow(gi, ti) * J->k[rk + i];", "kk[i] = J->k[rk + i];"),
                        ("acc += J->q[rk + i] * S", "acc += pow(J->g[rk + i], J->tau[rk + i]) * J->q[rk + i] * S")],
    "beta_missing": [("vv[j] = J->beta_hat[rv + j] * J->v[rv + j];", "vv[j] = J->v[rv + j];")],
    "beta_on_k_side": [("vv[j] = J->beta_hat[rv + j] * J->v[rv + j];", "vv[j] = J->v[rv + j];"),
                       ("kk[i] = pow(gi, ti) * J->k[rk + i];",
                        "kk[i] = pow(gi, ti) * J->beta_hat[rv + (i % dv)] * J->k[rk + i];")],
    "initial_state_ignored": [("if (J->S0)\n", "if (0)\n")],
    "q_from_next_token": [("acc += J->q[rk + i] *",
                           "acc += J->q[rk + i + (t + 1 < T ? (size_t)H * dk : 0)] *")],
    "readout_before_update": "readout_first",
    "write_uses_k_of_previous_token": [("kk[i] = pow(gi, ti) * J->k[rk + i];",
                                        "kk[i] = pow(gi, ti) * J->k[rk + i - (t > 0 ? (size_t)H * dk : 0)];")],
}


def _fwd_for(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    lib.ddts_oracle_fwd.restype = ctypes.c_int
    lib.ddts_oracle_fwd.argtypes = [ctypes.c_int] * 5 + [dp] * 9 + [ctypes.c_int]

    def ptr(a):
        return dp() if a is None else a.ctypes.data_as(dp)

    def fwd(q, k, v, g, tau, beta, S0=None):
        q, k, v, g, tau, beta = (np.ascontiguousarray(x, np.float64) for x in (q, k, v, g, tau, beta))
        S0 = None if S0 is None else np.ascontiguousarray(S0, np.float64)
        B, T, H, dk = q.shape
        dv = v.shape[3]
        out = np.empty((B, T, H, dv))
        sf = np.empty((B, H, dk, dv))
        rc = lib.ddts_oracle_fwd(B, T, H, dk, dv, ptr(q), ptr(k), ptr(g), ptr(tau), ptr(v),
                                 ptr(beta), ptr(S0), ptr(out), ptr(sf), 1)
        assert rc > 0
        return out, sf
    return fwd


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    src = open(SRC).read()
    m = MUTANTS[name]
    if m == "readout_first":
        mutated = _readout_first(src)
    else:
        mutated = src
        for old, new in m:
            assert old in mutated, f"mutation anchor not found: {old!r}"
            mutated = mutated.replace(old, new)
    assert mutated != src
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "m.c")
        so = os.path.join(d, "m.so")
        open(c, "w").write(mutated)
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                               "-pthread", "-o", so, c, "-lm"])
        fwd = _fwd_for(ctypes.CDLL(so))
        failed = []
        for pin in P.ALL_PINS:
            try:
                ok, _ = pin(fwd)
            except Exception:
                ok = False
            if not ok:
                failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"


# mistakes planted in the reverse mode (the forward left intact); the
# finite-difference pin of tests/test_oracle_bwd.py must catch each
BWD_MUTANTS = {
    "bwd_no_decay_of_adjoint": [("                    D[(size_t)i * dv + j] *= a[i];\n", "")],
    "bwd_dq_from_previous_state": [("acc += St[(size_t)i * dv + j] * dot[j];",
                                    "acc += Sp[(size_t)i * dv + j] * dot[j];")],
    "bwd_dalpha_from_current_state": [("accs += D[(size_t)i * dv + j] * Sp[(size_t)i * dv + j];",
                                       "accs += D[(size_t)i * dv + j] * St[(size_t)i * dv + j];")],
    "bwd_dk_without_gate": [("J->dk_[rk + i] = ah[i] * dkk[i];", "J->dk_[rk + i] = dkk[i];")],
    "bwd_dg_alpha_sign": [("double dgi = -ti * a[i] * da[i], dti = -gi * a[i] * da[i];",
                           "double dgi = ti * a[i] * da[i], dti = -gi * a[i] * da[i];")],
    "bwd_dtau_no_log": [("dti += log(gi) * ah[i] * dah;", "dti += ah[i] * dah;")],
    "bwd_dbeta_uses_beta": [("J->dbeta[rv + j] = J->v[rv + j] * dvv[j];",
                             "J->dbeta[rv + j] = J->beta_hat[rv + j] * dvv[j];")],
    "bwd_readout_adjoint_after_use": [(
        "            for (int i = 0; i < dk; ++i)\n                for (int j = 0; j < dv; ++j)\n"
        "                    D[(size_t)i * dv + j] += qt[i] * dot[j];\n", "")],
}


def _bwd_fd_error(lib):
    """Largest relative mismatch between the library's reverse mode and central
    finite differences of its forward, on a small random case."""
    dp = ctypes.POINTER(ctypes.c_double)
    lib.ddts_oracle_fwd.restype = ctypes.c_int
    lib.ddts_oracle_fwd.argtypes = [ctypes.c_int] * 5 + [dp] * 9 + [ctypes.c_int]
    lib.ddts_oracle_bwd.restype = ctypes.c_int
    lib.ddts_oracle_bwd.argtypes = [ctypes.c_int] * 5 + [dp] * 16 + [ctypes.c_int]
    ptr = lambda a: dp() if a is None else a.ctypes.data_as(dp)
    rng = np.random.default_rng(31)
    B, T, H, dk, dv = 1, 6, 1, 3, 2
    q, k, v = (rng.standard_normal((B, T, H, d)) for d in (dk, dk, dv))
    g, tau = 0.2 + 0.7 * rng.random((B, T, H, dk)), 0.1 + 0.8 * rng.random((B, T, H, dk))
    beta = rng.random((B, T, H, dv))
    S0, W, V = rng.standard_normal((B, H, dk, dv)), rng.standard_normal((B, T, H, dv)), rng.standard_normal((B, H, dk, dv))
    ins = [q, k, g, tau, v, beta]

    def loss():
        out, sf = np.empty((B, T, H, dv)), np.empty((B, H, dk, dv))
        assert lib.ddts_oracle_fwd(B, T, H, dk, dv, *(ptr(x) for x in ins), ptr(S0), ptr(out), ptr(sf), 1) > 0
        return float(np.sum(W * out) + np.sum(V * sf))

    grads = [np.empty_like(x) for x in ins] + [np.empty_like(S0)]
    assert lib.ddts_oracle_bwd(B, T, H, dk, dv, *(ptr(x) for x in ins), ptr(S0), ptr(W), ptr(V),
                               *(ptr(gr) for gr in grads), 1) > 0
    worst, h = 0.0, 1e-6
    for x, gr in zip(ins + [S0], grads[:6] + [grads[6]]):
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + h
            lp = loss()
            x[idx] = keep - h
            lm = loss()
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        worst = max(worst, float(np.max(np.abs(fd - gr)) / np.sqrt(np.mean(fd * fd))))
    return worst


def _build(src, d):
    c, so = os.path.join(d, "m.c"), os.path.join(d, "m.so")
    open(c, "w").write(src)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                           "-pthread", "-o", so, c, "-lm"])
    return ctypes.CDLL(so)


def test_bwd_pin_accepts_the_real_oracle():
    with tempfile.TemporaryDirectory() as d:
        assert _bwd_fd_error(_build(open(SRC).read(), d)) < 1e-6


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_bwd_mutant_is_caught(name):
    src = open(SRC).read()
    mutated = src
    for old, new in BWD_MUTANTS[name]:
        assert mutated.count(old) == 1, f"mutation anchor not unique: {old!r}"
        mutated = mutated.replace(old, new)
    with tempfile.TemporaryDirectory() as d:
        err = _bwd_fd_error(_build(mutated, d))
    assert err > 1e-3, f"mutant {name} passed the finite-difference pin ({err})"
