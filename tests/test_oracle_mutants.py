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
