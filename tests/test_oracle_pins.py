"""CPU tests: the fp64 oracle against its pins (no GPU needed)."""
import os

import numpy as np
import pytest

import oracle_pins as P

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle_mod, pin):
    ok, err = pin(oracle_mod.fwd)
    assert ok, f"{pin.__name__}: error {err}"


def test_thread_count_invariance(oracle_mod):
    rng = np.random.default_rng(7)
    ins = P.rand_inputs(rng, 3, 31, 5, 8, 6)
    o1, s1 = oracle_mod.fwd(*ins, nthreads=1)
    o8, s8 = oracle_mod.fwd(*ins, nthreads=8)
    assert np.array_equal(o1, o8) and np.array_equal(s1, s8)


def test_decode_is_one_step_of_fwd(oracle_mod):
    """The decode oracle applied to a resident state equals the forward oracle
    with T = 1 started from that state (bitwise), and T decode steps equal
    one T-token forward (bitwise)."""
    rng = np.random.default_rng(8)
    N, T, H, dk, dv = 3, 6, 2, 5, 4
    q, k, v, g, tau, beta, S0 = P.rand_inputs(rng, N, T, H, dk, dv)
    of, sf = oracle_mod.fwd(q, k, v, g, tau, beta, S0)
    st = S0.copy()
    for t in range(T):
        o, st = oracle_mod.decode(q[:, t], k[:, t], v[:, t], g[:, t], tau[:, t], beta[:, t], st)
        assert np.array_equal(o, of[:, t])
    assert np.array_equal(st, sf)


def test_decode_pins(oracle_mod):
    """The decode oracle on its own: g = 0 leaves the state unchanged; tau = 0
    and beta_hat = 1 add k v^T exactly."""
    rng = np.random.default_rng(9)
    N, H, dk, dv = 4, 3, 5, 6
    q = rng.standard_normal((N, H, dk)); k = rng.standard_normal((N, H, dk))
    v = rng.standard_normal((N, H, dv)); S = rng.standard_normal((N, H, dk, dv))
    tau = rng.uniform(0.1, 1, (N, H, dk)); beta = rng.uniform(0, 1, (N, H, dv))
    o, s1 = oracle_mod.decode(q, k, v, np.zeros_like(q), tau, beta, S)
    assert np.array_equal(s1, S)
    assert P.relerr(o, np.einsum("nhi,nhij->nhj", q, S)) < 1e-13
    g = rng.uniform(0.1, 1, (N, H, dk))
    o, s1 = oracle_mod.decode(q, k, v, g, np.zeros_like(tau), np.ones_like(beta), S)
    want = S + k[..., :, None] * v[..., None, :]
    assert P.relerr(s1, want) < 1e-14
    assert P.relerr(o, np.einsum("nhi,nhij->nhj", q, want)) < 1e-13


def test_tiny_workload_fixture(oracle_mod):
    """Regression lock: the oracle's output on the seeded tiny workload equals
    the stored fixture written by tests/golden/make_fixtures.py (which calls
    only the oracle)."""
    import ddts_inputs as D
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle_out.txt")
    want = np.loadtxt(path).reshape(1, 64, 2, 16)
    x = D.make("tiny")
    o, _ = oracle_mod.fwd(x.q, x.k, x.v, x.g, x.tau, x.beta_hat, None)
    assert np.max(np.abs(o - want)) <= 1e-15 * max(1.0, np.max(np.abs(want)))


def test_metric():
    import oracle
    x = np.array([3.0, -4.0])
    assert oracle.rel_to_rms_error(x + np.array([0.0, 0.5]), x) == pytest.approx(0.5 / np.sqrt(12.5))
