"""Pins for the fp64 oracle of the steps fused around the recurrence, written
as functions of an oracle module (the real one, or a copy with a planted
mistake in tests/test_oracle_fused.py, which must fail at least one pin).

What pins each function (the pages give these steps no formulas; the
readings are those stated in the oracle):
 - lowrank_beta: values computed by hand for a rank-2, three-column example
   over two heads with different factors, sigmoid(0) = 1/2, and the
   saturation limits;
 - short_conv: the impulse response (tap j appears j tokens after the
   impulse, only in the impulse's channel), the history rows, and splitting a
   sequence with the window carried over;
 - fwd_fused / decode_fused: q = 0 leaves exactly d * v; a one-tap unit filter
   with d = 0 reduces to the plain recurrence; a split sequence with the
   convolution window and the state carried over equals the whole; decode
   steps over rolling windows equal the fused forward.
"""
import math

import numpy as np


def relerr(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    rms = math.sqrt(float(np.mean(b * b))) or 1.0
    return float(np.max(np.abs(a - b))) / rms


def sig(x):
    return 1.0 / (1.0 + math.exp(-x))


def pin_lowrank_hand_values(O):
    # head 0: u = (1, -1), W = [[1, 2, 0], [0.5, 0, -1]] -> z = (0.5, 2, 1)
    # head 1: u = (2, 0.5), W = [[0, -1, 1], [4, 2, 0]]  -> z = (2, -1, 2)
    u = np.array([[[[1.0, -1.0], [2.0, 0.5]]]])                 # [1, 1, 2, 2]
    w = np.array([[[1.0, 2.0, 0.0], [0.5, 0.0, -1.0]],
                  [[0.0, -1.0, 1.0], [4.0, 2.0, 0.0]]])         # [2, 2, 3]
    got = O.lowrank_beta(u, w)
    want = np.array([[0.6224593312018546, 0.8807970779778823, 0.7310585786300049],
                     [0.8807970779778823, 0.2689414213699951, 0.8807970779778823]])
    assert got.shape == (1, 1, 2, 3)
    assert np.max(np.abs(got[0, 0] - want)) < 1e-15
    # sigmoid(0) = 1/2 exactly; saturation towards 1 and 0
    assert np.all(O.lowrank_beta(np.zeros((1, 1, 2, 2)), w) == 0.5)
    one = O.lowrank_beta(np.array([[[[40.0]]]]), np.array([[[1.0, -1.0]]]))
    assert one[0, 0, 0, 0] == 1.0 and 0.0 < one[0, 0, 0, 1] < 1e-17


def pin_conv_impulse(O):
    rng = np.random.default_rng(5)
    for W in (1, 2, 3, 4):
        T, H, D = 9, 2, 3
        c = rng.standard_normal((H, D, W))
        x = np.zeros((1, T + W - 1, H, D))
        s, h, i = 3, 1, 2
        x[0, W - 1 + s, h, i] = 1.0                     # raw token s
        y = O.short_conv(x, c)
        assert y.shape == (1, T, H, D)
        want = np.zeros((1, T, H, D))
        for j in range(W):
            if s + j < T:
                want[0, s + j, h, i] = c[h, i, j]
        assert np.array_equal(y, want), W
        # a history row (raw token -1) reaches tokens 0 .. W - 2
        if W > 1:
            x = np.zeros((1, T + W - 1, H, D))
            x[0, W - 2, 0, 0] = 1.0
            y = O.short_conv(x, c)
            for t in range(T):
                exp = c[0, 0, t + 1] if t + 1 < W else 0.0
                assert y[0, t, 0, 0] == exp


def pin_conv_carry(O):
    rng = np.random.default_rng(6)
    W, T1, T2, H, D = 4, 7, 5, 2, 3
    c = rng.standard_normal((H, D, W))
    x = rng.standard_normal((2, W - 1 + T1 + T2, H, D))
    whole = O.short_conv(x, c)
    first = O.short_conv(x[:, :W - 1 + T1], c)
    second = O.short_conv(x[:, T1:], c)                 # the last W - 1 rows of part 1 as history
    assert np.array_equal(np.concatenate([first, second], axis=1), whole)


def _rand(rng, B, T, H, dk, dv, r, W):
    q = rng.standard_normal((B, T + W - 1, H, dk))
    k = rng.standard_normal((B, T + W - 1, H, dk))
    v = rng.standard_normal((B, T + W - 1, H, dv))
    g = rng.uniform(0.0, 1.0, (B, T, H, dk))
    tau = rng.uniform(0.0, 1.0, (B, T, H, dk))
    u = rng.standard_normal((B, T, H, r))
    w = rng.standard_normal((H, r, dv))
    d = rng.standard_normal((H, dv))
    conv = tuple(rng.standard_normal((H, n, W)) for n in (dk, dk, dv))
    s0 = rng.standard_normal((B, H, dk, dv))
    return q, k, v, g, tau, u, w, d, conv, s0


def pin_fused_feedthrough(O):
    rng = np.random.default_rng(7)
    q, k, v, g, tau, u, w, d, conv, s0 = _rand(rng, 2, 6, 2, 3, 4, 2, 1)
    o, _ = O.fwd_fused(np.zeros_like(q), k, v, g, tau, u=u, w=w, d=d, initial_state=s0)
    assert np.array_equal(o, d[None, None] * v)
    # with the convolution, q = 0 leaves d times the convolved v
    q, k, v, g, tau, u, w, d, conv, s0 = _rand(rng, 1, 5, 2, 3, 4, 2, 3)
    o, _ = O.fwd_fused(np.zeros_like(q), k, v, g, tau, u=u, w=w, d=d, conv=conv, initial_state=s0)
    vc = np.zeros((1, 5, 2, 4))
    for t in range(5):
        for j in range(3):
            vc[0, t] += conv[2][:, :, j] * v[0, t + 2 - j]
    assert relerr(o, d[None, None] * vc) < 1e-14


def pin_fused_reduces_to_plain(O):
    rng = np.random.default_rng(8)
    q, k, v, g, tau, u, w, d, conv, s0 = _rand(rng, 2, 9, 2, 3, 4, 3, 1)
    ones = tuple(np.ones_like(c) for c in conv)
    beta = O.lowrank_beta(u, w)
    o1, s1 = O.fwd_fused(q, k, v, g, tau, u=u, w=w, conv=ones, initial_state=s0)
    o2, s2 = O.fwd(q, k, v, g, tau, beta, s0)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
    o3, _ = O.fwd_fused(q, k, v, g, tau, u=u, w=w, d=np.zeros_like(d), initial_state=s0)
    assert np.array_equal(o3, o2)


def pin_fused_split_carry(O):
    rng = np.random.default_rng(9)
    W, T1, T2 = 4, 6, 7
    q, k, v, g, tau, u, w, d, conv, s0 = _rand(rng, 2, T1 + T2, 2, 3, 4, 2, W)
    o, sf = O.fwd_fused(q, k, v, g, tau, u=u, w=w, d=d, conv=conv, initial_state=s0)
    a = O.fwd_fused(q[:, :W - 1 + T1], k[:, :W - 1 + T1], v[:, :W - 1 + T1], g[:, :T1],
                    tau[:, :T1], u=u[:, :T1], w=w, d=d, conv=conv, initial_state=s0)
    b = O.fwd_fused(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], tau[:, T1:], u=u[:, T1:], w=w,
                    d=d, conv=conv, initial_state=a[1])
    assert relerr(np.concatenate([a[0], b[0]], axis=1), o) < 1e-13
    assert relerr(b[1], sf) < 1e-13


def pin_decode_matches_forward(O):
    rng = np.random.default_rng(10)
    W, T = 3, 5
    q, k, v, g, tau, u, w, d, conv, s0 = _rand(rng, 2, T, 2, 3, 4, 2, W)
    o, sf = O.fwd_fused(q, k, v, g, tau, u=u, w=w, d=d, conv=conv, initial_state=s0)
    st = s0
    for t in range(T):
        win = [x[:, t:t + W] for x in (q, k, v)]
        ot, st = O.decode_fused(*win, g[:, t], tau[:, t], st, u=u[:, t], w=w, d=d, conv=conv)
        assert relerr(ot, o[:, t]) < 1e-13, t
    assert relerr(st, sf) < 1e-13


PINS = [pin_lowrank_hand_values, pin_conv_impulse, pin_conv_carry, pin_fused_feedthrough,
        pin_fused_reduces_to_plain, pin_fused_split_carry, pin_decode_matches_forward]
