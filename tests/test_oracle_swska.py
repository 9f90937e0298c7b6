"""CPU: the fp64 SW-SKA oracle (sliding-window attention with one key shared
by all heads) against what fixes it other than itself, and planted mistakes
that those pins must catch.

Pins: a hand-computed two-token example (weights 3/4, 1/4 come from scores
ln 3 and 0 after the 1/sqrt(dk) scale), window 1 returning v, constant keys
giving the moving average of v over the window (written with cumulative sums,
not softmax), the window's edges (a dominant key one token too old or in the
future changes nothing), the hard-attention limit, and the shared key (heads
differ only through q and v)."""
import importlib.util
import math
import os

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "__init__.py")


def pin_hand_example(O):
    # dk = 4, scale 1/2: q_1 = (2 ln 3, 0, 0, 0), k_0 = e_0, k_1 = 0 -> scores ln 3, 0
    q = np.zeros((1, 2, 1, 4)); k = np.zeros((1, 2, 4)); v = np.zeros((1, 2, 1, 2))
    q[0, 1, 0, 0] = 2 * math.log(3.0)
    k[0, 0, 0] = 1.0
    v[0, 0, 0] = [1.0, 10.0]
    v[0, 1, 0] = [5.0, -2.0]
    o = O.swska_fwd(q, k, v, window=2)
    assert np.allclose(o[0, 0, 0], [1.0, 10.0], rtol=0, atol=1e-15)      # token 0 sees itself
    want = 0.75 * np.array([1.0, 10.0]) + 0.25 * np.array([5.0, -2.0])
    assert np.max(np.abs(o[0, 1, 0] - want)) < 1e-14


def pin_window_one(O):
    rng = np.random.default_rng(1)
    q = rng.standard_normal((2, 9, 3, 8)); k = rng.standard_normal((2, 9, 8))
    v = rng.standard_normal((2, 9, 3, 5))
    assert np.array_equal(O.swska_fwd(q, k, v, window=1), v)


def pin_constant_keys_moving_average(O):
    rng = np.random.default_rng(2)
    B, T, H, dk, dv, w = 2, 23, 3, 8, 4, 5
    q = rng.standard_normal((B, T, H, dk))
    k = np.broadcast_to(rng.standard_normal((1, 1, dk)), (B, T, dk)).copy()
    v = rng.standard_normal((B, T, H, dv))
    o = O.swska_fwd(q, k, v, window=w)
    c = np.concatenate([np.zeros((B, 1, H, dv)), np.cumsum(v, axis=1)], axis=1)
    for t in range(T):
        s0 = max(0, t - w + 1)
        avg = (c[:, t + 1] - c[:, s0]) / (t + 1 - s0)
        assert np.max(np.abs(o[:, t] - avg)) < 1e-12, t


def pin_window_edges_and_causality(O):
    rng = np.random.default_rng(3)
    B, T, H, dk, dv, w = 1, 12, 2, 4, 3, 4
    q = np.ones((B, T, H, dk)); v = rng.standard_normal((B, T, H, dv))
    k = np.zeros((B, T, dk))
    t = 8
    base = O.swska_fwd(q, k, v, window=w)
    for s in (t - w, t + 1):                  # one token too old, one in the future
        k2 = k.copy()
        k2[0, s] = 50.0                       # a score that would dominate
        o2 = O.swska_fwd(q, k2, v, window=w)
        assert np.array_equal(o2[0, t], base[0, t]), s
    k3 = k.copy()
    k3[0, t - w + 1] = 50.0                   # the oldest token inside the window
    o3 = O.swska_fwd(q, k3, v, window=w)
    assert np.max(np.abs(o3[0, t] - v[0, t - w + 1])) < 1e-12


def pin_hard_attention_and_shared_key(O):
    rng = np.random.default_rng(4)
    B, T, H, dk, dv = 1, 10, 3, 6, 4
    q = rng.standard_normal((B, T, H, dk)); k = rng.standard_normal((B, T, dk))
    v = rng.standard_normal((B, T, H, dv))
    q[:, :, 1] = q[:, :, 0]                   # heads 0 and 1: same queries
    v[:, :, 1] = v[:, :, 0]                   # and same values
    o = O.swska_fwd(q, k, v, window=6)
    assert np.array_equal(o[:, :, 0], o[:, :, 1])
    # permuting the heads of q and v permutes the outputs: the key is shared
    perm = [2, 0, 1]
    op = O.swska_fwd(q[:, :, perm], k, v[:, :, perm], window=6)
    assert np.array_equal(op, o[:, :, perm])
    # a huge scale selects the highest-scoring visible key
    o_hard = O.swska_fwd(q, k, v, window=6, scale=1e6)
    for t in range(T):
        s0 = max(0, t - 5)
        for h in range(H):
            best = s0 + int(np.argmax(k[0, s0:t + 1] @ q[0, t, h]))
            assert np.max(np.abs(o_hard[0, t, h] - v[0, best, h])) < 1e-9


PINS = [pin_hand_example, pin_window_one, pin_constant_keys_moving_average,
        pin_window_edges_and_causality, pin_hard_attention_and_shared_key]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_swska_oracle_pin(pin):
    pin(oracle)


MUTANTS = {
    "no_scale": ("sc = 1.0 / np.sqrt(dk) if scale is None else float(scale)",
                 "sc = 1.0 if scale is None else float(scale)"),
    "window_too_long": ("s0 = max(0, t - window + 1)", "s0 = max(0, t - window)"),
    "window_too_short": ("s0 = max(0, t - window + 1)", "s0 = max(0, t - window + 2)"),
    "sees_future": [("z = (q[b, t] @ k[b, s0:t + 1].T) * sc",
                     "e = min(T, t + 2)\n            z = (q[b, t] @ k[b, s0:e].T) * sc"),
                    ('o[b, t] = np.einsum("hl,lhd->hd", p, v[b, s0:t + 1])',
                     'o[b, t] = np.einsum("hl,lhd->hd", p, v[b, s0:e])')],
    "no_normalisation": ("p /= p.sum(axis=1, keepdims=True)", "pass"),
    "key_of_other_token": ("z = (q[b, t] @ k[b, s0:t + 1].T) * sc", "z = (q[b, t] @ k[b, max(0, s0 - 1):t].T) * sc if t > 0 else (q[b, t] @ k[b, 0:1].T) * sc"),
    "values_shifted": ('o[b, t] = np.einsum("hl,lhd->hd", p, v[b, s0:t + 1])',
                       'o[b, t] = np.einsum("hl,lhd->hd", p, v[b, max(0, s0 - 1):max(0, s0 - 1) + p.shape[1]])'),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_swska_pins_catch_mutant(name, tmp_path):
    edits = MUTANTS[name]
    if isinstance(edits, tuple):
        edits = [edits]
    src = open(SRC).read()
    for old, new in edits:
        assert src.count(old) == 1, name
        src = src.replace(old, new)
    d = tmp_path / name
    d.mkdir()
    (d / "__init__.py").write_text(src)
    spec = importlib.util.spec_from_file_location(f"oracle_swska_mut_{name}", str(d / "__init__.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    failed = []
    for pin in PINS:
        try:
            pin(mod)
        except Exception as e:
            failed.append((pin.__name__, type(e).__name__))
    assert failed, f"mutant {name} passed every pin"
