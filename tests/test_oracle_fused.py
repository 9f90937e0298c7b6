"""CPU: the fp64 oracle of the fused steps (beta_hat from low-rank factors,
ShortConv, feedthrough d) against its pins, and the pins against planted
mistakes: each mutant is a copy of oracle/__init__.py with one plausible
error in a fused-step function, loaded as its own module; at least one pin
must fail (an assertion or an exception) for every mutant."""
import importlib.util
import os
import sys

import pytest

import oracle
import oracle_fused_pins as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "__init__.py")


@pytest.mark.parametrize("pin", P.PINS, ids=lambda f: f.__name__)
def test_fused_oracle_pin(pin):
    pin(oracle)


MUTANTS = {
    "sigmoid_sign": ("return 1.0 / (1.0 + np.exp(-z))", "return 1.0 / (1.0 + np.exp(z))"),
    "lowrank_other_head": ('z = np.einsum("...hr,hrj->...hj", u, w)',
                           'z = np.einsum("...hr,hrj->...hj", u, w[::-1])'),
    "lowrank_tanh": ("return 1.0 / (1.0 + np.exp(-z))", "return 0.5 * (1.0 + np.tanh(z))"),
    "conv_anticausal": ("y += c[None, None, :, :, j] * x[:, W - 1 - j:W - 1 - j + T]",
                        "y += c[None, None, :, :, j] * x[:, j:j + T]"),
    "conv_lag_off_by_one": ("y += c[None, None, :, :, j] * x[:, W - 1 - j:W - 1 - j + T]",
                            "y += c[None, None, :, :, W - 1 - j] * x[:, W - 1 - j:W - 1 - j + T]"),
    "conv_wrong_channel": ("y += c[None, None, :, :, j] * x[:, W - 1 - j:W - 1 - j + T]",
                           "y += c[None, None, ::-1, :, j] * x[:, W - 1 - j:W - 1 - j + T]"),
    "feedthrough_gated": ("        o = o + _f64(d)[None, None] * _f64(v)\n",
                          "        o = o + _f64(d)[None, None] * _f64(v) * _f64(beta_hat)\n"),
    "feedthrough_raw_v": ("        q, k, v = short_conv(q, cq), short_conv(k, ck), short_conv(v, cv)\n",
                          "        q, k = short_conv(q, cq), short_conv(k, ck)\n"
                          "        v_raw = v\n        v = short_conv(v, cv)\n"),
    "decode_window_reversed": ("        q, k, v = (short_conv(x, c)[:, 0] for x, c in ((q, cq), (k, ck), (v, cv)))",
                               "        q, k, v = (short_conv(x[:, ::-1], c)[:, 0] for x, c in ((q, cq), (k, ck), (v, cv)))"),
    "decode_feedthrough_missing": ("        o = o + _f64(d)[None] * _f64(v)\n", "        pass\n"),
}


def _load_mutant(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) >= 1, name
    src = src.replace(old, new)
    if name == "feedthrough_raw_v":
        src = src.replace("        o = o + _f64(d)[None, None] * _f64(v)\n",
                          "        o = o + _f64(d)[None, None] * _f64(v_raw if conv is not None else v)\n")
    d = tmp_path / name
    d.mkdir()
    (d / "__init__.py").write_text(src)
    # the mutant reuses the real oracle's compiled C recurrence
    os.symlink(oracle._load()._name, str(d / "libddts_oracle.so"))
    os.symlink(os.path.join(ROOT, "oracle", "ddts_oracle.c"), str(d / "ddts_oracle.c"))
    spec = importlib.util.spec_from_file_location(f"oracle_mut_{name}", str(d / "__init__.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_fused_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    mod = _load_mutant(name, old, new, tmp_path)
    failed = []
    for pin in P.PINS:
        try:
            pin(mod)
        except Exception as e:               # an assertion or a shape error
            failed.append((pin.__name__, type(e).__name__))
    assert failed, f"mutant {name} passed every pin"
