"""The layer prologue/epilogue oracle against its pins, and every plausible
mistake planted in it caught by some pin (CPU only).

Each mutant is oracle/layer.py with one textual change, loaded as a separate
module; the pins in layer_pins.py must reject it.
"""
import importlib.util
import os

import pytest

import oracle.layer
from layer_pins import LAYER_PINS

SRC = open(oracle.layer.__file__).read()

MUTANTS = {
    "conv taps reversed": ("y += weight[..., i] * xt[i:i + T]", "y += weight[..., W - 1 - i] * xt[i:i + T]"),
    "conv state ignored": ("xt = np.concatenate([state, x], axis=0)", "xt = np.concatenate([0 * state, x], axis=0)"),
    "conv state out from the front": ("return y, xt[T:T + W - 1].copy()", "return y, xt[:W - 1].copy()"),
    "conv looks one step ahead": ("y += weight[..., i] * xt[i:i + T]", "y += weight[..., i] * np.roll(xt, -1, 0)[i:i + T]"),
    "swish without x": ("return x * sigmoid(x)", "return sigmoid(x)"),
    "sigmoid branches swapped": ("np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))",
                                 "np.where(x >= 0, e / (1.0 + e), 1.0 / (1.0 + e))"),
    "l2norm mean": ("np.sqrt(np.sum(y * y,", "np.sqrt(np.mean(y * y,"),
    "q not normalised": ("q = l2norm(a[..., :Dk], qk_eps)", "q = a[..., :Dk]"),
    "k not normalised": ("k = l2norm(a[..., Dk:2 * Dk], qk_eps)", "k = a[..., Dk:2 * Dk]"),
    "k reads the query channels": ("k = l2norm(a[..., Dk:2 * Dk], qk_eps)", "k = l2norm(a[..., :Dk], qk_eps)"),
    "v without swish": ("v = a[..., 2 * Dk:]", "v = c[..., 2 * Dk:]"),
    "beta logit not squashed": ("return q, k, v, sigmoid(beta_logit),", "return q, k, v, beta_logit,"),
    "rmsnorm sum": ("np.sqrt(np.mean(o * o,", "np.sqrt(np.sum(o * o,"),
    "rmsnorm weight dropped": ("return _f64(weight) * o / np.sqrt", "return o / np.sqrt"),
    "gate not squashed": ("return sigmoid(gate_logit) * rmsnorm", "return gate_logit * rmsnorm"),
    "conv state of sequence 0 for all": ("else _f64(conv_state)[s]", "else _f64(conv_state)[0]"),
}


@pytest.mark.parametrize("pin", LAYER_PINS, ids=lambda p: p.__name__)
def test_layer_pin(pin):
    pin(oracle.layer)


def _load_mutant(src, path):
    path.write_text(src)
    spec = importlib.util.spec_from_file_location("layer_mutant", str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_layer_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, f"mutation anchor must occur once: {old!r}"
    mod = _load_mutant(SRC.replace(old, new), tmp_path / "layer_mutant.py")
    caught = None
    for pin in LAYER_PINS:
        try:
            pin(mod)
        except AssertionError:
            caught = pin.__name__
            break
    assert caught is not None, f"no pin catches mutant '{name}'"
