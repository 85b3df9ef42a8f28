"""Every plausible mistake planted in the oracle is caught by some pin.

Each mutant is a copy of oracle/kda_oracle.c with one textual change (a
dropped term, a wrong sign, a wrong index, a transposed operand), built with
gcc into a temporary directory and run through the pin suite on the CPU.
"""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = open(oracle._SRC).read()

MUTANTS = {
    "decay dropped": ("S[j * Dv + c] *= alpha[j];", "S[j * Dv + c] *= 1.0;"),
    "decay on columns": ("S[j * Dv + c] *= alpha[j];", "S[j * Dv + c] *= alpha[c % Dk];"),
    "delta sign": ("(vt[c] - u[c])", "(vt[c] + u[c])"),
    "beta dropped": ("+= bt * kt[j] * (vt[c] - u[c]);", "+= kt[j] * (vt[c] - u[c]);"),
    "erase reads q": ("u[c] += S[j * Dv + c] * kt[j];", "u[c] += S[j * Dv + c] * qt[j];"),
    "output reads k": ("(scale * qt[j]);", "(scale * kt[j]);"),
    "scale dropped": ("(scale * qt[j]);", "(qt[j]);"),
    "gate sigmoid sign": ("1.0 / (1.0 + exp(-x))", "1.0 / (1.0 + exp(x))"),
    "gate log-scale not exponentiated": ("double x = exp(A_h) * z;", "double x = (1.0 + A_h) * z;"),
    "gate head index": ("z_mode ? A_log[h] : 0.0", "z_mode ? A_log[0] : 0.0"),
    "initial state ignored": ("if (h0)\n", "if (0)\n"),
    "beta packing offset": ("beta + t0 * H + h,", "beta + t0 * H,"),
    "value stride": ("H * Dk, H * Dv, H,", "H * Dk, H * Dk, H,"),
    "output before update": (
        "        /* S <- S + beta_t k_t (v_t - u)^T */",
        "        for (int64_t c = 0; c < Dv; ++c) ot[c] = 0.0;\n"
        "        for (int64_t j = 0; j < Dk; ++j) for (int64_t c = 0; c < Dv; ++c) ot[c] += S[j*Dv+c]*(scale*qt[j]);\n"
        "        continue;\n"
        "        /* S <- S + beta_t k_t (v_t - u)^T */"),
}


def _caught(lib):
    for pin in ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            return pin.__name__
    return None


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    assert SRC.count(old) >= 1, f"mutation anchor missing: {old!r}"
    src = tmp_path / "mutant.c"
    src.write_text(SRC.replace(old, new, 1))
    lib = oracle.load(oracle.build(str(src), str(tmp_path / "libmutant.so")))
    assert _caught(lib) is not None, f"no pin catches mutant '{name}'"
