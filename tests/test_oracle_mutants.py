"""Each plausible mistake planted in a copy of the C oracle fails at least one pin.

The copies are compiled into a temporary directory; the committed oracle is untouched.
This shows the pins are strong enough: a dropped term, a wrong sign, a wrong index,
a transposed operand or a swapped operand does not pass unnoticed.
"""
import os
import subprocess

import pytest

import oracle
import pins

MUTANTS = {
    "no_decay": ("const double a = exp((double)gr[i]);", "const double a = 1.0;"),
    "decay_value_axis": ("row[j] *= a;", "row[j] *= exp((double)gr[j % dk]);"),
    "sign_flip": ("u[j] = b * ((double)vr[j] - u[j]);", "u[j] = b * (u[j] - (double)vr[j]);"),
    "no_beta": ("u[j] = b * ((double)vr[j] - u[j]);", "u[j] = ((double)vr[j] - u[j]);"),
    "transposed_read": ("u[j] += row[j] * kt[i];",
                        "u[j] += S[((size_t)j * dv + i) % ((size_t)dk * dv)] * kt[i];"),
    "read_before_decay": ("u[j] += row[j] * kt[i];", "u[j] += row[j] / exp((double)gr[i]) * kt[i];"),
    "g_index_shift": ("*gr = g + t * ldg;", "*gr = g + (t > 0 ? t - 1 : 0) * ldg;"),
    "readout_before_write": ("orow[j] += row[j] * qt[i];",
                             "orow[j] += (row[j] - kt[i] * u[j]) * qt[i];"),
    "readout_with_k": ("orow[j] += row[j] * qt[i];", "orow[j] += row[j] * kt[i];"),
    "write_with_q": ("row[j] += kt[i] * u[j];", "row[j] += qt[i] * u[j];"),
    "no_scale": ("orow[j] *= scale;", "orow[j] *= 1.0;"),
    "no_initial_state": ("S[e] = S0 ? (double)S0[e] : 0.0;", "S[e] = 0.0;"),
}


def _build_mutant(tmp_path, name):
    src = open(oracle._SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation target for {name} not found exactly once"
    path_c = os.path.join(tmp_path, f"{name}.c")
    path_so = os.path.join(tmp_path, f"lib{name}.so")
    with open(path_c, "w") as fh:
        fh.write(src.replace(old, new))
    subprocess.check_call(["gcc", "-O1", "-std=c99", "-fPIC", "-shared", path_c, "-o", path_so, "-lm"])
    return pins.load_chain_fn(path_so)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    chain_fn = _build_mutant(str(tmp_path), name)
    caught = []
    for pin in pins.PINS:
        try:
            err = pin(chain_fn)
        except Exception:  # a crash inside a pin (e.g. NaN in a solver) also counts
            err = float("inf")
        if not (err <= pin.tol):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passes every pin"
