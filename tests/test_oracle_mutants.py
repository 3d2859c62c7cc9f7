"""CPU test: plant plausible mistakes in copies of the oracle and check that the
pins of tests/oracle_pins.py catch every one of them. Each mutant stays within
the arrays' bounds (they run in this process)."""
import functools
import os
import subprocess

import pytest

import oracle
import oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.library_path()), "kda_oracle.c")

MUTANTS = {
    "error_sign": ("bt * (vt[j] - vhat[j])", "bt * (vt[j] + vhat[j])"),
    "error_without_beta": ("bt * (vt[j] - vhat[j])", "(vt[j] - vhat[j])"),
    "no_decay": ("const double a = exp(lat[i]);", "const double a = 1.0;"),
    "decay_by_column": ("S[(size_t)i * dv + j] *= a;",
                        "S[(size_t)i * dv + j] *= exp(lat[j % dk]);"),
    "recall_before_decay": ("vhat[j] += S[(size_t)i * dv + j] * kt[i];",
                            "vhat[j] += S[(size_t)i * dv + j] * kt[i] / exp(lat[i]);"),
    "no_write": ("S[(size_t)i * dv + j] += kt[i] * e[j];", "S[(size_t)i * dv + j] += 0.0 * e[j];"),
    "no_scale": ("(J->scale * qt[i])", "(qt[i])"),
    "beta_of_head0": ("J->beta[(size_t)t * H + h]", "J->beta[(size_t)t * H]"),
    "h0_of_head0": ("J->h0 + ((size_t)s * H + h) * dk * dv", "J->h0 + ((size_t)s * H) * dk * dv"),
    "readout_before_write_uses_old": ("acc += S[(size_t)i * dv + j] * (J->scale * qt[i]);",
                                      "acc += (S[(size_t)i * dv + j] - kt[i] * e[j]) * (J->scale * qt[i]);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    mut_c = tmp_path / f"{name}.c"
    mut_c.write_text(src.replace(old, new))
    lib = tmp_path / f"lib{name}.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", str(lib),
                           str(mut_c), "-lm", "-lpthread"])
    fwd = functools.partial(oracle.kda_reference, lib=str(lib))
    caught = []
    for check in P.ALL_CHECKS:
        try:
            check(fwd)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"mutant {name} passed every pin"
