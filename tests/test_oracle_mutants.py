"""Plant plausible mistakes in a copy of the oracle (CPU) and check the pins catch each.

The copy is compiled with gcc into a temporary directory; the real oracle is not
touched.  A mutant "survives" if every pin in ``pin_battery`` still passes -- the
test fails in that case, because the pins would not have caught that mistake.
"""
import json
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle import forms
from test_oracle_pins import GOLDEN, nerr, rand_problem

SRC = os.path.join(os.path.dirname(oracle.__file__), "ssd_oracle.c")

MUTANTS = {
    "input_term_sign": ("row[n] = decay * row[n] + u * Bt[n];",
                        "row[n] = decay * row[n] - u * Bt[n];"),
    "decay_sign": ("exp(d * A)", "exp(-d * A)"),
    "decay_drops_dt": ("exp(d * A)", "exp(A)"),
    "input_drops_dt": ("const double u = d * xt[p];", "const double u = xt[p];"),
    "output_reads_B": ("acc += Ct[n] * row[n];", "acc += Bt[n] * row[n];"),
    "skip_term_dropped": ("yt[p] = acc + D * xt[p];", "yt[p] = acc;"),
    "state_transposed_in_output": ("acc += Ct[n] * row[n];", "acc += Ct[n] * s[n * P + p];"),
    "dt_index_shifted": ("const double d = dt[t * dt_tstride];",
                         "const double d = dt[(t > 0 ? t - 1 : 0) * dt_tstride];"),
    "group_map_modulo": ("g = h / heads_per_group;", "g = h % G;"),
    "verify_selects_next_state": ("hist + (a - 1) * PN", "hist + (a < K ? a : K - 1) * PN"),
}


def pin_battery(lib):
    """A compact subset of the pins in test_oracle_pins; True iff all pass."""
    ok = True
    with open(GOLDEN) as f:
        examples = json.load(f)["examples"]
    for ex in examples:
        d = ex["dims"]
        b, L, H, P, N, G = d["b"], d["L"], d["H"], d["P"], d["N"], d["G"]
        x = np.array(ex["x"], float).reshape(b, L, H, P)
        dt = np.array(ex["dt"], float).reshape(b, L, H)
        B = np.array(ex["B"], float).reshape(b, L, G, N)
        C = np.array(ex["C"], float).reshape(b, L, G, N)
        h0 = None if ex["init_state"] is None else np.array(ex["init_state"]).reshape(b, H, P, N)
        y, fs = oracle.scan_f64(x, dt, np.array(ex["A"]), B, C, np.array(ex["D"]), h0, lib=lib)
        ok &= np.allclose(y.reshape(-1), np.array(ex["y"]).reshape(-1), atol=1e-13, rtol=0)
        ok &= np.allclose(fs.reshape(-1), np.array(ex["final_state"]).reshape(-1), atol=1e-13,
                          rtol=0)
    x, dt, A, B, C, D, h0 = rand_problem(0, G=2)
    y, _ = oracle.scan_f64(x, dt, A, B, C, D, h0, lib=lib)
    ok &= nerr(y, forms.quadratic_form(x, dt, A, B, C, D, h0)) < 1e-12
    # verify selection
    K = 4
    xv, dtv, Av, Bv, Cv, Dv, _ = rand_problem(1, b=5, L=K, init=False)
    st = np.random.default_rng(2).standard_normal((5, 4, 3, 5))
    acc = np.array([0, 1, 2, 3, 4], np.int32)
    _, so, _ = oracle.verify_f64(st, xv, dtv, Av, Bv, Cv, Dv, acc, lib=lib)
    for bi in range(5):
        a = int(acc[bi])
        _, fa = oracle.scan_f64(xv[bi:bi + 1, :a], dtv[bi:bi + 1, :a], Av, Bv[bi:bi + 1, :a],
                                Cv[bi:bi + 1, :a], Dv, st[bi:bi + 1])
        ok &= bool(np.array_equal(so[bi], fa[0]))
    return bool(ok)


def test_real_oracle_passes_battery():
    assert pin_battery(oracle.load_library())


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert old in src, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new, 1)
    cfile = tmp_path / "mut.c"
    cfile.write_text(mutated)
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
                           "-o", str(so), str(cfile), "-lm"])
    lib = oracle.load_library(str(so))
    assert not pin_battery(lib), f"mutant {name} survived the pins"
