"""Pins for the sequence-parallel scan pieces (``oracle.cp``, CPU only).

Run over n slices of a sequence (each slice scanned from zero by the scan oracle,
then total decay, combine and correction), the pieces must reproduce the scan
oracle of the whole sequence: the outputs of every slice and the final state.
Planted mistakes in copies of the module fail that check.
"""
import numpy as np
import pytest

import oracle
from oracle import cp
from test_oracle_pins import rand_problem


def _pipeline(mod, x, dt, A, B, C, D, h0, n):
    """Scan n equal slices from zero, combine, correct; returns (y, final_state)."""
    L = x.shape[1]
    cuts = np.linspace(0, L, n + 1).astype(int)
    ys, Ss, alphas, parts = [], [], [], []
    for j in range(n):
        sl = slice(cuts[j], cuts[j + 1])
        y_j, S_j = oracle.scan_f64(x[:, sl], dt[:, sl], A, B[:, sl], C[:, sl], D, None)
        ys.append(y_j)
        Ss.append(S_j)
        alphas.append(mod.total_decay_f64(dt[:, sl], A))
        parts.append(sl)
    h_in = mod.combine_f64(np.stack(alphas), np.stack(Ss), h0)
    y_out, fin = [], None
    for j in range(n):
        sl = parts[j]
        y_j, fin = mod.apply_entering_state_f64(ys[j], Ss[j], dt[:, sl], A, C[:, sl], h_in[j])
        y_out.append(y_j)
    return np.concatenate(y_out, axis=1), fin


def _err(mod, seed, n, **kw):
    x, dt, A, B, C, D, h0 = rand_problem(seed, **kw)
    y_ref, f_ref = oracle.scan_f64(x, dt, A, B, C, D, h0)
    y, f = _pipeline(mod, x, dt, A, B, C, D, h0, n)
    e = lambda a, r: float(np.max(np.abs(a - r)) / np.max(np.abs(r)))
    return max(e(y, y_ref), e(f, f_ref))


@pytest.mark.parametrize("n", [1, 2, 3, 8])
def test_slices_reproduce_whole_sequence(n):
    assert _err(cp, n, n, b=2, L=41, H=4, P=3, N=5, G=2) < 1e-12


def test_without_initial_state_and_one_group():
    assert _err(cp, 9, 4, b=1, L=24, H=2, P=2, N=3, G=1, init=False) < 1e-12


def test_total_decay_closed_form():
    dt = np.full((1, 7, 2), 0.25)
    A = np.array([-1.0, -2.0])
    assert np.allclose(cp.total_decay_f64(dt, A), np.exp([[-1.75, -3.5]]), rtol=1e-15)


# each mutant: literal (old, new) replacements applied to a copy of oracle/cp.py
MUTANTS = {
    # the entering state recorded after the slice's own update
    "entering_state_late": [("        out[j] = h\n        h = alpha[j][:, :, None, None] * h + S[j]",
                             "        h = alpha[j][:, :, None, None] * h + S[j]\n        out[j] = h")],
    # the correction decays by the sum before token t instead of through it
    "exclusive_cumsum": [("                cum += dt[bi, t, h] * A[h]\n"
                          "                y[bi, t, h] += np.exp(cum) * (h_in[bi, h] @ C[bi, t, g[h]])",
                          "                y[bi, t, h] += np.exp(cum) * (h_in[bi, h] @ C[bi, t, g[h]])\n"
                          "                cum += dt[bi, t, h] * A[h]")],
    "final_undecayed": [("fin[bi, h] += np.exp(cum) * h_in[bi, h]", "fin[bi, h] += h_in[bi, h]")],
    "decay_sign": [("np.exp(dt.sum(axis=1) * A[None, :])", "np.exp(-dt.sum(axis=1) * A[None, :])")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    src = open(cp.__file__).read()
    for old, new in MUTANTS[name]:
        assert old in src, f"mutation anchor for {name} not found"
        src = src.replace(old, new, 1)
    ns = {"__name__": "mutant_cp"}
    exec(compile(src, "mutant_cp", "exec"), ns)

    class M:
        pass
    mod = M()
    for k in ("total_decay_f64", "combine_f64", "apply_entering_state_f64"):
        setattr(mod, k, ns[k])
    assert _err(mod, 11, 3, b=1, L=18, H=2, P=2, N=3, G=1) > 1e-6, f"mutant {name} survived"
