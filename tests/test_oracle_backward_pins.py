"""Pins for the fp64 gradient oracle (``oracle.backward.scan_bwd_f64``).

The gradient oracle differentiates a torch transcription of the recurrence; it is
checked against things other than itself:
  * central finite differences of the C recurrence oracle (``oracle.scan_f64``, an
    independent implementation of the forward map) along random directions, for
    every input;
  * closed forms: dD is sum(x * dy); with dy = 0 the gradient of the initial state
    is the upstream final-state gradient times the total decay, and no other input
    receives gradient through the state except via B, x, dt and A;
  * planted mistakes in a copy of the forward transcription, which the
    finite-difference pin must reject.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import backward
from test_oracle_pins import rand_problem

NAMES = ("x", "dt", "A", "B", "C", "D", "init")


def _loss(inputs, dy, dfin):
    x, dt, A, B, C, D, h0 = inputs
    y, fs = oracle.scan_f64(x, dt, A, B, C, D, h0)
    return float(np.sum(y * dy) + np.sum(fs * dfin))


def _fd_check(grads, inputs, dy, dfin, seed, eps=1e-6):
    """max over inputs of |directional FD - <grad, v>| / max(|<grad, v>|, 1e-8)."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for i, name in enumerate(NAMES):
        v = rng.standard_normal(inputs[i].shape)
        if name == "dt":
            v *= 0.05          # keep dt positive and small
        plus = [a.copy() for a in inputs]
        minus = [a.copy() for a in inputs]
        plus[i] = plus[i] + eps * v
        minus[i] = minus[i] - eps * v
        fd = (_loss(plus, dy, dfin) - _loss(minus, dy, dfin)) / (2 * eps)
        an = float(np.sum(grads[i] * v))
        worst = max(worst, abs(fd - an) / max(abs(an), 1e-8))
    return worst


def _problem(seed, **kw):
    x, dt, A, B, C, D, h0 = rand_problem(seed, **kw)
    rng = np.random.default_rng(seed + 100)
    dy = rng.standard_normal(x.shape)
    dfin = rng.standard_normal(h0.shape)
    return [x, dt, A, B, C, D, h0], dy, dfin


@pytest.mark.parametrize("seed", [0, 1])
def test_gradients_match_finite_differences(seed):
    inputs, dy, dfin = _problem(seed, b=2, L=11, H=4, P=3, N=5, G=2)
    grads = backward.scan_bwd_f64(*inputs, dy, dfin)
    assert _fd_check(grads, inputs, dy, dfin, seed) < 1e-6


def test_gradients_single_group_and_no_final_gradient():
    inputs, dy, _ = _problem(3, b=1, L=9, H=2, P=2, N=3, G=1)
    zero = np.zeros_like(inputs[6])
    grads = backward.scan_bwd_f64(*inputs, dy, None)
    assert _fd_check(grads, inputs, dy, zero, 3) < 1e-6


def test_dD_closed_form():
    inputs, dy, dfin = _problem(4)
    grads = backward.scan_bwd_f64(*inputs, dy, dfin)
    x = inputs[0]
    assert np.allclose(grads[5], np.sum(x * dy, axis=(0, 1, 3)), rtol=1e-12, atol=1e-12)


def test_init_gradient_without_output_gradient_is_decayed_final_gradient():
    inputs, dy, dfin = _problem(5)
    dy = np.zeros_like(dy)
    grads = backward.scan_bwd_f64(*inputs, dy, dfin)
    dt, A = inputs[1], inputs[2]
    total = np.exp(np.sum(dt, axis=1) * A)                 # [b, H]
    assert np.allclose(grads[6], total[:, :, None, None] * dfin, rtol=1e-12, atol=1e-14)
    assert np.all(grads[4] == 0)                           # C only reaches y
    assert np.all(grads[5] == 0)                           # D only reaches y


def test_empty_sequence_passes_final_gradient_to_init():
    inputs, dy, dfin = _problem(6, L=0)
    grads = backward.scan_bwd_f64(*inputs, dy, dfin)
    assert np.array_equal(grads[6], dfin)
    assert grads[0].shape == inputs[0].shape and not np.any(grads[0])


MUTANTS = {
    "decay_sign": ("decay = torch.exp(dt[:, t] * A)", "decay = torch.exp(-dt[:, t] * A)"),
    "input_drops_dt": ("(dt[:, t, :, None] * x[:, t])[..., None]", "(x[:, t])[..., None]"),
    "output_reads_B": ("(s * Ct[:, :, None, :]).sum(-1)", "(s * Bt[:, :, None, :]).sum(-1)"),
    "group_map_modulo": ("g = torch.arange(H) // (H // G)", "g = torch.arange(H) % G"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_finite_difference_pin_catches_mutant(name):
    old, new = MUTANTS[name]
    src = open(backward.__file__).read()
    assert old in src, f"mutation anchor for {name} not found"
    ns = {}
    exec(compile(src.replace(old, new, 1), "mutant_backward", "exec"), ns)
    inputs, dy, dfin = _problem(7, b=1, L=7, H=4, P=2, N=3, G=2)
    grads = ns["scan_bwd_f64"](*inputs, dy, dfin)
    assert _fd_check(grads, inputs, dy, dfin, 7) > 1e-3, f"mutant {name} survived"
