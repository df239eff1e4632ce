"""Pins for the fp64 selective-scan oracle (one channel per head, diagonal A).

The oracle (``oracle.selective_scan_f64``) is checked against things other than
itself:
  * the SSD recurrence oracle, when every state of a channel shares its head's
    decay and the channels of a head share dt (SSD is that special case: the
    Bi-Mamba page, «Preliminary: Mamba Series»);
  * scipy's IIR filter in the time-invariant case, with a different decay per
    state (each state is then a first-order filter of x);
  * the closed form for A = 0 (no decay: the state is a prefix sum);
  * planted mistakes in a copy of the oracle, which these pins must reject.
"""
import math
import os
import subprocess

import numpy as np
import pytest
import scipy.signal

import oracle
from test_oracle_pins import nerr, rand_problem

SRC = os.path.join(os.path.dirname(oracle.__file__), "ssd_oracle.c")


def rand_selective(seed, b=2, L=19, Dch=6, N=5, G=2, init=True):
    rng = np.random.default_rng(seed)
    A = -np.exp(rng.uniform(0.0, math.log(4.0), (Dch, N)))
    D = rng.standard_normal(Dch)
    dt = rng.uniform(0.05, 0.6, (b, L, Dch))
    x = rng.standard_normal((b, L, Dch))
    B = rng.standard_normal((b, L, G, N))
    C = rng.standard_normal((b, L, G, N))
    h0 = rng.standard_normal((b, Dch, N)) if init else None
    return x, dt, A, B, C, D, h0


def _equals_ssd(lib=None, seed=0):
    """Selective scan with A[d][n] = A_h and dt[b,t,d] = dt[b,t,h] (d = h P + p) is the
    SSD scan; its y and final state must match the SSD oracle's."""
    x, dt, A, B, C, D, h0 = rand_problem(seed, b=2, L=17, H=4, P=3, N=5, G=2)
    b, L, H, P = x.shape
    N = B.shape[3]
    xs = x.reshape(b, L, H * P)
    dts = np.repeat(dt, P, axis=2)
    As = np.repeat(A, P)[:, None] * np.ones((1, N))
    Ds = np.repeat(D, P)
    h0s = h0.reshape(b, H * P, N)
    y, fs = oracle.selective_scan_f64(xs, dts, As, B, C, Ds, h0s, lib=lib)
    y_ref, fs_ref = oracle.scan_f64(x, dt, A, B, C, D, h0)
    return nerr(y, y_ref.reshape(b, L, H * P)) < 1e-13 and nerr(fs, fs_ref.reshape(b, H * P, N)) < 1e-13


def _lti_iir(lib=None, seed=1):
    """Constant dt per channel and constant B, C over time: state n of channel d is
    s_n[t] = a_n s_n[t-1] + dt B_n x_t with a_n = exp(dt A[d][n]), so
    y_t - D x_t = sum_n C_n lfilter([dt B_n], [1, -a_n], x)[t]."""
    rng = np.random.default_rng(seed)
    b, L, Dch, N, G = 1, 41, 3, 4, 1
    A = -np.exp(rng.uniform(0.0, math.log(8.0), (Dch, N)))   # distinct per state
    D = rng.standard_normal(Dch)
    delta = rng.uniform(0.05, 0.5, Dch)
    dt = np.broadcast_to(delta, (b, L, Dch)).copy()
    x = rng.standard_normal((b, L, Dch))
    Bc, Cc = rng.standard_normal(N), rng.standard_normal(N)
    B = np.broadcast_to(Bc, (b, L, G, N)).copy()
    C = np.broadcast_to(Cc, (b, L, G, N)).copy()
    y, _ = oracle.selective_scan_f64(x, dt, A, B, C, D, None, lib=lib)
    ok = True
    for d in range(Dch):
        ref = np.zeros(L)
        for n in range(N):
            ref += Cc[n] * scipy.signal.lfilter([delta[d] * Bc[n]], [1.0, -math.exp(delta[d] * A[d, n])],
                                                x[0, :, d])
        ok &= nerr(y[0, :, d] - D[d] * x[0, :, d], ref) < 1e-12
    return bool(ok)


def _a_zero_prefix_sum(lib=None, seed=2):
    """A = 0: s_t = s_0 + sum_{s<=t} dt_s x_s B_s, so y_t = C_t . s_t + D x_t."""
    x, dt, A, B, C, D, h0 = rand_selective(seed)
    A = np.zeros_like(A)
    y, fs = oracle.selective_scan_f64(x, dt, A, B, C, D, h0, lib=lib)
    b, L, Dch = x.shape
    G = B.shape[2]
    g = np.arange(Dch) // (Dch // G)
    Bd, Cd = B[:, :, g, :], C[:, :, g, :]                       # [b, L, Dch, N]
    s = h0[:, None] + np.cumsum((dt * x)[..., None] * Bd, axis=1)
    y_ref = np.sum(Cd * s, axis=-1) + D * x
    return nerr(y, y_ref) < 1e-12 and nerr(fs, s[:, -1]) < 1e-12


def _battery(lib=None):
    return _equals_ssd(lib) and _lti_iir(lib) and _a_zero_prefix_sum(lib)


def test_selective_equals_ssd_for_scalar_decay_per_head():
    assert _equals_ssd()


def test_selective_lti_matches_iir_filter_with_distinct_decays():
    assert _lti_iir()


def test_selective_a_zero_is_prefix_sum():
    assert _a_zero_prefix_sum()


def test_selective_empty_sequence_keeps_init():
    x, dt, A, B, C, D, h0 = rand_selective(3, L=0)
    y, fs = oracle.selective_scan_f64(x, dt, A, B, C, D, h0)
    assert y.shape == (2, 0, 6) and np.array_equal(fs, h0)


MUTANTS = {
    "decay_index_transposed": ("exp(dv * A[d * N + n])", "exp(dv * A[(n % Dch) * N + (d % N)])"),
    "output_before_update": ("s[n] = exp(dv * A[d * N + n]) * s[n] + dv * xv * Bt[n];\n"
                             "                    acc += Ct[n] * s[n];",
                             "acc += Ct[n] * s[n];\n"
                             "                    s[n] = exp(dv * A[d * N + n]) * s[n] + dv * xv * Bt[n];"),
    "input_drops_dt": ("+ dv * xv * Bt[n];", "+ xv * Bt[n];"),
    "group_map_modulo": ("const long g = d / per_group;", "const long g = d % G;"),
}


def test_real_oracle_passes_selective_battery():
    assert _battery(oracle.load_library())


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_selective_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert old in src, f"mutation anchor for {name} not found"
    cfile = tmp_path / "mut.c"
    cfile.write_text(src.replace(old, new, 1))
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
                           "-o", str(so), str(cfile), "-lm"])
    assert not _battery(oracle.load_library(str(so))), f"mutant {name} survived the pins"
