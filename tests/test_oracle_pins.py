"""Pins for the fp64 oracle (CPU only).

Each test ties the sequential recurrence in ``oracle/ssd_oracle.c`` to something
other than itself: a hand-computed worked example, closed forms, an IIR-filter
library routine, brute-force alternative forms and structural invariants.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.signal

import oracle
from oracle import forms

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_examples.json")


def rand_problem(seed, b=2, L=23, H=4, P=3, N=5, G=2, init=True, dt_range=(0.05, 0.6)):
    """Small dense fp64 problem with asymmetric B/C and a nonzero initial state."""
    rng = np.random.default_rng(seed)
    A = -np.exp(rng.uniform(0.0, math.log(4.0), H))
    D = rng.standard_normal(H)
    dt = rng.uniform(*dt_range, (b, L, H))
    x = rng.standard_normal((b, L, H, P))
    B = rng.standard_normal((b, L, G, N))
    C = rng.standard_normal((b, L, G, N))
    h0 = rng.standard_normal((b, H, P, N)) if init else None
    return x, dt, A, B, C, D, h0


def nerr(a, b):
    """max |a - b| / max |b| (slice-free normalised error)."""
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ------------------------------------------------------------ worked examples
def _load_golden():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


@pytest.mark.parametrize("ex", _load_golden(), ids=lambda e: e["name"])
def test_hand_worked_example(ex):
    d = ex["dims"]
    b, L, H, P, N, G = d["b"], d["L"], d["H"], d["P"], d["N"], d["G"]
    x = np.array(ex["x"], dtype=np.float64).reshape(b, L, H, P)
    dt = np.array(ex["dt"], dtype=np.float64).reshape(b, L, H)
    A = np.array(ex["A"], dtype=np.float64)
    D = np.array(ex["D"], dtype=np.float64)
    B = np.array(ex["B"], dtype=np.float64).reshape(b, L, G, N)
    C = np.array(ex["C"], dtype=np.float64).reshape(b, L, G, N)
    h0 = None if ex["init_state"] is None else np.array(ex["init_state"]).reshape(b, H, P, N)
    y, fs = oracle.scan_f64(x, dt, A, B, C, D, h0)
    np.testing.assert_allclose(y.reshape(-1), np.array(ex["y"]).reshape(-1), rtol=0, atol=1e-13)
    np.testing.assert_allclose(fs.reshape(-1), np.array(ex["final_state"]).reshape(-1),
                               rtol=0, atol=1e-13)
    # the same example through the verify entry (K = L, accept everything)
    state = np.zeros((b, H, P, N)) if h0 is None else h0
    yv, so, sa = oracle.verify_f64(state, x, dt, A, B, C, D, np.array([L], np.int32))
    np.testing.assert_allclose(yv.reshape(-1), np.array(ex["y"]).reshape(-1), rtol=0, atol=1e-13)
    np.testing.assert_allclose(so.reshape(-1), np.array(ex["final_state"]).reshape(-1),
                               rtol=0, atol=1e-13)


# ------------------------------------------------ quadratic (dual) form, brute force
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_recurrence_equals_quadratic_form(seed):
    x, dt, A, B, C, D, h0 = rand_problem(seed)
    y, _ = oracle.scan_f64(x, dt, A, B, C, D, h0)
    yq = forms.quadratic_form(x, dt, A, B, C, D, h0)
    assert nerr(y, yq) < 1e-12


def test_quadratic_form_zero_init_and_singleton_groups():
    x, dt, A, B, C, D, _ = rand_problem(7, b=1, L=17, H=3, G=3, init=False)
    y, _ = oracle.scan_f64(x, dt, A, B, C, D, None)
    assert nerr(y, forms.quadratic_form(x, dt, A, B, C, D, None)) < 1e-12


# --------------------------------------------------------- chunked decomposition
@pytest.mark.parametrize("Q", [1, 2, 3, 7, 16, 23, 28])
def test_chunked_equals_recurrence_any_Q(Q):
    x, dt, A, B, C, D, h0 = rand_problem(11)          # L = 23: ragged for most Q
    y, fs = oracle.scan_f64(x, dt, A, B, C, D, h0)
    yc, fc, entering = forms.chunked_form(x, dt, A, B, C, D, Q, h0)
    assert nerr(yc, y) < 1e-12
    assert nerr(fc, fs) < 1e-12
    # the state entering chunk c is the recurrence's final state after c*Q tokens
    L = x.shape[1]
    for c in range(entering.shape[2]):
        if c == 0:
            ref = h0
        else:
            _, ref = oracle.scan_f64(x[:, :c * Q], dt[:, :c * Q], A, B[:, :c * Q],
                                     C[:, :c * Q], D, h0)
        assert nerr(entering[:, :, c], ref) < 1e-12
    assert entering.shape[2] == (L + Q - 1) // Q


def test_chunked_Q1_and_Q_ge_L_reduce_to_recurrence_and_quadratic():
    x, dt, A, B, C, D, h0 = rand_problem(12, L=9)
    y1, _, _ = forms.chunked_form(x, dt, A, B, C, D, 1, h0)
    yL, _, _ = forms.chunked_form(x, dt, A, B, C, D, 9, h0)
    yq = forms.quadratic_form(x, dt, A, B, C, D, h0)
    y, _ = oracle.scan_f64(x, dt, A, B, C, D, h0)
    assert nerr(y1, y) < 1e-12 and nerr(yL, yq) < 1e-12


# ------------------------------------------------------------------ closed forms
def test_closed_form_constant_inputs():
    """Constant dt, x, B: h_t = q^t h0 + dt x (outer) B (1 - q^t) / (1 - q), q = e^{dt A}."""
    b, L, H, P, N, G = 1, 40, 2, 3, 4, 1
    rng = np.random.default_rng(3)
    delta = 0.37
    A = np.array([-0.8, -2.5])
    D = np.array([0.3, -1.2])
    xbar = rng.standard_normal((H, P))
    Bbar = rng.standard_normal(N)
    Cbar = rng.standard_normal(N)
    h0 = rng.standard_normal((b, H, P, N))
    x = np.broadcast_to(xbar, (b, L, H, P)).copy()
    dt = np.full((b, L, H), delta)
    B = np.broadcast_to(Bbar, (b, L, G, N)).copy()
    C = np.broadcast_to(Cbar, (b, L, G, N)).copy()
    y, fs = oracle.scan_f64(x, dt, A, B, C, D, h0)
    for h in range(H):
        q = math.exp(delta * A[h])
        for t in range(1, L + 1):
            ht = q ** t * h0[0, h] + delta * np.outer(xbar[h], Bbar) * (1 - q ** t) / (1 - q)
            yt = ht @ Cbar + D[h] * xbar[h]
            np.testing.assert_allclose(y[0, t - 1, h], yt, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(fs[0, h], ht, rtol=1e-12, atol=1e-12)


def test_lti_case_matches_iir_filter():
    """Constant dt, B, C and zero init: an LTI system, i.e. a causal IIR/convolution.

    y - D x = lfilter([dt (C.B)], [1, -e^{dt A}], x) along time, per (head, channel)
    ('另辟蹊径--Mamba介绍', «The Convolution Representation»: with fixed parameters
    the SSM is a convolution with kernel C Bbar, C Abar Bbar, ...).
    """
    b, L, H, P, N, G = 2, 64, 3, 4, 6, 1
    rng = np.random.default_rng(5)
    delta = 0.21
    A = np.array([-0.5, -1.7, -3.0])
    D = rng.standard_normal(H)
    x = rng.standard_normal((b, L, H, P))
    Bbar, Cbar = rng.standard_normal(N), rng.standard_normal(N)
    B = np.broadcast_to(Bbar, (b, L, G, N)).copy()
    C = np.broadcast_to(Cbar, (b, L, G, N)).copy()
    dt = np.full((b, L, H), delta)
    y, _ = oracle.scan_f64(x, dt, A, B, C, D, None)
    for h in range(H):
        ref = scipy.signal.lfilter([delta * float(Cbar @ Bbar)], [1.0, -math.exp(delta * A[h])],
                                   x[:, :, h, :], axis=1)
        np.testing.assert_allclose(y[:, :, h, :] - D[h] * x[:, :, h, :], ref, rtol=1e-11,
                                   atol=1e-12)


def test_A_zero_is_causal_linear_attention():
    """A = 0: no decay; y_t = sum_{s<=t} (C_t.B_s) dt_s x_s + C_t.h0 + D x_t."""
    x, dt, A, B, C, D, h0 = rand_problem(9, b=1, L=15, H=2, G=1)
    A = np.zeros_like(A)
    y, _ = oracle.scan_f64(x, dt, A, B, C, D, h0)
    for h in range(2):
        scores = np.tril(C[0, :, 0] @ B[0, :, 0].T)          # [L, L] causal
        v = dt[0, :, h, None] * x[0, :, h]
        ref = scores @ v + C[0, :, 0] @ h0[0, h].T + D[h] * x[0, :, h]
        np.testing.assert_allclose(y[0, :, h], ref, rtol=1e-12, atol=1e-12)


def test_zero_input_pure_decay():
    """x = 0, constant dt: ||h_t|| = e^{dt A t} ||h0|| and y_t = e^{dt A t} C_t.h0."""
    b, L, H, P, N, G = 1, 30, 2, 3, 4, 2
    rng = np.random.default_rng(13)
    A = np.array([-0.4, -1.9])
    D = rng.standard_normal(H)
    h0 = rng.standard_normal((b, H, P, N))
    x = np.zeros((b, L, H, P))
    B = rng.standard_normal((b, L, G, N))
    C = rng.standard_normal((b, L, G, N))
    dt = np.full((b, L, H), 0.3)
    y, fs = oracle.scan_f64(x, dt, A, B, C, D, h0)
    for h in range(H):
        q = math.exp(0.3 * A[h])
        assert abs(np.linalg.norm(fs[0, h]) - q ** L * np.linalg.norm(h0[0, h])) < 1e-12
        for t in range(L):
            ref = q ** (t + 1) * (h0[0, h] @ C[0, t, h])
            np.testing.assert_allclose(y[0, t, h], ref, rtol=1e-12, atol=1e-14)


# -------------------------------------------------------------------- invariants
def test_split_sequence_with_state_handoff():
    """Running [0, t0) and then [t0, L) from the handed-over state equals one run."""
    x, dt, A, B, C, D, h0 = rand_problem(21, L=31)
    y, fs = oracle.scan_f64(x, dt, A, B, C, D, h0)
    for t0 in (1, 10, 30):
        ya, fa = oracle.scan_f64(x[:, :t0], dt[:, :t0], A, B[:, :t0], C[:, :t0], D, h0)
        yb, fb = oracle.scan_f64(x[:, t0:], dt[:, t0:], A, B[:, t0:], C[:, t0:], D, fa)
        assert nerr(np.concatenate([ya, yb], axis=1), y) < 1e-13
        assert nerr(fb, fs) < 1e-13


def test_linearity_in_x_and_initial_state():
    x1, dt, A, B, C, D, h1 = rand_problem(31)
    x2, _, _, _, _, _, h2 = rand_problem(32)
    a, c = 0.7, -1.3
    y1, f1 = oracle.scan_f64(x1, dt, A, B, C, D, h1)
    y2, f2 = oracle.scan_f64(x2, dt, A, B, C, D, h2)
    y3, f3 = oracle.scan_f64(a * x1 + c * x2, dt, A, B, C, D, a * h1 + c * h2)
    assert nerr(y3, a * y1 + c * y2) < 1e-12
    assert nerr(f3, a * f1 + c * f2) < 1e-12


def test_skip_term_is_additive():
    x, dt, A, B, C, D, h0 = rand_problem(41)
    y, _ = oracle.scan_f64(x, dt, A, B, C, D, h0)
    y0, _ = oracle.scan_f64(x, dt, A, B, C, np.zeros_like(D), h0)
    np.testing.assert_allclose(y - y0, D[None, None, :, None] * x, rtol=1e-12, atol=1e-12)


def test_groups_share_B_and_C():
    """G = 1 equals G = H with B, C replicated per head; G = H heads are independent."""
    x, dt, A, B1, C1, D, h0 = rand_problem(51, G=1)
    H = x.shape[2]
    yg1, fg1 = oracle.scan_f64(x, dt, A, B1, C1, D, h0)
    Brep = np.repeat(B1, H, axis=2)
    Crep = np.repeat(C1, H, axis=2)
    ygH, fgH = oracle.scan_f64(x, dt, A, Brep, Crep, D, h0)
    assert nerr(yg1, ygH) < 1e-14 and nerr(fg1, fgH) < 1e-14
    # G = 2, H = 4: heads 0,1 read group 0, heads 2,3 read group 1
    x, dt, A, B, C, D, h0 = rand_problem(52, G=2)
    y, fs = oracle.scan_f64(x, dt, A, B, C, D, h0)
    for h in range(4):
        g = h // 2
        yh, fh = oracle.scan_f64(x[:, :, h:h + 1], dt[:, :, h:h + 1], A[h:h + 1],
                                 B[:, :, g:g + 1], C[:, :, g:g + 1], D[h:h + 1],
                                 h0[:, h:h + 1])
        assert nerr(yh[:, :, 0], y[:, :, h]) < 1e-14
        assert nerr(fh[:, 0], fs[:, h]) < 1e-14
    # permuting heads inside a group permutes the outputs
    perm = [1, 0, 3, 2]
    yp, fp = oracle.scan_f64(x[:, :, perm], dt[:, :, perm], A[perm], B, C, D[perm], h0[:, perm])
    assert nerr(yp, y[:, :, perm]) < 1e-14 and nerr(fp, fs[:, perm]) < 1e-14


def test_bh_range_computes_only_requested_units():
    x, dt, A, B, C, D, h0 = rand_problem(61)
    y, fs = oracle.scan_f64(x, dt, A, B, C, D, h0)
    ys, fss = oracle.scan_f64(x, dt, A, B, C, D, h0, bh_range=(3, 6))
    for bh in range(8):
        bi, h = divmod(bh, 4)
        if 3 <= bh < 6:
            assert np.array_equal(ys[bi, :, h], y[bi, :, h])
            assert np.array_equal(fss[bi, h], fs[bi, h])
        else:
            assert np.isnan(ys[bi, :, h]).all()


# ------------------------------------------------------------------- verify step
def test_verify_state_selection_semantics():
    """state_out = state after accept_len tokens; 0 -> exact copy of the input state."""
    rng = np.random.default_rng(71)
    b, K, H, P, N, G = 5, 4, 4, 3, 5, 2
    x, dt, A, B, C, D, _ = rand_problem(72, b=b, L=K, H=H, P=P, N=N, G=G, init=False)
    state = rng.standard_normal((b, H, P, N))
    accept = np.array([0, 1, 2, 3, 4], np.int32)
    y, so, sa = oracle.verify_f64(state, x, dt, A, B, C, D, accept)
    ys, _ = oracle.scan_f64(x, dt, A, B, C, D, state)
    assert np.array_equal(y, ys)                       # same arithmetic, same order
    for bi in range(b):
        a = accept[bi]
        if a == 0:
            assert np.array_equal(so[bi], state[bi])
        else:
            assert np.array_equal(so[bi], sa[bi, a - 1])
            _, fa = oracle.scan_f64(x[bi:bi + 1, :a], dt[bi:bi + 1, :a], A, B[bi:bi + 1, :a],
                                    C[bi:bi + 1, :a], D, state[bi:bi + 1])
            assert np.array_equal(so[bi], fa[0])
    with pytest.raises(ValueError):
        oracle.verify_f64(state, x, dt, A, B, C, D, np.array([0, 1, 2, 3, 5], np.int32))
