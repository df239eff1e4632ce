"""Pins for the multi-round verify oracle (``oracle.ring``, CPU only).

The ring oracle is tied to things other than itself:
  * after any sequence of rounds and rollbacks, the head state and every state behind
    it equal the final state of the scan oracle (``oracle.scan_f64``) run over the
    accepted tokens so far, and every round's y equals the scan's outputs on that
    prefix followed by the round's draft tokens;
  * the fused step activation equals the library routine ``numpy.logaddexp(0, v)`` and
    known values of softplus;
  * planted mistakes in copies of the oracle source fail these checks.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import ring


def _problem(seed, b=2, H=4, P=3, N=5, G=2):
    rng = np.random.default_rng(seed)
    A = -np.exp(rng.uniform(0.0, math.log(4.0), H))
    D = rng.standard_normal(H)
    h0 = rng.standard_normal((b, H, P, N))
    return rng, A, D, h0


def _round(rng, b, K, H, P, N, G, biased):
    x = rng.standard_normal((b, K, H, P))
    # raw steps: positive for the plain path, pre-activation values for the biased one
    dt = rng.normal(-1.0, 1.0, (b, K, H)) if biased else rng.uniform(0.05, 0.6, (b, K, H))
    B = rng.standard_normal((b, K, G, N))
    C = rng.standard_normal((b, K, G, N))
    return x, dt, B, C


def _scan_row(tokens, A, D, h0_row):
    """Scan oracle over one batch row's accepted tokens (lists of per-token arrays)."""
    if not tokens:
        return None, h0_row.copy()
    x = np.stack([t[0] for t in tokens])[None]
    dt = np.stack([t[1] for t in tokens])[None]
    B = np.stack([t[2] for t in tokens])[None]
    C = np.stack([t[3] for t in tokens])[None]
    y, fs = oracle.scan_f64(x, dt, A, B, C, D, h0_row[None])
    return y[0], fs[0]


def _run_and_check(mod, seed, b=2, K=3, R=5, H=4, P=3, N=5, G=2, rounds=7, biased=False,
                   rollbacks=True):
    """Drive ``mod`` (the ring oracle or a mutant) through rounds and rollbacks and
    return the worst normalised mismatch against the scan oracle."""
    rng, A, D, h0 = _problem(seed, b, H, P, N, G)
    bias = rng.normal(0.0, 0.5, H) if biased else None
    rg, meta = mod.ring_init_f64(h0, R)
    hist = [[] for _ in range(b)]          # accepted tokens per row: (x, step, B, C)
    exp_depth = [0] * b                    # states behind the head a rollback may reach
    worst = 0.0

    def nerr(a, r):
        return float(np.max(np.abs(a - r)) / max(np.max(np.abs(r)), 1e-300))

    for r in range(rounds):
        x, dt, B, C = _round(rng, b, K, H, P, N, G, biased)
        acc = rng.integers(0, K + 1, size=b)
        if r == 0:
            acc[0] = 0                      # a round that accepts nothing
        if r == 1:
            acc[-1] = K                     # a round that accepts everything
        y, rg, meta = mod.verify_ring_f64(rg, meta, x, dt, A, B, C, D, acc, dt_bias=bias)
        # the step the recurrence used, from the library routine
        step = np.logaddexp(0.0, dt + bias[None, None, :]) if biased else dt
        for bi in range(b):
            drafts = [(x[bi, k], step[bi, k], B[bi, k], C[bi, k]) for k in range(K)]
            yref, _ = _scan_row(hist[bi] + drafts, A, D, h0[bi])
            worst = max(worst, nerr(y[bi], yref[-K:]))
            hist[bi] += drafts[: acc[bi]]
            exp_depth[bi] = min(exp_depth[bi] + int(acc[bi]), R - 1)
        if rollbacks and r in (3, 5):
            steps = np.array([min(int(m[1]), 2 + bi) for bi, m in enumerate(meta)])
            meta = mod.ring_rollback(meta, steps, R)
            for bi in range(b):
                if steps[bi]:
                    hist[bi] = hist[bi][: len(hist[bi]) - steps[bi]]
                exp_depth[bi] -= int(steps[bi])
        # the head state and every state behind it (depth of them)
        for bi in range(b):
            head, depth = int(meta[bi, 0]), int(meta[bi, 1])
            assert depth == exp_depth[bi]
            for j in range(depth + 1):
                _, fs = _scan_row(hist[bi][: len(hist[bi]) - j], A, D, h0[bi])
                worst = max(worst, nerr(rg[bi, (head - j) % R], fs))
    return worst


@pytest.mark.parametrize("seed", [0, 1])
def test_rounds_match_scan_over_accepted_prefix(seed):
    assert _run_and_check(ring, seed, rollbacks=False) < 1e-12


def test_rounds_with_rollbacks_match_scan():
    assert _run_and_check(ring, 2, rollbacks=True) < 1e-12


def test_ring_wraps_many_times():
    # R = K + 1, the smallest ring; 12 rounds wrap it several times
    assert _run_and_check(ring, 3, K=3, R=4, rounds=12, rollbacks=False) < 1e-12


def test_fused_step_activation():
    assert _run_and_check(ring, 4, biased=True, rounds=5) < 1e-12


def test_softplus_values():
    v = np.array([-800.0, -40.0, -1.0, 0.0, 1e-8, 1.0, 30.0, 800.0])
    s = ring.softplus_f64(v)
    assert s[3] == math.log(2.0)
    assert np.allclose(s, np.logaddexp(0.0, v), rtol=1e-15, atol=0)
    assert s[0] == 0.0 or s[0] < 1e-300            # e^-800 underflows to 0
    assert s[-1] == 800.0
    assert np.allclose(s - ring.softplus_f64(-v), v, rtol=1e-15, atol=1e-15)


def test_rejects_invalid_calls():
    rng, A, D, h0 = _problem(5)
    rg, meta = ring.ring_init_f64(h0, 4)
    x, dt, B, C = _round(rng, 2, 4, 4, 3, 5, 2, False)
    with pytest.raises(ValueError):                 # K = R
        ring.verify_ring_f64(rg, meta, x, dt, A, B, C, D, [1, 1])
    x, dt, B, C = _round(rng, 2, 3, 4, 3, 5, 2, False)
    with pytest.raises(ValueError):                 # accept_len > K
        ring.verify_ring_f64(rg, meta, x, dt, A, B, C, D, [4, 0])
    with pytest.raises(ValueError):                 # rollback beyond depth
        ring.ring_rollback(meta, [1, 0], 4)


def test_clamped_rollback():
    meta = np.array([[3, 2], [0, 4], [1, 0]])
    ok, flag = ring.ring_rollback(meta, [1, 4, 0], 5, clamp=True)
    assert not flag and np.array_equal(ok, ring.ring_rollback(meta, [1, 4, 0], 5))
    out, flag = ring.ring_rollback(meta, [5, -1, 2], 5, clamp=True)
    assert flag
    assert np.array_equal(out, [[1, 0], [0, 4], [1, 0]])   # back to the oldest state


MUTANTS = {
    "slot_off_by_one": ("(head[bi] + k + 1) % R", "(head[bi] + k) % R"),
    "head_not_advanced": ("meta_out[bi, 0] = (head[bi] + a) % R", "meta_out[bi, 0] = head[bi] % R"),
    "depth_not_saturated": ("min(meta[bi, 1] + a, R - 1)", "meta[bi, 1] + a"),
    "rollback_forward": ("(meta[:, 0] - n) % R", "(meta[:, 0] + n) % R"),
    "softplus_no_log1p": ("np.log1p(np.exp(-np.abs(v)))", "np.exp(-np.abs(v))"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    old, new = MUTANTS[name]
    src = open(ring.__file__).read()
    assert old in src, f"mutation anchor for {name} not found"
    src = src.replace("from . import verify_f64", "from oracle import verify_f64")
    ns = {"__name__": "mutant_ring"}
    exec(compile(src.replace(old, new, 1), "mutant_ring", "exec"), ns)

    class M:
        pass
    mod = M()
    for k in ("ring_init_f64", "verify_ring_f64", "ring_rollback", "softplus_f64"):
        setattr(mod, k, ns[k])
    try:
        worst = max(_run_and_check(mod, 6, K=3, R=4, rounds=10, rollbacks=True),
                    _run_and_check(mod, 7, biased=True, rounds=4, rollbacks=False))
    except (AssertionError, ValueError, IndexError):
        return                                      # caught by an assertion
    assert worst > 1e-6, f"mutant {name} survived"
