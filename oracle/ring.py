"""Multi-round verify on a ring of states -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module; it shares no code with the HIP library.

What it computes (plain float64, one verify round at a time):

* A speculative-decoding verifier over a Mamba layer keeps a ring buffer of the most
  recent states and, when a draft token is rejected, restores the state of the last
  accepted position ("Llama 3与Mamba混合架构：加速推理的蒸馏技术解析", «状态管理机制»;
  "如何将 Llama 变成 Mamba？研究人员推出新工作并提高推理速度", «推测解码»: only the
  state at the position where the draft stops matching is kept).
* The ring holds, per batch row, R states of shape [H, P, N]; ``meta[b] = (head,
  depth)``: slot ``head`` holds the current state, and the ``depth`` slots behind it
  (head - 1, head - 2, ... modulo R) hold the states of the ``depth`` positions before
  it, so a later rollback can go back up to ``depth`` tokens.
* One round with K draft tokens and ``a = accept_len[b]`` accepted: the verify step
  (``oracle.verify_f64``, the fp64 recurrence) runs all K tokens from the head state
  and returns y for every position; the states after tokens 1..a go to slots
  head + 1 .. head + a (mod R), then ``head <- (head + a) mod R`` and
  ``depth <- min(depth + a, R - 1)``.  K < R, so the head slot is never overwritten
  during a round.
* A rollback by n (0 <= n <= depth) moves ``head`` back n slots and lowers ``depth``
  by n; the states ahead of the new head stay in the ring but are no longer reachable.
* Optional fused step activation (the discretisation step with step size Delta
  computed in the kernel: "另辟蹊径--Mamba介绍", «Hardware-aware Algorithm»): with a
  bias vector per head, the step used is softplus(dt + dt_bias[h]) instead of dt,
  softplus(v) = ln(1 + e^v), evaluated here as max(v, 0) + ln(1 + e^{-|v|}), an exact
  rearrangement that does not overflow.

Pinned in ``tests/test_oracle_ring_pins.py`` (multi-round equivalence with the scan
oracle over the accepted prefix, rollback, wrap-around, softplus values and the
library routine ``numpy.logaddexp``, planted mistakes).
"""
from __future__ import annotations

import numpy as np

from . import verify_f64


def softplus_f64(v):
    """ln(1 + e^v) in float64, as max(v, 0) + log1p(e^{-|v|})."""
    v = np.asarray(v, dtype=np.float64)
    return np.maximum(v, 0.0) + np.log1p(np.exp(-np.abs(v)))


def ring_init_f64(init_state, R):
    """A ring whose slot 0 holds init_state (zeros when None; shape [b, H, P, N]) and
    whose head and depth are 0.  Returns (ring [b, R, H, P, N], meta [b, 2])."""
    s = np.asarray(init_state, dtype=np.float64)
    ring = np.zeros((s.shape[0], R) + s.shape[1:])
    ring[:, 0] = s
    return ring, np.zeros((s.shape[0], 2), dtype=np.int64)


def verify_ring_f64(ring, meta, x, dt, A, B, C, D, accept_len, dt_bias=None):
    """One verify round on the ring.  Returns (y, ring', meta'); the inputs are not
    modified.  Raises on accept_len outside [0, K] or K >= R."""
    ring = np.asarray(ring, dtype=np.float64)
    meta = np.asarray(meta, dtype=np.int64)
    b, R = ring.shape[:2]
    K = x.shape[1]
    if K >= R:
        raise ValueError("the ring must hold more states than there are draft tokens")
    acc = np.asarray(accept_len, dtype=np.int64)
    if np.any(acc < 0) or np.any(acc > K):
        raise ValueError("accept_len outside [0, K]")
    step = np.asarray(dt, dtype=np.float64)
    if dt_bias is not None:
        step = softplus_f64(step + np.asarray(dt_bias, dtype=np.float64)[None, None, :])
    head = meta[:, 0]
    state_in = ring[np.arange(b), head]
    y, _, states_all = verify_f64(state_in, x, step, A, B, C, D, acc.astype(np.int32),
                                  want_all=True)
    ring_out = ring.copy()
    meta_out = meta.copy()
    for bi in range(b):
        a = int(acc[bi])
        for k in range(a):
            ring_out[bi, (head[bi] + k + 1) % R] = states_all[bi, k]
        meta_out[bi, 0] = (head[bi] + a) % R
        meta_out[bi, 1] = min(meta[bi, 1] + a, R - 1)
    return y, ring_out, meta_out


def ring_rollback(meta, steps, R, clamp=False):
    """Move every row's head back by steps[b] slots (0 <= steps[b] <= depth).
    Returns meta'.  A step count outside that range raises, or with ``clamp`` is
    clamped into it (the device's documented behaviour); then (meta', flag) is
    returned, flag telling whether any count was out of range."""
    meta = np.asarray(meta, dtype=np.int64)
    steps = np.asarray(steps, dtype=np.int64)
    bad = (steps < 0) | (steps > meta[:, 1])
    if np.any(bad) and not clamp:
        raise ValueError("rollback outside [0, depth]")
    n = np.clip(steps, 0, meta[:, 1])
    out = meta.copy()
    out[:, 0] = (meta[:, 0] - n) % R
    out[:, 1] = meta[:, 1] - n
    return (out, bool(np.any(bad))) if clamp else out
