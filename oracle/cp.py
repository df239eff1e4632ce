"""Sequence-parallel (context-parallel) scan pieces -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module; it shares no code with the HIP library.

The Mamba-2 article (msbhsh.com, «序列并行») splits a long sequence over devices: each
device scans its slice from a zero state, the devices exchange their final states
(and the total decay of their slice), each device folds its predecessors' pairs into
the state entering its slice, and its outputs are corrected by that state's
contribution.  The pairs compose associatively because the state passing is linear
(Mamba intro page, «The Scan Operation»; Mamba-2 article, «SSD 算法：分块和形态传递»,
step 3 over slices instead of chunks).  With a_t = dt_t A_h and, inside one slice,
cum_t = sum_{r <= t} a_r:

* total decay of a slice:  alpha = exp(cum_last)
* entering states:         h_in[0] = init_state,  h_in[j + 1] = alpha_j h_in[j] + S_j
  (S_j the final state of slice j scanned from zero)
* correction of slice j:   y_t += exp(cum_t) C_t . h_in[j]   (sum over N, for every p)
                           final_j += exp(cum_last) h_in[j]

Pinned in ``tests/test_oracle_cp_pins.py``: the pieces, run over n slices of a
sequence, reproduce the scan oracle (``oracle.scan_f64``) of the whole sequence.
"""
from __future__ import annotations

import numpy as np


def total_decay_f64(dt, A):
    """alpha[b, h] = exp(sum_t dt[b, t, h] A[h]) for dt [b, L, H], A [H]."""
    dt = np.asarray(dt, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    return np.exp(dt.sum(axis=1) * A[None, :])


def combine_f64(alpha, S, init_state=None):
    """Entering states of n slices: alpha [n, b, H], S [n, b, H, P, N], init_state
    [b, H, P, N] or None (zeros).  Returns h_in [n, b, H, P, N]."""
    alpha = np.asarray(alpha, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    h = np.zeros(S.shape[1:]) if init_state is None else np.asarray(init_state, dtype=np.float64)
    out = np.empty_like(S)
    for j in range(S.shape[0]):
        out[j] = h
        h = alpha[j][:, :, None, None] * h + S[j]
    return out


def apply_entering_state_f64(y, final_state, dt, A, C, h_in):
    """Corrected outputs and final state of one slice scanned from zero.

    y [b, L, H, P] and final_state [b, H, P, N] (or None) of the zero-state scan; dt
    [b, L, H]; A [H]; C [b, L, G, N]; h_in [b, H, P, N].  Returns (y', final')."""
    y = np.array(y, dtype=np.float64)
    dt = np.asarray(dt, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    h_in = np.asarray(h_in, dtype=np.float64)
    b, L, H, P = y.shape
    G = C.shape[2]
    g = np.arange(H) // (H // G)
    fin = None if final_state is None else np.array(final_state, dtype=np.float64)
    for bi in range(b):
        for h in range(H):
            cum = 0.0
            for t in range(L):
                cum += dt[bi, t, h] * A[h]
                y[bi, t, h] += np.exp(cum) * (h_in[bi, h] @ C[bi, t, g[h]])
            if fin is not None:
                fin[bi, h] += np.exp(cum) * h_in[bi, h]
    return y, fin
