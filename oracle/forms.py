"""Alternative fp64 formulations of the SSD map -- TEST INFRASTRUCTURE ONLY.

These exist to pin the sequential recurrence in ``ssd_oracle.c`` against forms
derived differently on the pages.  Plain NumPy, float64, loops kept visible.

* ``quadratic_form``: the dual "masked attention" form.  The whole sequence map
  is one lower-triangular (semiseparable) matrix M acting on the inputs:
  M[t,s] = (C_t . B_s) * exp(sum_{r=s+1..t} dt_r A) for s <= t, zero above the
  diagonal; y = M (dt o x) + (decay from the start) C_t . h0 + D x.
  Mamba-2 article (msbhsh.com), «SSD 层» and «SSD 算法» (the SSM equals a
  semiseparable-matrix multiply; linear and quadratic forms are dual).
* ``chunked_form``: the four-step block decomposition with chunk length Q.
  Mamba-2 article, «SSD 算法：分块矩阵分解» (diagonal Q x Q blocks computed
  quadratically, off-diagonal blocks are low rank) and «SSD 算法：分块和形态传递»
  (steps 1, 2, 4 parallel over chunks, step 3 a short scan over chunk states).
  The pages strip the step list; the step contents below are this library's
  reading: (1) intra-chunk masked form, (2) per-chunk state from B (x) x,
  (3) chunk-to-chunk state passing, (4) state-to-output through C.
"""
from __future__ import annotations

import numpy as np


def _groups(H, G):
    if H % G:
        raise ValueError("H must be a multiple of G")
    return H // G


def quadratic_form(x, dt, A, B, C, D, init_state=None):
    """Brute-force quadratic form; O(L^2) per head, for tiny inputs only."""
    x, dt, A, B, C, D = (np.asarray(v, dtype=np.float64) for v in (x, dt, A, B, C, D))
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = _groups(H, G)
    y = np.zeros((b, L, H, P))
    for bi in range(b):
        for h in range(H):
            g = h // hpg
            a = dt[bi, :, h] * A[h]                      # log-decay per token
            M = np.zeros((L, L))
            for t in range(L):
                for s in range(t + 1):
                    seg = a[s + 1:t + 1].sum()            # sum_{r=s+1..t} a_r
                    M[t, s] = np.dot(C[bi, t, g], B[bi, s, g]) * np.exp(seg)
            u = dt[bi, :, h, None] * x[bi, :, h, :]      # dt_s x_s, [L, P]
            yh = M @ u
            if init_state is not None:
                h0 = np.asarray(init_state, dtype=np.float64)[bi, h]   # [P, N]
                for t in range(L):
                    yh[t] += np.exp(a[:t + 1].sum()) * (h0 @ C[bi, t, g])
            y[bi, :, h, :] = yh + D[h] * x[bi, :, h, :]
    return y


def chunked_form(x, dt, A, B, C, D, Q, init_state=None):
    """Four-step chunked decomposition, chunk length Q >= 1 (last chunk ragged).

    Returns (y, final_state, chunk_states) where chunk_states[b,h,c] is the state
    entering chunk c (step-3 output).
    """
    x, dt, A, B, C, D = (np.asarray(v, dtype=np.float64) for v in (x, dt, A, B, C, D))
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = _groups(H, G)
    nc = (L + Q - 1) // Q
    y = np.zeros((b, L, H, P))
    final = np.zeros((b, H, P, N))
    entering = np.zeros((b, H, nc, P, N))
    for bi in range(b):
        for h in range(H):
            g = h // hpg
            Hprev = (np.zeros((P, N)) if init_state is None
                     else np.asarray(init_state, dtype=np.float64)[bi, h].copy())
            for c in range(nc):
                t0, t1 = c * Q, min((c + 1) * Q, L)
                a = dt[bi, t0:t1, h] * A[h]
                acum = np.cumsum(a)                       # inclusive, from chunk start
                Xc = x[bi, t0:t1, h, :]                   # [q, P]
                Bc = B[bi, t0:t1, g, :]                   # [q, N]
                Cc = C[bi, t0:t1, g, :]
                u = dt[bi, t0:t1, h, None] * Xc           # dt_s x_s
                q = t1 - t0
                # step 1: diagonal block, masked quadratic form inside the chunk
                Lmask = np.zeros((q, q))
                for t in range(q):
                    for s in range(t + 1):
                        Lmask[t, s] = np.exp(acum[t] - acum[s])
                Ydiag = ((Cc @ Bc.T) * Lmask) @ u
                # step 2: this chunk's own state contribution, decayed to chunk end
                w = np.exp(acum[-1] - acum)               # [q]
                S = (u * w[:, None]).T @ Bc               # [P, N]
                # step 4: incoming state -> outputs through C
                Yoff = np.exp(acum)[:, None] * (Cc @ Hprev.T)
                y[bi, t0:t1, h, :] = Ydiag + Yoff + D[h] * Xc
                entering[bi, h, c] = Hprev
                # step 3: pass the state to the next chunk
                Hprev = np.exp(acum[-1]) * Hprev + S
            final[bi, h] = Hprev
    return y, final, entering
