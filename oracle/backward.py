"""fp64 gradients of the SSD scan -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module; it shares no code with the HIP library.

Definition: for the recurrence of ``ssd_oracle.c`` ("另辟蹊径--Mamba介绍", «The
Recurrent Representation»; per (b, h), group g = h / (H/G))

    s_t = exp(dt_t A_h) s_{t-1} + dt_t x_t (outer) B_t,     s_{-1} = init_state
    y_t = C_t . s_t + D_h x_t,                              final_state = s_{L-1}

and upstream gradients dy (same shape as y) and d_final (same shape as the final
state, or none), the gradients are those of the scalar

    loss = sum(dy * y) + sum(d_final * final_state)

with respect to x, dt, A, B, C, D and init_state.  They are computed by reverse-mode
automatic differentiation (``torch.autograd``, used as a library primitive) through
a plain float64 transcription of the recurrence above: one token at a time, no
chunking.  Pinned in ``tests/test_oracle_backward_pins.py`` by central finite
differences of the C oracle and by closed forms.
"""
from __future__ import annotations

import numpy as np
import torch


def scan_bwd_f64(x, dt, A, B, C, D, init_state, dy, d_final=None):
    """Gradients (dx, ddt, dA, dB, dC, dD, d_init) as float64 numpy arrays.

    x[b,L,H,P], dt[b,L,H], A[H], B/C[b,L,G,N], D[H], init_state[b,H,P,N] or None,
    dy[b,L,H,P], d_final[b,H,P,N] or None.  d_init is returned even when
    init_state is None (the gradient with respect to a zero initial state).
    """
    f = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), dtype=torch.float64)
    x, dt, A, B, C, D, dy = (f(v) for v in (x, dt, A, B, C, D, dy))
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if H % G:
        raise ValueError("H must be a multiple of G")
    h0 = torch.zeros((b, H, P, N), dtype=torch.float64) if init_state is None else f(init_state)
    params = [x, dt, A, B, C, D, h0]
    for p in params:
        p.requires_grad_(True)
    g = torch.arange(H) // (H // G)          # group of every head
    s = h0
    ys = []
    for t in range(L):
        Bt = B[:, t][:, g]                   # [b, H, N]
        Ct = C[:, t][:, g]
        decay = torch.exp(dt[:, t] * A)      # [b, H]
        s = decay[:, :, None, None] * s + (dt[:, t, :, None] * x[:, t])[..., None] * Bt[:, :, None, :]
        ys.append((s * Ct[:, :, None, :]).sum(-1) + D[None, :, None] * x[:, t])
    loss = (torch.stack(ys, dim=1) * dy).sum() if L > 0 else torch.zeros((), dtype=torch.float64)
    if d_final is not None:
        loss = loss + (s * f(d_final)).sum()
    grads = torch.autograd.grad(loss, params, allow_unused=True)
    out = []
    for p, gr in zip(params, grads):
        out.append(np.zeros(tuple(p.shape)) if gr is None else gr.numpy())
    return tuple(out)
