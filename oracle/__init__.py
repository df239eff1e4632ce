"""Test-infrastructure oracle for the SSD hot path.  NOT PART OF THE PRODUCT.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  It shares no code with the
HIP library (``selective_state_space_ssd_amd``) and never imports it.

Contents
--------
``scan_f64`` / ``verify_f64``
    ctypes wrappers around ``ssd_oracle.c``: the plain sequential fp64
    recurrence (the definition of what the chunked scan and the verify step
    compute).  See the header of ``ssd_oracle.c`` for the cited passages.
``selective_scan_f64``
    the same recurrence with one channel per head and a diagonal A of N values
    per channel (the selective scan the SSD layer replaces; the comparison
    kernel's definition).
``backward.scan_bwd_f64``
    fp64 gradients of the scan (reverse-mode automatic differentiation through a
    plain torch transcription of the recurrence), pinned by finite differences of
    ``scan_f64``.
``ring.verify_ring_f64`` / ``ring.ring_rollback`` / ``ring.softplus_f64``
    multi-round verify on a ring of the most recent per-token states (rounds,
    rollback, and the optional fused step activation softplus(dt + bias)), built on
    ``verify_f64``; pinned by ``tests/test_oracle_ring_pins.py`` against the scan
    oracle over the accepted prefix and against ``numpy.logaddexp``.
``cp.total_decay_f64`` / ``cp.combine_f64`` / ``cp.apply_entering_state_f64``
    the per-device pieces of the sequence-parallel scan (total decay of a slice,
    entering states folded from the slices' pairs, correction of a slice scanned
    from zero); pinned by ``tests/test_oracle_cp_pins.py`` against the scan oracle of
    the whole sequence.
``forms``
    Two further fp64 NumPy formulations of the same map (the quadratic
    "masked attention" form over the semiseparable matrix, and the four-step
    chunked decomposition), used only to pin the recurrence in tests.

Parity status: every function here is pinned by ``tests/test_oracle_*pins.py``
(closed forms, a hand-computed worked example, an IIR-filter library routine,
brute force on tiny inputs, finite differences, invariants).  No function is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB = os.path.join(_HERE, "libssd_oracle.so")
_lib = None

# Error codes of ssd_oracle.c
ORACLE_OK, ORACLE_ERR_DIM, ORACLE_ERR_GROUPS, ORACLE_ERR_ACCEPT, ORACLE_ERR_ALLOC = range(5)


def build(force: bool = False) -> str:
    """Compile ssd_oracle.c with gcc (no HIP, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def load_library(path=None):
    """Open an oracle shared library (default: the built ``libssd_oracle.so``).

    Tests pass another path to load a deliberately broken copy of the oracle and
    check that the pins reject it.
    """
    if path is None:
        path = build()
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    L = ctypes.c_long
    lib.ssd_oracle_scan_f64.argtypes = [dp] * 9 + [L] * 8
    lib.ssd_oracle_scan_f64.restype = ctypes.c_int
    lib.ssd_oracle_verify_f64.argtypes = (
        [dp] * 7 + [ctypes.POINTER(ctypes.c_int32)] + [dp] * 3 + [L] * 6)
    lib.ssd_oracle_verify_f64.restype = ctypes.c_int
    lib.ssd_oracle_selective_scan_f64.argtypes = [dp] * 9 + [L] * 5
    lib.ssd_oracle_selective_scan_f64.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        _lib = load_library()
    return _lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def scan_f64(x, dt, A, B, C, D, init_state=None, bh_range=None, lib=None):
    """Sequential fp64 recurrence over the whole sequence.

    x[b,L,H,P], dt[b,L,H], A[H], B/C[b,L,G,N], D[H], init_state[b,H,P,N] or None.
    Returns (y[b,L,H,P], final_state[b,H,P,N]) as float64.  With ``bh_range``
    = (begin, end) only those flattened (batch*H + head) units are computed;
    the rest of y / final_state is NaN.
    """
    lib = lib or _load()
    x, dt, A, B, C, D = map(_f64, (x, dt, A, B, C, D))
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    init = None if init_state is None else _f64(init_state)
    y = np.full((b, L, H, P), np.nan)
    fs = np.full((b, H, P, N), np.nan)
    lo, hi = (0, b * H) if bh_range is None else bh_range
    rc = lib.ssd_oracle_scan_f64(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                 _ptr(init), _ptr(y), _ptr(fs), b, L, H, P, N, G, lo, hi)
    if rc != ORACLE_OK:
        raise ValueError(f"ssd_oracle_scan_f64 failed with code {rc}")
    return y, fs


def verify_f64(state_in, x, dt, A, B, C, D, accept_len, want_all=True, lib=None):
    """fp64 verify step: K draft tokens applied to ``state_in``.

    Returns (y[b,K,H,P], state_out[b,H,P,N], states_all[b,K,H,P,N] or None).
    ``accept_len`` must lie in [0, K]; the oracle raises otherwise.
    """
    lib = lib or _load()
    state_in, x, dt, A, B, C, D = map(_f64, (state_in, x, dt, A, B, C, D))
    acc = np.ascontiguousarray(accept_len, dtype=np.int32)
    b, K, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    y = np.empty((b, K, H, P))
    so = np.empty((b, H, P, N))
    sa = np.empty((b, K, H, P, N)) if want_all else None
    rc = lib.ssd_oracle_verify_f64(
        _ptr(state_in), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
        acc.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), _ptr(y), _ptr(so), _ptr(sa),
        b, K, H, P, N, G)
    if rc != ORACLE_OK:
        raise ValueError(f"ssd_oracle_verify_f64 failed with code {rc}")
    return y, so, sa


def selective_scan_f64(x, dt, A, B, C, D, init_state=None, lib=None):
    """Sequential fp64 selective scan with one channel per head (diagonal A).

    x[b,L,Dch], dt[b,L,Dch], A[Dch,N], B/C[b,L,G,N], D[Dch], init_state[b,Dch,N] or None.
    Returns (y[b,L,Dch], final_state[b,Dch,N]) as float64.
    """
    lib = lib or _load()
    x, dt, A, B, C, D = map(_f64, (x, dt, A, B, C, D))
    b, L, Dch = x.shape
    G, N = B.shape[2], B.shape[3]
    init = None if init_state is None else _f64(init_state)
    y = np.empty((b, L, Dch))
    fs = np.empty((b, Dch, N))
    rc = lib.ssd_oracle_selective_scan_f64(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                           _ptr(init), _ptr(y), _ptr(fs), b, L, Dch, N, G)
    if rc != ORACLE_OK:
        raise ValueError(f"ssd_oracle_selective_scan_f64 failed with code {rc}")
    return y, fs
