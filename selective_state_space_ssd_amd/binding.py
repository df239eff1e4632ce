"""Thin Python binding of libssd_mi355x.so (the C ABI in include/ssd_mi355x.h).

The functions named like the C entry points (``ssd_chunk_scan_fwd``,
``ssd_verify_step``, ...) only marshal torch tensors into pointers and sizes and
raise on a non-OK status; all computation happens in the HIP kernels.  The
convenience wrappers ``chunk_scan_fwd`` and ``verify_step`` additionally allocate
the outputs and the workspace with torch.  There is no fallback: if the library is
not built, or a tensor is not on the GPU, a call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssd_mi355x.so")

SSD_DTYPE_F32 = 0
SSD_DTYPE_BF16 = 1

STATUS_NAMES = {
    0: "SSD_OK", 1: "SSD_ERR_NULL_ARG", 2: "SSD_ERR_BAD_DIM", 3: "SSD_ERR_GROUPS",
    4: "SSD_ERR_UNSUPPORTED", 5: "SSD_ERR_ALIGN", 6: "SSD_ERR_WORKSPACE", 7: "SSD_ERR_ALIAS",
    8: "SSD_ERR_HIP",
}

# Every symbol declared in include/ssd_mi355x.h
EXPORTED = ("ssd_chunk_scan_workspace_bytes", "ssd_chunk_scan_workspace_init",
            "ssd_chunk_scan_workspace_error", "ssd_chunk_scan_fwd",
            "ssd_chunk_scan_fwd_noalloc", "ssd_verify_step", "ssd_selective_scan_fwd",
            "ssd_chunk_scan_bwd_workspace_bytes", "ssd_chunk_scan_bwd",
            "ssd_verify_ring_init", "ssd_verify_ring", "ssd_verify_ring_rollback",
            "ssd_seq_slice_state_workspace_bytes", "ssd_seq_slice_state",
            "ssd_seq_total_decay", "ssd_seq_combine", "ssd_seq_apply_state",
            "ssd_status_string", "ssd_version")

_lib = None


class SSDError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} "
                         f"({lib().ssd_status_string(status).decode()})")


def lib() -> ctypes.CDLL:
    """Open libssd_mi355x.so (built in-tree by selective_state_space_ssd_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -m selective_state_space_ssd_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.ssd_chunk_scan_workspace_bytes.argtypes = [i32] * 7 + [i32]
        L.ssd_chunk_scan_workspace_bytes.restype = sz
        L.ssd_chunk_scan_workspace_init.argtypes = [vp, sz, vp]
        L.ssd_chunk_scan_workspace_init.restype = i32
        L.ssd_chunk_scan_workspace_error.argtypes = [vp, sz, vp, i32, vp]
        L.ssd_chunk_scan_workspace_error.restype = i32
        L.ssd_chunk_scan_fwd.argtypes = [vp] * 9 + [i32] * 7 + [i32, vp, sz, vp]
        L.ssd_chunk_scan_fwd.restype = i32
        L.ssd_chunk_scan_fwd_noalloc.argtypes = [vp] * 9 + [i32] * 7 + [i32, vp]
        L.ssd_chunk_scan_fwd_noalloc.restype = i32
        L.ssd_verify_step.argtypes = [vp] * 12 + [i32] * 6 + [i32, vp]
        L.ssd_verify_step.restype = i32
        L.ssd_selective_scan_fwd.argtypes = [vp] * 9 + [i32] * 5 + [i32, vp]
        L.ssd_selective_scan_fwd.restype = i32
        L.ssd_chunk_scan_bwd_workspace_bytes.argtypes = [i32] * 6 + [i32]
        L.ssd_chunk_scan_bwd_workspace_bytes.restype = sz
        L.ssd_chunk_scan_bwd.argtypes = [vp] * 16 + [i32] * 6 + [i32, vp, sz, vp]
        L.ssd_chunk_scan_bwd.restype = i32
        L.ssd_verify_ring_init.argtypes = [vp, vp, vp] + [i32] * 5 + [vp]
        L.ssd_verify_ring_init.restype = i32
        L.ssd_verify_ring.argtypes = [vp] * 12 + [i32] * 7 + [i32, vp]
        L.ssd_verify_ring.restype = i32
        L.ssd_verify_ring_rollback.argtypes = [vp, vp, vp, i32, i32, vp]
        L.ssd_verify_ring_rollback.restype = i32
        L.ssd_seq_slice_state_workspace_bytes.argtypes = [i32] * 6 + [i32]
        L.ssd_seq_slice_state_workspace_bytes.restype = sz
        L.ssd_seq_slice_state.argtypes = [vp] * 6 + [i32] * 6 + [i32, vp, sz, vp]
        L.ssd_seq_slice_state.restype = i32
        L.ssd_seq_total_decay.argtypes = [vp, vp, vp, i32, i32, i32, vp]
        L.ssd_seq_total_decay.restype = i32
        L.ssd_seq_combine.argtypes = [vp] * 4 + [i32] * 5 + [vp]
        L.ssd_seq_combine.restype = i32
        L.ssd_seq_apply_state.argtypes = [vp] * 6 + [i32] * 6 + [i32, vp]
        L.ssd_seq_apply_state.restype = i32
        L.ssd_status_string.argtypes = [i32]
        L.ssd_status_string.restype = ctypes.c_char_p
        L.ssd_version.argtypes = []
        L.ssd_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def ssd_version() -> str:
    return lib().ssd_version().decode()


def ssd_status_string(status: int) -> str:
    return lib().ssd_status_string(status).decode()


def _io_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SSD_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return SSD_DTYPE_BF16
    raise TypeError(f"x/B/C/y must be float32 or bfloat16, got {t.dtype}")


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def ssd_chunk_scan_workspace_bytes(b, L, H, P, N, G, Q, io: int) -> int:
    n = lib().ssd_chunk_scan_workspace_bytes(b, L, H, P, N, G, Q, io)
    if n == ctypes.c_size_t(-1).value:
        raise SSDError(2, "ssd_chunk_scan_workspace_bytes")
    return n


def ssd_chunk_scan_workspace_init(workspace: torch.Tensor, stream=None) -> None:
    """Prepare a workspace (uint8 GPU tensor) once before its first chunk-scan call."""
    st = lib().ssd_chunk_scan_workspace_init(_ptr(workspace, "workspace"),
                                             workspace.numel() * workspace.element_size(),
                                             _stream(stream))
    if st != 0:
        raise SSDError(st, "ssd_chunk_scan_workspace_init")


def ssd_chunk_scan_workspace_error(workspace: torch.Tensor, err_out: torch.Tensor, clear=False,
                                   stream=None) -> None:
    """Enqueue a copy of the workspace's time-out error word into ``err_out`` (an int32
    GPU tensor of at least one element); ``clear`` resets the word afterwards."""
    st = lib().ssd_chunk_scan_workspace_error(
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _ptr(err_out, "err_out", torch.int32), 1 if clear else 0, _stream(stream))
    if st != 0:
        raise SSDError(st, "ssd_chunk_scan_workspace_error")


def ssd_chunk_scan_fwd(x, dt, A, B, C, D, init_state, y, final_state, Q, workspace,
                       stream=None) -> None:
    """Enqueue the chunked scan on ``stream`` (default: torch's current stream).

    x[b,L,H,P], B/C[b,L,G,N], y[b,L,H,P] share one dtype (float32 or bfloat16);
    dt[b,L,H], A[H], D[H], init_state/final_state[b,H,P,N] are float32
    (init_state and final_state may be None); workspace is a uint8 tensor of at
    least ssd_chunk_scan_workspace_bytes(...) bytes.
    """
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    io = _io_code(x)
    f32 = torch.float32
    st = lib().ssd_chunk_scan_fwd(
        _ptr(x, "x", x.dtype), _ptr(dt, "dt", f32), _ptr(A, "A", f32), _ptr(B, "B", x.dtype),
        _ptr(C, "C", x.dtype), _ptr(D, "D", f32), _ptr(init_state, "init_state", f32),
        _ptr(y, "y", x.dtype), _ptr(final_state, "final_state", f32), b, L, H, P, N, G, Q, io,
        _ptr(workspace, "workspace"), 0 if workspace is None else workspace.numel() *
        workspace.element_size(), _stream(stream))
    if st != 0:
        raise SSDError(st, "ssd_chunk_scan_fwd")


NOALLOC_WORKSPACE_BYTES = 64 << 20


def ssd_chunk_scan_fwd_noalloc(x, dt, A, B, C, D, init_state, y, final_state, Q,
                               stream=None) -> None:
    """Enqueue the chunked scan with the library's own per-GPU workspace buffer (no
    workspace argument, nothing allocated); arguments otherwise as ssd_chunk_scan_fwd."""
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    io = _io_code(x)
    f32 = torch.float32
    st = lib().ssd_chunk_scan_fwd_noalloc(
        _ptr(x, "x", x.dtype), _ptr(dt, "dt", f32), _ptr(A, "A", f32), _ptr(B, "B", x.dtype),
        _ptr(C, "C", x.dtype), _ptr(D, "D", f32), _ptr(init_state, "init_state", f32),
        _ptr(y, "y", x.dtype), _ptr(final_state, "final_state", f32), b, L, H, P, N, G, Q, io,
        _stream(stream))
    if st != 0:
        raise SSDError(st, "ssd_chunk_scan_fwd_noalloc")


def ssd_verify_step(state_in, x, dt, A, B, C, D, accept_len, y, state_out, states_all=None,
                    err_flag=None, stream=None) -> None:
    """Enqueue the verify step on ``stream`` (default: torch's current stream)."""
    b, K, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    io = _io_code(x)
    f32 = torch.float32
    st = lib().ssd_verify_step(
        _ptr(state_in, "state_in", f32), _ptr(x, "x", x.dtype), _ptr(dt, "dt", f32),
        _ptr(A, "A", f32), _ptr(B, "B", x.dtype), _ptr(C, "C", x.dtype), _ptr(D, "D", f32),
        _ptr(accept_len, "accept_len", torch.int32), _ptr(y, "y", x.dtype),
        _ptr(state_out, "state_out", f32), _ptr(states_all, "states_all", f32),
        _ptr(err_flag, "err_flag", torch.int32), b, K, H, P, N, G, io, _stream(stream))
    if st != 0:
        raise SSDError(st, "ssd_verify_step")


def ssd_selective_scan_fwd(x, dt, A, B, C, D, init_state, y, final_state, stream=None) -> None:
    """Enqueue the one-channel-per-head selective scan (diagonal A) on ``stream``.

    x[b,L,Dch], B/C[b,L,G,N], y[b,L,Dch] share one dtype (float32 or bfloat16);
    dt[b,L,Dch], A[Dch,N], D[Dch], init_state/final_state[b,Dch,N] are float32
    (init_state and final_state may be None).
    """
    b, L, Dch = x.shape
    G, N = B.shape[2], B.shape[3]
    io = _io_code(x)
    f32 = torch.float32
    st = lib().ssd_selective_scan_fwd(
        _ptr(x, "x", x.dtype), _ptr(dt, "dt", f32), _ptr(A, "A", f32), _ptr(B, "B", x.dtype),
        _ptr(C, "C", x.dtype), _ptr(D, "D", f32), _ptr(init_state, "init_state", f32),
        _ptr(y, "y", x.dtype), _ptr(final_state, "final_state", f32), b, L, Dch, N, G, io,
        _stream(stream))
    if st != 0:
        raise SSDError(st, "ssd_selective_scan_fwd")


def ssd_chunk_scan_bwd_workspace_bytes(b, L, H, P, N, G, io: int) -> int:
    n = lib().ssd_chunk_scan_bwd_workspace_bytes(b, L, H, P, N, G, io)
    if n == ctypes.c_size_t(-1).value:
        raise SSDError(2, "ssd_chunk_scan_bwd_workspace_bytes")
    return n


def ssd_chunk_scan_bwd(x, dt, A, B, C, D, init_state, dy, d_final, dx, ddt, dA, dB, dC, dD,
                       d_init, workspace, stream=None) -> None:
    """Enqueue the gradients of the chunked scan on ``stream``.

    Inputs as for ssd_chunk_scan_fwd plus dy (like x) and d_final[b,H,P,N] float32
    (may be None); outputs dx (like x), ddt[b,L,H], dA[H], dD[H] float32, dB/dC (like
    B), d_init[b,H,P,N] float32 (may be None); workspace is a uint8 tensor of at least
    ssd_chunk_scan_bwd_workspace_bytes(...) bytes.
    """
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    io = _io_code(x)
    f32 = torch.float32
    st = lib().ssd_chunk_scan_bwd(
        _ptr(x, "x", x.dtype), _ptr(dt, "dt", f32), _ptr(A, "A", f32), _ptr(B, "B", x.dtype),
        _ptr(C, "C", x.dtype), _ptr(D, "D", f32), _ptr(init_state, "init_state", f32),
        _ptr(dy, "dy", x.dtype), _ptr(d_final, "d_final", f32), _ptr(dx, "dx", x.dtype),
        _ptr(ddt, "ddt", f32), _ptr(dA, "dA", f32), _ptr(dB, "dB", x.dtype),
        _ptr(dC, "dC", x.dtype), _ptr(dD, "dD", f32), _ptr(d_init, "d_init", f32),
        b, L, H, P, N, G, io, _ptr(workspace, "workspace"),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream))
    if st != 0:
        raise SSDError(st, "ssd_chunk_scan_bwd")


def ssd_verify_ring_init(ring, meta, init_state=None, stream=None) -> None:
    """Slot 0 of every row of ``ring`` [b,R,H,P,N] float32 <- init_state [b,H,P,N]
    (None = zeros); ``meta`` [b,2] int32 <- (0, 0)."""
    b, R, H, P, N = ring.shape
    st = lib().ssd_verify_ring_init(_ptr(ring, "ring", torch.float32), _ptr(meta, "meta", torch.int32),
                                    _ptr(init_state, "init_state", torch.float32), b, R, H, P, N,
                                    _stream(stream))
    if st != 0:
        raise SSDError(st, "ssd_verify_ring_init")


def ssd_verify_ring(ring, meta, x, dt, A, B, C, D, accept_len, y, dt_bias=None, err_flag=None,
                    stream=None) -> None:
    """Enqueue one verify round on the ring (see include/ssd_mi355x.h)."""
    b, R = ring.shape[:2]
    _, K, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    io = _io_code(x)
    f32 = torch.float32
    st = lib().ssd_verify_ring(
        _ptr(ring, "ring", f32), _ptr(meta, "meta", torch.int32), _ptr(x, "x", x.dtype),
        _ptr(dt, "dt", f32), _ptr(dt_bias, "dt_bias", f32), _ptr(A, "A", f32),
        _ptr(B, "B", x.dtype), _ptr(C, "C", x.dtype), _ptr(D, "D", f32),
        _ptr(accept_len, "accept_len", torch.int32), _ptr(y, "y", x.dtype),
        _ptr(err_flag, "err_flag", torch.int32), b, K, R, H, P, N, G, io, _stream(stream))
    if st != 0:
        raise SSDError(st, "ssd_verify_ring")


def ssd_verify_ring_rollback(meta, steps, err_flag=None, R=None, stream=None) -> None:
    """Move every row's ring head back by steps[b] (int32 [b]) slots; R is the ring
    length."""
    b = meta.shape[0]
    st = lib().ssd_verify_ring_rollback(_ptr(meta, "meta", torch.int32),
                                        _ptr(steps, "steps", torch.int32),
                                        _ptr(err_flag, "err_flag", torch.int32), b, R,
                                        _stream(stream))
    if st != 0:
        raise SSDError(st, "ssd_verify_ring_rollback")


def ssd_seq_slice_state_workspace_bytes(b, L, H, P, N, G, io) -> int:
    n = lib().ssd_seq_slice_state_workspace_bytes(b, L, H, P, N, G, io)
    if n == ctypes.c_size_t(-1).value:
        raise SSDError(4, "ssd_seq_slice_state_workspace_bytes")
    return n


def ssd_seq_slice_state(x, dt, A, B, state, alpha, workspace, stream=None) -> None:
    """state [b,H,P,N] and alpha [b,H] (float32) of the slice x, dt, B from a zero state;
    workspace: a uint8 GPU tensor of ssd_seq_slice_state_workspace_bytes (or None when 0)."""
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    f32 = torch.float32
    ws_bytes = 0 if workspace is None else workspace.numel()
    st = lib().ssd_seq_slice_state(_ptr(x, "x", x.dtype), _ptr(dt, "dt", f32), _ptr(A, "A", f32),
                                   _ptr(B, "B", x.dtype), _ptr(state, "state", f32),
                                   _ptr(alpha, "alpha", f32), b, L, H, P, N, G, _io_code(x),
                                   _ptr(workspace, "workspace", torch.uint8), ws_bytes,
                                   _stream(stream))
    if st != 0:
        raise SSDError(st, "ssd_seq_slice_state")


def ssd_seq_total_decay(dt, A, alpha, stream=None) -> None:
    """alpha[b,h] = exp(sum_t dt[b,t,h] A[h]) (all float32)."""
    b, L, H = dt.shape
    f32 = torch.float32
    st = lib().ssd_seq_total_decay(_ptr(dt, "dt", f32), _ptr(A, "A", f32), _ptr(alpha, "alpha", f32),
                                   b, L, H, _stream(stream))
    if st != 0:
        raise SSDError(st, "ssd_seq_total_decay")


def ssd_seq_combine(alpha, S, init_state, h_in, stream=None) -> None:
    """Entering states of n slices from alpha [n,b,H] and final states S [n,b,H,P,N]."""
    n, b, H, P, N = S.shape
    f32 = torch.float32
    st = lib().ssd_seq_combine(_ptr(alpha, "alpha", f32), _ptr(S, "S", f32),
                               _ptr(init_state, "init_state", f32), _ptr(h_in, "h_in", f32),
                               n, b, H, P, N, _stream(stream))
    if st != 0:
        raise SSDError(st, "ssd_seq_combine")


def ssd_seq_apply_state(y, final_state, dt, A, C, h_in, stream=None) -> None:
    """Correct a slice scanned from zero by its entering state h_in (in place)."""
    b, L, H, P = y.shape
    G, N = C.shape[2], C.shape[3]
    f32 = torch.float32
    st = lib().ssd_seq_apply_state(_ptr(y, "y", y.dtype), _ptr(final_state, "final_state", f32),
                                   _ptr(dt, "dt", f32), _ptr(A, "A", f32), _ptr(C, "C", y.dtype),
                                   _ptr(h_in, "h_in", f32), b, L, H, P, N, G, _io_code(y),
                                   _stream(stream))
    if st != 0:
        raise SSDError(st, "ssd_seq_apply_state")


# ------------------------------------------------------------ allocating wrappers
def chunk_scan_workspace(x, B, Q, stream=None) -> torch.Tensor:
    """Allocate and prepare a workspace for chunk scans of x's and B's shapes."""
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    n = ssd_chunk_scan_workspace_bytes(b, L, H, P, N, G, Q, _io_code(x))
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=x.device)
    ssd_chunk_scan_workspace_init(ws, stream)
    return ws


def seq_slice_state(x, dt, A, B, stream=None):
    """Allocate the outputs and the workspace; returns (state, alpha) of the slice."""
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    n = ssd_seq_slice_state_workspace_bytes(b, L, H, P, N, G, _io_code(x))
    ws = torch.empty(n, dtype=torch.uint8, device=x.device) if n else None
    state = torch.empty((b, H, P, N), dtype=torch.float32, device=x.device)
    alpha = torch.empty((b, H), dtype=torch.float32, device=x.device)
    ssd_seq_slice_state(x, dt, A, B, state, alpha, ws, stream)
    return state, alpha


def chunk_scan_fwd(x, dt, A, B, C, D, Q, init_state=None, workspace=None, stream=None):
    """Allocate y, final_state (and the workspace if not given); returns (y, final_state)."""
    b, L, H, P = x.shape
    N = B.shape[3]
    y = torch.empty_like(x)
    final_state = torch.empty((b, H, P, N), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = chunk_scan_workspace(x, B, Q)
    ssd_chunk_scan_fwd(x, dt, A, B, C, D, init_state, y, final_state, Q, workspace, stream)
    return y, final_state


def chunk_scan_bwd(x, dt, A, B, C, D, dy, init_state=None, d_final=None, workspace=None,
                   stream=None):
    """Allocate the gradients (and the workspace if not given); returns
    (dx, ddt, dA, dB, dC, dD, d_init)."""
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev = x.device
    f32 = torch.float32
    dx, dB, dC = torch.empty_like(x), torch.empty_like(B), torch.empty_like(C)
    ddt = torch.empty((b, L, H), dtype=f32, device=dev)
    dA = torch.empty((H,), dtype=f32, device=dev)
    dD = torch.empty((H,), dtype=f32, device=dev)
    d_init = torch.empty((b, H, P, N), dtype=f32, device=dev)
    if workspace is None:
        n = ssd_chunk_scan_bwd_workspace_bytes(b, L, H, P, N, G, _io_code(x))
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
    ssd_chunk_scan_bwd(x, dt, A, B, C, D, init_state, dy, d_final, dx, ddt, dA, dB, dC, dD,
                       d_init, workspace, stream)
    return dx, ddt, dA, dB, dC, dD, d_init


def verify_step(state, x, dt, A, B, C, D, accept_len, return_all_states=False, stream=None):
    """Allocate outputs; returns (y, state_out) or (y, state_out, states_all)."""
    b, K, H, P = x.shape
    N = B.shape[3]
    y = torch.empty_like(x)
    state_out = torch.empty_like(state)
    states_all = (torch.empty((b, K, H, P, N), dtype=torch.float32, device=x.device)
                  if return_all_states else None)
    ssd_verify_step(state, x, dt, A, B, C, D, accept_len, y, state_out, states_all, None, stream)
    return (y, state_out, states_all) if return_all_states else (y, state_out)


def selective_scan_fwd(x, dt, A, B, C, D, init_state=None, stream=None):
    """Allocate y and final_state; returns (y, final_state)."""
    b, L, Dch = x.shape
    N = B.shape[3]
    y = torch.empty_like(x)
    final_state = torch.empty((b, Dch, N), dtype=torch.float32, device=x.device)
    ssd_selective_scan_fwd(x, dt, A, B, C, D, init_state, y, final_state, stream)
    return y, final_state


def to_device(arr, device="cuda"):
    """Move one generator array (selective_state_space_ssd_amd.inputs.Tensor or an
    ndarray) to the GPU in its storage type."""
    import numpy as np

    from .inputs import Tensor
    if arr is None:
        return None
    if isinstance(arr, Tensor):
        if arr.dtype == "bf16":
            return torch.from_numpy(arr.data.view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(arr.data).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)
