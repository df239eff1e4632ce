"""Shared helpers of the GPU parity tests: run the HIP library through the binding,
run the oracle on the same seeded inputs, and compare."""
import concurrent.futures
import os

import numpy as np
import torch

import oracle
from selective_state_space_ssd_amd import binding as bd

# Tolerances on the slice-normalised max error (per (batch, head) slice:
# max |gpu - oracle| / max |oracle|): fp32 I/O path and bf16 I/O path.
TOL = {"f32": 1e-4, "bf16": 2e-2}
# States produced by the verify step are fp32 arithmetic on exactly represented
# inputs in both I/O modes.
TOL_VERIFY_STATE = 1e-4


def slice_err(gpu, ref, axes):
    """max over slices of max|gpu-ref| / max|ref|, slices indexed by all axes not in `axes`."""
    num = np.max(np.abs(gpu - ref), axis=axes)
    den = np.maximum(np.max(np.abs(ref), axis=axes), 1e-30)
    return float(np.max(num / den))


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def workspace_error(ws) -> int:
    """The workspace's hand-off time-out word, read through the C ABI (0 = healthy)."""
    err = torch.full((1,), -1, dtype=torch.int32, device=ws.device)
    bd.ssd_chunk_scan_workspace_error(ws, err)
    torch.cuda.synchronize()
    return int(err.item())


def run_scan(inp, device="cuda", workspace=None, check_error_word=True):
    dev = lambda a: bd.to_device(a, device)
    x, dt, A, B, C, D = (dev(getattr(inp, n)) for n in ("x", "dt", "A", "B", "C", "D"))
    init = dev(inp.init_state)
    if workspace is None:
        workspace = bd.chunk_scan_workspace(x, B, inp.Q)
    y, fs = bd.chunk_scan_fwd(x, dt, A, B, C, D, inp.Q, init_state=init, workspace=workspace)
    torch.cuda.synchronize()
    if check_error_word and workspace.numel() >= 256:
        # no chunk of a healthy call gives up waiting for its predecessor's state
        assert workspace_error(workspace) == 0
    return y, fs


def oracle_scan(inp, bh_range=None):
    init = None if inp.init_state is None else inp.init_state.f64()
    return oracle.scan_f64(inp.x.f64(), inp.dt.f64(), inp.A.f64(), inp.B.f64(), inp.C.f64(),
                           inp.D.f64(), init, bh_range=bh_range)


def scan_errors(inp, y, fs, units=None):
    """Slice errors of y and final_state against the oracle, optionally on a sample of
    flattened (batch*H + head) units only."""
    d = inp.dims
    H = d["H"]
    yg, fg = to_f64(y), to_f64(fs)
    if units is None:
        yo, fo = oracle_scan(inp)
        return slice_err(yg, yo, (1, 3)), slice_err(fg, fo, (2, 3))
    ey = ef = 0.0
    for u in units:
        yo, fo = oracle_scan(inp, bh_range=(u, u + 1))
        bi, h = divmod(u, H)
        ey = max(ey, slice_err(yg[bi, :, h], yo[bi, :, h], (0, 1)))
        ef = max(ef, slice_err(fg[bi, h], fo[bi, h], (0, 1)))
    return ey, ef


def oracle_threads() -> int:
    """Host threads for the oracle: the cores this process may use, at most 16 (a
    GPU machine's share of its host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def scan_errors_all_units(inp, y, fs, threads=None):
    """Slice errors of y and final_state against the oracle over EVERY (batch, head)
    unit.  Each unit runs through the oracle on its own slice of the inputs (one batch
    row, one head, its group's B and C), on a thread pool; returns (err_y, err_final,
    units compared)."""
    d = inp.dims
    b, H, G = d["b"], d["H"], d["G"]
    hpg = H // G
    x, dt, A, B, C, D = (getattr(inp, n).f64() for n in ("x", "dt", "A", "B", "C", "D"))
    init = None if inp.init_state is None else inp.init_state.f64()
    yg, fg = to_f64(y), to_f64(fs)

    def one(u):
        bi, h = divmod(u, H)
        g = h // hpg
        sl = lambda a: np.ascontiguousarray(a)
        yo, fo = oracle.scan_f64(sl(x[bi:bi + 1, :, h:h + 1]), sl(dt[bi:bi + 1, :, h:h + 1]),
                                 A[h:h + 1], sl(B[bi:bi + 1, :, g:g + 1]),
                                 sl(C[bi:bi + 1, :, g:g + 1]), D[h:h + 1],
                                 None if init is None else sl(init[bi:bi + 1, h:h + 1]))
        return (slice_err(yg[bi, :, h], yo[0, :, 0], (0, 1)),
                slice_err(fg[bi, h], fo[0, 0], (0, 1)))

    with concurrent.futures.ThreadPoolExecutor(max_workers=threads or oracle_threads()) as ex:
        errs = list(ex.map(one, range(b * H)))
    return max(e[0] for e in errs), max(e[1] for e in errs), len(errs)


def backward_row_oracle(args):
    """Gradient oracle for one batch row of a named workload (every head, in blocks of
    8 heads), for a process pool: the inputs are regenerated from the workload's seed
    here rather than sent over.  Returns the row's dx, ddt, d_init, dB, dC and its
    contributions to dA, dD."""
    name, grad_seed, row, threads = args
    from oracle import backward
    from selective_state_space_ssd_amd import inputs

    torch.set_num_threads(threads)
    inp = inputs.make_workload(name)
    dy, d_final = inputs.make_upstream_grads(inp, seed=grad_seed)
    f = lambda t: None if t is None else t.f64()
    x, dt, A, B, C, D = (f(getattr(inp, n)) for n in ("x", "dt", "A", "B", "C", "D"))
    h0, dfin, dyf = f(inp.init_state), f(d_final), dy.f64()
    H = inp.dims["H"]
    r = slice(row, row + 1)
    out = None
    for h0_ in range(0, H, 8):
        hs = slice(h0_, h0_ + 8)
        part = backward.scan_bwd_f64(
            x[r][:, :, hs], dt[r][:, :, hs], A[hs], B[r], C[r], D[hs],
            None if h0 is None else h0[r][:, hs], dyf[r][:, :, hs],
            None if dfin is None else dfin[r][:, hs])
        if out is None:
            out = {"dx": np.zeros(x[r].shape), "ddt": np.zeros(dt[r].shape),
                   "d_init": np.zeros((1, H) + part[6].shape[2:]), "dB": np.zeros_like(part[3]),
                   "dC": np.zeros_like(part[4]), "dA": np.zeros(H), "dD": np.zeros(H)}
        out["dx"][:, :, hs] = part[0]
        out["ddt"][:, :, hs] = part[1]
        out["dA"][hs] = part[2]
        out["dB"] += part[3]
        out["dC"] += part[4]
        out["dD"][hs] = part[5]
        out["d_init"][:, hs] = part[6]
    return out
