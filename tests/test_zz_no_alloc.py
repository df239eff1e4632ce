"""ssd_chunk_scan_fwd_noalloc, the entry point that takes its workspace from the
library's own per-GPU buffer, against ssd_chunk_scan_fwd with a caller's workspace,
through the C ABI (MI355X only).  Several calls in a row share the buffer: the
benchmark layer, then smaller problems on both kernel paths."""
import numpy as np
import pytest
import torch

from gpu_helpers import TOL, scan_errors, scan_errors_all_units
from selective_state_space_ssd_amd import binding as bd
from selective_state_space_ssd_amd import inputs

pytestmark = pytest.mark.gpu


def _both(inp):
    dev = lambda a: bd.to_device(a)
    x, dt, A, B, C, D = (dev(getattr(inp, n)) for n in ("x", "dt", "A", "B", "C", "D"))
    init = dev(inp.init_state)
    d = inp.dims
    y_ref, fs_ref = bd.chunk_scan_fwd(x, dt, A, B, C, D, inp.Q, init_state=init)
    y = torch.full_like(y_ref, float("nan"))
    fs = torch.full_like(fs_ref, float("nan"))
    bd.ssd_chunk_scan_fwd_noalloc(x, dt, A, B, C, D, init, y, fs, d["Q"])
    torch.cuda.synchronize()
    return y, fs, y_ref, fs_ref


def test_noalloc_matches_workspace_entry_on_calls_in_a_row():
    cases = [
        # the benchmark layer (21 MB of workspace), compared on every unit
        ("full", inputs.make_workload("mamba2_2p7b_L2k")),
        # a smaller bf16 problem on the single-pass kernel, ragged, with an init state
        ("small", inputs.make_scan_inputs(2, 1100, 8, 64, 128, 2, 256, io="bf16", init=True,
                                          seed=41)),
        # smaller still, fp32 I/O (the three-kernel path), one chunk plus a tail
        ("fp32", inputs.make_scan_inputs(1, 70, 4, 32, 16, 2, 64, io="f32", init=True,
                                         seed=42)),
        # and the single-pass kernel again after the three-kernel path used the buffer
        ("again", inputs.make_scan_inputs(1, 600, 4, 64, 64, 1, 128, io="bf16", init=False,
                                          seed=43)),
    ]
    for name, inp in cases:
        print(f"  case {name}: dims {inp.dims}", flush=True)
        y, fs, y_ref, fs_ref = _both(inp)
        # same kernels on the same inputs: identical bits
        assert torch.equal(y, y_ref) and torch.equal(fs, fs_ref), name
        if name == "full":
            ey, ef, _ = scan_errors_all_units(inp, y, fs)
        else:
            ey, ef = scan_errors(inp, y, fs)
        print(f"    y err {ey:.3e}  final_state err {ef:.3e}", flush=True)
        assert np.isfinite(ey) and np.isfinite(ef)
        assert ey <= TOL[inp.io] and ef <= TOL[inp.io], name


def test_noalloc_refuses_a_problem_beyond_its_buffer():
    # fp32 I/O at Q = 64 on the benchmark layer needs 671 MB of chunk states
    b, L, H, P, N, G, Q = 4, 2048, 80, 64, 128, 1, 64
    assert bd.ssd_chunk_scan_workspace_bytes(b, L, H, P, N, G, Q, bd.SSD_DTYPE_F32) > \
        bd.NOALLOC_WORKSPACE_BYTES
    x = torch.zeros((b, L, H, P), device="cuda")
    dt = torch.zeros((b, L, H), device="cuda")
    A = torch.zeros(H, device="cuda")
    B = torch.zeros((b, L, G, N), device="cuda")
    y = torch.empty_like(x)
    with pytest.raises(bd.SSDError) as e:
        bd.ssd_chunk_scan_fwd_noalloc(x, dt, A, B, B, A, None, y, None, Q)
    assert e.value.status == 6   # SSD_ERR_WORKSPACE
