"""GPU parity of ssd_selective_scan_fwd (one channel per head, diagonal A) against the
fp64 oracle (MI355X only)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL, slice_err, to_f64
from selective_state_space_ssd_amd import binding as bd
from selective_state_space_ssd_amd import inputs

pytestmark = pytest.mark.gpu


def _run(inp):
    dev = lambda a: bd.to_device(a)
    x, dt, A, B, C, D = (dev(getattr(inp, n)) for n in ("x", "dt", "A", "B", "C", "D"))
    y, fs = bd.selective_scan_fwd(x, dt, A, B, C, D, init_state=dev(inp.init_state))
    torch.cuda.synchronize()
    return to_f64(y), to_f64(fs)


def _oracle(inp, channels=None):
    """Oracle outputs, optionally for a sample of channels only (channels are
    independent; with one group every channel reads the same B and C)."""
    x, dt, A, B, C, D = (getattr(inp, n).f64() for n in ("x", "dt", "A", "B", "C", "D"))
    h0 = None if inp.init_state is None else inp.init_state.f64()
    if channels is not None:
        x, dt, A, D = x[:, :, channels], dt[:, :, channels], A[channels], D[channels]
        h0 = None if h0 is None else h0[:, channels]
    return oracle.selective_scan_f64(x, dt, A, B, C, D, h0)


def _check(inp, tol=None):
    yg, fg = _run(inp)
    yo, fo = _oracle(inp)
    ey, ef = slice_err(yg, yo, (1,)), slice_err(fg, fo, (2,))   # per (batch, channel)
    tol = tol or TOL[inp.io]
    print(f"  y err {ey:.3e}  final_state err {ef:.3e}  (tol {tol})", flush=True)
    assert np.isfinite(ey) and np.isfinite(ef)
    assert ey <= tol and ef <= tol


# Several time tiles with a ragged last one, initial states, every supported N, two
# groups, both dtypes.  The channels of a group are a multiple of one workgroup's (32).
SMALL = [
    # b,  L,  Dch,  N, G,  io,    init
    (2, 100, 64, 16, 1, "f32", True),
    (2, 130, 128, 16, 2, "bf16", False),
    (1, 77, 32, 32, 1, "bf16", True),
    (1, 45, 128, 32, 2, "f32", False),
    (2, 65, 64, 64, 2, "f32", True),
    (2, 150, 64, 128, 2, "bf16", True),
    (1, 33, 32, 128, 1, "f32", True),
    (1, 70, 64, 256, 2, "bf16", False),
    (1, 40, 32, 256, 1, "f32", True),
    (1, 1, 64, 16, 1, "bf16", True),                   # one token
]


@pytest.mark.parametrize("b,L,Dch,N,G,io,init", SMALL)
def test_selective_small(b, L, Dch, N, G, io, init):
    _check(inputs.make_selective_inputs(b, L, Dch, N, G, io=io, init=init, seed=L + N))


def test_selective_empty_sequence_copies_init():
    inp = inputs.make_selective_inputs(2, 0, 64, 16, 1, io="f32", init=True, seed=3)
    dev = lambda a: bd.to_device(a)
    x, dt, A, B, C, D, h0 = (dev(getattr(inp, n)) for n in ("x", "dt", "A", "B", "C", "D",
                                                             "init_state"))
    _, fs = bd.selective_scan_fwd(x, dt, A, B, C, D, init_state=h0)
    torch.cuda.synchronize()
    assert torch.equal(fs, h0)


def test_selective_unsupported_channel_count_is_rejected():
    inp = inputs.make_selective_inputs(1, 8, 48, 16, 1, io="f32", seed=4)   # 48 % 32 != 0
    dev = lambda a: bd.to_device(a)
    x, dt, A, B, C, D = (dev(getattr(inp, n)) for n in ("x", "dt", "A", "B", "C", "D"))
    with pytest.raises(bd.SSDError) as e:
        bd.selective_scan_fwd(x, dt, A, B, C, D)
    assert e.value.status == 4   # SSD_ERR_UNSUPPORTED


@pytest.mark.parametrize("name", ["mamba1_L2k_N16", "mamba1_L2k_N128"])
def test_selective_benchmark_shapes_sampled(name):
    """The benchmark layers (b=4, L=2048, 5120 channels), checked on four channels of
    every workgroup the launch uses (at different lanes and waves of it), in every
    batch row."""
    inp = inputs.make_workload(name)
    yg, fg = _run(inp)
    Dch = inp.dims["Dch"]
    dc = 32   # channels per workgroup
    ch = np.unique(np.concatenate([w * dc + (np.r_[0, 9, 18, 27] + 5 * w) % dc
                                   for w in range(Dch // dc)]))
    yo, fo = _oracle(inp, ch)
    ey = slice_err(yg[:, :, ch], yo, (1,))
    ef = slice_err(fg[:, ch], fo, (2,))
    print(f"  {name}: y err {ey:.3e}  final_state err {ef:.3e}", flush=True)
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"]
