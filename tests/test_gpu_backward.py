"""GPU parity of ssd_chunk_scan_bwd (gradients of the chunked scan) against the fp64
gradient oracle (MI355X only)."""
import numpy as np
import pytest
import torch

from gpu_helpers import TOL, slice_err, to_f64
from oracle import backward
from selective_state_space_ssd_amd import binding as bd
from selective_state_space_ssd_amd import inputs

pytestmark = pytest.mark.gpu

NAMES = ("dx", "ddt", "dA", "dB", "dC", "dD", "d_init")


def _run(inp, dy, d_final):
    dev = lambda a: bd.to_device(a)
    x, dt, A, B, C, D = (dev(getattr(inp, n)) for n in ("x", "dt", "A", "B", "C", "D"))
    grads = bd.chunk_scan_bwd(x, dt, A, B, C, D, dev(dy), init_state=dev(inp.init_state),
                              d_final=dev(d_final))
    torch.cuda.synchronize()
    return [to_f64(g) for g in grads]


def _oracle(inp, dy, d_final, rows=slice(None), heads=slice(None)):
    """Oracle gradients for a block of batch rows and heads (one group only when heads
    is not the full range)."""
    f = lambda t: None if t is None else t.f64()
    x, dt, A, B, C, D = (f(getattr(inp, n)) for n in ("x", "dt", "A", "B", "C", "D"))
    h0 = f(inp.init_state)
    dfin = f(d_final)
    return backward.scan_bwd_f64(
        x[rows][:, :, heads], dt[rows][:, :, heads], A[heads], B[rows], C[rows], D[heads],
        None if h0 is None else h0[rows][:, heads], dy.f64()[rows][:, :, heads],
        None if dfin is None else dfin[rows][:, heads])


# slice axes of every gradient: per (batch, head) for dx, ddt, d_init; per (batch,
# group) for dB, dC; the whole vector for dA, dD
AXES = {"dx": (1, 3), "ddt": (1,), "dA": (0,), "dB": (1, 3), "dC": (1, 3), "dD": (0,),
        "d_init": (2, 3)}


def _errors(got, ref, names=NAMES):
    return {n: slice_err(got[NAMES.index(n)], ref[NAMES.index(n)], AXES[n]) for n in names}


def _assert(errs, tol):
    print("  " + "  ".join(f"{n} {e:.2e}" for n, e in errs.items()) + f"  (tol {tol})", flush=True)
    for n, e in errs.items():
        assert np.isfinite(e) and e <= tol, f"{n}: {e:.3e} > {tol}"


# Several 64-token chunks with ragged last ones, initial states, final-state gradients
# or none, P in {32, 64}, N from 16 to 128, groups of 1, 2, 3, 4 and 12 heads, both
# dtypes; bf16 with P = 64 and N in {64, 128} takes the bf16 matrix-core path (blocks
# of heads of a group per workgroup, sized by the launch's round model: one head at
# the shortest shapes, 2 and 8 at the two longer ones below; forward state walks over
# two heads of a group when the group has an even number of heads, one otherwise),
# the rest the fp32 path.
SMALL = [
    # b,  L,  H,  P,   N, G,  io,    init, final
    (2, 300, 4, 64, 128, 2, "bf16", True, True),
    (1, 200, 4, 32, 16, 1, "bf16", False, False),
    (2, 130, 2, 32, 64, 1, "f32", True, True),
    (1, 64, 2, 64, 32, 2, "f32", False, True),        # exactly one chunk
    (1, 63, 4, 64, 48, 4, "f32", True, False),        # one group per head, short
    (1, 1, 2, 32, 16, 1, "f32", True, True),          # one token
    (2, 517, 4, 64, 128, 1, "f32", True, True),
    (1, 190, 12, 64, 64, 1, "bf16", True, True),      # twelve heads in one group
    (2, 129, 2, 64, 128, 2, "bf16", False, False),    # one head per group
    (1, 200, 3, 64, 64, 1, "bf16", True, True),       # odd group: one head per forward walk
    (2, 150, 6, 64, 128, 2, "bf16", True, False),     # odd groups of 3, two groups
    (2, 1100, 12, 64, 128, 1, "bf16", True, False),   # blocks of 2 heads
    (4, 630, 48, 64, 64, 2, "bf16", True, True),      # blocks of 8 heads, two groups
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "b{}L{}H{}P{}N{}G{}{}{}{}".format(
    *c[:7], "init" if c[7] else "", "dfin" if c[8] else ""))
def test_backward_small_full_oracle(case):
    b, L, H, P, N, G, io, init, final = case
    inp = inputs.make_scan_inputs(b, L, H, P, N, G, 64, io=io, init=init, seed=L + N + P)
    dy, d_final = inputs.make_upstream_grads(inp, seed=1000 + L, final=final)
    got = _run(inp, dy, d_final)
    _assert(_errors(got, _oracle(inp, dy, d_final)), TOL[io])


def test_backward_is_deterministic():
    inp = inputs.make_scan_inputs(2, 300, 8, 64, 64, 2, 64, io="bf16", init=True, seed=5)
    dy, d_final = inputs.make_upstream_grads(inp, seed=6)
    a, b = _run(inp, dy, d_final), _run(inp, dy, d_final)
    for n, u, v in zip(NAMES, a, b):
        assert np.array_equal(u, v), n


def test_backward_empty_sequence():
    inp = inputs.make_scan_inputs(2, 0, 4, 64, 32, 1, 64, io="f32", init=True, seed=8)
    dy, d_final = inputs.make_upstream_grads(inp, seed=9)
    dx, ddt, dA, dB, dC, dD, d_init = _run(inp, dy, d_final)
    assert dx.size == 0 and ddt.size == 0 and dB.size == 0 and dC.size == 0
    assert not np.any(dA) and not np.any(dD)
    assert np.array_equal(d_init, d_final.f64())


def test_backward_unsupported_head_dim_is_rejected():
    inp = inputs.make_scan_inputs(1, 64, 2, 16, 16, 1, 64, io="f32", seed=10)
    dy, _ = inputs.make_upstream_grads(inp, seed=11, final=False)
    with pytest.raises(bd.SSDError) as e:
        _run(inp, dy, None)
    assert e.value.status == 4   # SSD_ERR_UNSUPPORTED


@pytest.fixture(scope="module")
def full_size():
    """The Mamba-2-2.7B-shaped layer at L = 2048 (b=4, H=80, P=64, N=128, bf16) with
    upstream gradients for y and the final state, run once on the GPU."""
    inp = inputs.make_workload("mamba2_2p7b_L2k")
    dy, d_final = inputs.make_upstream_grads(inp, seed=77)
    return inp, dy, d_final, _run(inp, dy, d_final)


@pytest.mark.timeout(480)   # the fp64 gradient oracle over 4 x 2048 tokens x 80 heads
def test_backward_full_size_every_unit(full_size):
    """Every (batch row, head) of the full-size layer: dx, ddt, d_init per head; dB, dC
    per batch row (the sum over all 80 heads); dA and dD per head (sums over all rows
    and tokens).  The oracle runs one batch row per process (fresh interpreters that
    never touch the GPU), each regenerating the seeded inputs."""
    import multiprocessing as mp

    from gpu_helpers import backward_row_oracle, oracle_threads

    inp, dy, d_final, got = full_size
    b = inp.dims["b"]
    threads = max(1, oracle_threads() // b)
    with mp.get_context("spawn").Pool(b) as pool:
        rows = pool.map(backward_row_oracle,
                        [("mamba2_2p7b_L2k", 77, r, threads) for r in range(b)])
    ref = [np.concatenate([row["dx"] for row in rows]),
           np.concatenate([row["ddt"] for row in rows]),
           sum(row["dA"] for row in rows),
           np.concatenate([row["dB"] for row in rows]),
           np.concatenate([row["dC"] for row in rows]),
           sum(row["dD"] for row in rows),
           np.concatenate([row["d_init"] for row in rows])]
    _assert(_errors(got, ref), TOL["bf16"])
