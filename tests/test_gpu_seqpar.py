"""GPU parity of the sequence-parallel pieces (ssd_seq_slice_state, ssd_seq_total_decay,
ssd_seq_combine, ssd_seq_apply_state) against the fp64 oracles (MI355X only).

Both orders of work are run over the slices of one sequence.  Outputs first: every
slice is scanned from zero by ssd_chunk_scan_fwd, the pairs (total decay, final
state) are combined into entering states, and every slice is corrected.  States
first: ssd_seq_slice_state gives every slice's pair, the pairs are combined, and every
slice is scanned from its entering state.  Either way the result must equal the scan
oracle of the whole sequence.  On one GPU the slices stand in for the devices of the
sequence-parallel layout; the exchange between devices is not part of the library."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL, oracle_scan, scan_errors_all_units, slice_err, to_f64
from oracle import cp
from selective_state_space_ssd_amd import binding as bd
from selective_state_space_ssd_amd import inputs

pytestmark = pytest.mark.gpu


def _pipeline_states_first(inp, cuts):
    """Slice states, combine, then a scan of every slice from its entering state;
    returns (y, final_state)."""
    d = inp.dims
    dev = bd.to_device
    x, dt, A, B, C, D = (dev(getattr(inp, n)) for n in ("x", "dt", "A", "B", "C", "D"))
    init = dev(inp.init_state)
    n = len(cuts) - 1
    b, H, P, N = d["b"], d["H"], d["P"], d["N"]
    S = torch.empty((n, b, H, P, N), dtype=torch.float32, device="cuda")
    alpha = torch.empty((n, b, H), dtype=torch.float32, device="cuda")
    parts = []
    for j in range(n):
        sl = slice(cuts[j], cuts[j + 1])
        xs, dts, Bs, Cs = (t[:, sl].contiguous() for t in (x, dt, B, C))
        S[j], alpha[j] = bd.seq_slice_state(xs, dts, A, Bs)
        parts.append((xs, dts, Bs, Cs))
    h_in = torch.empty_like(S)
    bd.ssd_seq_combine(alpha, S, init, h_in)
    ys, final = [], None
    for j, (xs, dts, Bs, Cs) in enumerate(parts):
        y_j, final = bd.chunk_scan_fwd(xs, dts, A, Bs, Cs, D, d["Q"], init_state=h_in[j])
        ys.append(y_j)
    torch.cuda.synchronize()
    return torch.cat(ys, dim=1), final


def _pipeline(inp, cuts, flow="outputs_first"):
    """Run the pieces over the slices [cuts[j], cuts[j+1]); returns (y, final_state)."""
    if flow == "states_first":
        return _pipeline_states_first(inp, cuts)
    d = inp.dims
    dev = bd.to_device
    x, dt, A, B, C, D = (dev(getattr(inp, n)) for n in ("x", "dt", "A", "B", "C", "D"))
    init = dev(inp.init_state)
    n = len(cuts) - 1
    b, H, P, N = d["b"], d["H"], d["P"], d["N"]
    ys, S = [], torch.empty((n, b, H, P, N), dtype=torch.float32, device="cuda")
    alpha = torch.empty((n, b, H), dtype=torch.float32, device="cuda")
    for j in range(n):
        sl = slice(cuts[j], cuts[j + 1])
        xs, dts, Bs, Cs = (t[:, sl].contiguous() for t in (x, dt, B, C))
        y_j, f_j = bd.chunk_scan_fwd(xs, dts, A, Bs, Cs, D, d["Q"])      # from a zero state
        S[j] = f_j
        bd.ssd_seq_total_decay(dts, A, alpha[j])
        ys.append((y_j, dts, Cs))
    h_in = torch.empty_like(S)
    bd.ssd_seq_combine(alpha, S, init, h_in)
    final = None
    for j, (y_j, dts, Cs) in enumerate(ys):
        f_j = S[j].clone()
        bd.ssd_seq_apply_state(y_j, f_j, dts, A, Cs, h_in[j])
        final = f_j
    torch.cuda.synchronize()
    return torch.cat([t[0] for t in ys], dim=1), final


SMALL = [
    # b,  L,  H,  P,   N, G,  io,   init, cuts
    (2, 700, 4, 64, 64, 2, "bf16", True, [0, 250, 450, 700]),
    (1, 513, 2, 32, 128, 1, "f32", True, [0, 1, 300, 513]),     # a one-token slice
    (2, 384, 4, 16, 32, 4, "f32", False, [0, 128, 256, 384]),
    (1, 300, 2, 64, 48, 2, "bf16", True, [0, 300, 300]),         # an empty last slice
    (1, 400, 2, 128, 32, 1, "bf16", True, [0, 150, 400]),        # P > 64: two channel passes
    (1, 600, 2, 64, 256, 2, "bf16", True, [0, 333, 600]),        # N = 256: state staged twice
    (2, 300, 2, 16, 80, 1, "bf16", False, [0, 17, 300]),         # one channel tile, padded N,
                                                                 # a slice of one token tile
]


FLOWS = ["outputs_first", "states_first"]


@pytest.mark.parametrize("flow", FLOWS)
@pytest.mark.parametrize("case", SMALL, ids=lambda c: "b{}L{}H{}P{}N{}G{}{}{}n{}".format(
    *c[:7], "init" if c[7] else "", len(c[8]) - 1))
def test_slices_reproduce_whole_sequence(case, flow):
    b, L, H, P, N, G, io, init, cuts = case
    inp = inputs.make_scan_inputs(b, L, H, P, N, G, 64, io=io, init=init, seed=L + P)
    y, fs = _pipeline(inp, cuts, flow)
    yo, fo = oracle_scan(inp)
    ey, ef = slice_err(to_f64(y), yo, (1, 3)), slice_err(to_f64(fs), fo, (2, 3))
    print(f"  y err {ey:.2e}  final err {ef:.2e}", flush=True)
    assert ey <= TOL[io] and ef <= TOL[io]


def test_pieces_against_their_oracles():
    inp = inputs.make_scan_inputs(2, 200, 4, 32, 64, 2, 64, io="f32", init=True, seed=21)
    dev = bd.to_device
    dt, A, C = dev(inp.dt), dev(inp.A), dev(inp.C)
    alpha = torch.empty((2, 4), dtype=torch.float32, device="cuda")
    bd.ssd_seq_total_decay(dt, A, alpha)
    rng = np.random.default_rng(22)
    S = rng.standard_normal((3, 2, 4, 32, 64)).astype(np.float32)
    al = rng.uniform(0.2, 1.0, (3, 2, 4)).astype(np.float32)
    h0 = inp.init_state.data
    h_in = torch.empty((3, 2, 4, 32, 64), dtype=torch.float32, device="cuda")
    bd.ssd_seq_combine(dev(al), dev(S), dev(h0), h_in)
    y0 = rng.standard_normal((2, 200, 4, 32)).astype(np.float32)
    f0 = rng.standard_normal((2, 4, 32, 64)).astype(np.float32)
    y, f = dev(y0), dev(f0)
    bd.ssd_seq_apply_state(y, f, dt, A, C, dev(h0))
    torch.cuda.synchronize()
    a_o = cp.total_decay_f64(inp.dt.f64(), inp.A.f64())
    h_o = cp.combine_f64(al, S, h0)
    y_o, f_o = cp.apply_entering_state_f64(y0, f0, inp.dt.f64(), inp.A.f64(), inp.C.f64(), h0)
    assert slice_err(to_f64(alpha), a_o, (1,)) <= 1e-5
    assert slice_err(to_f64(h_in), h_o, (3, 4)) <= 1e-5
    assert slice_err(to_f64(y), y_o, (1, 3)) <= TOL["f32"]
    assert slice_err(to_f64(f), f_o, (2, 3)) <= TOL["f32"]


# The slice state on its own.  bf16 with P = 64 and N in {64, 128, 256} takes the
# dedicated kernel (runs of 128-token segments; about 512 workgroups, so many heads
# make runs of several segments); the other shapes take the chunk-state kernel (fp32
# at P = 128, N = 256 with the shortest chunk).  Ragged last segments, several groups.
SLICE = [
    # b,  L,   H,  P,   N,  G,  io
    (2, 600, 4, 64, 128, 2, "bf16"),     # 5 runs of one segment per head
    (4, 1000, 64, 64, 128, 4, "bf16"),   # 2 runs of 4 segments
    (2, 700, 64, 64, 64, 4, "bf16"),     # N = 64: 3 runs of 2 segments
    (1, 600, 256, 64, 256, 2, "bf16"),   # N = 256: runs of 3 and 2 segments
    (1, 300, 2, 16, 16, 1, "f32"),
    (2, 129, 4, 32, 48, 2, "f32"),
    (1, 520, 2, 128, 256, 1, "bf16"),
    (1, 200, 2, 128, 256, 2, "f32"),
    (1, 1, 2, 64, 64, 1, "bf16"),       # one token
    (1, 0, 2, 64, 64, 1, "bf16"),       # empty slice: zero state, decay 1
]


@pytest.mark.parametrize("b,L,H,P,N,G,io", SLICE)
def test_slice_state_against_oracle(b, L, H, P, N, G, io):
    inp = inputs.make_scan_inputs(b, L, H, P, N, G, 64, io=io, init=False, seed=7 * L + N)
    dev = bd.to_device
    state, alpha = bd.seq_slice_state(dev(inp.x), dev(inp.dt), dev(inp.A), dev(inp.B))
    torch.cuda.synchronize()
    f = lambda a: a.f64()
    _, fo = oracle.scan_f64(f(inp.x), f(inp.dt), f(inp.A), f(inp.B), f(inp.C), f(inp.D), None)
    ao = cp.total_decay_f64(f(inp.dt), f(inp.A))
    es = slice_err(to_f64(state), fo, (2, 3)) if L > 0 else float(np.abs(to_f64(state)).max())
    ea = float(np.abs(to_f64(alpha) - ao).max() / max(np.abs(ao).max(), 1e-30))
    print(f"  state err {es:.2e}  alpha err {ea:.2e}", flush=True)
    assert es <= TOL[io] and ea <= 1e-5


@pytest.mark.parametrize("flow", FLOWS)
def test_long_context_layer_in_eight_slices_every_head(flow):
    """The L=16384 layer (b=1, H=80, P=64, N=128, bf16, initial state) as 8 slices of
    2048 tokens, one GPU's share each; every head compared with the oracle of the
    whole sequence."""
    inp = inputs.make_workload("mamba2_2p7b_L16k")
    y, fs = _pipeline(inp, list(range(0, 16385, 2048)), flow)
    ey, ef, n = scan_errors_all_units(inp, y, fs)
    print(f"  {n} units: y err {ey:.2e}  final err {ef:.2e}", flush=True)
    assert n == inp.dims["b"] * inp.dims["H"]
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"]
