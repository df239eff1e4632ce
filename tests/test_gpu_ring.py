"""GPU parity of the multi-round verify on a state ring (ssd_verify_ring_init,
ssd_verify_ring, ssd_verify_ring_rollback) against the fp64 ring oracle (MI355X only).

Every round compares y with the oracle; after every round and rollback the ring
bookkeeping (head, depth) must match exactly and every state a rollback can still
reach (the head slot and the depth slots behind it) must match the oracle's."""
import numpy as np
import pytest
import torch

from gpu_helpers import TOL, TOL_VERIFY_STATE, slice_err, to_f64
from oracle import ring as oring
from selective_state_space_ssd_amd import binding as bd
from selective_state_space_ssd_amd import inputs

pytestmark = pytest.mark.gpu


def _run(b, K, H, P, N, G, R, rounds, io, biased, seed):
    inp = inputs.make_verify_ring_inputs(b, K, H, P, N, G, R, rounds, io=io, biased=biased,
                                         seed=seed)
    dev = bd.to_device
    A, D, h0 = dev(inp.A), dev(inp.D), dev(inp.init_state)
    bias = dev(inp.dt_bias)
    ring = torch.empty((b, R, H, P, N), dtype=torch.float32, device="cuda")
    meta = torch.empty((b, 2), dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    bd.ssd_verify_ring_init(ring, meta, h0)
    rg, mt = oring.ring_init_f64(inp.init_state.f64(), R)
    worst_y = worst_s = 0.0
    flag_expected = False
    for r in inp.rounds:
        x, dt, B, C = dev(r["x"]), dev(r["dt"]), dev(r["B"]), dev(r["C"])
        acc = dev(r["accept_len"])
        y = torch.empty_like(x)
        bd.ssd_verify_ring(ring, meta, x, dt, A, B, C, D, acc, y, dt_bias=bias, err_flag=err)
        yo, rg, mt = oring.verify_ring_f64(
            rg, mt, r["x"].f64(), r["dt"].f64(), inp.A.f64(), r["B"].f64(), r["C"].f64(),
            inp.D.f64(), r["accept_len"], dt_bias=None if bias is None else inp.dt_bias.f64())
        if r["rollback"] is not None:
            bd.ssd_verify_ring_rollback(meta, dev(r["rollback"]), err_flag=err, R=R)
            mt, flag = oring.ring_rollback(mt, r["rollback"], R, clamp=True)
            flag_expected |= flag
        torch.cuda.synchronize()
        worst_y = max(worst_y, slice_err(to_f64(y), yo, (1, 3)))
        mg = meta.cpu().numpy()
        assert np.array_equal(mg, mt), f"ring bookkeeping differs: {mg.tolist()} vs {mt.tolist()}"
        rgg = ring.cpu().numpy().astype(np.float64)
        for bi in range(b):
            head, depth = int(mt[bi, 0]), int(mt[bi, 1])
            for j in range(depth + 1):
                sl = (head - j) % R
                worst_s = max(worst_s, slice_err(rgg[bi, sl], rg[bi, sl], (1, 2)))
    print(f"  y err {worst_y:.2e}  state err {worst_s:.2e}  flag {int(err.item())}", flush=True)
    assert worst_y <= TOL[io] and worst_s <= TOL_VERIFY_STATE
    assert bool(err.item()) == flag_expected
    return inp


CASES = [
    # b, K, H,   P,   N, G, R, rounds, io,    biased
    (3, 4, 4, 64, 128, 2, 6, 9, "bf16", False),
    (3, 4, 4, 64, 128, 2, 6, 9, "bf16", True),
    (2, 1, 2, 16, 16, 1, 2, 12, "f32", False),     # decode: one token a round, smallest ring
    (2, 3, 4, 32, 64, 4, 4, 14, "f32", True),      # wraps the ring several times
    (1, 16, 2, 128, 256, 1, 20, 4, "bf16", True),  # longest draft, largest state
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}K{}H{}P{}N{}G{}R{}x{}{}{}".format(
    *c[:9], "bias" if c[9] else ""))
def test_ring_rounds_match_oracle(case):
    _run(*case, seed=sum(case[:8]))


def test_ring_equals_verify_step_on_one_round():
    """One round on a fresh ring gives the y and accepted state of ssd_verify_step."""
    b, K, H, P, N, G, R = 4, 4, 4, 64, 64, 2, 5
    inp = inputs.make_verify_ring_inputs(b, K, H, P, N, G, R, 1, io="bf16", seed=9)
    r = inp.rounds[0]
    dev = bd.to_device
    A, D, h0 = dev(inp.A), dev(inp.D), dev(inp.init_state)
    x, dt, B, C, acc = dev(r["x"]), dev(r["dt"]), dev(r["B"]), dev(r["C"]), dev(r["accept_len"])
    ring = torch.empty((b, R, H, P, N), dtype=torch.float32, device="cuda")
    meta = torch.empty((b, 2), dtype=torch.int32, device="cuda")
    bd.ssd_verify_ring_init(ring, meta, h0)
    y1 = torch.empty_like(x)
    bd.ssd_verify_ring(ring, meta, x, dt, A, B, C, D, acc, y1)
    y2, so = bd.verify_step(h0, x, dt, A, B, C, D, acc)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    heads = meta[:, 0].long()
    assert torch.equal(ring[torch.arange(b, device="cuda"), heads], so)


def test_ring_head_out_of_range_is_reduced_and_flagged():
    """A head outside [0, R) in meta (e.g. a ring never initialised) is reduced modulo R
    inside the kernel, so every access stays inside the ring, and is reported."""
    b, K, H, P, N, G, R = 2, 2, 2, 32, 32, 1, 4
    inp = inputs.make_verify_ring_inputs(b, K, H, P, N, G, R, 1, io="f32", seed=11)
    r = inp.rounds[0]
    dev = bd.to_device
    A, D, h0 = dev(inp.A), dev(inp.D), dev(inp.init_state)
    ring = torch.zeros((b, R, H, P, N), dtype=torch.float32, device="cuda")
    meta = torch.empty((b, 2), dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    bd.ssd_verify_ring_init(ring, meta, h0)
    meta[:, 0] = torch.tensor([R + 1, -3], dtype=torch.int32)      # reduce to 1 and 1
    y = torch.empty_like(dev(r["x"]))
    bd.ssd_verify_ring(ring, meta, dev(r["x"]), dev(r["dt"]), A, dev(r["B"]), dev(r["C"]), D,
                       dev(r["accept_len"]), y, err_flag=err)
    torch.cuda.synchronize()
    rg, mt = oring.ring_init_f64(inp.init_state.f64(), R)
    mt[:, 0] = 1                                                   # slot 1 holds zeros
    yo, rg, mt = oring.verify_ring_f64(rg, mt, r["x"].f64(), r["dt"].f64(), inp.A.f64(),
                                       r["B"].f64(), r["C"].f64(), inp.D.f64(), r["accept_len"])
    assert int(err.item()) == 1
    assert np.array_equal(meta.cpu().numpy(), mt)
    assert slice_err(to_f64(y), yo, (1, 3)) <= TOL["f32"]
