"""Seeded input generator: determinism, ranges and bf16 rounding (CPU only)."""
import hashlib

import numpy as np
import torch

from selective_state_space_ssd_amd import inputs


def _digest(t):
    return hashlib.sha256(np.ascontiguousarray(t.data).tobytes()).hexdigest()


def test_seeded_determinism_and_seed_sensitivity():
    a = inputs.make_workload("tiny_fp32")
    b = inputs.make_workload("tiny_fp32")
    c = inputs.make_workload("tiny_fp32", seed=99)
    for name in ("x", "dt", "A", "B", "C", "D"):
        assert _digest(getattr(a, name)) == _digest(getattr(b, name))
    assert _digest(a.x) != _digest(c.x)


def test_distributions_and_ranges():
    s = inputs.make_scan_inputs(b=2, L=4096, H=16, P=8, N=8, G=4, Q=64, io="bf16", init=True,
                                seed=5)
    dt = s.dt.data
    assert dt.dtype == np.float32 and dt.min() >= np.float32(1e-3) and dt.max() <= np.float32(0.1)
    assert 0.0085 < float(np.median(dt)) < 0.0115           # median softplus(bias) = 0.01
    A = s.A.data
    assert A.dtype == np.float32 and A.max() <= -1.0 and A.min() >= -16.0
    assert s.x.dtype == "bf16" and s.x.data.dtype == np.uint16
    xs = s.x.f64()
    assert abs(xs.mean()) < 0.01 and abs(xs.std() - 1.0) < 0.01
    assert abs(s.init_state.data.std() - 0.1) < 0.002


def test_bf16_rounding_matches_torch_nearest_even():
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(200_000) * 10.0 ** rng.uniform(-20, 20, 200_000)).astype(np.float32)
    # exact ties in both directions
    a[:4] = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x7F7FFFFF], np.uint32).view(np.float32)
    mine = inputs.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    back = inputs.bf16_bits_to_f32(mine)
    assert np.array_equal(back.view(np.uint32) & 0xFFFF, np.zeros_like(back.view(np.uint32)))


def test_verify_inputs_shapes():
    v = inputs.make_workload("verify_b32_K4", b=6)
    assert v.state.shape == (6, 32, 128, 128)
    assert v.x.shape == (6, 4, 32, 128) and v.B.shape == (6, 4, 8, 128)
    assert v.accept_len.dtype == np.int32
    assert v.accept_len.min() >= 0 and v.accept_len.max() <= 4
