"""Seeded synthetic inputs for the SSD chunked scan and the verify step.

This module only draws random numbers and rounds them to the storage types; it
holds none of the method's arithmetic.  Both sides of every parity check (the
fp64 CPU oracle and the HIP library) receive the exact arrays produced here.

Recipe (the same for tests and for the benchmark):

* Generator: ``numpy.random.default_rng(seed)`` (PCG64), values drawn in float64.
* Draw order, chunked scan: A, D, z (for dt), x, B, C, init_state.
  Draw order, verify step: A, D, state, z, x, B, C, accept_len.
  Draw order, selective scan (one channel per head): A, D, z, x, B, C, init_state;
  there A is drawn per (channel, state) and dt per (token, channel), with the same
  distributions as below.
* A_h = -exp(U(0, ln 16))            scalar per head, in [-16, -1]
* D_h ~ N(0, 1)
* dt = clip(softplus(z + DT_BIAS), 1e-3, 1e-1) with z ~ N(0, 1) and
  DT_BIAS = softplus^-1(0.01), so the median step is 0.01 and dt stays in the
  stated range.  The library takes dt as given (no softplus inside).
* x, B, C ~ N(0, 1)
* init_state / state ~ N(0, 0.1^2)   (standard deviation 0.1)
* accept_len ~ U{0, ..., K}
* Upstream gradients of the chunked scan (its backward pass), from a generator of
  their own seed: dy ~ N(0, 1) stored like x, then d_final ~ N(0, 1) in float32.
* Multi-round verify on a state ring: A, D, init_state as above, then (with a fused
  step activation) dt_bias = softplus^-1(0.01) + N(0, 0.5^2) per head; then per
  round x, dt, B, C, accept_len ~ U{0..K}, a rollback request ~ U{0..3} and whether
  it is made (probability 0.3).  dt follows the recipe above without the activation,
  and is the raw pre-activation value z ~ N(0, 1) with it.
* Storage: dt, A, D and every state in float32.  x, B, C are float32 for the
  fp32 workload and bfloat16 (float64 -> float32 -> bfloat16, both roundings to
  nearest-even) for the bf16 workloads.

The workload shapes are those of a Mamba-2 style SSD layer (see ``WORKLOADS``);
no dataset is involved.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

DT_MIN, DT_MAX = 1e-3, 1e-1
DT_BIAS = math.log(math.expm1(0.01))          # softplus^-1(0.01) = -4.6002...

# Named workloads.  "scan" entries feed the chunked scan, "verify" the verify step.
WORKLOADS = {
    # tiny fp32 layer, the case the oracle finishes instantly
    "tiny_fp32": dict(kind="scan", b=1, L=256, H=4, P=16, N=16, G=1, Q=64, io="f32",
                      init=False, seed=0),
    # Mamba-2-2.7B-shaped layer at L=2k
    "mamba2_2p7b_L2k": dict(kind="scan", b=4, L=2048, H=80, P=64, N=128, G=1, Q=256,
                            io="bf16", init=False, seed=1),
    # long-context layer, 64 chunks, nonzero initial state
    "mamba2_2p7b_L16k": dict(kind="scan", b=1, L=16384, H=80, P=64, N=128, G=1, Q=256,
                             io="bf16", init=True, seed=2),
    # state-size sweep
    "dstate_sweep_N16": dict(kind="scan", b=8, L=4096, H=32, P=64, N=16, G=4, Q=128,
                             io="bf16", init=False, seed=30),
    "dstate_sweep_N64": dict(kind="scan", b=8, L=4096, H=32, P=64, N=64, G=4, Q=128,
                             io="bf16", init=False, seed=31),
    "dstate_sweep_N128": dict(kind="scan", b=8, L=4096, H=32, P=64, N=128, G=4, Q=128,
                              io="bf16", init=False, seed=32),
    "dstate_sweep_N256": dict(kind="scan", b=8, L=4096, H=32, P=64, N=256, G=4, Q=128,
                              io="bf16", init=False, seed=33),
    # the selective scan SSD replaces (one channel per head, diagonal A) on the same
    # layer: 80 x 64 = 5120 channels, at the state size 16 it was used with and at
    # SSD's 128
    "mamba1_L2k_N16": dict(kind="selective", b=4, L=2048, Dch=5120, N=16, G=1, io="bf16",
                           init=False, seed=40),
    "mamba1_L2k_N128": dict(kind="selective", b=4, L=2048, Dch=5120, N=128, G=1, io="bf16",
                            init=False, seed=41),
    # speculative-decoding verify on a Llama-3-8B-distilled hybrid layer shape
    "verify_b32_K4": dict(kind="verify", b=32, K=4, H=32, P=128, N=128, G=8, io="bf16",
                          seed=4),
}


# ---------------------------------------------------------------- rounding helpers
def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    nan = np.isnan(a)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _softplus(v):
    return np.logaddexp(0.0, v)


@dataclasses.dataclass
class Tensor:
    """An array in its storage type: float32 values, or bfloat16 as uint16 bits."""
    data: np.ndarray
    dtype: str                                # "f32" or "bf16"

    def f64(self) -> np.ndarray:
        """Exact float64 copy of the stored values (what the oracle consumes)."""
        if self.dtype == "bf16":
            return bf16_bits_to_f32(self.data).astype(np.float64)
        return self.data.astype(np.float64)

    @property
    def shape(self):
        return self.data.shape


def _store(v64: np.ndarray, dtype: str) -> Tensor:
    v32 = v64.astype(np.float32)
    if dtype == "bf16":
        return Tensor(f32_to_bf16_bits(v32), "bf16")
    if dtype == "f32":
        return Tensor(v32, "f32")
    raise ValueError(dtype)


@dataclasses.dataclass
class ScanInputs:
    x: Tensor
    dt: Tensor
    A: Tensor
    B: Tensor
    C: Tensor
    D: Tensor
    init_state: Optional[Tensor]
    Q: int
    io: str

    @property
    def dims(self):
        b, L, H, P = self.x.shape
        return dict(b=b, L=L, H=H, P=P, N=self.B.shape[3], G=self.B.shape[2], Q=self.Q)


@dataclasses.dataclass
class VerifyInputs:
    state: Tensor
    x: Tensor
    dt: Tensor
    A: Tensor
    B: Tensor
    C: Tensor
    D: Tensor
    accept_len: np.ndarray
    io: str

    @property
    def dims(self):
        b, K, H, P = self.x.shape
        return dict(b=b, K=K, H=H, P=P, N=self.B.shape[3], G=self.B.shape[2])


@dataclasses.dataclass
class SelectiveInputs:
    x: Tensor
    dt: Tensor
    A: Tensor
    B: Tensor
    C: Tensor
    D: Tensor
    init_state: Optional[Tensor]
    io: str

    @property
    def dims(self):
        b, L, Dch = self.x.shape
        return dict(b=b, L=L, Dch=Dch, N=self.B.shape[3], G=self.B.shape[2])


def _dt(rng, shape):
    z = rng.standard_normal(shape)
    return np.clip(_softplus(z + DT_BIAS), DT_MIN, DT_MAX)


def make_scan_inputs(b, L, H, P, N, G, Q, io="bf16", init=False, seed=0) -> ScanInputs:
    """Draw one chunked-scan problem (see the module docstring for the recipe)."""
    if H % G:
        raise ValueError("H must be a multiple of G")
    rng = np.random.default_rng(seed)
    A = -np.exp(rng.uniform(0.0, math.log(16.0), H))
    D = rng.standard_normal(H)
    dt = _dt(rng, (b, L, H))
    x = rng.standard_normal((b, L, H, P))
    x = _store(x, io)
    B = _store(rng.standard_normal((b, L, G, N)), io)
    C = _store(rng.standard_normal((b, L, G, N)), io)
    init_state = _store(0.1 * rng.standard_normal((b, H, P, N)), "f32") if init else None
    return ScanInputs(x=x, dt=_store(dt, "f32"), A=_store(A, "f32"), B=B, C=C,
                      D=_store(D, "f32"), init_state=init_state, Q=Q, io=io)


def make_verify_inputs(b, K, H, P, N, G, io="bf16", seed=0) -> VerifyInputs:
    """Draw one verify-step problem (see the module docstring for the recipe)."""
    if H % G:
        raise ValueError("H must be a multiple of G")
    rng = np.random.default_rng(seed)
    A = -np.exp(rng.uniform(0.0, math.log(16.0), H))
    D = rng.standard_normal(H)
    state = 0.1 * rng.standard_normal((b, H, P, N))
    dt = _dt(rng, (b, K, H))
    x = rng.standard_normal((b, K, H, P))
    B = rng.standard_normal((b, K, G, N))
    C = rng.standard_normal((b, K, G, N))
    accept = rng.integers(0, K + 1, size=b).astype(np.int32)
    return VerifyInputs(state=_store(state, "f32"), x=_store(x, io), dt=_store(dt, "f32"),
                        A=_store(A, "f32"), B=_store(B, io), C=_store(C, io),
                        D=_store(D, "f32"), accept_len=accept, io=io)


def make_selective_inputs(b, L, Dch, N, G=1, io="bf16", init=False, seed=0) -> SelectiveInputs:
    """Draw one selective-scan problem, one channel per head (see the module docstring)."""
    if Dch % G:
        raise ValueError("Dch must be a multiple of G")
    rng = np.random.default_rng(seed)
    A = -np.exp(rng.uniform(0.0, math.log(16.0), (Dch, N)))
    D = rng.standard_normal(Dch)
    dt = _dt(rng, (b, L, Dch))
    x = rng.standard_normal((b, L, Dch))
    B = rng.standard_normal((b, L, G, N))
    C = rng.standard_normal((b, L, G, N))
    init_state = _store(0.1 * rng.standard_normal((b, Dch, N)), "f32") if init else None
    return SelectiveInputs(x=_store(x, io), dt=_store(dt, "f32"), A=_store(A, "f32"),
                           B=_store(B, io), C=_store(C, io), D=_store(D, "f32"),
                           init_state=init_state, io=io)


def make_upstream_grads(inp: ScanInputs, seed: int, final: bool = True):
    """Upstream gradients (dy, d_final) for the backward pass of a chunked-scan problem:
    dy like x, d_final like the state (None unless ``final``)."""
    d = inp.dims
    rng = np.random.default_rng(seed)
    dy = _store(rng.standard_normal((d["b"], d["L"], d["H"], d["P"])), inp.io)
    d_final = (_store(rng.standard_normal((d["b"], d["H"], d["P"], d["N"])), "f32")
               if final else None)
    return dy, d_final


@dataclasses.dataclass
class RingInputs:
    A: Tensor
    D: Tensor
    init_state: Tensor
    dt_bias: Optional[Tensor]
    rounds: list          # per round: dict(x, dt, B, C, accept_len, rollback)
    R: int
    io: str


def make_verify_ring_inputs(b, K, H, P, N, G, R, rounds, io="bf16", biased=False,
                            seed=0) -> RingInputs:
    """Draw a multi-round verify problem (see the module docstring for the recipe).
    ``rollback`` of a round is None or int32 [b] step requests (which may exceed what
    the ring can undo)."""
    if H % G:
        raise ValueError("H must be a multiple of G")
    rng = np.random.default_rng(seed)
    A = -np.exp(rng.uniform(0.0, math.log(16.0), H))
    D = rng.standard_normal(H)
    init = 0.1 * rng.standard_normal((b, H, P, N))
    bias = _store(DT_BIAS + 0.5 * rng.standard_normal(H), "f32") if biased else None
    out = []
    for _ in range(rounds):
        x = rng.standard_normal((b, K, H, P))
        dt = rng.standard_normal((b, K, H)) if biased else _dt(rng, (b, K, H))
        Bv = rng.standard_normal((b, K, G, N))
        Cv = rng.standard_normal((b, K, G, N))
        acc = rng.integers(0, K + 1, size=b).astype(np.int32)
        steps = rng.integers(0, 4, size=b).astype(np.int32)
        made = rng.uniform() < 0.3
        out.append(dict(x=_store(x, io), dt=_store(dt, "f32"), B=_store(Bv, io), C=_store(Cv, io),
                        accept_len=acc, rollback=steps if made else None))
    return RingInputs(A=_store(A, "f32"), D=_store(D, "f32"), init_state=_store(init, "f32"),
                      dt_bias=bias, rounds=out, R=R, io=io)


def make_workload(name: str, **override):
    """Inputs of a named workload; keyword overrides change shape or seed."""
    cfg = dict(WORKLOADS[name])
    cfg.update(override)
    kind = cfg.pop("kind")
    if kind == "scan":
        return make_scan_inputs(**cfg)
    if kind == "selective":
        return make_selective_inputs(**cfg)
    return make_verify_inputs(**cfg)
