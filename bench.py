#!/usr/bin/env python3
"""Benchmark of the SSD hot path on one MI355X (gfx950).

A step is one ssd_chunk_scan_fwd call (discretisation, in-chunk decay scan, steps 1-4
of the chunked SSD algorithm) over the Mamba-2-2.7B-shaped layer at L=2048
(batch 4, 80 heads, headdim 64, dstate 128, 1 group, chunk 256, bf16 I/O, fp32
state).  Inputs are seeded synthetic data resident in HBM before timing starts.  To
keep the 256 MB Infinity Cache from serving a step's inputs out of cache, the steps
rotate over several identical copies of the inputs whose total exceeds the cache.

Printed: one JSON line with the contract fields plus
  roofline      algorithmic bytes of one call / its mean duration (HIP events on the
                launch stream around the K timed calls), against 8 TB/s; "traffic" is
                the measured HBM bytes per call from the committed counter summary in
                profiles/, used only while the kernel source still hashes to what was
                profiled
  call_stats_us median, 10th and 90th percentile of per-call durations, from a second
                pass of at least 50 calls with an event before each (so the event
                records stay out of the K timed steps)
  device        CU count and maximum engine clock of the GPU (rocminfo)
  scan_configs  the other chunk-scan configs of the workload list, each with its own
                tokens/s, call statistics and roofline object: the long-context layer
                (L=16384, nonzero initial state) and the state-size sweep (b=8, L=4096,
                H=32, G=4, Q=128, N in {16, 64, 128, 256})
  cpu_baseline  the fp64 CPU oracle as it stands, on a bounded sample of the headline
                workload: one run on 1 thread and one on the host pool (the box's share,
                at most 16 threads), with the CPU model and core counts; the pool run's
                outputs are compared with the timed GPU call's (parity_vs_timed_call)
  cpu_baseline_configs
                the same on 16 units of every other chunk-scan config
  parity_ok     every oracle comparison above within its tolerance
  cpu_oracle_extras
                the verify, comparison-scan and gradient oracles timed on bounded
                samples of their legs' workloads
  verify        the K=4 verify step (GB/s of algorithmic bytes), beside an elementwise
                kernel that reads and writes the same 64 MiB (inputs rotated alike)
  selective_scan_comparison
                the one-channel-per-head selective scan (diagonal A, the recurrence
                SSD replaces) on the same layer shape (4 x 2048 tokens, 5120
                channels) at N=16 and N=128, and how many times faster the SSD
                chunked scan (N=128) is than each, with the comparison kernel's own
                roofline (state updates/s against the vector-ALU ceiling) and the
                speed-up the SSD scan would keep over a comparison kernel at that
                ceiling
  decode_K1     the verify step with one token (a decode step), GB/s
  verify_ring   one round of the multi-round verify on a ring of 8 states (K=4, every
                draft accepted, fused softplus step), GB/s
  sequence_parallel
                one device's share of the L=16k layer split into 8 slices, in both
                orders of work: states first (the slice's (decay, state) pair without
                outputs, the combine of 8 pairs, the slice's scan from its entering
                state) and outputs first (the slice's scan from zero, its total decay,
                the combine, the correction by the entering state); share_us is the
                faster (the exchange between devices is not measured: this build runs
                on one GPU)
  backward      ssd_chunk_scan_bwd (all seven gradients, states recomputed) on the
                L=2048 layer with upstream gradients for y and the final state:
                tokens/s and algorithmic bytes / call time against 8 TB/s
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SSD fwd tokens/s per layer at L=2k/16k; % MFMA/HBM roofline; verify-step GB/s"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 << 20
# Vector-ALU ceiling of the comparison scan, in state updates per second.  One update
# of one state for one token needs one exponential (dt a, the decay factor) and four
# plain vector operations (the product dt a, the product dt x B, the fused decay-and-add,
# the fused C h accumulation).  On MI355X (256 CUs of 4 SIMDs at 2.4 GHz; 157.3 TFLOP/s
# fp32 = 32 fused multiply-adds per SIMD per clock) a wave of 64 lanes issues a plain
# fp32 operation in 2 clocks and a transcendental (quarter rate) in 8, so an update
# costs at least (4 * 2 + 8) / 64 SIMD clocks: 4 updates per SIMD per clock.
SEL_ALU_PEAK_UPDATES = 256 * 4 * 2.4e9 * 4.0


KERNEL_SOURCES = [os.path.join(ROOT, "selective_state_space_ssd_amd", "csrc", f)
                  for f in ("ssd_chunk_fused.hip", "ssd_device.h", "ssd_kernels.h", "ssd_api.hip")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_ssd_fused_mamba2_2p7b_L2k.json")


def kernel_source_hash():
    """Hash of the sources that decide what the scan kernels do."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per call from the committed rocprofv3 counter summary, or None when
    there is none or the kernel source changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t.get("bytes_per_call")


def scan_alg_bytes(d, io_bytes, init):
    """Bytes the method must move: x, y, dt, B, C, A, D, final state (+ initial state)."""
    tokens = d["b"] * d["L"]
    per_tok = d["H"] * d["P"] * io_bytes * 2 + 4 * d["H"] + 2 * d["G"] * d["N"] * io_bytes
    state = d["b"] * d["H"] * d["P"] * d["N"] * 4
    return tokens * per_tok + 8 * d["H"] + state * (2 if init else 1)


def scan_alg_flops(d):
    """2 x MACs of the causal chunked algorithm (C B^T per group, Y_diag, S, Y_off)."""
    b, L, H, P, N, G, Q = (d[k] for k in ("b", "L", "H", "P", "N", "G", "Q"))
    macs = 0
    for c in range(math.ceil(L / Q)):
        q = min(Q, L - c * Q)
        tri = q * (q + 1) // 2
        macs += G * tri * N + H * (tri * P + 2 * q * P * N)
    return 2 * b * macs


def verify_alg_bytes(d, io_bytes):
    b, K, H, P, N, G = (d[k] for k in ("b", "K", "H", "P", "N", "G"))
    state = b * H * P * N * 4
    return (2 * state + 2 * b * K * H * P * io_bytes + b * K * H * 4 +
            2 * b * K * G * N * io_bytes + 4 * b + 8 * H)


def _copies(inp, count, bd):
    sets = []
    for _ in range(count):
        sets.append({k: bd.to_device(getattr(inp, k))
                     for k in ("x", "dt", "A", "B", "C", "D", "init_state")})
    return sets


def time_scan(name, steps, warmup, bd, inputs, torch, stats_calls=50):
    inp = inputs.make_workload(name)
    d = inp.dims
    io_bytes = 2 if inp.io == "bf16" else 4
    alg = scan_alg_bytes(d, io_bytes, inp.init_state is not None)
    footprint = alg + d["b"] * d["L"] * d["H"] * d["P"] * io_bytes
    nsets = max(2, math.ceil(3 * MALL_BYTES / footprint))
    sets = _copies(inp, nsets, bd)
    ys = [torch.empty_like(s["x"]) for s in sets]
    fss = [torch.empty((d["b"], d["H"], d["P"], d["N"]), dtype=torch.float32, device="cuda")
           for _ in sets]
    ws = bd.chunk_scan_workspace(sets[0]["x"], sets[0]["B"], d["Q"])
    stream = torch.cuda.current_stream()

    def call(i):
        s = sets[i % nsets]
        bd.ssd_chunk_scan_fwd(s["x"], s["dt"], s["A"], s["B"], s["C"], s["D"], s["init_state"],
                              ys[i % nsets], fss[i % nsets], d["Q"], ws, stream)

    for i in range(warmup):
        call(i)
    mean_ms, wall = _timed(call, warmup, steps, stream, torch)
    last = (warmup + steps - 1) % nsets          # the set the last timed call wrote
    stats = _call_stats(call, warmup + steps, max(stats_calls, steps), stream, torch)
    # outputs of one call for the oracle comparison: the stats pass ran after the timed
    # calls, so run the last timed call's inputs once more into its own buffers
    call(last)
    err = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    bd.ssd_chunk_scan_workspace_error(ws, err)
    torch.cuda.synchronize()
    return dict(name=name, inp=inp, dims=d, alg_bytes=alg, flops=scan_alg_flops(d), wall_s=wall,
                ms_per_step=wall * 1e3 / steps, call_ms_mean=mean_ms, nsets=nsets,
                stats=stats, y=ys[last], final_state=fss[last], handoff_error=int(err.item()))


def time_selective(name, steps, warmup, bd, inputs, torch):
    """The comparison scan on its workload, inputs rotated like time_scan's."""
    inp = inputs.make_workload(name)
    d = inp.dims
    io_bytes = 2 if inp.io == "bf16" else 4
    # x, y, dt per (token, channel), B and C per token, A per (channel, state)
    alg = (d["b"] * d["L"] * d["Dch"] * (2 * io_bytes + 4) + 2 * d["b"] * d["L"] * d["G"] * d["N"] *
           io_bytes + d["Dch"] * d["N"] * 4 + 8 * d["Dch"])
    nsets = max(2, math.ceil(3 * MALL_BYTES / alg))
    sets = _copies(inp, nsets, bd)
    ys = [torch.empty_like(s["x"]) for s in sets]
    stream = torch.cuda.current_stream()

    def call(i):
        s = sets[i % nsets]
        bd.ssd_selective_scan_fwd(s["x"], s["dt"], s["A"], s["B"], s["C"], s["D"], s["init_state"],
                                  ys[i % nsets], None, stream)

    for i in range(warmup):
        call(i)
    mean_ms, _ = _timed(call, warmup, steps, stream, torch)
    return dict(dims=d, alg_bytes=alg, call_ms_mean=mean_ms)


def _timed(call, first, steps, stream, torch):
    """Run `steps` calls back to back between one pair of HIP events on `stream` (the
    stream the kernels are launched on); returns (mean event ms per call, wall s)."""
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        call(first + i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall


def _call_stats(call, first, n, stream, torch):
    """n more calls with a HIP event recorded on `stream` before each call and after the
    last: per-call durations (event to event, so back-to-back launches) -> median, 10th
    and 90th percentile in microseconds.  A separate pass from the K timed steps, so the
    extra event records do not touch the headline timing."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(n):
        call(first + i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    us = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(n))
    q = lambda f: us[min(n - 1, max(0, int(round(f * (n - 1)))))]
    return {"calls": n, "median_us": q(0.5), "p10_us": q(0.1), "p90_us": q(0.9),
            "min_us": us[0], "max_us": us[-1]}


def time_verify(steps, warmup, bd, inputs, torch, K=None):
    v = inputs.make_workload("verify_b32_K4", **({} if K is None else {"K": K}))
    d = v.dims
    io_bytes = 2 if v.io == "bf16" else 4
    alg = verify_alg_bytes(d, io_bytes)
    nsets = max(2, math.ceil(3 * MALL_BYTES / alg))
    sets = []
    for _ in range(nsets):
        t = {k: bd.to_device(getattr(v, k)) for k in ("state", "x", "dt", "A", "B", "C", "D",
                                                       "accept_len")}
        t["y"] = torch.empty_like(t["x"])
        t["out"] = torch.empty_like(t["state"])
        sets.append(t)
    stream = torch.cuda.current_stream()

    def call(i):
        t = sets[i % nsets]
        bd.ssd_verify_step(t["state"], t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"],
                           t["accept_len"], t["y"], t["out"], None, None, stream)

    for i in range(warmup):
        call(i)
    mean_ms, _ = _timed(call, warmup, steps, stream, torch)
    stats = _call_stats(call, warmup + steps, max(50, steps), stream, torch)
    return dict(dims=d, alg_bytes=alg, call_ms_mean=mean_ms, gbs=alg / (mean_ms * 1e-3) / 1e9,
                stats=stats)


def bwd_alg_bytes(d, io_bytes, init, final):
    """Bytes the gradient call must move at least: x, dy, B, C, dt, A, D, the initial
    state and d_final read; dx, ddt, dA, dB, dC, dD and d_init written."""
    b, L, H, P, N, G = (d[k] for k in ("b", "L", "H", "P", "N", "G"))
    xb, bc, st = b * L * H * P * io_bytes, b * L * G * N * io_bytes, b * H * P * N * 4
    return (3 * xb + 4 * bc + 2 * b * L * H * 4 + (st if init else 0) + (st if final else 0) +
            st + 4 * H * 4)


def time_backward(name, steps, warmup, bd, inputs, torch):
    """ssd_chunk_scan_bwd on a scan workload with upstream gradients for y and the final
    state; inputs rotated like time_scan's."""
    inp = inputs.make_workload(name)
    dy, dfin = inputs.make_upstream_grads(inp, seed=77)
    d = inp.dims
    io_bytes = 2 if inp.io == "bf16" else 4
    alg = bwd_alg_bytes(d, io_bytes, inp.init_state is not None, True)
    nsets = max(2, math.ceil(3 * MALL_BYTES / alg))
    sets = _copies(inp, nsets, bd)
    for s in sets:
        s["dy"], s["dfin"] = bd.to_device(dy), bd.to_device(dfin)
        s["out"] = [torch.empty_like(s["x"]), torch.empty_like(s["dt"]), torch.empty_like(s["A"]),
                    torch.empty_like(s["B"]), torch.empty_like(s["C"]), torch.empty_like(s["D"]),
                    torch.empty((d["b"], d["H"], d["P"], d["N"]), dtype=torch.float32,
                                device="cuda")]
    n = bd.ssd_chunk_scan_bwd_workspace_bytes(d["b"], d["L"], d["H"], d["P"], d["N"], d["G"],
                                              bd._io_code(sets[0]["x"]))
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def call(i):
        s = sets[i % nsets]
        bd.ssd_chunk_scan_bwd(s["x"], s["dt"], s["A"], s["B"], s["C"], s["D"], s["init_state"],
                              s["dy"], s["dfin"], *s["out"], ws, stream)

    for i in range(warmup):
        call(i)
    mean_ms, _ = _timed(call, warmup, steps, stream, torch)
    return dict(dims=d, alg_bytes=alg, call_ms_mean=mean_ms, workspace_bytes=n)


def time_ring(steps, warmup, bd, inputs, torch, K=4, R=8):
    """Verify rounds on a state ring at the verify workload's layer shape (b=32, H=32,
    P=128, N=128, G=8, bf16 I/O), every draft accepted (K states written per round), with
    the fused step activation."""
    w = inputs.WORKLOADS["verify_b32_K4"]
    b, H, P, N, G = w["b"], w["H"], w["P"], w["N"], w["G"]
    ri = inputs.make_verify_ring_inputs(b, K, H, P, N, G, R, 1, io="bf16", biased=True, seed=5)
    r = ri.rounds[0]
    dev = bd.to_device
    A, D, bias = dev(ri.A), dev(ri.D), dev(ri.dt_bias)
    x, dt, B, C = dev(r["x"]), dev(r["dt"]), dev(r["B"]), dev(r["C"])
    acc = torch.full((b,), K, dtype=torch.int32, device="cuda")
    ring = torch.zeros((b, R, H, P, N), dtype=torch.float32, device="cuda")
    meta = torch.empty((b, 2), dtype=torch.int32, device="cuda")
    bd.ssd_verify_ring_init(ring, meta, dev(ri.init_state))
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()

    def call(i):
        bd.ssd_verify_ring(ring, meta, x, dt, A, B, C, D, acc, y, dt_bias=bias, stream=stream)

    for i in range(warmup):
        call(i)
    mean_ms, _ = _timed(call, warmup, steps, stream, torch)
    alg = ring_alg_bytes(b, H, P, N, G, K)
    return dict(call_ms_mean=mean_ms, alg_bytes=alg, gbs=alg / (mean_ms * 1e-3) / 1e9, R=R, K=K)


def ring_alg_bytes(b, H, P, N, G, K):
    """One ring round with every draft accepted: the head state read, K states written,
    bf16 x and y, fp32 dt, bf16 B and C, fp32 A, D, dt_bias and the per-row scalars."""
    st = b * H * P * N * 4
    return (1 + K) * st + 2 * b * K * H * P * 2 + b * K * H * 4 + 2 * b * K * G * N * 2 + 16 * H + 12 * b


def time_seqpar(steps, warmup, bd, inputs, torch, n=8):
    """One device's share of the L=16k layer split into n slices (sequence parallel),
    in both orders of work, each call timed with HIP events.  Outputs first: the
    slice's scan from a zero state, its total decay, the combine of n pairs and the
    correction of the slice by its entering state.  States first: the slice's state and
    decay without outputs, the combine, and the slice's scan from its entering state.
    The slices' pairs stand in for the ones the other devices would send."""
    inp = inputs.make_workload("mamba2_2p7b_L16k")
    d = inp.dims
    b, L, H, P, N, G = d["b"], d["L"], d["H"], d["P"], d["N"], d["G"]
    Ls = L // n
    dev = bd.to_device
    x, dt, A, B, C, D = (dev(getattr(inp, k)) for k in ("x", "dt", "A", "B", "C", "D"))
    xs, dts, Bs, Cs = (t[:, :Ls].contiguous() for t in (x, dt, B, C))
    ys = torch.empty_like(xs)
    fs = torch.empty((b, H, P, N), dtype=torch.float32, device="cuda")
    ws = bd.chunk_scan_workspace(xs, Bs, d["Q"])
    nss = bd.ssd_seq_slice_state_workspace_bytes(b, Ls, H, P, N, G, bd.SSD_DTYPE_BF16)
    ws_state = torch.empty(nss, dtype=torch.uint8, device="cuda")
    alpha = torch.empty((n, b, H), dtype=torch.float32, device="cuda")
    S = torch.randn((n, b, H, P, N), dtype=torch.float32, device="cuda")
    h_in = torch.empty_like(S)
    init = dev(inp.init_state)
    stream = torch.cuda.current_stream()
    flows = {
        "outputs_first": {
            "scan_slice": lambda i: bd.ssd_chunk_scan_fwd(xs, dts, A, Bs, Cs, D, None, ys, fs,
                                                          d["Q"], ws, stream),
            "total_decay": lambda i: bd.ssd_seq_total_decay(dts, A, alpha[0], stream),
            "combine": lambda i: bd.ssd_seq_combine(alpha, S, init, h_in, stream),
            "apply_state": lambda i: bd.ssd_seq_apply_state(ys, fs, dts, A, Cs, h_in[1], stream),
        },
        "states_first": {
            "slice_state": lambda i: bd.ssd_seq_slice_state(xs, dts, A, Bs, S[0], alpha[0],
                                                            ws_state, stream),
            "combine": lambda i: bd.ssd_seq_combine(alpha, S, init, h_in, stream),
            "scan_slice_from_entering_state": lambda i: bd.ssd_chunk_scan_fwd(
                xs, dts, A, Bs, Cs, D, h_in[1], ys, fs, d["Q"], ws, stream),
        },
    }
    out = {}
    for flow, calls in flows.items():
        rec = {}
        for k, call in calls.items():
            for i in range(warmup):
                call(i)
            rec[k + "_us"] = _timed(call, warmup, steps, stream, torch)[0] * 1e3
        rec["share_us"] = sum(rec.values())
        out[flow] = rec
    best = min(flows, key=lambda f: out[f]["share_us"])
    out["share_us"] = out[best]["share_us"]
    out["share_flow"] = best
    out["slice_tokens"] = b * Ls
    out["exchange_bytes_per_device"] = b * H * (P * N + 1) * 4
    return out


def copy_bandwidth(torch, mib=1024, reps=10):
    """Read+write GB/s of a plain elementwise kernel over a buffer far larger than the
    caches: the practical HBM ceiling beside the 8 TB/s specification."""
    n = (mib << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    torch.neg(src, out=dst)
    ms, _ = _timed(lambda i: torch.neg(src, out=dst), 0, reps, stream, torch)
    del src, dst
    return 2 * (n * 4) / (ms * 1e-3) / 1e9


def copy_bandwidth_rotated(torch, mib, steps):
    """Read+write GB/s of the same elementwise kernel over `mib` MiB each way, the buffers
    rotated like a leg's inputs so that none is served from the Infinity Cache: the
    practical ceiling for a kernel that moves that many bytes in one launch."""
    n = (mib << 20) // 4
    nsets = max(2, math.ceil(3 * MALL_BYTES / (2 * n * 4)))
    bufs = [(torch.ones(n, dtype=torch.float32, device="cuda"),
             torch.empty(n, dtype=torch.float32, device="cuda")) for _ in range(nsets)]
    stream = torch.cuda.current_stream()

    def call(i):
        src, dst = bufs[i % nsets]
        torch.neg(src, out=dst)

    for i in range(3):
        call(i)
    ms, _ = _timed(call, 3, steps, stream, torch)
    del bufs
    return 2 * (n * 4) / (ms * 1e-3) / 1e9


def host_cpu():
    """CPU model and the core counts the host reports (the box's share may be smaller
    than os.cpu_count(): the oracle's pool uses the affinity count, at most 16)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity_cpus": affinity,
            "pool_threads": max(1, min(16, affinity))}


def _oracle_units(inp, units, threads):
    """Run the fp64 oracle on the given (batch, head) units, each on its own slice of the
    inputs (one batch row, one head, its group's B and C), on `threads` host threads.
    Returns ({unit: (y [L, P], final_state [P, N])}, wall seconds)."""
    import concurrent.futures

    import numpy as np

    import oracle
    d = inp.dims
    H, G = d["H"], d["G"]
    hpg = H // G
    x, dt, A, B, C, D = (getattr(inp, k).f64() for k in ("x", "dt", "A", "B", "C", "D"))
    init = None if inp.init_state is None else inp.init_state.f64()
    sl = np.ascontiguousarray

    def one(u):
        bi, h = divmod(u, H)
        g = h // hpg
        y, fs = oracle.scan_f64(sl(x[bi:bi + 1, :, h:h + 1]), sl(dt[bi:bi + 1, :, h:h + 1]),
                                A[h:h + 1], sl(B[bi:bi + 1, :, g:g + 1]),
                                sl(C[bi:bi + 1, :, g:g + 1]), D[h:h + 1],
                                None if init is None else sl(init[bi:bi + 1, h:h + 1]))
        return u, (y[0, :, 0], fs[0, 0])

    one(units[0])   # load the library, page in the inputs
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
        res = dict(ex.map(one, units))
    return res, time.perf_counter() - t0


def _compare(res, y, fs, H, tol):
    """Slice-normalised max errors of the GPU outputs against the oracle's, per unit."""
    import numpy as np
    yg = y.float().cpu().numpy().astype(np.float64)
    fg = fs.cpu().numpy().astype(np.float64)
    ey = ef = 0.0
    for u, (yo, fo) in res.items():
        bi, h = divmod(u, H)
        ey = max(ey, float(np.max(np.abs(yg[bi, :, h] - yo)) / max(np.max(np.abs(yo)), 1e-30)))
        ef = max(ef, float(np.max(np.abs(fg[bi, h] - fo)) / max(np.max(np.abs(fo)), 1e-30)))
    ok = bool(np.isfinite(ey) and np.isfinite(ef) and ey <= tol and ef <= tol)
    return {"units": len(res), "err_y": ey, "err_final_state": ef, "tol": tol, "ok": ok}


def cpu_baseline(r, one_thread_units, all_units, host):
    """The fp64 oracle as it stands, timed on the host cores on a bounded sample of the
    workload: one run on 1 thread, one on the pool (up to 16 threads, the box's share).
    The units of the pool run are also compared with the outputs of the timed GPU call
    (slice-normalised max error, the tolerance the parity tests use)."""
    inp, d = r["inp"], r["dims"]
    units = d["b"] * d["H"]
    tokens_per_unit = d["b"] * d["L"] / units
    n1 = min(units, one_thread_units)
    stride1 = max(1, units // n1)
    u1 = list(range(0, units, stride1))[:n1]
    _, w1 = _oracle_units(inp, u1, 1)
    na = min(units, all_units)
    stridea = max(1, units // na)
    ua = list(range(0, units, stridea))[:na]
    threads = host["pool_threads"]
    resa, wa = _oracle_units(inp, ua, threads)
    tol = 2e-2 if inp.io == "bf16" else 1e-4
    return {"value": tokens_per_unit * len(ua) / wa, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{len(ua)} of {units} (batch, head) units of {d['b']}x{d['L']} tokens "
                      f"on {threads} threads, tokens scaled by {len(ua)}/{units}; wall {wa:.2f} s",
            "one_thread": {"value": tokens_per_unit * len(u1) / w1, "unit": "tokens/s",
                           "cores": 1,
                           "sample": f"{len(u1)} of {units} units, tokens scaled by "
                                     f"{len(u1)}/{units}; wall {w1:.2f} s"},
            "cpu_model": host["cpu_model"], "os_cpu_count": host["os_cpu_count"],
            "affinity_cpus": host["affinity_cpus"],
            "parity_vs_timed_call": _compare(resa, r["y"], r["final_state"], d["H"], tol)}


def cpu_oracle_extras(inputs):
    """The other oracles as they stand, on bounded samples of the extra legs'
    workloads (one host thread each; a few seconds in all)."""
    import numpy as np

    import oracle
    from oracle import backward, cp, ring
    out = {}
    # verify step: the whole verify workload through the fp64 verify oracle
    v = inputs.make_workload("verify_b32_K4")
    d = v.dims
    args = [getattr(v, k).f64() for k in ("state", "x", "dt", "A", "B", "C", "D")]
    t0 = time.perf_counter()
    oracle.verify_f64(*args, v.accept_len, want_all=False)
    wall = time.perf_counter() - t0
    out["verify"] = {"value": verify_alg_bytes(d, 2) / wall / 1e9, "unit": "GB/s", "cores": 1,
                     "kind": "oracle", "sample": f"the whole verify workload; wall {wall:.2f} s"}
    # ring: one round of the ring leg's workload, every draft accepted
    K, R = 4, 8
    ri = inputs.make_verify_ring_inputs(d["b"], K, d["H"], d["P"], d["N"], d["G"], R, 1,
                                        io="bf16", biased=True, seed=5)
    rr = ri.rounds[0]
    rg, meta = ring.ring_init_f64(ri.init_state.f64(), R)
    acc = np.full(d["b"], K, dtype=np.int32)
    t0 = time.perf_counter()
    ring.verify_ring_f64(rg, meta, rr["x"].f64(), rr["dt"].f64(), ri.A.f64(), rr["B"].f64(),
                         rr["C"].f64(), ri.D.f64(), acc, dt_bias=ri.dt_bias.f64())
    wall = time.perf_counter() - t0
    out["verify_ring"] = {"value": ring_alg_bytes(d["b"], d["H"], d["P"], d["N"], d["G"], K)
                          / wall / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                          "sample": f"one whole round; wall {wall:.2f} s"}
    # comparison scan: 64 of 5120 channels at N = 128
    sel = inputs.make_workload("mamba1_L2k_N128")
    ch = np.arange(64)
    x, dt, A, D = (getattr(sel, k).f64() for k in ("x", "dt", "A", "D"))
    t0 = time.perf_counter()
    oracle.selective_scan_f64(x[:, :, ch], dt[:, :, ch], A[ch], sel.B.f64(), sel.C.f64(), D[ch])
    wall = time.perf_counter() - t0
    ds = sel.dims
    out["selective_scan_N128"] = {
        "value": ds["b"] * ds["L"] * len(ch) / ds["Dch"] / wall, "unit": "tokens/s", "cores": 1,
        "kind": "oracle", "sample": f"{len(ch)} of {ds['Dch']} channels, tokens scaled by "
                                    f"{len(ch)}/{ds['Dch']}; wall {wall:.2f} s"}
    # sequence-parallel correction: 16 heads of batch row 0 over one 2048-token slice of
    # the L16k layer (one group: C is shared by those heads)
    l16 = inputs.make_workload("mamba2_2p7b_L16k")
    d16 = l16.dims
    Ls, nh = d16["L"] // 8, 16
    rng = np.random.default_rng(3)
    h_in = rng.standard_normal((1, nh, d16["P"], d16["N"]))
    ys = rng.standard_normal((1, Ls, nh, d16["P"]))
    t0 = time.perf_counter()
    cp.apply_entering_state_f64(ys, None, l16.dt.f64()[:1, :Ls, :nh], l16.A.f64()[:nh],
                                l16.C.f64()[:1, :Ls, :1], h_in)
    wall = time.perf_counter() - t0
    u16 = d16["b"] * d16["H"]
    out["sequence_parallel_apply"] = {
        "value": d16["b"] * Ls * nh / u16 / wall, "unit": "tokens/s", "cores": 1,
        "kind": "oracle",
        "sample": f"{nh} of {u16} (batch, head) units of one {Ls}-token slice, tokens scaled "
                  f"by {nh}/{u16}; wall {wall:.2f} s"}
    # backward: one head of one batch row of the L2k layer through the gradient oracle
    inp = inputs.make_workload("mamba2_2p7b_L2k")
    dy, dfin = inputs.make_upstream_grads(inp, seed=77)
    db = inp.dims
    sl = (slice(0, 1), slice(None), slice(0, 1))
    t0 = time.perf_counter()
    backward.scan_bwd_f64(inp.x.f64()[sl], inp.dt.f64()[:1, :, :1], inp.A.f64()[:1],
                          inp.B.f64()[:1], inp.C.f64()[:1], inp.D.f64()[:1], None,
                          dy.f64()[sl], dfin.f64()[:1, :1])
    wall = time.perf_counter() - t0
    units = db["b"] * db["H"]
    out["backward"] = {"value": db["b"] * db["L"] / units / wall, "unit": "tokens/s",
                       "cores": 1, "kind": "oracle",
                       "sample": f"1 of {units} (batch, head) units, tokens scaled by 1/{units}; "
                                 f"wall {wall:.2f} s"}
    return out


def device_info():
    """CU count and maximum engine clock of the GPU agent, from rocminfo (run as a child
    process before this process touches the GPU)."""
    import subprocess
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return {}
    info = {}
    for agent in out.split("*******")[1:]:
        if "gfx950" not in agent:
            continue
        for line in agent.splitlines():
            key, _, val = line.strip().partition(":")
            val = val.strip()
            if key == "Compute Unit" and "compute_units" not in info:
                info["compute_units"] = int(val.split()[0])
            elif key == "Max Clock Freq. (MHz)" and "max_sclk_mhz" not in info:
                info["max_sclk_mhz"] = int(val.split()[0])
            elif key == "Marketing Name" and "name" not in info:
                info["name"] = val
        break
    return info


def scan_record(r, copy_gbs, traffic=None):
    """One chunk-scan config: tokens/s, per-call statistics and its own roofline object
    (algorithmic bytes of one call / the mean call time on the launch stream)."""
    d = r["dims"]
    achieved = r["alg_bytes"] / (r["call_ms_mean"] * 1e-3) / 1e9
    tf = r["flops"] / (r["call_ms_mean"] * 1e-3) / 1e12
    return {
        "workload": r["name"],
        "shape": {k: d[k] for k in ("b", "L", "H", "P", "N", "G", "Q")},
        "tokens_per_s": d["b"] * d["L"] / (r["call_ms_mean"] * 1e-3),
        "call_ms_mean": r["call_ms_mean"],
        "call_stats_us": r["stats"],
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "alg_bytes_per_launch": r["alg_bytes"], "measured_copy_GBs": copy_gbs,
                     "frac_of_measured_copy": achieved / copy_gbs,
                     "mfma_tflops_alg": tf, "mfma_frac_alg": tf / BF16_PEAK_TFLOPS},
        "handoff_error_word": r["handoff_error"],
    }


def _progress(msg):
    """One line per finished leg on stderr (stdout carries only the JSON line)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mamba2_2p7b_L2k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the L=16k and verify-step measurements")
    ap.add_argument("--calibration-copy-mb", type=int, default=0,
                    help="first run one elementwise kernel that reads and writes this many "
                         "MiB (a known-size reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    dev_info = device_info()   # rocminfo, before this process touches the GPU

    import torch

    from selective_state_space_ssd_amd import binding as bd
    from selective_state_space_ssd_amd import inputs
    bd.lib()
    torch.cuda.set_device(0)
    if args.calibration_copy_mb:
        # one elementwise kernel that reads and writes exactly this many bytes
        n = (args.calibration_copy_mb << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    r = time_scan(args.workload, args.steps, args.warmup, bd, inputs, torch)
    _progress(f"{args.workload} timed")
    d = r["dims"]
    tokens = d["b"] * d["L"]
    copy_gbs = copy_bandwidth(torch)
    head = scan_record(r, copy_gbs, measured_traffic())
    roof = dict(head["roofline"])
    roof["kernel"] = "ssd_chunk_scan_fwd = k_ssd_fused<256,128> (one launch per call)"
    roof["call_ms_mean"] = r["call_ms_mean"]
    out = {
        "metric": METRIC,
        "value": tokens / (r["ms_per_step"] * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if r["inp"].io == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": d["b"], "seqlen": d["L"],
                   "nheads": d["H"], "headdim": d["P"], "dstate": d["N"], "ngroups": d["G"],
                   "chunk": d["Q"], "io": r["inp"].io, "state": "f32",
                   "input_copies_rotated": r["nsets"]},
        "roofline": roof,
        "call_stats_us": r["stats"],
        "handoff_error_word": r["handoff_error"],
        "device": dev_info,
    }
    scans = {args.workload: r}
    if not args.no_extra:
        # every chunk-scan config of the workload list: the long-context layer and the
        # four state sizes of the sweep, each with its own roofline object
        configs = {}
        for name in ("mamba2_2p7b_L16k", "dstate_sweep_N16", "dstate_sweep_N64",
                     "dstate_sweep_N128", "dstate_sweep_N256"):
            if name == args.workload:
                continue
            rc = time_scan(name, max(5, args.steps // 2), 2, bd, inputs, torch)
            scans[name] = rc
            configs[name] = scan_record(rc, copy_gbs)
            _progress(f"{name} timed")
        out["scan_configs"] = configs
        if "mamba2_2p7b_L16k" in configs:
            c16 = configs["mamba2_2p7b_L16k"]
            out["L16k"] = {"tokens_per_s": c16["tokens_per_s"],
                           "call_ms_mean": c16["call_ms_mean"],
                           "achieved_GBs": c16["roofline"]["achieved"],
                           "hbm_frac": c16["roofline"]["frac"]}
        r2 = scans.get("mamba2_2p7b_L16k")
        rv = time_verify(max(10, args.steps), 3, bd, inputs, torch)
        # the verify step moves one 64 MiB state each way: the same-size copy is its
        # practical ceiling
        same = copy_bandwidth_rotated(torch, 64, max(10, args.steps))
        out["verify"] = {"workload": "verify_b32_K4", "GB_per_s": rv["gbs"],
                         "hbm_frac": rv["gbs"] / HBM_PEAK_GBS, "call_ms_mean": rv["call_ms_mean"],
                         "call_stats_us": rv["stats"],
                         "alg_bytes": rv["alg_bytes"], "same_size_copy_GBs": same,
                         "frac_of_same_size_copy": rv["gbs"] / same,
                         "roofline": {"bound": "hbm", "achieved": rv["gbs"],
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": rv["gbs"] / HBM_PEAK_GBS, "traffic": None}}
        r1 = time_verify(max(10, args.steps), 3, bd, inputs, torch, K=1)
        out["decode_K1"] = {"workload": "verify_b32_K4 with K=1", "GB_per_s": r1["gbs"],
                            "hbm_frac": r1["gbs"] / HBM_PEAK_GBS,
                            "call_ms_mean": r1["call_ms_mean"], "alg_bytes": r1["alg_bytes"]}
        rr = time_ring(max(10, args.steps), 3, bd, inputs, torch)
        _progress("verify, decode and ring rounds timed")
        out["verify_ring"] = {"workload": "verify_b32_K4 layer, ring of 8, all 4 drafts accepted, "
                                          "fused softplus step",
                              "GB_per_s": rr["gbs"], "hbm_frac": rr["gbs"] / HBM_PEAK_GBS,
                              "call_ms_mean": rr["call_ms_mean"], "alg_bytes": rr["alg_bytes"]}
        cmp = {}
        ssd_tps = d["b"] * d["L"] / (r["call_ms_mean"] * 1e-3)   # both timed by HIP events
        for n in (16, 128):
            rs = time_selective(f"mamba1_L2k_N{n}", max(3, args.steps // 10), 1, bd, inputs, torch)
            ds = rs["dims"]
            tps = ds["b"] * ds["L"] / (rs["call_ms_mean"] * 1e-3)
            ups = ds["b"] * ds["L"] * ds["Dch"] * ds["N"] / (rs["call_ms_mean"] * 1e-3)
            cmp[f"N{n}"] = {"workload": f"mamba1_L2k_N{n}", "tokens_per_s": tps,
                            "call_ms_mean": rs["call_ms_mean"],
                            "ssd_N128_speedup": ssd_tps / tps,
                            "roofline": {"bound": "alu", "achieved": ups / 1e12,
                                         "peak": SEL_ALU_PEAK_UPDATES / 1e12,
                                         "unit": "T state updates/s",
                                         "frac": ups / SEL_ALU_PEAK_UPDATES, "traffic": None},
                            "ssd_N128_speedup_vs_alu_floor":
                                ssd_tps / (ds["b"] * ds["L"] * SEL_ALU_PEAK_UPDATES /
                                           (ds["b"] * ds["L"] * ds["Dch"] * ds["N"]))}
        out["selective_scan_comparison"] = cmp
        _progress("comparison scan timed")
        sp = time_seqpar(max(10, args.steps), 3, bd, inputs, torch)
        _progress("sequence-parallel pieces timed")
        sp["workload"] = "mamba2_2p7b_L16k in 8 slices of 2048 tokens, one slice's share"
        if r2 is not None:
            sp["monolithic_L16k_per_slice_us"] = r2["call_ms_mean"] * 1e3 / 8
        out["sequence_parallel"] = sp
        rb = time_backward(args.workload, max(5, args.steps // 3), 2, bd, inputs, torch)
        _progress("backward timed")
        db = rb["dims"]
        ab = rb["alg_bytes"] / (rb["call_ms_mean"] * 1e-3) / 1e9
        out["backward"] = {"workload": args.workload,
                           "tokens_per_s": db["b"] * db["L"] / (rb["call_ms_mean"] * 1e-3),
                           "call_ms_mean": rb["call_ms_mean"], "alg_bytes": rb["alg_bytes"],
                           "achieved_GBs": ab, "hbm_frac": ab / HBM_PEAK_GBS,
                           "workspace_bytes": rb["workspace_bytes"],
                           "kernels": "k_bwd_chain<N, 2> (both walks), k_bwd_chunk_bf<N>, "
                                      "k_bwd_reduce_bc, k_bwd_reduce_h"}
    if not args.no_cpu_baseline:
        host = host_cpu()
        out["cpu_baseline"] = cpu_baseline(r, 1 << 30, 1 << 30, host)
        _progress("oracle timed on the headline workload")
        if not args.no_extra:
            # the other chunk-scan configs: the oracle on 16 units each (pool threads),
            # its outputs compared with the timed call's
            per = {}
            for name, rc in scans.items():
                if name == args.workload:
                    continue
                cb = cpu_baseline(rc, 4, 16, host)
                per[name] = {k: cb[k] for k in ("value", "unit", "cores", "sample",
                                                "one_thread", "parity_vs_timed_call")}
            out["cpu_baseline_configs"] = per
            out["cpu_oracle_extras"] = cpu_oracle_extras(inputs)
            _progress("oracles timed on the other legs")
        checks = [out["cpu_baseline"]["parity_vs_timed_call"]["ok"]] + [
            v["parity_vs_timed_call"]["ok"] for v in out.get("cpu_baseline_configs", {}).values()]
        out["parity_ok"] = all(checks)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
