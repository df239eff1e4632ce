"""The C-ABI library: loads, exports every declared symbol, and rejects bad
arguments on the host before anything is enqueued (CPU only: no compute call)."""
import ctypes
import os
import re

import pytest

from selective_state_space_ssd_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd_mi355x.h")

OK, NULL, DIM, GROUPS, UNSUP, ALIGN, WS, ALIAS, HIP = range(9)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.LIB_PATH):
        from selective_state_space_ssd_amd import build
        build.build()
    return bd.lib()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(bd.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert bd.ssd_version().startswith("ssd_mi355x")
    for code in range(9):
        assert bd.ssd_status_string(code).startswith(bd.STATUS_NAMES[code])


def test_workspace_bytes(lib):
    # bf16, P = 64: single-pass kernel, workspace = header + one flag per (b, h, chunk)
    # + a two-slot fp32 state ring per (b, h)
    b, L, H, P, N, G, Q = 4, 2048, 80, 64, 128, 1, 256
    n = bd.ssd_chunk_scan_workspace_bytes(b, L, H, P, N, G, Q, bd.SSD_DTYPE_BF16)
    ring = b * H * 2 * P * N * 4
    flags = b * H * (L // Q) * 4
    assert ring + flags + 256 <= n < ring + flags + 256 + 2 * 256
    # fp32 I/O: three-kernel path, fp32 chunk states + per-chunk decay + entering states
    n32 = bd.ssd_chunk_scan_workspace_bytes(b, L, H, P, N, G, Q, bd.SSD_DTYPE_F32)
    units = b * H * (L // Q)
    # (after the same 256-byte header, which a prepared workspace keeps whichever path
    # a call takes)
    base = 256 + units * P * N * 8 + units * 4
    assert base <= n32 < base + 3 * 256
    assert bd.ssd_chunk_scan_workspace_bytes(0, L, H, P, N, G, Q, 1) == 0
    assert bd.ssd_chunk_scan_workspace_bytes(b, 0, H, P, N, G, Q, 1) == 0
    with pytest.raises(bd.SSDError):
        bd.ssd_chunk_scan_workspace_bytes(b, L, 0, P, N, G, Q, 1)


# Fake device addresses: never dereferenced, because every case below fails a
# host-side check before any launch.
BASE = 0x7F0000000000


def addr(i, misalign=0):
    return BASE + i * 0x100000000 + misalign


def scan_call(lib, over=None, dims=None, io=1, ws_bytes=1 << 40):
    ptrs = dict(x=addr(1), dt=addr(2), A=addr(3), B=addr(4), C=addr(5), D=addr(6),
                init=None, y=addr(7), final=addr(8), ws=addr(9))
    ptrs.update(over or {})
    d = dict(b=1, L=256, H=4, P=16, N=16, G=1, Q=64)
    d.update(dims or {})
    return lib.ssd_chunk_scan_fwd(ptrs["x"], ptrs["dt"], ptrs["A"], ptrs["B"], ptrs["C"],
                                  ptrs["D"], ptrs["init"], ptrs["y"], ptrs["final"], d["b"],
                                  d["L"], d["H"], d["P"], d["N"], d["G"], d["Q"], io,
                                  ptrs["ws"], ws_bytes, None)


@pytest.mark.parametrize("name", ["x", "dt", "A", "B", "C", "D", "y"])
def test_scan_null_required_pointer(lib, name):
    assert scan_call(lib, {name: None}) == NULL


@pytest.mark.parametrize("dims,code", [
    (dict(b=-1), DIM), (dict(L=-5), DIM), (dict(H=0), DIM), (dict(P=0), DIM), (dict(N=0), DIM),
    (dict(G=0), DIM), (dict(Q=0), DIM), (dict(G=3), GROUPS),
    (dict(Q=32), UNSUP), (dict(Q=100), UNSUP), (dict(P=24), UNSUP), (dict(N=24), UNSUP),
    (dict(N=512), UNSUP), (dict(P=128, N=256, Q=256), UNSUP),
])
def test_scan_bad_dims(lib, dims, code):
    assert scan_call(lib, dims=dims) == code


def test_scan_bad_dtype(lib):
    assert scan_call(lib, io=7) == UNSUP


@pytest.mark.parametrize("name,mis", [("x", 8), ("B", 2), ("C", 4), ("y", 8), ("final", 4),
                                      ("init", 8), ("ws", 8), ("dt", 2), ("A", 1), ("D", 2)])
def test_scan_misaligned(lib, name, mis):
    idx = {"x": 1, "dt": 2, "A": 3, "B": 4, "C": 5, "D": 6, "y": 7, "final": 8, "ws": 9,
           "init": 10}[name]
    assert scan_call(lib, {name: addr(idx, mis)}) == ALIGN


def test_workspace_init_checks(lib):
    assert lib.ssd_chunk_scan_workspace_init(None, 0, None) == OK          # nothing to do
    assert lib.ssd_chunk_scan_workspace_init(None, 4096, None) == NULL
    assert lib.ssd_chunk_scan_workspace_init(addr(9, 8), 4096, None) == ALIGN


def test_workspace_error_checks(lib):
    err = addr(11)
    assert lib.ssd_chunk_scan_workspace_error(None, 4096, err, 0, None) == NULL
    assert lib.ssd_chunk_scan_workspace_error(addr(9), 4096, None, 0, None) == NULL
    assert lib.ssd_chunk_scan_workspace_error(addr(9, 8), 4096, err, 0, None) == ALIGN
    assert lib.ssd_chunk_scan_workspace_error(addr(9), 4096, addr(11, 2), 0, None) == ALIGN
    assert lib.ssd_chunk_scan_workspace_error(addr(9), 255, err, 1, None) == WS
    assert lib.ssd_chunk_scan_workspace_error(addr(9), 0, err, 1, None) == WS
    # err_out inside the 256-byte header
    assert lib.ssd_chunk_scan_workspace_error(addr(9), 4096, addr(9, 8), 0, None) == ALIAS
    assert lib.ssd_chunk_scan_workspace_error(addr(9), 4096, addr(9, 252), 1, None) == ALIAS


def test_scan_q256_n256_p64_is_unsupported(lib):
    # Q = 256 with N = 256 at P = 64 fits neither kernel's LDS (160 KiB per CU): the
    # call is refused on the host, before anything is enqueued
    dims = dict(b=1, L=600, H=2, P=64, N=256, G=1, Q=256)
    assert scan_call(lib, dims=dims, io=1) == UNSUP
    # Q = 128 is supported: the same call gets past that check and stops at the next
    # one (a workspace too small), still before any launch
    assert scan_call(lib, dims=dict(dims, Q=128), io=1, ws_bytes=1) == WS


def noalloc_call(lib, dims=None, io=1, over=None):
    ptrs = dict(x=addr(1), dt=addr(2), A=addr(3), B=addr(4), C=addr(5), D=addr(6),
                init=None, y=addr(7), final=addr(8))
    ptrs.update(over or {})
    d = dict(b=1, L=256, H=4, P=16, N=16, G=1, Q=64)
    d.update(dims or {})
    return lib.ssd_chunk_scan_fwd_noalloc(ptrs["x"], ptrs["dt"], ptrs["A"], ptrs["B"],
                                          ptrs["C"], ptrs["D"], ptrs["init"], ptrs["y"],
                                          ptrs["final"], d["b"], d["L"], d["H"], d["P"],
                                          d["N"], d["G"], d["Q"], io, None)


def test_noalloc_host_checks(lib):
    # every case fails (or finishes) on the host before the buffer is looked up
    assert bd.NOALLOC_WORKSPACE_BYTES == 64 << 20
    big = dict(b=4, L=2048, H=80, P=64, N=128, G=1, Q=64)      # fp32: three-kernel path
    need = bd.ssd_chunk_scan_workspace_bytes(*big.values(), bd.SSD_DTYPE_F32)
    assert need > bd.NOALLOC_WORKSPACE_BYTES
    assert noalloc_call(lib, dims=big, io=0) == WS
    assert noalloc_call(lib, dims=dict(H=0)) == DIM
    assert noalloc_call(lib, dims=dict(G=3)) == GROUPS
    assert noalloc_call(lib, io=7) == UNSUP
    assert noalloc_call(lib, dims=dict(b=0), over=dict(x=None, y=None)) == OK   # empty


def test_scan_workspace_checks(lib):
    need = bd.ssd_chunk_scan_workspace_bytes(1, 256, 4, 16, 16, 1, 64, 1)
    assert scan_call(lib, ws_bytes=need - 1) == WS
    assert scan_call(lib, {"ws": None}) == WS


def test_scan_alias_checks(lib):
    assert scan_call(lib, {"y": addr(1)}) == ALIAS                   # y == x
    assert scan_call(lib, {"ws": addr(4)}) == ALIAS                  # workspace on B
    assert scan_call(lib, {"final": addr(5)}) == ALIAS               # final_state on C
    assert scan_call(lib, {"init": addr(10), "final": addr(10, 16)}) == ALIAS   # partial


def test_scan_empty_problem_needs_no_pointers(lib):
    # b == 0: nothing to do, returns OK without touching anything
    assert scan_call(lib, {k: None for k in ("x", "dt", "A", "B", "C", "D", "y", "final",
                                             "ws")}, dims=dict(b=0)) == OK


def verify_call(lib, over=None, dims=None, io=1):
    p = dict(state_in=addr(1), x=addr(2), dt=addr(3), A=addr(4), B=addr(5), C=addr(6),
             D=addr(7), acc=addr(8), y=addr(9), state_out=addr(10), all=None, err=None)
    p.update(over or {})
    d = dict(b=2, K=4, H=4, P=16, N=32, G=2)
    d.update(dims or {})
    return lib.ssd_verify_step(p["state_in"], p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"],
                               p["acc"], p["y"], p["state_out"], p["all"], p["err"], d["b"],
                               d["K"], d["H"], d["P"], d["N"], d["G"], io, None)


@pytest.mark.parametrize("name", ["state_in", "x", "dt", "A", "B", "C", "D", "acc", "y",
                                  "state_out"])
def test_verify_null_required_pointer(lib, name):
    assert verify_call(lib, {name: None}) == NULL


@pytest.mark.parametrize("dims,code", [
    (dict(b=-1), DIM), (dict(K=0), DIM), (dict(H=0), DIM), (dict(P=0), DIM), (dict(N=0), DIM),
    (dict(G=0), DIM), (dict(G=3), GROUPS), (dict(K=17), UNSUP), (dict(N=48), UNSUP),
    (dict(N=512), UNSUP),
])
def test_verify_bad_dims(lib, dims, code):
    assert verify_call(lib, dims=dims) == code


def test_verify_alignment_and_alias(lib):
    assert verify_call(lib, {"state_in": addr(1, 4)}) == ALIGN
    assert verify_call(lib, {"state_out": addr(10, 8)}) == ALIGN
    assert verify_call(lib, {"all": addr(11, 4)}) == ALIGN
    assert verify_call(lib, {"B": addr(5, 2)}) == ALIGN
    assert verify_call(lib, {"state_out": addr(1, 16)}) == ALIAS     # partial overlap
    assert verify_call(lib, {"all": addr(1)}) == ALIAS               # states_all on state_in
    assert verify_call(lib, {"y": addr(2)}) == ALIAS                 # y on x
    assert verify_call(lib, {"err": addr(8)}) == ALIAS               # flag on accept_len


def test_verify_empty_batch_is_ok(lib):
    assert verify_call(lib, {k: None for k in ("state_in", "x", "y", "state_out")},
                       dims=dict(b=0)) == OK


def bwd_call(lib, over=None, dims=None, io=1, ws_bytes=1 << 40):
    p = dict(x=addr(1), dt=addr(2), A=addr(3), B=addr(4), C=addr(5), D=addr(6), init=None,
             dy=addr(7), dfin=None, dx=addr(8), ddt=addr(9), dA=addr(10), dB=addr(11),
             dC=addr(12), dD=addr(13), dinit=addr(14), ws=addr(15))
    p.update(over or {})
    d = dict(b=1, L=256, H=4, P=64, N=32, G=1)
    d.update(dims or {})
    return lib.ssd_chunk_scan_bwd(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["init"],
                                  p["dy"], p["dfin"], p["dx"], p["ddt"], p["dA"], p["dB"],
                                  p["dC"], p["dD"], p["dinit"], d["b"], d["L"], d["H"], d["P"],
                                  d["N"], d["G"], io, p["ws"], ws_bytes, None)


def test_bwd_workspace_bytes(lib):
    b, L, H, P, N, G = 4, 2048, 80, 64, 128, 1
    units = b * H * (L // 64)
    # bf16 I/O, P = 64: bf16 entering states and state gradients, fp32 dB / dC
    # partials per block of heads, two per-chunk scalars.  At this shape the blocks hold
    # 40 heads: 32 chunks x 2 blocks x 4 rows = 256 workgroups, one per CU of gfx950
    n = bd.ssd_chunk_scan_bwd_workspace_bytes(b, L, H, P, N, G, bd.SSD_DTYPE_BF16)
    need = 2 * units * P * N * 2 + 2 * b * L * (H // 40) * N * 4 + 2 * units * 4
    assert need <= n < need + 6 * 256
    # fp32 I/O: fp32 states and state gradients, per-head partials, three scalars
    n32 = bd.ssd_chunk_scan_bwd_workspace_bytes(b, L, H, P, N, G, bd.SSD_DTYPE_F32)
    need32 = 2 * units * P * N * 4 + 2 * b * L * H * N * 4 + 3 * units * 4
    assert need32 <= n32 < need32 + 7 * 256
    # the blocks of heads the plan takes, read back from the size of the dB / dC
    # partials: the workgroups of a block of d heads cost about d + 0.75 head times and
    # run ceil(workgroups / 256) rounds; the cheapest divisor of the group size wins
    for (b2, L2, H2, G2), d in [((2, 300, 4, 2), 1), ((2, 1100, 12, 1), 2),
                                ((4, 630, 48, 2), 8), ((8, 4096, 32, 4), 8),
                                ((4, 2048, 80, 1), 40)]:
        nc2 = -(-L2 // 64)
        fixed = 2 * (b2 * H2 * nc2) * 64 * 64 * 2 + 2 * (b2 * H2 * nc2) * 4
        m = bd.ssd_chunk_scan_bwd_workspace_bytes(b2, L2, H2, 64, 64, G2, bd.SSD_DTYPE_BF16)
        parts = 2 * b2 * L2 * (H2 // d) * 64 * 4
        assert fixed + parts <= m < fixed + parts + 6 * 256, (b2, L2, H2, G2, d)
    assert bd.ssd_chunk_scan_bwd_workspace_bytes(0, L, H, P, N, G, 1) == 0
    assert bd.ssd_chunk_scan_bwd_workspace_bytes(b, 0, H, P, N, G, 1) == 0
    with pytest.raises(bd.SSDError):
        bd.ssd_chunk_scan_bwd_workspace_bytes(b, L, H, -1, N, G, 1)


@pytest.mark.parametrize("name", ["x", "dt", "A", "B", "C", "D", "dy", "dx", "ddt", "dA",
                                  "dB", "dC", "dD"])
def test_bwd_null_required_pointer(lib, name):
    assert bwd_call(lib, {name: None}) == NULL


@pytest.mark.parametrize("dims,code", [
    (dict(b=-1), DIM), (dict(L=-1), DIM), (dict(H=0), DIM), (dict(P=0), DIM), (dict(N=0), DIM),
    (dict(G=0), DIM), (dict(G=3), GROUPS), (dict(P=16), UNSUP), (dict(P=128), UNSUP),
    (dict(N=24), UNSUP), (dict(N=256), UNSUP),
])
def test_bwd_bad_dims(lib, dims, code):
    assert bwd_call(lib, dims=dims) == code


def test_bwd_bad_dtype(lib):
    assert bwd_call(lib, io=3) == UNSUP


@pytest.mark.parametrize("name,idx,mis", [("x", 1, 8), ("dy", 7, 2), ("dx", 8, 8), ("dB", 11, 4),
                                          ("ddt", 9, 2), ("dA", 10, 1), ("dinit", 14, 8),
                                          ("ws", 15, 8), ("dfin", 16, 4)])
def test_bwd_misaligned(lib, name, idx, mis):
    assert bwd_call(lib, {name: addr(idx, mis)}) == ALIGN


def test_bwd_workspace_and_alias_checks(lib):
    need = bd.ssd_chunk_scan_bwd_workspace_bytes(1, 256, 4, 64, 32, 1, 1)
    assert bwd_call(lib, ws_bytes=need - 1) == WS
    assert bwd_call(lib, {"ws": None}) == WS
    assert bwd_call(lib, {"dx": addr(7)}) == ALIAS                  # dx on dy
    assert bwd_call(lib, {"dB": addr(12)}) == ALIAS                 # dB on dC
    assert bwd_call(lib, {"ws": addr(1)}) == ALIAS                  # workspace on x
    assert bwd_call(lib, {"dinit": addr(16), "dfin": addr(16)}) == ALIAS
    assert bwd_call(lib, {"dD": addr(10)}) == ALIAS                 # dD on dA


def ring_call(lib, over=None, dims=None, io=1):
    p = dict(ring=addr(1), meta=addr(2), x=addr(3), dt=addr(4), bias=None, A=addr(5), B=addr(6),
             C=addr(7), D=addr(8), acc=addr(9), y=addr(10), err=None)
    p.update(over or {})
    d = dict(b=2, K=4, R=6, H=4, P=16, N=32, G=2)
    d.update(dims or {})
    return lib.ssd_verify_ring(p["ring"], p["meta"], p["x"], p["dt"], p["bias"], p["A"], p["B"],
                               p["C"], p["D"], p["acc"], p["y"], p["err"], d["b"], d["K"], d["R"],
                               d["H"], d["P"], d["N"], d["G"], io, None)


@pytest.mark.parametrize("name", ["ring", "meta", "x", "dt", "A", "B", "C", "D", "acc", "y"])
def test_ring_null_required_pointer(lib, name):
    assert ring_call(lib, {name: None}) == NULL


@pytest.mark.parametrize("dims,code", [
    (dict(b=-1), DIM), (dict(K=0), DIM), (dict(R=4), DIM), (dict(R=3), DIM), (dict(H=0), DIM),
    (dict(G=3), GROUPS), (dict(K=17, R=20), UNSUP), (dict(N=48), UNSUP),
])
def test_ring_bad_dims(lib, dims, code):
    assert ring_call(lib, dims=dims) == code


def test_ring_alignment_and_alias(lib):
    assert ring_call(lib, {"ring": addr(1, 8)}) == ALIGN
    assert ring_call(lib, {"bias": addr(11, 2)}) == ALIGN
    assert ring_call(lib, {"meta": addr(2, 2)}) == ALIGN
    assert ring_call(lib, {"y": addr(3)}) == ALIAS                   # y on x
    assert ring_call(lib, {"meta": addr(1, 16)}) == ALIAS            # meta inside the ring
    assert ring_call(lib, {"ring": addr(5)}) == ALIAS                # ring on A
    assert ring_call(lib, {"err": addr(9)}) == ALIAS                 # flag on accept_len
    assert ring_call(lib, {"bias": addr(10)}) == ALIAS               # y on dt_bias


def test_ring_init_and_rollback_checks(lib):
    assert lib.ssd_verify_ring_init(addr(1), addr(2), None, 2, 1, 4, 16, 32, None) == DIM
    assert lib.ssd_verify_ring_init(None, addr(2), None, 2, 4, 4, 16, 32, None) == NULL
    assert lib.ssd_verify_ring_init(addr(1, 4), addr(2), None, 2, 4, 4, 16, 32, None) == ALIGN
    assert lib.ssd_verify_ring_init(addr(1), addr(1, 64), None, 2, 4, 4, 16, 32, None) == ALIAS
    assert lib.ssd_verify_ring_init(None, None, None, 0, 4, 4, 16, 32, None) == OK
    assert lib.ssd_verify_ring_rollback(addr(1), addr(2), None, 2, 1, None) == DIM
    assert lib.ssd_verify_ring_rollback(None, addr(2), None, 2, 4, None) == NULL
    assert lib.ssd_verify_ring_rollback(addr(1), addr(1), None, 2, 4, None) == ALIAS
    assert lib.ssd_verify_ring_rollback(addr(1, 2), addr(2), None, 2, 4, None) == ALIGN


def test_seqpar_host_checks(lib):
    # total decay
    assert lib.ssd_seq_total_decay(addr(1), addr(2), addr(3), -1, 8, 4, None) == DIM
    assert lib.ssd_seq_total_decay(None, addr(2), addr(3), 1, 8, 4, None) == NULL
    assert lib.ssd_seq_total_decay(addr(1), addr(2), addr(1), 1, 8, 4, None) == ALIAS
    assert lib.ssd_seq_total_decay(addr(1, 2), addr(2), addr(3), 1, 8, 4, None) == ALIGN
    # combine
    assert lib.ssd_seq_combine(addr(1), addr(2), None, addr(3), -1, 1, 4, 16, 16, None) == DIM
    assert lib.ssd_seq_combine(addr(1), None, None, addr(3), 2, 1, 4, 16, 16, None) == NULL
    assert lib.ssd_seq_combine(addr(1), addr(2, 8), None, addr(3), 2, 1, 4, 16, 16, None) == ALIGN
    assert lib.ssd_seq_combine(addr(1), addr(2), None, addr(2), 2, 1, 4, 16, 16, None) == ALIAS
    assert lib.ssd_seq_combine(None, None, None, None, 0, 1, 4, 16, 16, None) == OK
    # apply
    call = lambda y=addr(1), f=addr(2), dt=addr(3), A=addr(4), C=addr(5), h=addr(6), \
        P=64, N=64, G=1, io=1: lib.ssd_seq_apply_state(y, f, dt, A, C, h, 1, 16, 4, P, N, G, io, None)
    assert call(P=24) == UNSUP
    assert call(N=512) == UNSUP
    assert call(G=3) == GROUPS
    assert call(io=5) == UNSUP
    assert call(C=None) == NULL
    assert call(C=addr(5, 8)) == ALIGN
    assert call(y=addr(5)) == ALIAS                  # y on C
    assert call(f=addr(6)) == ALIAS                  # final_state on h_in


def test_slice_state_host_checks(lib):
    # b=1, L=512, H=4, P=64, N=128, G=1, bf16: the dedicated kernel, 4 runs of one
    # 128-token segment per head (at most one run per segment, about 512 workgroups)
    need = lib.ssd_seq_slice_state_workspace_bytes(1, 512, 4, 64, 128, 1, 1)
    ws = lambda units, pn: ((units * pn * 4 + 255) // 256 + (units * 4 + 255) // 256) * 256
    assert need == ws(1 * 4 * 4, 64 * 128)
    # b=8, L=4096, H=32: 256 heads fill the 512 workgroups with 2 runs of 16 segments
    assert lib.ssd_seq_slice_state_workspace_bytes(8, 4096, 32, 64, 128, 1, 1) == ws(8 * 32 * 2, 64 * 128)
    # fp32 I/O takes the chunk-state kernel: 128-token chunks fit the LDS at N = 128
    assert lib.ssd_seq_slice_state_workspace_bytes(1, 512, 4, 64, 128, 1, 0) == ws(4 * 4, 64 * 128)
    assert lib.ssd_seq_slice_state_workspace_bytes(1, 0, 4, 64, 128, 1, 1) == 0
    bad = ctypes.c_size_t(-1).value
    assert lib.ssd_seq_slice_state_workspace_bytes(1, 512, 4, 48, 128, 1, 1) == bad   # P
    assert lib.ssd_seq_slice_state_workspace_bytes(1, 512, 4, 64, 128, 3, 1) == bad   # G
    assert lib.ssd_seq_slice_state_workspace_bytes(1, 512, 4, 64, 128, 1, 7) == bad   # dtype

    def call(x=addr(1), dt=addr(2), A=addr(3), B=addr(4), s=addr(5), a=addr(6), ws=addr(7),
             wsb=need, L=512, P=64, N=128, G=1, io=1, b=1):
        return lib.ssd_seq_slice_state(x, dt, A, B, s, a, b, L, 4, P, N, G, io, ws, wsb, None)
    assert call(b=-1) == DIM
    assert call(io=5) == UNSUP
    assert call(G=3) == GROUPS
    assert call(P=48) == UNSUP
    assert call(N=272) == UNSUP
    assert call(b=0, x=None, dt=None, A=None, B=None, s=None, a=None, ws=None) == OK
    assert call(x=None) == NULL
    assert call(s=None) == NULL
    assert call(B=addr(4, 8)) == ALIGN
    assert call(s=addr(5, 4)) == ALIGN
    assert call(ws=addr(7, 8)) == ALIGN
    assert call(ws=None) == WS
    assert call(wsb=need - 1) == WS
    assert call(s=addr(4)) == ALIAS                  # state on B
    assert call(a=addr(2)) == ALIAS                  # alpha on dt
    assert call(ws=addr(1)) == ALIAS                 # workspace on x
    assert call(a=addr(5)) == ALIAS                  # alpha on state
