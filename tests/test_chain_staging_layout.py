"""Host check of the swizzled LDS staging of the backward kernels (CPU only).

The loader waves of k_bwd_chain store 4-byte token pairs of the decay-weighted u (rows
p, 64 per head) and of v (rows n, N of them) transposed into rows of 64 tokens with a
row stride of 72 bf16 (36 dwords); k_bwd_chunk_bf stores dy the same way with a row
stride of 80 bf16.  Chunk c (8 tokens, 16 bytes) of row r sits at chunk position
c ^ ((r / 8) mod 8).  The MFMA operand reads take one whole chunk per lane (row
16 t + lane % 16, chunk 4 kk + lane / 16).  This replays both sides' index arithmetic
for N = 64 and 128: every read must find the token chunk it asks for, the decay
factors kept in the padding of row 0 must not be overwritten, and each pass of a
4-byte store (32 lanes, as the LDS serves it: measured with the bank-conflict counter)
must fall on 32 distinct banks of 4 bytes.
"""
import pytest

HP = 64
LOADERS = 256          # loader threads of a state walk (4 waves)


def swz8(r):
    return (r >> 3) & 7


def u_stores(stride, tid0=0):
    """(wave, j) -> [(dword offset, (row, first token))] for the u (or dy) stores."""
    out = {}
    for t in range(LOADERS):
        tpu, pgu = t >> 3, t & 7
        for j in range(8):
            p = 8 * pgu + j
            off = p * stride + 8 * ((tpu >> 2) ^ swz8(p)) + 2 * (tpu & 3)
            out.setdefault((t >> 6, j), []).append((off, (p, 2 * tpu)))
    return out


def v_stores(N, stride=72):
    NG = N // 8
    out = {}
    for t in range(LOADERS):
        for k in range((32 * NG + LOADERS - 1) // LOADERS):
            item = t + LOADERS * k
            if item >= 32 * NG:
                continue
            tp, ng = (item >> 3) & 31, (item & 7) | ((item >> 8) << 3)
            for j in range(8):
                n = 8 * ng + j
                off = n * stride + 8 * ((tp >> 2) ^ swz8(n)) + 2 * (tp & 3)
                out.setdefault((k, t >> 6, j), []).append((off, (n, 2 * tp)))
    return out


def placed(stores):
    cell = {}
    for lst in stores.values():
        for off, (row, tok) in lst:
            for e in range(2):
                assert off + e not in cell
                cell[off + e] = (row, tok + e)
    return cell


def check_reads(cell, rows, stride):
    for lane in range(64):
        r16, g4 = lane & 15, lane >> 4
        for kk in range(2):
            cc = 4 * kk + g4
            for t in range(rows // 16):
                r = 16 * t + r16
                base = r * stride + 8 * (cc ^ swz8(r))
                assert [cell[base + e] for e in range(8)] == [(r, 8 * cc + e) for e in range(8)]


@pytest.mark.parametrize("N", [64, 128])
def test_reads_find_their_chunks(N):
    cu, cv = placed(u_stores(72)), placed(v_stores(N))
    assert len(cu) == HP * 64 and len(cv) == N * 64
    assert not any(64 <= off < 72 for off in cu)        # row 0 padding: decay factors
    check_reads(cu, HP, 72)
    check_reads(cv, N, 72)
    cd = placed(u_stores(80))                            # dy^T of the chunk kernel
    check_reads(cd, HP, 80)


@pytest.mark.parametrize("N", [64, 128])
def test_every_store_pass_spans_32_banks(N):
    for stores in (u_stores(72), v_stores(N), u_stores(80)):
        for lst in stores.values():
            assert len(lst) == 64
            for half in (lst[:32], lst[32:]):
                assert len({(off // 2) % 32 for off, _ in half}) == 32


def gh_swz(e):
    return e ^ (((e >> 6) & 3) << 3)


@pytest.mark.parametrize("N", [64, 128])
def test_gh_copy_swizzle(N):
    """k_bwd_chunk_bf's LDS copy of a head's Gh^T tiles (accumulator layout: element
    (p, n) of tile (n / 16) * 4 + p / 16 at 4 (16 ((p % 16) / 4) + n % 16) + p % 4)
    is stored at gh_swz(e).  Both operand reads must find their elements, 16-byte copy
    pieces and 8-byte read pieces must stay whole, and the 2-byte row reads of a
    32-lane pass must not meet on a bank in more than one dword."""
    total = 64 * N
    assert sorted(gh_swz(e) for e in range(total)) == list(range(total))
    for k in range(total // 8):
        assert all(gh_swz(8 * k + i) == gh_swz(8 * k) + i for i in range(8))

    def elem(p, n):
        return ((n // 16) * 4 + p // 16) * 256 + 4 * (16 * ((p % 16) // 4) + n % 16) + p % 4

    where = {gh_swz(elem(p, n)): (p, n) for p in range(64) for n in range(N)}
    for q in range(4):
        for kq in range(N // 32):
            dwords = []
            for lane in range(64):
                rr, gg = lane & 15, lane >> 4
                m = rr >> 2
                base = ((2 * kq + (gg >> 1)) * 4 + q) * 256 + 4 * (16 * m + 8 * (gg & 1)) + (rr & 3)
                p, n0 = 16 * q + rr, 32 * kq + 8 * gg
                got = []
                for j in range(4):
                    e = base + 8 * (j ^ m)
                    got += [where[e], where[e + 4]]
                assert got == [(p, n0 + i) for i in range(8)]
                dwords.append((base + 8 * (0 ^ m)) // 2)
            for half in (dwords[:32], dwords[32:]):
                banks = {}
                for d in set(half):
                    banks.setdefault(d % 32, set()).add(d)
                assert max(len(v) for v in banks.values()) == 1
    for ntw in range(N // 16):                     # rows n, k = p: two 8-byte pieces
        for kp in range(2):
            for lane in range(64):
                r16, g4 = lane & 15, lane >> 4
                tile = ntw * 4 + 2 * kp + (g4 >> 1)
                l = r16 + 32 * (g4 & 1)
                n = 16 * ntw + r16
                p0 = 32 * kp + 8 * g4
                got = []
                for ll in (l, l + 16):
                    e = gh_swz(tile * 256 + 4 * ll)
                    assert gh_swz(tile * 256 + 4 * ll + 3) == e + 3
                    got += [where[e + i] for i in range(4)]
                assert got == [(p0 + i, n) for i in range(8)]
