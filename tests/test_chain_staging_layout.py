"""Host check of the LDS staging layout of the backward state walks (CPU only).

The loader waves of k_bwd_chain store 4-byte token pairs of the decay-weighted u
(rows p, 64 per head) and of v (rows n, N of them) transposed into rows of 64 tokens
with a row stride of 72 bf16 (36 dwords); chunk c (8 tokens, 16 bytes) of row r sits
at chunk position c ^ f(r), with f(r) = 2 ((r / 16) mod 4) for u and
(r / 16 or 2 (r / 16), by state size) mod 8 for v.  The state waves read 16-byte MFMA
operands (row 16 t + lane % 16, chunk 4 kk + lane / 16).  This replays both sides'
index arithmetic for N = 64 and 128: every read must find the token chunk it asks
for, the decay factors kept in the padding of row 0 must not be overwritten, and the
64 lanes of each store must fall on 64 distinct banks (64 banks of 4 bytes).
"""
import pytest

HP, RSA = 64, 72
LOADERS = 256          # loader threads (4 waves)


def swz_u(r):
    return 2 * ((r >> 4) & 3)


def swz_v(r, NG):
    return (r >> 4 if NG >= 16 else 2 * (r >> 4)) & 7


def u_stores():
    """(wave, j) -> list of (element offset, (p, token)) for the u staging stores."""
    out = {}
    for tid in range(LOADERS):
        tpu, pgu = tid >> 3, tid & 7
        for j in range(8):
            p = 8 * pgu + j
            off = p * RSA + 8 * ((tpu >> 2) ^ swz_u(p)) + 2 * (tpu & 3)
            out.setdefault((tid >> 6, j), []).append((off, (p, 2 * tpu)))
    return out


def v_stores(N):
    NG = N // 8
    out = {}
    for tid in range(LOADERS):
        for k in range((32 * NG + LOADERS - 1) // LOADERS):
            item = tid + LOADERS * k
            if item >= 32 * NG:
                continue
            tp, ng = item // NG, item % NG
            for j in range(8):
                n = 8 * ng + j
                off = n * RSA + 8 * ((tp >> 2) ^ swz_v(n, NG)) + 2 * (tp & 3)
                out.setdefault((k, tid >> 6, j), []).append((off, (n, 2 * tp)))
    return out


def placed(stores):
    cell = {}
    for lst in stores.values():
        for off, (row, tok) in lst:
            for e in range(2):
                assert off + e not in cell
                cell[off + e] = (row, tok + e)
    return cell


@pytest.mark.parametrize("N", [64, 128])
def test_reads_find_their_chunks(N):
    NG = N // 8
    cu, cv = placed(u_stores()), placed(v_stores(N))
    assert len(cu) == HP * 64 and len(cv) == N * 64
    assert not any(64 <= off < RSA for off in cu)        # row 0 padding: decay factors
    for lane in range(64):
        r16, g4 = lane & 15, lane >> 4
        for kk in range(2):
            cc = 4 * kk + g4
            for sw in range(4):                          # u: state wave sw, rows 16 sw + r16
                p = 16 * sw + r16
                base = p * RSA + 8 * (cc ^ swz_u(16 * sw))
                assert [cu[base + e] for e in range(8)] == [(p, 8 * cc + e) for e in range(8)]
            for nt in range(N // 16):                    # v: column tile nt
                n = 16 * nt + r16
                base = n * RSA + 8 * (cc ^ swz_v(16 * nt, NG))
                assert [cv[base + e] for e in range(8)] == [(n, 8 * cc + e) for e in range(8)]


@pytest.mark.parametrize("N", [64, 128])
def test_every_store_spans_all_banks(N):
    for stores in (u_stores(), v_stores(N)):
        for lst in stores.values():
            banks = {(off // 2) % 64 for off, _ in lst}
            assert len(lst) == 64 and len(banks) == 64
