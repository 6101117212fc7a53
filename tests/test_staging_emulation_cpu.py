"""CPU emulation of the MFMA kernel's direct global->LDS staging (no GPU).

Every wavefront lane of the MFMA kernel loads W = 4 floats (one 16-byte
global_load_lds_dwordx4, from any 4-byte aligned address: leading dimensions
need not be multiples of 4) of one k-tile into LDS.  Its source offset follows the kernel's
staging code: LDS float e of a k-contiguous tile row holds logical chunk
(e % BK / 4) XOR swz(row) of that row; rows past M (and, for op(B) = B^T, past
N) are clamped to the last valid row on edge tiles, and op(B) = B columns past
N to the last whole group of W columns.  This test replays that arithmetic for
every wavefront and lane of each tile geometry the library launches and checks:

* bounds: every source address lies inside the operand's M x lda (or K x ldb,
  N x ldb) allocation, interior and edge tiles, aligned and unaligned ld;
* coverage: every LDS float of the stage is written exactly once;
* content: the LDS float the MFMA fragment reads for logical (row, k) holds
  A[row, k] (op(B)(k, col) for B) wherever row < M (col < N) -- clamped rows
  and columns only feed outputs the masked epilogue drops.

Operands are filled with their own flat addresses, so content checks compare
addresses.  The geometries are the kernel configurations in use: 64 x 64 with
4 wavefronts, 64 x 64, 128 x 128 and 128 x 64 with 8 wavefronts as two
k-slices, 256 x 256 with 8 wavefronts, and 32 x 32 with 4 wavefronts as four
k-slices, BK 32.
"""
import numpy as np
import pytest


def swz(r, cpr):
    return ((r >> 1) ^ (r >> 2)) & 3 if cpr == 4 else (r ^ (r >> 3)) & 7


def stage_and_check(BM, BN, BK, NW, KS, trans_b, edge, M, N, K, lda, ldb, m0, n0, kt, write_swz=swz):
    cpr = BK // 4
    a_sz, b_sz = BM * BK, BK * BN
    slice_sz = a_sz + b_sz
    kt_len = KS * BK
    W = 4
    bw = 64 * W
    a_n, b_n = KS * a_sz // bw // NW, KS * b_sz // bw // NW
    assert a_n * bw * NW == KS * a_sz and b_n * bw * NW == KS * b_sz
    a_bps, b_bps = a_sz // bw, b_sz // bw
    A = np.arange(M * lda, dtype=np.int64).reshape(M, lda)
    b_rows = N if trans_b else K
    B = np.arange(b_rows * ldb, dtype=np.int64).reshape(b_rows, ldb) + 10**12
    lds = np.full(KS * slice_sz, -1, dtype=np.int64)
    writes = np.zeros(KS * slice_sz, dtype=np.int64)

    def kcontig(e, sl, ld, last):
        r, q = e // BK, e % BK
        c = (q // 4) ^ write_swz(r, cpr)
        rg = min(r, last) if edge else r
        return rg * ld + sl * BK + 4 * c + q % 4

    for wave in range(NW):
        for lane in range(64):
            for j in range(a_n):
                b = wave * a_n + j
                sl, lb = b // a_bps, b % a_bps
                off = kcontig(lb * bw + W * lane, sl, lda, M - 1 - m0)
                base = m0 * lda + kt * kt_len
                for w in range(W):
                    addr = base + off + w
                    assert 0 <= addr < M * lda, ("A out of bounds", wave, lane, j, addr)
                    p = sl * slice_sz + lb * bw + W * lane + w
                    lds[p] = A.flat[addr]
                    writes[p] += 1
            for j in range(b_n):
                b = wave * b_n + j
                sl, lb = b // b_bps, b % b_bps
                e = lb * bw + W * lane
                if trans_b:
                    off = kcontig(e, sl, ldb, N - 1 - n0)
                    base = n0 * ldb + kt * kt_len
                else:
                    col = e % BN
                    cg = min(col, N - W - n0) if edge else col
                    off = (sl * BK + e // BN) * ldb + cg
                    base = n0 + kt * kt_len * ldb
                for w in range(W):
                    addr = base + off + w
                    assert 0 <= addr < b_rows * ldb, ("B out of bounds", wave, lane, j, addr)
                    p = sl * slice_sz + a_sz + lb * bw + W * lane + w
                    lds[p] = B.flat[addr]
                    writes[p] += 1
    assert np.all(writes == 1), "every LDS float written exactly once"
    for sl in range(KS):
        for r in range(BM):
            for k in range(BK):
                p = sl * slice_sz + r * BK + 4 * ((k // 4) ^ swz(r, cpr)) + k % 4
                if m0 + r < M:
                    assert lds[p] == A[m0 + r, kt * kt_len + sl * BK + k], ("A content", sl, r, k)
        for n in range(BN):
            for k in range(BK):
                kk = kt * kt_len + sl * BK + k
                if n0 + n >= N:
                    continue
                if trans_b:
                    p = sl * slice_sz + a_sz + n * BK + 4 * ((k // 4) ^ swz(n, cpr)) + k % 4
                    assert lds[p] == B[n0 + n, kk], ("B^T content", sl, n, k)
                else:
                    p = sl * slice_sz + a_sz + k * BN + n
                    assert lds[p] == B[kk, n0 + n], ("B content", sl, n, k)


GEOMETRIES = [(64, 64, 32, 4, 1), (64, 64, 32, 8, 2), (128, 128, 32, 8, 2), (256, 256, 32, 8, 1), (32, 32, 32, 4, 4),
              (128, 64, 32, 8, 2)]


@pytest.mark.parametrize("geo", GEOMETRIES, ids=lambda g: f"{g[0]}x{g[1]}_w{g[3]}_ks{g[4]}")
@pytest.mark.parametrize("trans_b", [False, True])
@pytest.mark.parametrize("pad", [(4, 0), (1, 3), (3, 1)], ids=["aligned", "unaligned13", "unaligned31"])
def test_direct_staging(geo, trans_b, pad):
    BM, BN, BK, NW, KS = geo
    pa, pb = pad
    K = 4 * KS * BK
    # an interior tile; leading dimensions a multiple of 4 or not
    M, N = 3 * BM, 3 * BN
    stage_and_check(BM, BN, BK, NW, KS, trans_b, False, M, N, K, K + pa, (K if trans_b else N) + pb, BM, BN, 1)
    # an edge tile in M and N (the edge path of op(B) = B needs N % 4 == 0)
    M2, N2 = BM + 37, BN + (21 if trans_b else 20)
    stage_and_check(BM, BN, BK, NW, KS, trans_b, True, M2, N2, K, K + pb, (K if trans_b else N2) + pa, BM, BN, 2)
    # an edge tile with a single valid row and column group
    N3 = BN + (1 if trans_b else 4)
    stage_and_check(BM, BN, BK, NW, KS, trans_b, True, BM + 1, N3, K, K + pa, (K if trans_b else N3) + pb, BM, BN,
                    0)


def test_emulation_catches_planted_mistakes():
    # the checks are not vacuous: a writer swizzle that differs from the
    # reader's fails on content, and an edge tile staged without the row clamp
    # fails on bounds
    with pytest.raises(AssertionError, match="content"):
        stage_and_check(64, 64, 32, 4, 1, True, False, 192, 192, 128, 132, 132, 64, 64, 1,
                        write_swz=lambda r, cpr: 0)
    with pytest.raises(AssertionError, match="out of bounds"):
        stage_and_check(64, 64, 32, 4, 1, True, False, 64 + 37, 64 + 21, 128, 128, 128, 64, 64, 2)
