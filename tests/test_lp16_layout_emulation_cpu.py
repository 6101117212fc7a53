"""CPU replay of the two-pass mixed-precision index arithmetic (no GPU).

The rounding passes store each operand as 16-bit "slabs": slab s holds
k in [32s, 32s + 32) of every (padded) row, 64 bytes per row, rows
consecutive, so element (row, k) of an Rp x Kp operand sits at 16-bit index
((k // 32) * Rp + row) * 32 + k % 32 and a 16-row block of a slab is 1 KB of
contiguous memory.  The GEMM pass loads such 1 KB blocks straight into LDS,
each lane 16 bytes: lane l of a block covers row 16b + l // 4 and stores that
row's logical chunk (l % 4) XOR swz(row) at physical chunk l % 4; a fragment
read of logical chunk c then reads physical chunk c XOR swz(row).

This test replays, on small shapes, every work-item of:
* the row rounding pass (k-contiguous source: A, or B stored N x K),
* the transposing rounding pass (B stored K x N: a 64 x 64 LDS tile),
* the GEMM pass's direct loads and fragment reads for both tile geometries,
and checks that every write lands once inside the workspace, every source
read stays inside its matrix (zero written past R rows and K columns), and
every fragment read sees the element it multiplies.  Values are replaced by
their (row, k) coordinates.
"""
import numpy as np
import pytest

QK = 32


def swz(r):
    return ((r >> 1) ^ (r >> 2)) & 3


def up(v, m):
    return -(-v // m) * m


def slab_index(row, k, Rp):
    return ((k // QK) * Rp + row) * QK + k % QK


def round_rows(R, K, Rp, Kp):
    """Items i = (slab * Rp + r) * 4 + c: 8 values at k = 32 slab + 8c of row r,
    written to 16-bit index 8i.  Returns dst[Rp*Kp] of (row, k) codes, -1 for zero."""
    dst = np.full(Rp * Kp, -2, dtype=np.int64)
    for i in range(Rp * (Kp // 8)):
        c, rs = i & 3, i >> 2
        r, slab = rs % Rp, rs // Rp
        k = QK * slab + 8 * c
        for q in range(8):
            assert dst[8 * i + q] == -2, "written twice"
            inside = r < R and k + q < K
            dst[8 * i + q] = r * 100000 + (k + q) if inside else -1
            assert 8 * i + q == slab_index(r, k + q, Rp)
    assert np.all(dst != -2), "every element written"
    return dst


def round_transpose(K, N, Np, Kp):
    """B is K x N; grid (Np / 64, ceil(Kp / 64)) of 256 work-items; the result
    is r(B^T) in the slab layout with Np rows."""
    dst = np.full(Np * Kp, -2, dtype=np.int64)
    for bx in range(Np // 64):
        for by in range(-(-Kp // 64)):
            n0, k0 = 64 * bx, 64 * by
            t = np.full((64, 64), -3, dtype=np.int64)
            for tid in range(256):
                for i in range(4):
                    e = tid + 256 * i
                    kr, nc = e // 16, 4 * (e % 16)
                    k, n = k0 + kr, n0 + nc
                    for q in range(4):
                        assert t[nc + q, kr] == -3
                        t[nc + q, kr] = n + q + 100000 * k if (k < K and n + q < N) else -1
            assert np.all(t != -3)
            for tid in range(256):
                for i in range(2):
                    e = tid + 256 * i
                    sl, nr, c = e // 256, (e // 4) % 64, e % 4
                    n, k = n0 + nr, k0 + QK * sl + 8 * c
                    if n < Np and k < Kp:
                        base = ((k // QK) * Np + n) * QK + 8 * c
                        for q in range(8):
                            assert dst[base + q] == -2, "written twice"
                            v = t[nr, QK * sl + 8 * c + q]
                            # stored as (row n, k) like the row pass's codes
                            dst[base + q] = -1 if v == -1 else n * 100000 + (k + q)
                            assert v == -1 or v == n + 100000 * (k + q)
                            assert base + q == slab_index(n, k + q, Np)
    assert np.all(dst != -2), "every element written"
    return dst


def gemm_stage(A16, B16, Mp, Np, Kp, BM, BN, WGM, WGN, m0, n0, kt):
    """One stage (k-tile kt) of the direct loads of tile (m0, n0), then every
    fragment read of it, in (row, k) codes."""
    NW = WGM * WGN
    NA, NB = BM // 16 // NW, BN // 16 // NW
    lds = np.full((BM + BN) * QK, -2, dtype=np.int64)   # 16-bit units
    for w in range(NW):
        for lane in range(64):
            for j in range(NA):
                r = 16 * (w * NA + j) + lane // 4
                src = (m0 + r) * QK + 8 * ((lane & 3) ^ swz(r)) + kt * Mp * QK
                dst = (w * NA + j) * 512 + lane * 8
                assert 0 <= src and src + 8 <= Mp * Kp
                assert np.all(lds[dst:dst + 8] == -2)
                lds[dst:dst + 8] = A16[src:src + 8]
            for j in range(NB):
                r = 16 * (w * NB + j) + lane // 4
                src = (n0 + r) * QK + 8 * ((lane & 3) ^ swz(r)) + kt * Np * QK
                dst = BM * QK + (w * NB + j) * 512 + lane * 8
                assert 0 <= src and src + 8 <= Np * Kp
                assert np.all(lds[dst:dst + 8] == -2)
                lds[dst:dst + 8] = B16[src:src + 8]
    assert np.all(lds != -2), "every LDS element written once"
    WM, WN = BM // WGM, BN // WGN
    for w in range(NW):
        wm, wn = w // WGN, w % WGN
        for lane in range(64):
            l32, hi = lane & 31, lane >> 5
            for ks in range(2):
                c = 2 * ks + hi
                for fm in range(WM // 32):
                    r = wm * WM + fm * 32 + l32
                    got = lds[r * QK + 8 * (c ^ swz(r)):][:8]
                    for q in range(8):
                        assert got[q] == A16[slab_index(m0 + r, kt * QK + 8 * c + q, Mp)]
                for fn in range(WN // 32):
                    r = wn * WN + fn * 32 + l32
                    got = lds[BM * QK + r * QK + 8 * (c ^ swz(r)):][:8]
                    for q in range(8):
                        assert got[q] == B16[slab_index(n0 + r, kt * QK + 8 * c + q, Np)]


@pytest.mark.parametrize("R,K,Rp", [(5, 7, 128), (130, 33, 256), (128, 64, 128), (1, 1, 128)])
def test_row_rounding(R, K, Rp):
    round_rows(R, K, Rp, up(K, QK))


@pytest.mark.parametrize("K,N,Np", [(7, 5, 128), (33, 130, 256), (64, 128, 128), (100, 64, 128)])
def test_transposing_rounding_matches_row_rounding_of_bt(K, N, Np):
    # r(B^T) written by the transposing pass equals what the row pass writes
    # for B stored N x K
    Kp = up(K, QK)
    assert np.array_equal(round_transpose(K, N, Np, Kp), round_rows(N, K, Np, Kp))


@pytest.mark.parametrize("geo", [(256, 256, 4, 4), (256, 256, 4, 2), (128, 128, 2, 4), (128, 128, 2, 2)],
                         ids=["256x256_w4x4", "256x256_w4x2", "128x128_w2x4", "128x128_w2x2"])
def test_gemm_staging_and_fragments(geo):
    BM, BN, WGM, WGN = geo
    M, N, K = BM + 17, BN + 3, 70            # edge rows and columns, a k tail
    Mp, Np, Kp = up(M, BM), up(N, BN), up(K, QK)
    A16, B16 = round_rows(M, K, Mp, Kp), round_rows(N, K, Np, Kp)
    for (m0, n0) in [(0, 0), (BM, BN)]:
        for kt in range(Kp // QK):
            gemm_stage(A16, B16, Mp, Np, Kp, BM, BN, WGM, WGN, m0, n0, kt)


def test_replay_catches_a_planted_mistake():
    # a loader that ignores the swizzle stores chunks where the reader does
    # not look: the fragment check must fail
    global swz
    keep = swz
    A16 = round_rows(128, 32, 128, 32)
    B16 = round_rows(128, 32, 128, 32)
    try:
        calls = {"n": 0}

        def loader_only_swz(r):
            calls["n"] += 1
            return 0 if calls["n"] <= 128 * 2 * 4 else keep(r)   # the first stage's loads use no swizzle
        swz = loader_only_swz
        with pytest.raises(AssertionError):
            gemm_stage(A16, B16, 128, 128, 32, 128, 128, 2, 2, 0, 0, 0)
    finally:
        swz = keep
