"""CPU replay of the stream-K schedule (no GPU).

The stream-K launch (Osama et al., "Stream-K: Work-centric Parallel
Decomposition for Dense Matrix-Matrix Multiplication on the GPU") runs the
whole waves of output tiles data-parallel and deals the k-iterations of the
remaining tiles evenly over `workers` workgroups; a worker's range is cut at
tile boundaries into pieces, and a piece that is not a whole tile goes to slot
2w (the worker's first piece) or 2w + 1 (its last) of the workspace, where the
fix-up kernel sums the slots of each shared tile in worker order.  This test
replays that index arithmetic (workgroup -> iteration range, XCD remapping of
workgroup ids, tile order, slot choice, and the fix-up's worker range per tile)
and checks, for each shape and both stream-K tiles:

* the schedule's sizes equal what the library's own plan query reports;
* every (tile, k-iteration) is computed exactly once, with k inside [0, K);
* slots are unique and within the 2 * workers the workspace holds;
* for every shared tile the fix-up finds exactly the pieces written for it,
  contiguous in k and in worker order, covering all its iterations; a tile
  finished by a single worker has no pieces.
"""
import os
import random

import pytest

import fp32_gemm_08_amd as lib

OK = 0
WORKERS_MAX = 256
TILES = {256: (256, 256, 32), 128: (128, 128, 64)}   # BM, BN, k per iteration (one LDS stage)


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(lib.LIB_PATH):
        pytest.skip("libsgemm_f32.so not built")


def cdiv(a, b):
    return -(-a // b)


def xcd_remap(bid, total):
    return (bid & 7) * (total >> 3) + (bid >> 3) if total % 8 == 0 else bid


def group_order(t, nbm, nbn):
    per = 8 * nbn
    gi = t // per
    first = gi * 8
    gsz = min(nbm - first, 8)
    i = t - gi * per
    return first + i % gsz, i // gsz


def replay(M, N, K, tile):
    BM, BN, KT = TILES[tile]
    nbm, nbn = cdiv(M, BM), cdiv(N, BN)
    T, I = nbm * nbn, cdiv(K, KT)
    rem = T % WORKERS_MAX
    dp = T - rem
    P = 0 if rem == 0 else min(rem * I, WORKERS_MAX)
    st, kid, q_dp, q_skt, q_workers, q_bytes = lib.sgemm_f32_streamk_plan(tile, M, N, K, 0)
    assert st == OK and (q_dp, q_skt, q_workers) == (dp, rem, P), (M, N, K, tile)
    assert q_bytes == 2 * P * BM * BN * 4
    S, base = rem * I, dp * I
    cover, slots = set(), {}
    for bid in range(dp + P):
        w = -1
        if bid < dp:
            it = xcd_remap(bid, dp) * I
            end = it + I
        else:
            raw = bid - dp
            w = (raw & 7) * (P >> 3) + (raw >> 3) if P % 8 == 0 else raw
            it, end = base + w * S // P, base + (w + 1) * S // P
        assert it < end, ("empty workgroup", bid)
        first = it
        while it < end:
            t = it // I
            kb = it - t * I
            ke = min(I, kb + (end - it))
            tm, tn = group_order(t, nbm, nbn)
            assert 0 <= tm < nbm and 0 <= tn < nbn
            assert 0 <= kb * KT < min(K, ke * KT) <= K
            for k in range(kb, ke):
                assert (tm, tn, k) not in cover, ("computed twice", tm, tn, k)
                cover.add((tm, tn, k))
            if not (kb == 0 and ke == I):
                assert w >= 0, "a data-parallel workgroup wrote a piece"
                slot = 2 * w + (0 if it == first else 1)
                assert 0 <= slot < 2 * P and slot not in slots
                slots[slot] = (t, kb, ke)
            it += ke - kb
    assert len(cover) == T * I, "every (tile, k-iteration) computed"
    for j in range(rem):
        lo, hi = j * I, j * I + I - 1
        w_lo, w_hi = ((lo + 1) * P - 1) // S, ((hi + 1) * P - 1) // S
        pieces = [v for v in slots.values() if v[0] == dp + j]
        if w_lo == w_hi:
            assert not pieces, ("a whole tile left pieces", j)
            continue
        k = 0
        for w in range(w_lo, w_hi + 1):
            slot = 2 * w + (0 if lo <= w * S // P else 1)
            t, kb, ke = slots[slot]
            assert t == dp + j and kb == k, ("fix-up order", j, w)
            k = ke
        assert k == I and len(pieces) == w_hi - w_lo + 1
    return dp, rem, P


FIXED = [(4608, 4608, 4608), (3000, 3000, 3000), (2304, 2304, 8192), (1536, 1536, 4096), (1024, 1024, 1024),
         (257 * 256, 256, 100), (256, 256, 33), (1, 1, 1), (300, 300, 31), (6144, 6144, 2048), (4096, 4096, 4096),
         (4097, 4096, 64), (100, 5000, 7), (3584, 3584, 3584)]
_rng = random.Random(1)
RANDOM = [(_rng.randint(1, 6000), _rng.randint(1, 6000), _rng.randint(1, 5000)) for _ in range(40)]


@pytest.mark.parametrize("tile", [256, 128])
@pytest.mark.parametrize("shape", FIXED + RANDOM, ids=lambda s: "x".join(map(str, s)))
def test_streamk_schedule(shape, tile):
    replay(*shape, tile)


def test_replay_sees_a_stream_k_part():
    # the fixed shapes exercise shared tiles (pieces and fix-up), not only
    # whole waves
    assert replay(4608, 4608, 4608, 256)[1] == 324 - 256
    assert replay(300, 300, 31, 128)[2] > 0
