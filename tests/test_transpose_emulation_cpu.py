"""CPU replay of the transpose kernels' index arithmetic (no GPU).

The GPU tests check the transpose bit for bit with canaries around the
destination, which catches stray writes; this replay also bounds every read.
For each launch shape the library uses -- the 128 x 128 padded (or unpadded)
LDS tile in its persistent pipelined form (256 work-items, at most 512
workgroups) and its streaming form (512 work-items, grouped tile order, 4- or
1-float loads), the 64 x 64 tile for small matrices, the narrow kernel (one
work-item per destination element) and the naive kernel -- it recomputes every
work-item's source and destination offsets, over grids smaller than the tile
count too (persistent loops), and checks:

* every source read lies inside the (rows - 1) * ld_src + cols floats of the
  source and every write inside the (cols - 1) * ld_dst + rows of the
  destination; full tiles need no mask;
* every LDS float of a tile (without the padding column) is written once;
* every destination element dst(j, i), j < cols, i < rows, is written once.
"""
import numpy as np
import pytest


def tile_of(t, tiles_r, tiles_c, group, T):
    if group == 0:
        tr, tc = t // tiles_c, t % tiles_c
    else:
        per = group * tiles_c
        g, rem = t // per, t % per
        gh = min(tiles_r - g * group, group)
        tr, tc = g * group + rem % gh, rem // gh
    return tr * T, tc * T


def run_tile(T, TH, PAD, V4, rows, cols, lsrc, ldst, r0, c0, written, mask=True):
    P, NW = T + PAD, TH // 64
    rpi = 4 if V4 else 1
    loads, stores = (T // rpi) * (T // 64) // NW, T * (T // 64) // NW
    full = r0 + T <= rows and c0 + T <= cols
    src_n, dst_n = (rows - 1) * lsrc + cols, (cols - 1) * ldst + rows
    lane = np.arange(64)
    cover = np.zeros(T * P, np.int32)
    for w in range(NW):
        for i in range(loads):
            ch = w + NW * i
            if V4:
                r, c = (ch // (T // 64)) * 4 + (lane >> 4), (ch % (T // 64)) * 64 + 4 * (lane & 15)
            else:
                r, c = np.full(64, ch // (T // 64)), (ch % (T // 64)) * 64 + lane
            for q in range(rpi if V4 else 1):
                inside = (r0 + r < rows) & (c0 + c + q < cols)
                if full:
                    assert np.all(inside), "a full tile reads outside the source"
                ok = np.ones(64, bool) if full else inside
                off = (r0 + r) * lsrc + (c0 + c + q)
                assert np.all(off[ok] >= 0) and np.all(off[ok] < src_n), "read out of bounds"
                np.add.at(cover, r * P + c + q, 1)
    assert np.all(cover.reshape(T, P)[:, :T] == 1), "LDS tile written once"
    for w in range(NW):
        for i in range(stores):
            ch = w + NW * i
            j, r = ch // (T // 64), (ch % (T // 64)) * 64 + lane
            inside = (c0 + j < cols) & (r0 + r < rows)
            if full:
                assert np.all(inside)
            ok = np.ones(64, bool) if (full or not mask) else inside
            off = (c0 + j) * ldst + (r0 + r)
            assert np.all(off[ok] >= 0) and np.all(off[ok] < dst_n), "write out of bounds"
            assert np.all(r * P + j < T * P)
            if np.any(ok):
                np.add.at(written, (np.full(int(ok.sum()), c0 + j), (r0 + r)[ok]), 1)


def tile_launch(rows, cols, lsrc, ldst, T, TH, PAD, V4, group, cap):
    tiles_r, tiles_c = -(-rows // T), -(-cols // T)
    tiles = tiles_r * tiles_c
    written = np.zeros((cols, rows), np.int32)
    seen = set()
    for b in range(min(tiles, cap)):
        for t in range(b, tiles, min(tiles, cap)):
            r0, c0 = tile_of(t, tiles_r, tiles_c, group, T)
            seen.add((r0, c0))
            run_tile(T, TH, PAD, V4, rows, cols, lsrc, ldst, r0, c0, written)
    assert len(seen) == tiles, "every tile visited"
    assert np.all(written == 1), "every destination element written once"


def narrow_launch(rows, cols, lsrc, ldst, cap):
    tiles_i = -(-rows // 64)
    tiles = tiles_i * -(-cols // 16)
    written = np.zeros((cols, rows), np.int32)
    src_n, dst_n = (rows - 1) * lsrc + cols, (cols - 1) * ldst + rows
    tid = np.arange(256)
    for b in range(min(tiles, cap)):
        for t in range(b, tiles, min(tiles, cap)):
            j0, i = (t // tiles_i) * 16, (t % tiles_i) * 64 + (tid & 63)
            for k in range(4):
                j = j0 + (tid >> 6) + 4 * k
                ok = (i < rows) & (j < cols)
                assert np.all((i * lsrc + j)[ok] < src_n) and np.all((j * ldst + i)[ok] < dst_n)
                np.add.at(written, (j[ok], i[ok]), 1)
    assert np.all(written == 1)


def naive_launch(rows, cols, lsrc, ldst, cap):
    tiles_c = -(-cols // 64)
    tiles = tiles_c * -(-rows // 16)
    written = np.zeros((cols, rows), np.int32)
    src_n, dst_n = (rows - 1) * lsrc + cols, (cols - 1) * ldst + rows
    tid = np.arange(256)
    for b in range(min(tiles, cap)):
        for t in range(b, tiles, min(tiles, cap)):
            r0, c = (t // tiles_c) * 16, (t % tiles_c) * 64 + (tid & 63)
            for i in range(4):
                r = r0 + (tid >> 6) + 4 * i
                ok = (c < cols) & (r < rows)
                assert np.all((r * lsrc + c)[ok] < src_n) and np.all((c * ldst + r)[ok] < dst_n)
                np.add.at(written, (c[ok], r[ok]), 1)
    assert np.all(written == 1)


TILE_SHAPES = [(1, 1), (1, 300), (300, 1), (128, 128), (127, 129), (129, 127), (200, 64), (64, 200),
               (301, 517), (130, 3), (3, 130), (1025, 260)]


@pytest.mark.parametrize("shape", TILE_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("pad", [0, 1])
def test_pipelined_and_streaming_tiles(shape, pad):
    rows, cols = shape
    tile_launch(rows, cols, cols + 3, rows + 5, 128, 256, pad, False, 0, 512)   # pipelined
    tile_launch(rows, cols, cols + 3, rows + 5, 128, 256, pad, False, 0, 3)     # ... on a small grid
    tile_launch(rows, cols, cols + 3, rows + 5, 128, 512, pad, False, 8, 1 << 20)   # streaming, 1-float loads
    tile_launch(rows, cols, cols + 4, rows + 5, 128, 512, pad, True, 8, 1 << 20)    # streaming, 4-float loads
    tile_launch(rows, cols, cols + 3, rows + 5, 128, 512, pad, False, 8, 5)


@pytest.mark.parametrize("shape", [(1, 1), (65, 63), (130, 3), (3, 130), (300, 333)], ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("pad", [0, 1])
def test_small_tiles(shape, pad):
    rows, cols = shape
    tile_launch(rows, cols, cols + 3, rows + 5, 64, 256, pad, False, 0, 1 << 20)
    tile_launch(rows, cols, cols + 3, rows + 5, 64, 256, pad, False, 0, 7)


@pytest.mark.parametrize("shape", TILE_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_narrow_and_naive(shape):
    rows, cols = shape
    for cap in (1 << 20, 3):
        narrow_launch(rows, cols, cols + 1, rows + 2, cap)
        naive_launch(rows, cols, cols + 1, rows + 2, cap)


def test_replay_catches_a_planted_mistake():
    # an edge tile stored without its mask writes past the destination
    with pytest.raises(AssertionError, match="write out of bounds"):
        run_tile(128, 256, 1, False, 100, 90, 93, 105, 0, 0, np.zeros((90, 100), np.int32), mask=False)
