"""GPU parity of the transpose kernels against the transpose oracle, through the C ABI.

Bar: bit-exact.  A transpose moves bits, so every destination element must equal
the oracle's element bit for bit (NaN payloads, signed zeros and subnormals
included), and nothing outside the destination window may change (guard rows
above and below it, padding columns beside it, all holding a canary pattern).
Full compares at every size the oracle finishes in seconds (4096 x 4096, the
measured workload, included); the grid-loop case compares sampled row blocks,
each of which the oracle transposes on its own.
"""
import numpy as np
import pytest

import fp32_gemm_08_amd as lib
from fp32_gemm_08_amd.inputs import TRANSPOSE_CONFIGS, make_transpose_config, make_transpose_input
from oracle import transpose as oracle_transpose

from gpu_helpers import say

pytestmark = pytest.mark.gpu

ALGOS = ["naive", "lds", "lds_nopad", "narrow", "auto"]
CANARY_BITS = np.uint32(0x7FBADBAD)  # a signalling NaN no input here contains
GUARD = 2


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert lib.sgemm_f32_version()  # the HIP library must load: no fallback exists


def _canary(shape):
    return np.full(shape, CANARY_BITS, dtype=np.uint32).view(np.float32)


def run_transpose(src, rows, cols, algo, ld_dst=None, src_offset=0, dst_offset=0, stream=None):
    """Transpose the rows x cols matrix held in ``src`` (rows x ld_src storage) on
    the GPU; returns (status, dst window as a (cols, rows) float32 array).  Guard
    rows and padding columns of the destination are checked for the canary."""
    import torch

    dev = torch.device("cuda", 0)
    ld_src = src.shape[1]
    ld_dst = max(1, rows) if ld_dst is None else ld_dst
    full = _canary((cols + 2 * GUARD, ld_dst))
    dS = torch.from_numpy(np.concatenate([np.zeros(src_offset, np.float32), src.ravel()])).to(dev)
    dD = torch.from_numpy(np.concatenate([_canary(dst_offset), full.ravel()])).to(dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    algo_id = lib.TRANSPOSE_ALGO[algo]
    say(f"transpose algo={algo} rows={rows} cols={cols} ld_src={ld_src} ld_dst={ld_dst} "
        f"src_offset={src_offset} dst_offset={dst_offset}")
    st = lib.sgemm_f32_transpose_algo(algo_id, rows, cols, dS.data_ptr() + 4 * src_offset, ld_src,
                                      dD.data_ptr() + 4 * (dst_offset + GUARD * ld_dst), ld_dst,
                                      s.cuda_stream)
    torch.cuda.synchronize()
    out = dD.cpu().numpy()
    head = out[:dst_offset]
    out = out[dst_offset:].reshape(cols + 2 * GUARD, ld_dst)
    bits = out.view(np.uint32)
    assert np.all(head.view(np.uint32) == CANARY_BITS), "write before the destination"
    assert np.all(bits[:GUARD] == CANARY_BITS), "write above the destination"
    assert np.all(bits[GUARD + cols:] == CANARY_BITS), "write below the destination"
    if ld_dst > rows:
        assert np.all(bits[GUARD:GUARD + cols, rows:] == CANARY_BITS), "write into row padding"
    return st, out[GUARD:GUARD + cols, :rows]


def assert_bits_equal(got, want, what):
    g, w = np.ascontiguousarray(got).view(np.uint32), np.ascontiguousarray(want).view(np.uint32)
    assert g.shape == w.shape, f"{what}: shape {g.shape} vs {w.shape}"
    bad = np.argwhere(g != w)
    say(f"{what}: mismatches={len(bad)}")
    assert len(bad) == 0, f"{what}: {len(bad)} mismatches, first at {tuple(bad[0])}"


# Square, single row/column, narrow (AUTO's element kernels), tile edges +-1,
# the persistent pipelined launch with ragged tiles, and (6000 x 6100, 2256
# tiles) the one-tile-per-workgroup launch with ragged tiles.
SHAPES = [(1, 1), (1, 1000), (1000, 1), (31, 300), (300, 31), (64, 64), (127, 129), (129, 127),
          (128, 192), (200, 64), (64, 200), (1000, 1017), (4097, 4095), (6000, 6100)]


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("rows,cols", SHAPES)
def test_shapes_bit_exact_with_special_values(algo, rows, cols):
    # Padded storage on both sides and special bit patterns in the data.
    src = make_transpose_input(rows, cols, seed=rows * 7 + cols, ld_src=cols + 3, specials=True)
    st, got = run_transpose(src, rows, cols, algo, ld_dst=rows + 5)
    assert st == 0
    assert_bits_equal(got, oracle_transpose(src, rows, cols), f"{algo} {rows}x{cols}")


@pytest.mark.parametrize("name", sorted(TRANSPOSE_CONFIGS))
@pytest.mark.parametrize("algo", ["lds", "auto", "naive"])
def test_configs_full(name, algo):
    cfg = TRANSPOSE_CONFIGS[name]
    rows, cols = cfg["rows"], cfg["cols"]
    src = make_transpose_config(name)
    st, got = run_transpose(src, rows, cols, algo)
    assert st == 0
    assert_bits_equal(got, oracle_transpose(src, rows, cols), f"{algo} {name}")


@pytest.mark.parametrize("algo", ALGOS)
def test_misaligned_pointers_and_odd_strides(algo):
    rows, cols = 301, 517
    src = make_transpose_input(rows, cols, seed=9, ld_src=cols + 1)
    st, got = run_transpose(src, rows, cols, algo, ld_dst=rows + 2, src_offset=1, dst_offset=3)
    assert st == 0
    assert_bits_equal(got, oracle_transpose(src, rows, cols), f"{algo} misaligned")


@pytest.mark.parametrize("algo,rows", [("lds", (1 << 27) + 77), ("naive", (1 << 26) + 77),
                                       ("narrow", (1 << 26) + 77)])
def test_grid_loop_sampled(algo, rows):
    # More work units than the grid holds (2^20 workgroups): each workgroup loops.
    # A block of source rows transposes to the same block of destination
    # columns, so the oracle checks sampled row blocks one at a time.
    cols = 1
    src = make_transpose_input(rows, cols, seed=10)
    st, got = run_transpose(src, rows, cols, algo)
    assert st == 0
    blk = 4096
    starts = [0, 1 << 20, (1 << 24) + 13, (1 << 25) - 5, rows - 3 * blk, rows - blk]
    for r0 in starts:
        r1 = min(rows, r0 + blk)
        assert_bits_equal(got[:, r0:r1], oracle_transpose(src[r0:r1], r1 - r0, cols),
                          f"{algo} rows {r0}:{r1}")


@pytest.mark.parametrize("algo", ["lds", "lds_nopad"])
@pytest.mark.parametrize("ld_extra,offset", [(0, 0), (4, 0), (1, 0), (0, 1)])
def test_stream_launch_alignment(algo, ld_extra, offset):
    # 8192 x 4160 (4160 tiles, one per workgroup): with a 16-byte aligned source
    # and leading dimension the padded kernel loads 128 bits per lane, otherwise
    # 32; both must give the same bits.
    rows, cols = 8192, 4160
    src = make_transpose_input(rows, cols, seed=14, ld_src=cols + ld_extra)
    st, got = run_transpose(src, rows, cols, algo, src_offset=offset)
    assert st == 0
    assert_bits_equal(got, oracle_transpose(src, rows, cols), f"{algo} ld+{ld_extra} offset {offset}")


@pytest.mark.parametrize("rows,cols", [(0, 5), (5, 0)])
def test_empty_touches_nothing(rows, cols):
    import torch

    dev = torch.device("cuda", 0)
    dS = torch.zeros(16, device=dev)
    dD = torch.from_numpy(_canary(16)).to(dev)
    st = lib.sgemm_f32_transpose(rows, cols, dS.data_ptr(), max(1, cols), dD.data_ptr(), max(1, rows), 0)
    torch.cuda.synchronize()
    assert st == 0
    assert np.all(dD.cpu().numpy().view(np.uint32) == CANARY_BITS)


def test_alias_is_rejected_and_nothing_written():
    import torch

    dev = torch.device("cuda", 0)
    x = make_transpose_input(64, 64, seed=12)
    dX = torch.from_numpy(x.copy()).to(dev)
    st = lib.sgemm_f32_transpose(64, 64, dX.data_ptr(), 64, dX.data_ptr() + 4 * 64, 64, 0)
    torch.cuda.synchronize()
    assert st == 2
    assert np.array_equal(dX.cpu().numpy().view(np.uint32), x.view(np.uint32))


def test_side_stream_and_wrapper_views():
    import torch

    dev = torch.device("cuda", 0)
    rows, cols = 333, 444
    src = make_transpose_input(rows, cols, seed=13, ld_src=cols + 9)
    want = oracle_transpose(src, rows, cols)
    big_src = torch.from_numpy(src).to(dev)
    s_view = big_src[:, :cols]                      # row stride cols + 9
    big_dst = torch.full((cols, rows + 4), -1.0, device=dev)
    d_view = big_dst[:, 2:2 + rows]                 # row stride rows + 4, offset base
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        lib.transpose(s_view, d_view, algo="auto")
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    out = big_dst.cpu().numpy()
    assert_bits_equal(out[:, 2:2 + rows], want, "wrapper views")
    assert np.all(out[:, :2] == -1.0) and np.all(out[:, 2 + rows:] == -1.0)
    with pytest.raises(ValueError):
        lib.transpose(s_view, big_dst)              # wrong destination shape


def test_repeated_calls_identical():
    rows, cols = 4096, 4096
    src = make_transpose_config("t_4096")
    _, a = run_transpose(src, rows, cols, "auto")
    _, b = run_transpose(src, rows, cols, "auto")
    assert_bits_equal(a, b, "repeat")
