"""C-ABI boundary tests of the transpose entry points that need no GPU.

Validation, quick returns and the planning query run on the host before any
HIP call, so every status they produce is checked here without a device.
"""
import numpy as np
import pytest

import fp32_gemm_08_amd as lib

OK, INVALID, ALIAS = 0, 1, 2
KID_NONE, KID_NAIVE, KID_PAD, KID_NOPAD, KID_NARROW = 0, 50, 51, 52, 53
PS, PD = 1 << 32, 1 << 40   # fake, well-separated device addresses


@pytest.fixture(scope="module", autouse=True)
def built():
    import os
    if not os.path.exists(lib.LIB_PATH):
        pytest.skip("libsgemm_f32.so not built")


def plan(algo=0, rows=64, cols=64, src=PS, ld_src=None, dst=PD, ld_dst=None):
    ld_src = cols if ld_src is None else ld_src
    ld_dst = rows if ld_dst is None else ld_dst
    return lib.sgemm_f32_transpose_plan(algo, rows, cols, src, ld_src, dst, ld_dst)


def call(algo=0, rows=64, cols=64, src=PS, ld_src=None, dst=PD, ld_dst=None):
    ld_src = cols if ld_src is None else ld_src
    ld_dst = rows if ld_dst is None else ld_dst
    return lib.sgemm_f32_transpose_algo(algo, rows, cols, src, ld_src, dst, ld_dst, 0)


@pytest.mark.parametrize("kw", [
    dict(rows=-1), dict(cols=-1), dict(rows=1 << 31), dict(cols=(1 << 31) - 1024),
    dict(ld_src=63), dict(ld_dst=63), dict(rows=1, ld_dst=0), dict(cols=1, ld_src=0),
    dict(src=0), dict(dst=0), dict(algo=5), dict(algo=-1),
    dict(rows=2, cols=2, ld_src=1 << 61),
])
def test_invalid_arguments(kw):
    assert plan(**kw)[0] == INVALID
    assert call(**kw) == INVALID


def test_largest_dimension_is_accepted():
    big = (1 << 31) - 1025
    st, kid, blocks, _ = plan(rows=big, cols=1, ld_src=1, ld_dst=big, dst=1 << 46)
    assert st == OK and kid == KID_NARROW and blocks == min(-(-big // 64), 1 << 20)
    st, kid, blocks, _ = plan(algo=2, rows=big, cols=1, ld_src=1, ld_dst=big, dst=1 << 46)
    assert st == OK and kid == KID_PAD and blocks == 1 << 20


def test_grid_is_capped():
    # 2^15 x 2^13 tiles of 128 x 128: the workgroups loop over them.
    rows, cols = 1 << 22, 1 << 20
    st, kid, blocks, name = plan(rows=rows, cols=cols, ld_src=cols, ld_dst=rows, src=1 << 48, dst=1 << 58)
    assert (st, kid, blocks) == (OK, KID_PAD, 1 << 20) and name.endswith("_stream_v4")


def test_too_many_tiles():
    # 2^23 x 2^9 = 2^32 tiles of 128 x 128: rejected before any launch.
    rows, cols = 1 << 30, 1 << 16
    assert plan(rows=rows, cols=cols, ld_src=cols, ld_dst=rows, src=1 << 48, dst=1 << 59)[0] == INVALID


@pytest.mark.parametrize("rows,cols", [(0, 5), (5, 0), (0, 0)])
def test_empty_is_a_no_op(rows, cols):
    # Nothing is read or written: NULL pointers are fine, and no device is needed.
    st, kid, blocks, _ = plan(rows=rows, cols=cols, src=0, dst=0, ld_src=max(cols, 1), ld_dst=max(rows, 1))
    assert (st, kid, blocks) == (OK, KID_NONE, 0)
    assert call(rows=rows, cols=cols, src=0, dst=0, ld_src=max(cols, 1), ld_dst=max(rows, 1)) == OK


def test_alias_is_rejected():
    src_bytes = ((64 - 1) * 64 + 64) * 4
    assert plan(dst=PS + src_bytes - 4)[0] == ALIAS
    assert plan(dst=PS - 64 * 64 * 4 + 4)[0] == ALIAS
    assert plan(dst=PS)[0] == ALIAS
    assert call(dst=PS + 4) == ALIAS
    # Adjacent but not overlapping ranges are fine.
    assert plan(dst=PS + src_bytes)[0] == OK
    assert plan(dst=PS - 64 * 64 * 4)[0] == OK


@pytest.mark.parametrize("algo,kid", [(0, KID_PAD), (1, KID_NAIVE), (2, KID_PAD), (3, KID_NOPAD), (4, KID_NARROW)])
def test_algorithm_choice(algo, kid):
    st, k, blocks, name = plan(algo=algo, rows=2000, cols=2017)
    assert st == OK and k == kid
    if kid == KID_NAIVE:
        assert blocks == -(-2000 // 16) * -(-2017 // 64) and name == "transpose_naive_64x16"
    elif kid == KID_NARROW:
        assert blocks == -(-2000 // 64) * -(-2017 // 16) and name == "transpose_narrow_64x16"
    else:
        # 16 x 16 tiles of 128 x 128: the persistent, pipelined shape
        assert blocks == 256 and name == f"transpose_lds_128x128_pad{int(kid == KID_PAD)}_pipe"


@pytest.mark.parametrize("rows,cols,kid", [(31, 5000, KID_NAIVE), (5000, 31, KID_NARROW), (32, 32, KID_PAD),
                                           (3, 3, KID_NAIVE), (32, 31, KID_NARROW)])
def test_auto_sends_narrow_shapes_to_element_kernels(rows, cols, kid):
    assert plan(rows=rows, cols=cols)[:2] == (OK, kid)


def test_launch_shape_by_tile_count():
    # fewer 128 x 128 tiles than CUs: 64 x 64 tiles, one per workgroup
    st, _, blocks, name = plan(rows=1000, cols=1017)        # 8 x 8 tiles of 128
    assert (st, blocks, name) == (OK, 16 * 16, "transpose_lds_64x64_pad1")
    st, _, blocks, name = plan(algo=3, rows=1920, cols=2048)  # 15 x 16 = 240 tiles of 128
    assert (st, blocks, name) == (OK, 30 * 32, "transpose_lds_64x64_pad0")
    st, _, blocks, name = plan(rows=2048, cols=2048)        # 256 tiles of 128
    assert (st, blocks) == (OK, 256) and name.endswith("_pipe")
    # up to 2048 tiles: persistent grid of 512 workgroups; above: one tile per workgroup
    st, _, blocks, name = plan(rows=4096, cols=8192)        # 32 x 64 = 2048 tiles
    assert (st, blocks) == (OK, 512) and name.endswith("_pipe")
    st, _, blocks, name = plan(rows=4096, cols=8193)        # 32 x 65 tiles
    assert (st, blocks) == (OK, 32 * 65) and name.endswith("_stream")   # ld 8193: no 16-byte loads
    st, _, blocks, name = plan(rows=8192, cols=8192)
    assert (st, blocks) == (OK, 4096) and name.endswith("_stream_v4")
    st, _, _, name = plan(rows=8192, cols=8192, src=PS + 4)  # misaligned base: no 16-byte loads
    assert name.endswith("_stream")
    st, _, _, name = plan(algo=3, rows=8192, cols=8192)     # only the padded kernel uses them
    assert name == "transpose_lds_128x128_pad0_stream"


def test_python_wrapper_checks_before_the_library():
    torch = pytest.importorskip("torch")
    x = torch.zeros(4, 5)
    with pytest.raises(TypeError):
        lib.transpose(x, torch.zeros(5, 4))          # host tensors are refused
    with pytest.raises(KeyError):
        lib.sgemm._algo_id("bogus", lib.TRANSPOSE_ALGO)


def test_transpose_algorithm_table_matches_header():
    assert lib.TRANSPOSE_ALGO == {"auto": 0, "naive": 1, "lds": 2, "lds_nopad": 3, "narrow": 4}
    assert np.all(np.array(list(lib.TRANSPOSE_ALGO.values())) == np.arange(5))
