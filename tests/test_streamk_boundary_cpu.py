"""Stream-K entry points without a GPU: validation and the planning queries.
Every call here is rejected before any HIP call (fake addresses)."""
import os

import pytest

import fp32_gemm_08_amd as lib

OK, INVALID, ALIAS = 0, 1, 2
KID_L, KID_M, KID_S, KID_L_SK, KID_M_SK = 40, 41, 42, 43, 44
PA, PB, PC, PW = 1 << 32, 1 << 40, 1 << 44, 1 << 46
MB = 1 << 20


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(lib.LIB_PATH):
        pytest.skip("libsgemm_f32.so not built")


def call(tile=0, M=1000, N=1000, K=1000, alpha=1.0, A=PA, lda=None, B=PB, ldb=None, transB=0, beta=0.0, C=PC,
         ldc=None, W=PW, wb=0):
    lda = K if lda is None else lda
    ldb = (K if transB else N) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return lib.sgemm_f32_streamk(tile, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, W, wb, 0)


@pytest.mark.parametrize("shape,tile,want", [
    # 324 tiles of 256: one whole wave, 68 tiles shared by 256 workers (two 256x256 slots each)
    ((4608, 4608, 4608), 256, (KID_L_SK, 256, 68, 256, 2 * 256 * 256 * 256 * 4)),
    # 576 tiles of 128: two whole waves, 64 shared
    ((3072, 3072, 3072), 128, (KID_M_SK, 512, 64, 256, 2 * 256 * 128 * 128 * 4)),
    # fewer tiles than CUs: all shared
    ((1000, 1017, 999), 256, (KID_L_SK, 0, 16, 256, 128 * MB)),
    # whole waves only: the plain schedule, no workspace
    ((4096, 4096, 4096), 256, (KID_L_SK, 256, 0, 0, 0)),
    # one tile, one k-iteration: one worker, which covers it whole
    ((1, 1, 1), 256, (KID_L_SK, 0, 1, 1, 2 * 256 * 256 * 4)),
    # 3 tiles x 47 iterations = 141 < 256: one worker per iteration
    ((100, 300, 3000), 128, (KID_M_SK, 0, 3, 141, 2 * 141 * 128 * 128 * 4)),
])
def test_plan(shape, tile, want):
    st, kid, dp, skt, wk, need = lib.sgemm_f32_streamk_plan(tile, *shape, 0)
    assert (st, kid, dp, skt, wk, need) == (OK,) + want


def test_plan_auto_tile_is_one_of_the_two():
    for shape in [(4608, 4608, 4608), (3000, 3000, 3000), (1536, 1536, 4096), (2304, 2304, 8192)]:
        st, kid, *_ = lib.sgemm_f32_streamk_plan(0, *shape, 0)
        assert st == OK and kid in (KID_L_SK, KID_M_SK)


@pytest.mark.parametrize("tile", [64, -1, 512, 1])
def test_invalid_tile(tile):
    assert lib.sgemm_f32_streamk_plan(tile, 1000, 1000, 1000, 0)[0] == INVALID
    assert call(tile=tile, wb=256 * MB) == INVALID


@pytest.mark.parametrize("kw", [dict(M=-1), dict(lda=999), dict(transB=2), dict(A=0), dict(C=0),
                                dict(W=0, wb=256 * MB), dict(wb=-1)])
def test_invalid_arguments(kw):
    assert call(**kw) == INVALID


def test_workspace_too_small():
    need = lib.sgemm_f32_streamk_plan(256, 1000, 1000, 1000, 0)[5]
    assert call(tile=256, wb=need - 4) == INVALID
    assert call(tile=256, wb=0) == INVALID


@pytest.mark.parametrize("off", [4, 8, 12, 1])
def test_workspace_misaligned(off):
    # the fix-up kernel reads the workspace with 128-bit loads
    assert call(tile=256, W=PW + off, wb=256 * MB) == INVALID
    assert call(tile=128, W=PW + off, wb=256 * MB) == INVALID


@pytest.mark.parametrize("W", [PA + 64, PB + 64, PC + 64])
def test_workspace_alias(W):
    assert call(tile=256, W=W, wb=256 * MB) == ALIAS


def test_quick_returns():
    assert call(M=0) == OK and call(N=0, ldb=1, ldc=1) == OK
    assert call(alpha=0.0, beta=1.0) == OK
    st, kid, dp, skt, wk, need = lib.sgemm_f32_streamk_plan(0, 0, 10, 10, 0)
    assert (st, dp, skt, wk, need) == (OK, 0, 0, 0, 0)


@pytest.mark.parametrize("shape,method", [((4608, 4608, 4608), 2), ((3072, 3072, 3072), 2), ((512, 512, 512), 0),
                                          ((300, 333, 1500), 1),
                                          ((256, 256, 8192), 1), ((4096, 4096, 4096), 0), ((8192, 8192, 8192), 0),
                                          ((1024, 1024, 1024), 0)])
def test_ws_plan_method(shape, method):
    st, m, kid, need = lib.sgemm_f32_ws_plan(*shape, 0)
    assert (st, m) == (OK, method)
    assert (need > 0) == (method != 0)
    if method == 2:
        assert kid in (KID_L_SK, KID_M_SK)
        assert need == lib.sgemm_f32_streamk_plan(0, *shape, 0)[5]
    if method == 1:
        assert need == lib.sgemm_f32_splitk_plan(0, *shape, 0)[3]
