"""k-split entry points without a GPU: the planning query, and every argument
check that returns before a device call.  The addresses are fake, so every
call here must be rejected or be a quick return: a call that passed
validation would launch on a GPU host."""
import os

import pytest

import fp32_gemm_08_amd as lib

OK, INVALID, ALIAS = 0, 1, 2
KID_L, KID_M, KID_S, KID_S2, KID_T = 40, 41, 42, 45, 46
PA, PB, PC, PW = 1 << 32, 1 << 40, 1 << 44, 1 << 48


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(lib.LIB_PATH):
        pytest.skip("libsgemm_f32.so not built")


@pytest.mark.parametrize("shape,auto", [
    ((4096, 4096, 4096), (1, KID_L, 0)),          # fills the chip: never split
    ((2048, 2048, 2048), (1, KID_M, 0)),
    ((1024, 1024, 1024), (1, KID_S2, 0)),         # 256 tiles of 64 x 64: the plain call's kernel
    ((512, 512, 512), (1, KID_T, 0)),            # 4 splits: no more workgroups than the plain 32 x 32 grid
    ((700, 333, 1500), (1, KID_T, 0)),           # 3 splits
    ((300, 333, 1500), (8, KID_S, 8 * 300 * 333 * 4)),
    ((768, 768, 768), (1, KID_T, 0)),              # 144 tiles: over half the CUs busy already
    ((512, 512, 8192), (8, KID_S, 8 * 512 * 512 * 4)),       # two workgroups per CU, 1024 of k each
    ((256, 256, 8192), (16, KID_S, 16 * 256 * 256 * 4)),     # two per CU would leave only 256 of k
    ((256, 256, 32768), (32, KID_S, 32 * 256 * 256 * 4)),
    ((512, 256, 16384), (16, KID_S, 16 * 512 * 256 * 4)),
    ((384, 384, 8192), (7, KID_S, 7 * 384 * 384 * 4)),       # 36 tiles: 14 splits would get 585 of k
    ((64, 64, 65536), (64, KID_S, 64 * 64 * 64 * 4)),
    ((128, 128, 128), (1, KID_T, 0)),             # k too short to split at 256 per split
])
def test_auto_split_choice(shape, auto):
    st, used, kid, nbytes = lib.sgemm_f32_splitk_plan(0, *shape)
    assert st == OK and (used, kid, nbytes) == auto


def test_explicit_split_geometry():
    # K = 100 in 8 splits: 32 per split (whole k-tiles) leaves 4 non-empty splits.
    assert lib.sgemm_f32_splitk_plan(8, 512, 512, 100)[:2] == (OK, 4)
    # K <= 32 cannot split.
    assert lib.sgemm_f32_splitk_plan(4, 512, 512, 32)[1:] == (1, KID_T, 0)    # the plain call's kernel
    # an explicit count splits any shape, always with the 64 x 64 partial tile
    assert lib.sgemm_f32_splitk_plan(4, 1024, 1024, 1024)[1:] == (4, KID_S, 4 * 1024 * 1024 * 4)
    assert lib.sgemm_f32_splitk_plan(16, 4096, 4096, 4096)[1:] == (16, KID_S, 16 * 4096 * 4096 * 4)
    # transB does not change the plan
    assert lib.sgemm_f32_splitk_plan(3, 1000, 1017, 999, 1) == lib.sgemm_f32_splitk_plan(3, 1000, 1017, 999, 0)


@pytest.mark.parametrize("args", [(-1, 64, 64, 64, 0), (65, 64, 64, 64, 0), (2, -1, 64, 64, 0),
                                  (2, 64, 64, 1 << 31, 0), (2, 64, 64, 64, 2)])
def test_plan_rejects_invalid(args):
    assert lib.sgemm_f32_splitk_plan(*args)[0] == INVALID


def call(splits, M=512, N=512, K=512, alpha=1.0, A=PA, lda=None, B=PB, ldb=None, transB=0, beta=0.0, C=PC,
         ldc=None, W=PW, wbytes=None):
    lda = K if lda is None else lda
    ldb = (K if transB else N) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    wbytes = 16 * M * N * 4 if wbytes is None else wbytes
    if splits is None:
        return lib.sgemm_f32_ws(M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, W, wbytes, 0)
    return lib.sgemm_f32_splitk(splits, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, W, wbytes, 0)


@pytest.mark.parametrize("kw", [dict(splits=0), dict(splits=-2), dict(splits=65), dict(splits=2, M=-1),
                                dict(splits=2, lda=100), dict(splits=2, transB=3), dict(splits=2, A=0),
                                dict(splits=4, wbytes=4 * 512 * 512 * 4 - 4), dict(splits=2, W=0),
                                dict(splits=None, wbytes=-1)])
def test_invalid_calls(kw):
    assert call(**kw) == INVALID


@pytest.mark.parametrize("kw", [dict(W=PA), dict(W=PC + 16), dict(W=PB - 2 * 512 * 512 * 4 + 16),
                                dict(splits=None, K=8192, W=PA + 16)])   # AUTO splits 512 x 512 x 8192
def test_workspace_alias(kw):
    # the 2-split partials need 2 * 512 * 512 * 4 bytes from W on
    kw.setdefault("splits", 2)
    assert call(**kw) == ALIAS


@pytest.mark.parametrize("off", [4, 8, 12, 2])
def test_workspace_misaligned(off):
    # every workspace starts on a 16-byte boundary; an explicit split count
    # with a misaligned one is an error (sgemm_f32_ws would run the plain call)
    assert call(4, W=PW + off) == INVALID


SCRATCH_LIMIT = 6


def noalloc(splits, M=512, N=512, K=512, alpha=1.0, A=PA, B=PB, transB=0, beta=0.0, C=PC):
    ldb = K if transB else N
    return lib.sgemm_f32_splitk_noalloc(splits, M, N, K, alpha, A, K, B, ldb, transB, beta, C, N, 0)


def test_noalloc_rejects_partials_beyond_the_scratch():
    # 64 splits of 1024 x 1024 need 256 MiB; 5 of 1024 x 1024 need 20 MiB
    assert noalloc(64, M=1024, N=1024, K=4096) == SCRATCH_LIMIT
    assert noalloc(5, M=1024, N=1024, K=4096) == SCRATCH_LIMIT
    assert lib.sgemm_f32_splitk_plan(4, 1024, 1024, 4096)[3] == lib.SCRATCH_BYTES   # 4 splits fit exactly
    assert "16 MiB" in lib.sgemm_f32_status_string(SCRATCH_LIMIT)


@pytest.mark.parametrize("kw", [dict(splits=-1), dict(splits=65), dict(splits=2, M=-1), dict(splits=2, A=0),
                                dict(splits=2, transB=2)])
def test_noalloc_invalid(kw):
    assert noalloc(**kw) == INVALID


def test_noalloc_alias_and_quick_returns():
    assert noalloc(2, C=PA + 64) == ALIAS
    assert noalloc(2, M=0) == OK and noalloc(0, alpha=0.0, beta=1.0) == OK


@pytest.mark.parametrize("M,N,K", [(512, 512, 512), (256, 256, 32768), (64, 64, 65536), (100, 700, 9000),
                                   (2000, 60, 50000), (800, 800, 800), (1, 1, 1 << 20)])
def test_auto_split_fits_the_scratch(M, N, K):
    # the AUTO rule keeps splits x 64x64 tiles <= 512, i.e. at most 8 MiB of partials
    st, used, _, need = lib.sgemm_f32_splitk_plan(0, M, N, K)
    assert st == OK and need <= lib.SCRATCH_BYTES // 2


def test_quick_returns_touch_nothing():
    # No launch happens for these, so fake addresses are safe.
    assert call(2, M=0) == OK and call(None, N=0, ldb=1, ldc=1) == OK
    assert call(2, alpha=0.0, beta=1.0) == OK and call(None, K=0, lda=1, beta=1.0) == OK
