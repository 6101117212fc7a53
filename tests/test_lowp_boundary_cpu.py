"""Mixed-precision entry points without a GPU: validation and the planning
query.  Every call here is rejected or a quick return (fake addresses)."""
import os

import pytest

import fp32_gemm_08_amd as lib

OK, INVALID, ALIAS = 0, 1, 2
KID_SCALE, KID_LP_F16, KID_LP_BF16, KID_LP_F16_S, KID_LP_BF16_S = 1, 60, 61, 62, 63
PA, PB, PC = 1 << 32, 1 << 40, 1 << 44


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(lib.LIB_PATH):
        pytest.skip("libsgemm_f32.so not built")


def plan(prec=1, M=64, N=64, K=64, alpha=1.0, A=PA, lda=None, B=PB, ldb=None, transB=0, beta=0.0, C=PC, ldc=None):
    lda = K if lda is None else lda
    ldb = (K if transB else N) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return lib.sgemm_f32_lowp_plan(prec, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc)


def call(prec=1, M=64, N=64, K=64, alpha=1.0, A=PA, lda=None, B=PB, ldb=None, transB=0, beta=0.0, C=PC, ldc=None):
    lda = K if lda is None else lda
    ldb = (K if transB else N) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return lib.sgemm_f32_lowp(prec, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, 0)


@pytest.mark.parametrize("kw", [dict(prec=0), dict(prec=3), dict(prec=-1), dict(M=-1), dict(lda=63),
                                dict(transB=2), dict(A=0), dict(C=0), dict(K=(1 << 31) - 1024)])
def test_invalid(kw):
    assert plan(**kw)[0] == INVALID
    assert call(**kw) == INVALID


@pytest.mark.parametrize("kw", [dict(C=PA + 4), dict(B=PC + 8, transB=1)])
def test_alias(kw):
    assert plan(**kw)[0] == ALIAS and call(**kw) == ALIAS


@pytest.mark.parametrize("prec,tag", [(1, "f16"), (2, "bf16")])
@pytest.mark.parametrize("shape,large,tiles", [
    ((4096, 4096, 4096), True, (16, 16)),     # 256 tiles of 256 x 256: every CU busy
    ((4096, 4000, 64), True, (16, 16)),
    ((4000, 3840, 512), False, (63, 60)),     # 16 x 15 = 240 large tiles: the 64 x 64 tile
    ((2048, 2048, 2048), False, (32, 32)),
    ((1000, 1017, 999), False, (16, 16)),
    ((1, 1, 1), False, (1, 1)),
    ((257, 256, 5), False, (5, 4))])
def test_plan(prec, tag, shape, large, tiles):
    st, k, tm, tn, name = plan(prec, *shape)
    kid = {(1, True): KID_LP_F16, (2, True): KID_LP_BF16, (1, False): KID_LP_F16_S, (2, False): KID_LP_BF16_S}
    assert (st, k, (tm, tn)) == (OK, kid[(prec, large)], tiles)
    assert name.startswith(f"mfma_lp_{tag}_256x256x32" if large else f"mfma_lp_{tag}_64x64x32")


def test_quick_returns_and_product_free():
    assert call(M=0) == OK and call(N=0, ldb=1, ldc=1) == OK
    assert call(alpha=0.0, beta=1.0) == OK
    # alpha == 0 with beta != 1: C <- beta*C, the FP32 call's scale kernel (no operands read)
    assert plan(alpha=0.0, beta=2.0)[1] == KID_SCALE
    assert plan(K=0, lda=1, beta=0.5)[1] == KID_SCALE


def test_precision_table():
    assert lib.PRECISION == {"fp16": 1, "bf16": 2}
