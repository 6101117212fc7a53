"""Mixed-precision entry points without a GPU: validation and the planning
query.  Every call here is rejected or a quick return (fake addresses)."""
import os

import pytest

import fp32_gemm_08_amd as lib

OK, INVALID, ALIAS = 0, 1, 2
KID_SCALE, KID_LP_F16, KID_LP_BF16, KID_LP_F16_S, KID_LP_BF16_S = 1, 60, 61, 62, 63
KID_Q_F16, KID_Q_BF16, KID_Q_F16_S, KID_Q_BF16_S = 64, 65, 66, 67
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
    ((4000, 3840, 512), True, (16, 15)),      # 240 large tiles: still the 256 x 256 tile
    ((3000, 3000, 3000), True, (12, 12)),     # 144: at least half the CUs
    ((2560, 2560, 2560), False, (40, 40)),    # 100 large tiles: the 64 x 64 tile
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


@pytest.mark.parametrize("shape,want", [
    ((4096, 4096, 4096), ("two", True, (16, 16))),    # >= 1e10 FLOPs, 256 tiles of 256
    ((3000, 3000, 3000), ("two", True, (12, 12))),    # 144 tiles of 256: more than half the CUs
    ((4096, 2048, 2048), ("two", False, (32, 16))),   # exactly 128 tiles of 256: the 128 x 128 tile
    ((4096, 2064, 2048), ("two", True, (16, 9))),     # 144 tiles of 256
    ((2560, 2560, 2560), ("two", False, (20, 20))),   # 100: the 128 x 128 tile
    ((2048, 2048, 2048), ("two", False, (16, 16))),
    ((1000, 1017, 999), ("two", False, (8, 8))),      # 2e9 FLOPs with edges and a k tail
    ((1024, 1024, 1024), ("one", False, (16, 16))),   # aligned and small: the one-pass call
    ((1536, 1536, 1536), ("two", False, (12, 12))),   # 7.2e9 FLOPs with K >= min(M, N)
    ((1280, 1280, 1280), ("two", False, (10, 10))),   # 4.2e9, K = M = N
    ((1024, 1024, 4096), ("two", False, (8, 8))),
    ((2048, 2048, 1024), ("one", False, (32, 32))),   # 8.6e9 but shallow: one pass
    ((2048, 2048, 512), ("one", False, (32, 32))),
    ((1024, 1024, 1856), ("one", False, (16, 16))),   # 3.9e9 < 4e9: one pass
    ((100, 100, 100), ("one", False, (2, 2))),
])
@pytest.mark.parametrize("prec", [1, 2])
def test_ws_plan(shape, want, prec):
    st, kid, tm, tn, need = lib.sgemm_f32_lowp_ws_plan(prec, *shape, 0)
    kind, large, tiles = want
    assert st == OK and (tm, tn) == tiles
    if kind == "two":
        q = {(1, True): KID_Q_F16, (2, True): KID_Q_BF16, (1, False): KID_Q_F16_S, (2, False): KID_Q_BF16_S}
        assert kid == q[(prec, large)]
        b = 256 if large else 128
        mp, np_, kp = -(-shape[0] // b) * b, -(-shape[1] // b) * b, -(-shape[2] // 32) * 32
        assert need == -(-(mp * kp * 2) // 256) * 256 + np_ * kp * 2
    else:
        assert kid in (KID_LP_F16_S, KID_LP_BF16_S) and need == 0


def call_ws(prec=2, M=1000, N=1017, K=999, A=PA, B=PB, C=PC, W=1 << 46, wb=1 << 30, transB=0, lda=None):
    lda = K if lda is None else lda
    ldb = K if transB else N
    return lib.sgemm_f32_lowp_ws(prec, M, N, K, 1.0, A, lda, B, ldb, transB, 0.0, C, N, W, wb, 0)


@pytest.mark.parametrize("kw,want", [(dict(prec=3), INVALID), (dict(M=-1), INVALID), (dict(lda=5), INVALID),
                                     (dict(wb=-1), INVALID), (dict(W=PA + 64), ALIAS), (dict(W=PB + 64), ALIAS),
                                     (dict(W=PC + 64), ALIAS)])
def test_ws_rejections(kw, want):
    assert call_ws(**kw) == want


@pytest.mark.parametrize("tile,large", [(0, False), (256, True), (128, False)])
def test_2pass_plan(tile, large):
    st, kid, tm, tn, need = lib.sgemm_f32_lowp_2pass_plan(2, tile, 300, 200, 50, 0)
    b = 256 if large else 128
    assert (st, kid) == (OK, KID_Q_BF16 if large else KID_Q_BF16_S)
    assert (tm, tn) == (-(-300 // b), -(-200 // b))
    assert need == -(-(-(-300 // b) * b * 64 * 2) // 256) * 256 + -(-200 // b) * b * 64 * 2


@pytest.mark.parametrize("tile", [64, -1, 1, 512])
def test_2pass_bad_tile(tile):
    assert lib.sgemm_f32_lowp_2pass_plan(2, tile, 300, 200, 50, 0)[0] == INVALID
    assert lib.sgemm_f32_lowp_2pass(2, tile, 300, 200, 50, 1.0, PA, 50, PB, 200, 0, 0.0, PC, 200, 1 << 46,
                                    1 << 30, 0) == INVALID


def test_2pass_small_workspace():
    need = lib.sgemm_f32_lowp_2pass_plan(2, 0, 300, 200, 50, 0)[4]
    assert lib.sgemm_f32_lowp_2pass(2, 0, 300, 200, 50, 1.0, PA, 50, PB, 200, 0, 0.0, PC, 200, 1 << 46,
                                    need - 1, 0) == INVALID
    assert lib.sgemm_f32_lowp_2pass(2, 0, 300, 200, 50, 1.0, PA, 50, PB, 200, 0, 0.0, PC, 200, 0,
                                    need, 0) == INVALID


@pytest.mark.parametrize("off", [4, 8, 12, 2])
def test_2pass_misaligned_workspace(off):
    # the GEMM pass stages the rounded operands with 16-byte loads
    assert lib.sgemm_f32_lowp_2pass(2, 0, 300, 200, 50, 1.0, PA, 50, PB, 200, 0, 0.0, PC, 200, (1 << 46) + off,
                                    1 << 30, 0) == INVALID


def test_two_passes_stop_at_the_grid_limit_in_k():
    # the rounding transpose launches ceil(K / 64) workgroup rows, at most 65535
    kmax = 64 * 65535
    st, kid, _, _, need = lib.sgemm_f32_lowp_ws_plan(2, 2048, 2048, kmax, 0)
    assert st == OK and kid == KID_Q_BF16_S and need > 0
    st, kid, _, _, need = lib.sgemm_f32_lowp_ws_plan(2, 2048, 2048, kmax + 1, 0)
    assert st == OK and kid == KID_LP_BF16_S and need == 0      # the one-pass call
    assert lib.sgemm_f32_lowp_2pass_plan(2, 0, 256, 256, kmax + 1, 0)[0] == INVALID
    assert lib.sgemm_f32_lowp_2pass_plan(2, 0, 256, 256, kmax, 0)[0] == OK
