"""sgemm_f32_splitk_noalloc on the GPU: the k-split with its partials in the
library's static device scratch must give exactly the bits of
sgemm_f32_splitk on a caller workspace (same kernels, same split count, same
k order), and satisfy the oracle's bound, on consecutive calls whose sizes
shrink (the scratch keeps the previous call's partials; each call must
overwrite every partial it reads).  A call whose partials exceed the scratch
is rejected before any launch.
"""
import numpy as np
import pytest

import fp32_gemm_08_amd as lib
from fp32_gemm_08_amd.inputs import make_case
from oracle import check

from gpu_helpers import oracle_rows, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert lib.sgemm_f32_version()


def run_both(case, splits):
    import torch

    dev = torch.device("cuda", 0)
    M, N, K, t = case.M, case.N, case.K, int(case.trans_b)
    st, used, _, need = lib.sgemm_f32_splitk_plan(splits, M, N, K, t)
    assert st == 0 and used > 1 and 0 < need <= lib.SCRATCH_BYTES
    # sgemm_f32_splitk takes explicit counts only: the count the AUTO rule
    # (splits = 0) plans gives the same split geometry
    ref_splits = splits if splits else used
    A = torch.from_numpy(case.A).to(dev)
    B = torch.from_numpy(case.B).to(dev)
    C0 = case.C if case.C is not None else np.full((M, case.ldc), np.nan, np.float32)
    C_ref = torch.from_numpy(C0.copy()).to(dev)
    C_new = torch.from_numpy(C0.copy()).to(dev)
    W = torch.empty(need // 4, dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream(dev).cuda_stream
    say(f"noalloc splits={splits} (used {used}, {need} B) M={M} N={N} K={K} transB={t} alpha={case.alpha} "
        f"beta={case.beta}")
    st_ref = lib.sgemm_f32_splitk(ref_splits, M, N, K, case.alpha, A.data_ptr(), case.lda, B.data_ptr(), case.ldb, t,
                                  case.beta, C_ref.data_ptr(), case.ldc, W.data_ptr(), need, s)
    st_new = lib.sgemm_f32_splitk_noalloc(splits, M, N, K, case.alpha, A.data_ptr(), case.lda, B.data_ptr(),
                                          case.ldb, t, case.beta, C_new.data_ptr(), case.ldc, s)
    torch.cuda.synchronize()
    assert st_ref == 0 and st_new == 0
    return C_ref.cpu().numpy(), C_new.cpu().numpy(), used


def check_pair(oracle_lib, case, splits, what):
    ref, new, used = run_both(case, splits)
    assert np.array_equal(ref.view(np.uint32), new.view(np.uint32)), f"{what}: bits differ from sgemm_f32_splitk"
    D, S = oracle_rows(oracle_lib, case)
    r = check(new[:, :case.N], D, S, case.K)
    say(f"{what}: {used} splits, max_abs={r['max_abs']:.3e} max_rho={r['max_rho']:.3f} fails={r['n_fail']}")
    assert r["ok"], f"{what}: {r}"


def test_two_calls_second_smaller(oracle_lib):
    big = make_case(256, 256, 4096, trans_b=False, alpha=1.0, beta=1.0, dist="normal", seed=61)
    check_pair(oracle_lib, big, 0, "256x256x4096 auto")
    small = make_case(200, 136, 1000, trans_b=True, alpha=1.5, beta=-0.5, dist="uniform", seed=62)
    check_pair(oracle_lib, small, 0, "200x136x1000 B^T auto")


def test_explicit_splits_then_smaller(oracle_lib):
    a = make_case(300, 300, 2048, trans_b=False, alpha=-0.75, beta=0.0, dist="uniform", seed=63)
    check_pair(oracle_lib, a, 8, "300x300x2048 8 splits")
    b = make_case(129, 65, 333, trans_b=False, alpha=1.0, beta=0.5, dist="uniform", seed=64, lda=337)
    check_pair(oracle_lib, b, 3, "129x65x333 3 splits")


def test_scratch_limit_touches_nothing():
    import torch

    dev = torch.device("cuda", 0)
    A = torch.zeros(1024, 4096, device=dev)
    B = torch.zeros(4096, 1024, device=dev)
    C = torch.full((1024, 1024), 5.0, device=dev)
    st = lib.sgemm_f32_splitk_noalloc(8, 1024, 1024, 4096, 1.0, A.data_ptr(), 4096, B.data_ptr(), 1024, 0, 0.0,
                                      C.data_ptr(), 1024, 0)
    torch.cuda.synchronize()
    assert st == lib.SGEMM_ERR_SCRATCH_LIMIT and torch.all(C == 5.0)
