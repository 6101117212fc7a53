"""GPU parity of the k-split path (sgemm_f32_splitk / sgemm_f32_ws) against the
FP64 oracle, through the C ABI.

Same bar as the unsplit GEMM: |D_gpu - D| <= 4*K*2^-24*S + 1e-6 elementwise,
finite; bit-exact for small-integer inputs (every summation order is exact
there, so any misplaced or missing partial shows).  The workspace has a canary
tail past the bytes the plan asks for, and C has canary guard rows and padding.
"""
import numpy as np
import pytest

import fp32_gemm_08_amd as lib
from fp32_gemm_08_amd.inputs import make_case, make_config
from oracle import check

from gpu_helpers import CANARY, GUARD_ROWS, oracle_rows, say

pytestmark = pytest.mark.gpu

W_CANARY = np.float32(-3333.5)
W_TAIL = 1024  # floats of canary after the planned workspace


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert lib.sgemm_f32_version()


def run_split(case, splits, ws_bytes=None, a_offset=0, ldc_pad=0, ws_offset=0, c_fill=np.nan):
    """Run one GEMM through sgemm_f32_splitk (splits >= 1) or sgemm_f32_ws
    (splits = 0).  Returns (status, D, planned splits)."""
    import torch

    dev = torch.device("cuda", 0)
    M, N, K = case.M, case.N, case.K
    st, used, kid, need = lib.sgemm_f32_splitk_plan(splits, M, N, K, int(case.trans_b))
    assert st == 0
    ws_bytes = need if ws_bytes is None else ws_bytes
    ldc = case.ldc + ldc_pad
    g = GUARD_ROWS
    full = np.full((M + 2 * g, ldc), CANARY, dtype=np.float32)
    full[g:g + M, :N] = case.C[:, :N] if case.C is not None else c_fill
    dA = torch.from_numpy(np.concatenate([np.zeros(a_offset, np.float32), case.A.ravel()])).to(dev)
    dB = torch.from_numpy(case.B.ravel().copy()).to(dev)
    dC = torch.from_numpy(full.ravel().copy()).to(dev)
    n_ws = ws_offset + max(ws_bytes, 0) // 4 + W_TAIL
    dW = torch.full((n_ws,), float(W_CANARY), dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream(dev)
    say(f"splitk splits={splits} (plan {used}, kid {kid}, {need} B) M={M} N={N} K={K} transB={int(case.trans_b)} "
        f"alpha={case.alpha} beta={case.beta} lda={case.lda} ldb={case.ldb} ldc={ldc} ws_bytes={ws_bytes} "
        f"a_offset={a_offset} ws_offset={ws_offset}")
    args = (M, N, K, case.alpha, dA.data_ptr() + 4 * a_offset, case.lda, dB.data_ptr(), case.ldb,
            int(case.trans_b), case.beta, dC.data_ptr() + 4 * g * ldc, ldc, dW.data_ptr() + 4 * ws_offset,
            ws_bytes, s.cuda_stream)
    st = lib.sgemm_f32_splitk(splits, *args) if splits else lib.sgemm_f32_ws(*args)
    torch.cuda.synchronize()
    out = dC.cpu().numpy().reshape(M + 2 * g, ldc)
    w = dW.cpu().numpy()
    assert np.all(w[:ws_offset].view(np.uint32) == W_CANARY.view(np.uint32)), "write before the workspace"
    assert np.all(w[ws_offset + max(ws_bytes, 0) // 4:].view(np.uint32) == W_CANARY.view(np.uint32)), \
        "write past the planned workspace"
    assert np.all(out[:g].view(np.uint32) == CANARY.view(np.uint32)), "write above C"
    assert np.all(out[g + M:].view(np.uint32) == CANARY.view(np.uint32)), "write below C"
    if ldc > N:
        assert np.all(out[g:g + M, N:].view(np.uint32) == CANARY.view(np.uint32)), "write into C padding"
    return st, out[g:g + M], used


def assert_parity(o, case, D_gpu, what):
    D, S = oracle_rows(o, case)
    r = check(D_gpu[:, :case.N], D, S, case.K)
    say(f"{what}: max_abs={r['max_abs']:.3e} max_rho={r['max_rho']:.3f} fails={r['n_fail']}")
    assert r["ok"], f"{what}: {r}"


SHAPES = [
    # M, N, K, transB, alpha, beta, extra
    (512, 512, 512, False, 1.0, 0.0, {}),
    (1000, 1017, 999, True, 1.5, -0.5, {}),       # ragged config: unaligned lda, odd ldc
    (256, 256, 8192, False, 1.0, 1.0, dict(dist="normal")),
    (257, 130, 4133, True, -0.75, 0.25, dict(ldb=4140)),
    (64, 64, 65536, False, 1.0, 0.0, {}),
    (128, 128, 128, False, 1.0, 0.0, {}),
]


@pytest.mark.parametrize("splits", [2, 3, 5, 8, 12, 16, 64])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}x{s[1]}x{s[2]}{'T' if s[3] else ''}")
def test_split_parity(oracle_lib, shape, splits):
    M, N, K, tb, alpha, beta, extra = shape
    case = make_case(M, N, K, trans_b=tb, alpha=alpha, beta=beta, seed=M + N + K, **extra)
    st, D, used = run_split(case, splits)
    assert st == 0
    assert_parity(oracle_lib, case, D, f"split {splits} (used {used}) {M}x{N}x{K}")


@pytest.mark.parametrize("splits", [0, 2, 7, 31])
@pytest.mark.parametrize("tb", [False, True])
def test_split_integers_bit_exact(oracle_lib, splits, tb):
    # small integers: every partial and every order is exact, so the split path
    # must reproduce the oracle bit for bit
    case = make_case(300, 260, 2000, trans_b=tb, alpha=1.0, beta=1.0, dist="int2", seed=17)
    st, D, used = run_split(case, splits)
    assert st == 0
    Dref, _ = oracle_rows(oracle_lib, case)
    assert np.array_equal(D[:, :case.N].astype(np.float64), Dref), f"splits {splits} (used {used})"


def test_auto_with_and_without_workspace(oracle_lib):
    case = make_case(256, 256, 4096, alpha=1.0, beta=1.0, dist="normal", seed=4)   # AUTO splits in 16
    st, D, used = run_split(case, 0)
    assert st == 0 and used == 16
    assert_parity(oracle_lib, case, D, "ws auto")
    # too small a workspace: the plain path, identical to sgemm_f32 bit for bit
    st, D0, _ = run_split(case, 0, ws_bytes=1024)
    assert st == 0
    import torch
    dev = torch.device("cuda", 0)
    A, B = torch.from_numpy(case.A).to(dev), torch.from_numpy(case.B).to(dev)
    C = torch.from_numpy(case.C.copy()).to(dev)
    lib.gemm(A, B, C, alpha=case.alpha, beta=case.beta)
    torch.cuda.synchronize()
    assert np.array_equal(D0.view(np.uint32), C.cpu().numpy().view(np.uint32))


def test_misaligned_operands(oracle_lib):
    case = make_case(700, 333, 1500, trans_b=False, alpha=1.0, beta=0.0, seed=21, lda=1503)
    st, D, used = run_split(case, 4, a_offset=1, ldc_pad=3, ws_offset=4)
    assert st == 0 and used == 4
    assert_parity(oracle_lib, case, D, "misaligned")


def test_misaligned_workspace(oracle_lib):
    # A workspace off a 16-byte boundary: the explicit split count is rejected
    # before any launch (C and the workspace keep their canaries); the
    # automatic call runs the plain kernel instead.
    case = make_case(300, 333, 1500, trans_b=False, alpha=1.0, beta=0.0, seed=21)
    st, D, _ = run_split(case, 4, ws_offset=1, c_fill=7.0)
    assert st == 1 and np.all(D[:, :333] == 7.0)
    assert lib.sgemm_f32_splitk_plan(0, 300, 333, 1500, 0)[1] > 1
    st, D, _ = run_split(case, 0, ws_offset=3)
    assert st == 0
    assert_parity(oracle_lib, case, D, "misaligned workspace, plain call")


def test_beta_zero_does_not_read_c(oracle_lib):
    case = make_case(400, 400, 3000, alpha=2.0, beta=0.0, seed=22)
    st, D, _ = run_split(case, 6, c_fill=np.nan)
    assert st == 0 and np.all(np.isfinite(D[:, :400]))
    assert_parity(oracle_lib, case, D, "beta 0, NaN C")


def test_deterministic():
    case = make_case(512, 512, 4096, seed=23)
    _, D1, _ = run_split(case, 8)
    _, D2, _ = run_split(case, 8)
    assert np.array_equal(D1.view(np.uint32), D2.view(np.uint32))


def test_small_workspace_for_explicit_split_is_an_error():
    case = make_case(256, 256, 1024, seed=24)
    st, D, _ = run_split(case, 4, ws_bytes=4 * 256 * 256 * 4 - 4)
    assert st == 1
    assert np.all(np.isnan(D[:, :256]))           # C untouched


def test_torch_wrapper_with_workspace(oracle_lib):
    import torch

    dev = torch.device("cuda", 0)
    case = make_case(512, 384, 2048, trans_b=True, alpha=0.5, beta=0.0, seed=25)
    A, B = torch.from_numpy(case.A).to(dev), torch.from_numpy(case.B).to(dev)
    C = torch.empty(512, 384, device=dev)
    _, used, _, need = lib.sgemm_f32_splitk_plan(0, 512, 384, 2048, 1)
    ws = torch.empty(need // 4, device=dev)
    lib.gemm(A, B, C, alpha=0.5, trans_b=True, workspace=ws)
    lib.gemm(A, B, C, alpha=0.5, trans_b=True, workspace=ws)   # reuse on the same stream
    torch.cuda.synchronize()
    assert used > 1
    assert_parity(oracle_lib, case, C.cpu().numpy(), "wrapper")
