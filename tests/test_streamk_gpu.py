"""GPU parity of the stream-K schedule (sgemm_f32_streamk, and sgemm_f32_ws
where it picks stream-K) against the FP64 oracle, through the C ABI.

Same bar as the plain GEMM: |D_gpu - D| <= 4*K*2^-24*S + 1e-6 elementwise,
finite; bit-exact for small-integer inputs, where every summation order is
exact, so a piece added twice, dropped or placed in the wrong tile shows.  The
workspace carries canary floats before and after the planned bytes, and C
canary guard rows and padding columns.
"""
import numpy as np
import pytest

import fp32_gemm_08_amd as lib
from fp32_gemm_08_amd.inputs import make_case
from oracle import check

from gpu_helpers import CANARY, GUARD_ROWS, oracle_rows, sample_rows, say

pytestmark = pytest.mark.gpu

W_CANARY = np.float32(-7777.25)
W_TAIL = 1024
KID_L_SK, KID_M_SK = 43, 44


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert lib.sgemm_f32_version()


def run_sk(case, tile, ws_bytes=None, a_offset=0, ldc_pad=0, ws_offset=4, c_fill=np.nan, auto=False):
    """One call of sgemm_f32_streamk (or sgemm_f32_ws when auto).  Returns
    (status, D, plan)."""
    import torch

    dev = torch.device("cuda", 0)
    M, N, K = case.M, case.N, case.K
    t = int(case.trans_b)
    if auto:
        st, method, kid, need = lib.sgemm_f32_ws_plan(M, N, K, t)
        plan = (st, kid, method, need)
    else:
        st, kid, dp, skt, wk, need = lib.sgemm_f32_streamk_plan(tile, M, N, K, t)
        plan = (st, kid, dp, skt, wk, need)
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
    say(f"streamk tile={tile} auto={auto} plan={plan} M={M} N={N} K={K} transB={t} alpha={case.alpha} "
        f"beta={case.beta} lda={case.lda} ldb={case.ldb} ldc={ldc} ws_bytes={ws_bytes} a_offset={a_offset}")
    args = (M, N, K, case.alpha, dA.data_ptr() + 4 * a_offset, case.lda, dB.data_ptr(), case.ldb, t, case.beta,
            dC.data_ptr() + 4 * g * ldc, ldc, dW.data_ptr() + 4 * ws_offset, ws_bytes, s.cuda_stream)
    st = lib.sgemm_f32_ws(*args) if auto else lib.sgemm_f32_streamk(tile, *args)
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
    return st, out[g:g + M], plan


def assert_parity(o, case, D_gpu, what, rows=None):
    D, S = oracle_rows(o, case, rows)
    Dg = D_gpu[:, :case.N] if rows is None else D_gpu[rows, :case.N]
    r = check(Dg, D, S, case.K)
    say(f"{what}: max_abs={r['max_abs']:.3e} max_rho={r['max_rho']:.3f} fails={r['n_fail']}")
    assert r["ok"], f"{what}: {r}"


# (M, N, K, transB, alpha, beta): all tiles shared (T < 256), whole waves plus a
# remainder, ragged edges, K tails, K shorter than one iteration, one tile.
SHAPES = [(1000, 1017, 999, 1, 1.5, -0.5), (1000, 1000, 1024, 0, 1.0, 0.0), (700, 1300, 333, 0, -0.75, 1.0),
          (2049, 2051, 517, 1, 1.25, 0.5), (256, 256, 4096, 0, 1.0, 1.0), (300, 200, 20, 1, 2.0, 0.0),
          (64, 64, 1, 0, 1.0, 0.5), (1, 700, 3000, 1, 1.0, 0.0)]


@pytest.mark.parametrize("tile", [256, 128])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(str(v) for v in s[:4]))
def test_streamk_full(oracle_lib, tile, shape):
    M, N, K, t, alpha, beta = shape
    case = make_case(M, N, K, trans_b=t, alpha=alpha, beta=beta, dist="uniform", seed=M + 3 * N + K)
    st, D, plan = run_sk(case, tile, ldc_pad=3)
    assert st == 0 and plan[1] == (KID_L_SK if tile == 256 else KID_M_SK)
    assert_parity(oracle_lib, case, D, f"streamk {tile} {M}x{N}x{K} t{t}")


@pytest.mark.parametrize("tile", [256, 128])
@pytest.mark.parametrize("t", [0, 1])
def test_streamk_integers_bit_exact(oracle_lib, tile, t):
    case = make_case(1003, 1004, 1000, trans_b=t, alpha=1.0, beta=1.0, dist="int2", seed=29)
    st, D, plan = run_sk(case, tile)
    assert st == 0 and plan[3] > 0  # tiles were shared out
    Dref, _ = oracle_rows(oracle_lib, case)
    assert np.array_equal(D[:, :1004], Dref.astype(np.float32))


@pytest.mark.parametrize("tile", [256, 128])
def test_streamk_unaligned_and_misaligned(oracle_lib, tile):
    # lda odd (register staging on the 256 tile, 4-byte direct loads on the 128 tile), A off by one float
    case = make_case(1001, 1003, 999, trans_b=0, alpha=1.5, beta=0.25, dist="uniform", seed=31)
    st, D, plan = run_sk(case, tile, a_offset=1, ldc_pad=1)
    assert st == 0
    assert_parity(oracle_lib, case, D, f"streamk {tile} unaligned")


@pytest.mark.parametrize("tile", [256, 128])
def test_streamk_beta_zero_ignores_nan(oracle_lib, tile):
    case = make_case(900, 800, 700, alpha=2.0, beta=0.0, seed=37)
    st, D, _ = run_sk(case, tile, c_fill=np.nan)
    assert st == 0 and np.all(np.isfinite(D[:, :800]))
    assert_parity(oracle_lib, case, D, f"streamk {tile} beta 0")


# Large shapes at the sizes the schedule is for, checked on sampled rows.
LARGE = [(4608, 4608, 4608, 0, 0), (3000, 3000, 3000, 1, 0), (2304, 2304, 8192, 0, 0), (1536, 1536, 4096, 0, 0),
         (6144, 6144, 2048, 1, 256), (5120, 5120, 1024, 0, 128)]


@pytest.mark.parametrize("shape", LARGE, ids=lambda s: "x".join(str(v) for v in s[:4]) + f"_tile{s[4]}")
def test_streamk_large_sampled(oracle_lib, shape):
    M, N, K, t, tile = shape
    case = make_case(M, N, K, trans_b=t, alpha=1.0, beta=1.0, dist="normal", seed=M + K)
    st, D, plan = run_sk(case, tile, ldc_pad=0)
    assert st == 0
    rows = np.unique(np.concatenate([sample_rows(M, n=12, seed=K, tile=128), np.arange(M - 8, M)]))
    assert_parity(oracle_lib, case, D, f"streamk large {M}x{N}x{K}", rows=rows)


def test_ws_auto_picks_streamk(oracle_lib):
    case = make_case(4608, 4608, 1536, trans_b=0, alpha=1.0, beta=0.0, dist="uniform", seed=41)
    st, D, plan = run_sk(case, 0, auto=True)
    assert st == 0 and plan[2] == 2 and plan[1] in (KID_L_SK, KID_M_SK)
    rows = sample_rows(4608, n=16, seed=3, tile=256)
    assert_parity(oracle_lib, case, D, "ws auto stream-K", rows=rows)


def test_streamk_deterministic():
    case = make_case(1000, 1017, 999, trans_b=1, alpha=1.5, beta=-0.5, dist="uniform", seed=43)
    st1, D1, _ = run_sk(case, 256)
    st2, D2, _ = run_sk(case, 256)
    assert st1 == st2 == 0 and np.array_equal(D1.view(np.uint32), D2.view(np.uint32))


def test_streamk_full_waves_need_no_workspace(oracle_lib):
    # 1024 tiles of 128 x 128: whole waves only, the plain schedule, no workspace
    case = make_case(4096, 4096, 256, seed=47)
    st, kid, dp, skt, wk, need = lib.sgemm_f32_streamk_plan(128, 4096, 4096, 256, 0)
    assert (st, dp, skt, wk, need) == (0, 1024, 0, 0, 0)
    st, D, _ = run_sk(case, 128, ws_bytes=0)
    assert st == 0
    assert_parity(oracle_lib, case, D, "streamk whole waves", rows=sample_rows(4096, n=8, seed=5, tile=128))


def test_streamk_misaligned_workspace(oracle_lib):
    # rejected before any launch; sgemm_f32_ws falls back to the plain call
    case = make_case(1000, 1017, 999, trans_b=1, alpha=1.5, beta=-0.5, dist="uniform", seed=44)
    st, D, _ = run_sk(case, 256, ws_offset=1)
    assert st == 1 and np.array_equal(D[:, :1017], case.C[:, :1017])
    big = make_case(4608, 4608, 1536, trans_b=0, alpha=1.0, beta=0.0, dist="uniform", seed=45)
    assert lib.sgemm_f32_ws_plan(4608, 4608, 1536, 0)[1] == 2
    st, D, _ = run_sk(big, 0, auto=True, ws_offset=2)
    assert st == 0
    assert_parity(oracle_lib, big, D, "ws auto, misaligned workspace", rows=sample_rows(4608, n=8, seed=4, tile=256))


def test_streamk_small_workspace_rejected():
    import torch

    dev = torch.device("cuda", 0)
    M = N = K = 1000
    st, kid, dp, skt, wk, need = lib.sgemm_f32_streamk_plan(256, M, N, K, 0)
    assert need > 0
    A = torch.zeros(M, K, device=dev)
    B = torch.zeros(K, N, device=dev)
    C = torch.full((M, N), 5.0, device=dev)
    W = torch.zeros(need // 4, device=dev)
    st = lib.sgemm_f32_streamk(256, M, N, K, 1.0, A.data_ptr(), K, B.data_ptr(), N, 0, 0.0, C.data_ptr(), N,
                               W.data_ptr(), need - 4, 0)
    torch.cuda.synchronize()
    assert st == 1 and torch.all(C == 5.0)
