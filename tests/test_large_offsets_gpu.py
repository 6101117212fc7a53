"""Element offsets beyond 2^31 and 2^32: operands and outputs whose rows sit
gigabytes apart.

The leading dimensions here put a matrix's last row more than 2^31 floats
(8 GiB) past its first, and for the 520-row cases more than 2^32 floats, so
any 32-bit product of a row index and a leading dimension would wrap.  Two
regimes of the MFMA kernels are covered: a leading dimension of 2^23 or more,
where the host routes the operands through the register staging path with
64-bit row offsets, and one just below 2^23, the largest the 16-byte direct
path takes (a 256-row tile's offsets then stay under 2^31, and the tile's base
row is a 64-bit offset).  The gaps between an operand's rows hold NaN, so a
read from a wrong row shows in the result.  C's storage is filled with a
canary, which the words before its first row and after each row's end must
keep.  Results meet the oracle's bound (the same values
computed on compact copies), for every algorithm, the workspace schedules, the
mixed-precision calls and the transpose.
"""
import numpy as np
import pytest

import fp32_gemm_08_amd as lib
from fp32_gemm_08_amd.inputs import make_case
from oracle import check, gemm_lowp_rows
from oracle import transpose as oracle_transpose

from gpu_helpers import ALGOS, CANARY, oracle_rows, say

pytestmark = pytest.mark.gpu

FAR = (1 << 23) + 3      # register staging path (>= 2^23), rows not 16-byte aligned
FAR_VEC = (1 << 23) + 4  # the same with 16-byte aligned rows
NEAR = (1 << 23) - 5     # the largest leading dimensions the direct path takes
LEAD = 64                # canary words before each big allocation's first element
TAIL = 256               # and after its last row

MFMA_ALGOS = ALGOS + ["mfma_256", "mfma_128", "mfma_64"]


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert lib.sgemm_f32_version()


@pytest.fixture(autouse=True)
def free_device_memory():
    yield
    import torch
    torch.cuda.empty_cache()


def _strided(values, ld, fill=None):
    """Device storage of `values` (rows x cols) with leading dimension ld,
    LEAD words before the first element and TAIL after the last row.
    Returns (storage, view, address of element (0, 0))."""
    import torch

    dev = torch.device("cuda", 0)
    rows, cols = values.shape
    total = LEAD + (rows - 1) * ld + cols + TAIL
    say(f"  storage {rows}x{cols} ld={ld}: {total * 4 / 2 ** 30:.2f} GiB, last row at float {(rows - 1) * ld}")
    store = torch.empty(total, dtype=torch.float32, device=dev)
    if fill is not None:
        store.fill_(float(fill))
    view = store.as_strided((rows, cols), (ld, 1), LEAD)
    view.copy_(torch.from_numpy(np.ascontiguousarray(values)).to(dev))
    return store, view, store.data_ptr() + 4 * LEAD


def _read(view):
    return view.contiguous().cpu().numpy()


def _assert_canary_around_rows(store, rows, cols, ld, what):
    """The words before the first row, in the gaps after sampled rows and after
    the last row still hold the canary."""
    want = CANARY.view(np.uint32)
    head = store[:LEAD].cpu().numpy()
    assert np.all(head.view(np.uint32) == want), f"{what}: write before the first row"
    for r in sorted({0, 1, rows // 2, rows - 2, rows - 1}):
        gap = TAIL if r == rows - 1 else min(TAIL, ld - cols)
        if gap <= 0:
            continue
        start = LEAD + r * ld + cols
        seg = store[start:start + gap].cpu().numpy()
        assert np.all(seg.view(np.uint32) == want), f"{what}: write after row {r}"


def _compact(M, N, K, t, alpha, beta, seed):
    return make_case(M, N, K, trans_b=t, alpha=alpha, beta=beta, dist="uniform", seed=seed)


# (name, M, N, K, transB, lda, ldb, ldc, beta)
FAR_CASES = [
    ("A_register_path", 300, 136, 96, 0, FAR, None, None, 0.0),
    ("A_direct_path", 520, 200, 64, 0, NEAR, None, None, 0.0),
    ("Bt_register_path", 136, 300, 96, 1, None, FAR, None, 0.0),
    ("Bt_direct_path", 200, 520, 64, 1, None, NEAR, None, 0.0),
    ("A_register_path_aligned", 260, 136, 96, 0, FAR_VEC, None, None, 0.0),
    ("B_register_path_aligned", 136, 64, 300, 0, None, FAR_VEC, None, 0.0),
    ("C_far_rows", 300, 136, 96, 0, None, None, FAR, 0.5),
    ("C_far_rows_aligned", 300, 136, 96, 0, None, None, FAR_VEC, 0.5),
]


def _device_operands(case, lda, ldb, ldc):
    """A, B and C on the device; a None leading dimension keeps that matrix
    compact (no gaps).  C is canary-filled around its rows."""
    import torch

    dev = torch.device("cuda", 0)
    keep = []
    if lda is None:
        dA = torch.from_numpy(case.A.copy()).to(dev)
        pa, lda = dA.data_ptr(), case.lda
    else:
        dA, _, pa = _strided(case.A, lda, fill=np.nan)
    keep.append(dA)
    if ldb is None:
        dB = torch.from_numpy(case.B.copy()).to(dev)
        pb, ldb = dB.data_ptr(), case.ldb
    else:
        dB, _, pb = _strided(case.B, ldb, fill=np.nan)
    keep.append(dB)
    ldc = case.N if ldc is None else ldc
    C0 = case.C if case.C is not None else np.full((case.M, case.N), np.nan, np.float32)
    dC, vC, pc = _strided(C0[:, :case.N], ldc, fill=CANARY)
    return keep, (pa, lda, pb, ldb, pc, ldc), dC, vC


@pytest.mark.parametrize("shape", FAR_CASES, ids=lambda s: s[0])
def test_far_rows_every_algorithm(oracle_lib, shape):
    import torch

    name, M, N, K, t, lda, ldb, ldc, beta = shape
    case = _compact(M, N, K, t, 1.25, beta, seed=M + N + K)
    Dr, S = oracle_rows(oracle_lib, case)
    keep, (pa, lda_, pb, ldb_, pc, ldc_), dC, vC = _device_operands(case, lda, ldb, ldc)
    C0 = torch.from_numpy(case.C[:, :N].copy()).to(dC.device) if case.C is not None else None
    for algo in MFMA_ALGOS:
        if C0 is not None:
            vC.copy_(C0)
        say(f"{name} algo={algo} M={M} N={N} K={K} transB={t} lda={lda_} ldb={ldb_} ldc={ldc_} beta={beta}")
        st = lib.sgemm_f32_algo(lib.ALGO[algo], M, N, K, case.alpha, pa, lda_, pb, ldb_, t, beta, pc, ldc_,
                                torch.cuda.current_stream(dC.device).cuda_stream)
        torch.cuda.synchronize()
        assert st == 0, lib.sgemm_f32_status_string(st)
        r = check(_read(vC), Dr, S, K)
        say(f"   max_rho={r['max_rho']:.3f}")
        assert r["ok"], f"{name} {algo}: {r}"
        _assert_canary_around_rows(dC, M, N, ldc_, f"{name} {algo}")
    del keep, dC, vC


@pytest.mark.parametrize("kind", ["splitk", "streamk", "noalloc"])
def test_far_rows_workspace_schedules(oracle_lib, kind):
    import torch

    M, N, K, t = 300, 136, 2048, 0
    case = _compact(M, N, K, t, 0.75, 0.5, seed=K + 3)
    Dr, S = oracle_rows(oracle_lib, case)
    keep, (pa, lda, pb, ldb, pc, ldc), dC, vC = _device_operands(case, FAR, None, FAR)
    dev = dC.device
    sp = torch.cuda.current_stream(dev).cuda_stream
    args = (M, N, K, case.alpha, pa, lda, pb, ldb, t, case.beta, pc, ldc)
    say(f"far rows {kind} M={M} N={N} K={K} lda={lda} ldc={ldc}")
    if kind == "splitk":
        need = lib.sgemm_f32_splitk_plan(4, M, N, K, t)[3]
        W = torch.empty(max(need, 4) // 4, device=dev)
        st = lib.sgemm_f32_splitk(4, *args, W.data_ptr(), need, sp)
    elif kind == "streamk":
        need = lib.sgemm_f32_streamk_plan(128, M, N, K, t)[5]
        W = torch.empty(max(need, 4) // 4, device=dev)
        st = lib.sgemm_f32_streamk(128, *args, W.data_ptr(), need, sp)
    else:
        st = lib.sgemm_f32_splitk_noalloc(4, *args, sp)
    torch.cuda.synchronize()
    assert st == 0, lib.sgemm_f32_status_string(st)
    r = check(_read(vC), Dr, S, K)
    say(f"   max_rho={r['max_rho']:.3f}")
    assert r["ok"], f"{kind}: {r}"
    _assert_canary_around_rows(dC, M, N, ldc, kind)
    del keep, dC, vC


@pytest.mark.parametrize("prec", ["fp16", "bf16"])
@pytest.mark.parametrize("two_pass", [False, True])
def test_far_rows_mixed_precision(prec, two_pass):
    import torch

    M, N, K, t = 300, 136, 96, 1
    case = _compact(M, N, K, t, 1.0, -0.5, seed=11)
    D, S, _ = gemm_lowp_rows(prec, M, N, K, case.alpha, case.A, case.B, t, case.beta, case.C)
    keep, (pa, lda, pb, ldb, pc, ldc), dC, vC = _device_operands(case, FAR, FAR, FAR)
    dev = dC.device
    sp = torch.cuda.current_stream(dev).cuda_stream
    p = lib.PRECISION[prec]
    say(f"far rows lowp {prec} two_pass={two_pass} M={M} N={N} K={K} lda={lda} ldb={ldb} ldc={ldc}")
    if two_pass:
        need = lib.sgemm_f32_lowp_2pass_plan(p, 0, M, N, K, t)[4]
        assert need > 0
        W = torch.empty(need // 4, device=dev)
        st = lib.sgemm_f32_lowp_2pass(p, 0, M, N, K, case.alpha, pa, lda, pb, ldb, t, case.beta, pc, ldc,
                                      W.data_ptr(), need, sp)
    else:
        st = lib.sgemm_f32_lowp(p, M, N, K, case.alpha, pa, lda, pb, ldb, t, case.beta, pc, ldc, sp)
    torch.cuda.synchronize()
    assert st == 0, lib.sgemm_f32_status_string(st)
    r = check(_read(vC), D, S, K)
    say(f"   max_rho={r['max_rho']:.3f}")
    assert r["ok"], f"lowp {prec}: {r}"
    _assert_canary_around_rows(dC, M, N, ldc, f"lowp {prec}")
    del keep, dC, vC


@pytest.mark.parametrize("algo", list(lib.TRANSPOSE_ALGO))
@pytest.mark.parametrize("far", ["src", "src_vec", "dst"])
def test_far_rows_transpose(algo, far):
    import torch

    dev = torch.device("cuda", 0)
    rows, cols = (300, 64) if far != "dst" else (64, 300)
    src_h = np.random.default_rng(rows + cols).standard_normal((rows, cols)).astype(np.float32)
    want = oracle_transpose(src_h, rows, cols)
    if far == "dst":
        src = torch.from_numpy(src_h).to(dev)
        ps, ld_src = src.data_ptr(), cols
        dst, vdst, pd = _strided(np.full((cols, rows), CANARY, np.float32), FAR, fill=CANARY)
        ld_dst = FAR
    else:
        ld_src = FAR if far == "src" else FAR_VEC
        src, _, ps = _strided(src_h, ld_src, fill=np.nan)
        dst = torch.full((LEAD + cols * rows + TAIL,), float(CANARY), device=dev)
        vdst = dst.as_strided((cols, rows), (rows, 1), LEAD)
        pd, ld_dst = dst.data_ptr() + 4 * LEAD, rows
    say(f"far rows transpose {algo} {rows}x{cols} ld_src={ld_src} ld_dst={ld_dst}")
    st = lib.sgemm_f32_transpose_algo(lib.TRANSPOSE_ALGO[algo], rows, cols, ps, ld_src, pd, ld_dst,
                                      torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.synchronize()
    assert st == 0, lib.sgemm_f32_status_string(st)
    assert np.array_equal(_read(vdst).view(np.uint32), want.view(np.uint32))
    _assert_canary_around_rows(dst, cols, rows, ld_dst, f"transpose {algo}")
    del src, dst, vdst
