"""The entry points under HIP graph capture.

The library enqueues kernels on the caller's stream and nothing else: no
allocation, no copy, no memset, no synchronisation.  So a caller can record a
call into a HIP graph (here through torch.cuda.graph, whose capture stream is
the current stream during the `with` block) and replay it.  Each case records
one call after an eager call of the same arguments (which fills the library's
per-device caches outside the capture), then replays the graph five times,
with eager work of the program between the replays (C reset to its input by
a copy, the caller's own kernels), and checks every replay's output bit for
bit against the eager result, which itself meets the oracle's bound.
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


def _replay_matches(call, C, C0, what):
    """call(stream_handle) enqueues the GEMM; C is the output tensor, C0 its
    input state.  Returns the eager output."""
    import torch

    dev = C.device
    C.copy_(C0)
    st = call(torch.cuda.current_stream(dev).cuda_stream)
    assert st == 0, lib.sgemm_f32_status_string(st)
    torch.cuda.synchronize()
    eager = C.clone()
    g = torch.cuda.CUDAGraph()
    C.copy_(C0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        st = call(torch.cuda.current_stream(dev).cuda_stream)
    assert st == 0, lib.sgemm_f32_status_string(st)
    scratch = torch.empty(1 << 20, device=dev)
    for rep in range(5):
        say(f"graph {what}: replay {rep}")
        C.copy_(C0)
        scratch.normal_()                  # the program's own work between the replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C.view(torch.int32), eager.view(torch.int32)), f"{what}: replay {rep} differs"
    return eager


def _device_case(case):
    import torch

    dev = torch.device("cuda", 0)
    A = torch.from_numpy(case.A).to(dev)
    B = torch.from_numpy(case.B).to(dev)
    C0 = torch.from_numpy(case.c_storage(0.0)).to(dev)
    return A, B, C0, C0.clone()


def _assert_oracle(oracle_lib, case, D, what):
    Dr, S = oracle_rows(oracle_lib, case)
    r = check(D[:, :case.N], Dr, S, case.K)
    say(f"{what}: max_rho={r['max_rho']:.3f}")
    assert r["ok"], f"{what}: {r}"


@pytest.mark.parametrize("shape", [(1000, 1017, 999, 1, 1.5, -0.5), (512, 512, 512, 0, 1.0, 1.0),
                                   (2048, 2048, 1024, 0, 1.0, 0.0)], ids=lambda s: "x".join(map(str, s[:4])))
def test_plain_call_in_a_graph(oracle_lib, shape):
    M, N, K, t, alpha, beta = shape
    case = make_case(M, N, K, trans_b=t, alpha=alpha, beta=beta, dist="uniform", seed=M + K)
    A, B, C0, C = _device_case(case)
    call = lambda s: lib.sgemm_f32(M, N, K, alpha, A.data_ptr(), case.lda, B.data_ptr(), case.ldb, t, beta,  # noqa
                                   C.data_ptr(), case.ldc, s)
    D = _replay_matches(call, C, C0, f"sgemm_f32 {M}x{N}x{K}")
    _assert_oracle(oracle_lib, case, D.cpu().numpy(), "graph plain")


@pytest.mark.parametrize("kind", ["splitk", "streamk", "noalloc"])
def test_workspace_schedules_in_a_graph(oracle_lib, kind):
    import torch

    if kind == "streamk":
        M, N, K, t = 1000, 1017, 999, 1
    else:
        M, N, K, t = 256, 256, 4096, 0
    case = make_case(M, N, K, trans_b=t, alpha=1.25, beta=0.5, dist="uniform", seed=K + 7)
    A, B, C0, C = _device_case(case)
    args = (M, N, K, case.alpha, A.data_ptr(), case.lda, B.data_ptr(), case.ldb, t, case.beta, C.data_ptr(),
            case.ldc)
    if kind == "splitk":
        need = lib.sgemm_f32_splitk_plan(0, M, N, K, t)[3]
        assert need > 0
        W = torch.empty(need // 4, device=A.device)
        call = lambda s: lib.sgemm_f32_ws(*args, W.data_ptr(), need, s)  # noqa: E731
    elif kind == "streamk":
        need = lib.sgemm_f32_streamk_plan(256, M, N, K, t)[5]
        W = torch.empty(need // 4, device=A.device)
        call = lambda s: lib.sgemm_f32_streamk(256, *args, W.data_ptr(), need, s)  # noqa: E731
    else:
        call = lambda s: lib.sgemm_f32_splitk_noalloc(0, *args, s)  # noqa: E731
    D = _replay_matches(call, C, C0, kind)
    _assert_oracle(oracle_lib, case, D.cpu().numpy(), f"graph {kind}")


def test_transpose_in_a_graph():
    import torch

    from oracle import transpose as oracle_transpose

    dev = torch.device("cuda", 0)
    rows, cols = 3000, 2100
    src_h = np.random.default_rng(5).standard_normal((rows, cols)).astype(np.float32)
    src = torch.from_numpy(src_h).to(dev)
    dst0 = torch.zeros((cols, rows), device=dev)
    dst = dst0.clone()
    call = lambda s: lib.sgemm_f32_transpose(rows, cols, src.data_ptr(), cols, dst.data_ptr(), rows, s)  # noqa
    out = _replay_matches(call, dst, dst0, "transpose")
    assert np.array_equal(out.cpu().numpy().view(np.uint32), oracle_transpose(src_h, rows, cols).view(np.uint32))
