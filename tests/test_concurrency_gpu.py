"""Host threads calling the library at once, each on its own stream.

The library keeps per-device state that threads share (the cached result of
the architecture check, the static scratch's address) and otherwise only
enqueues kernels on the caller's stream.  Eight Python threads (ctypes drops
the interpreter lock for the duration of each call) start together at a
barrier and each makes its call 25 times on its own torch stream: the plain
call, the call with a workspace of its own, and the transpose, on shapes that
take different kernels.  Every output must carry the bits of the same call
made alone beforehand, which itself meets the oracle's bound.  The
no-allocation k-split shares one scratch per device, and its calls that
overlap race by contract, so it is not among them.
"""
import threading

import numpy as np
import pytest

import fp32_gemm_08_amd as lib
from fp32_gemm_08_amd.inputs import make_case
from oracle import check
from oracle import transpose as oracle_transpose

from gpu_helpers import oracle_rows, say

pytestmark = pytest.mark.gpu

REPEATS = 25

# (kind, M, N, K, transB, alpha, beta) for GEMM jobs; (kind, rows, cols) for the transpose
JOBS = [
    ("plain", 1000, 1017, 999, 1, 1.5, -0.5),
    ("plain", 512, 512, 512, 0, 1.0, 1.0),
    ("plain", 2048, 2048, 256, 0, 1.0, 0.0),
    ("plain", 300, 260, 96, 1, 0.75, 0.0),
    ("ws", 256, 256, 4096, 0, 1.25, 0.5),
    ("ws", 1000, 1017, 999, 1, 1.0, 1.0),
    ("transpose", 3000, 2100),
    ("transpose", 37, 4099),
]


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert lib.sgemm_f32_version()


class Job:
    """One thread's work: device inputs, the output's initial state, and the
    call that enqueues it on a given stream handle."""

    def __init__(self, spec, seed):
        import torch

        dev = torch.device("cuda", 0)
        self.spec = spec
        self.kind = spec[0]
        if self.kind == "transpose":
            _, rows, cols = spec
            self.src_h = np.random.default_rng(seed).standard_normal((rows, cols)).astype(np.float32)
            self.src = torch.from_numpy(self.src_h).to(dev)
            self.out0 = torch.zeros((cols, rows), device=dev)
            self.call = lambda out, s: lib.sgemm_f32_transpose(rows, cols, self.src.data_ptr(), cols,  # noqa
                                                               out.data_ptr(), rows, s)
            return
        _, M, N, K, t, alpha, beta = spec
        self.case = make_case(M, N, K, trans_b=t, alpha=alpha, beta=beta, dist="uniform", seed=seed)
        self.A = torch.from_numpy(self.case.A).to(dev)
        self.B = torch.from_numpy(self.case.B).to(dev)
        self.out0 = torch.from_numpy(self.case.c_storage(0.0)).to(dev)
        args = (M, N, K, alpha, self.A.data_ptr(), self.case.lda, self.B.data_ptr(), self.case.ldb, t, beta)
        if self.kind == "plain":
            self.call = lambda out, s: lib.sgemm_f32(*args, out.data_ptr(), self.case.ldc, s)  # noqa: E731
        else:
            need = max(lib.sgemm_f32_ws_plan(M, N, K, t)[3], 16)
            self.W = torch.empty(need // 4, device=dev)
            self.call = lambda out, s: lib.sgemm_f32_ws(*args, out.data_ptr(), self.case.ldc,  # noqa: E731
                                                        self.W.data_ptr(), need, s)

    def check_reference(self, oracle_lib, D):
        if self.kind == "transpose":
            _, rows, cols = self.spec
            assert np.array_equal(D.view(np.uint32), oracle_transpose(self.src_h, rows, cols).view(np.uint32))
            return
        Dr, S = oracle_rows(oracle_lib, self.case)
        r = check(D[:, :self.case.N], Dr, S, self.case.K)
        assert r["ok"], f"{self.spec}: {r}"


def test_threads_on_their_own_streams(oracle_lib):
    import torch

    dev = torch.device("cuda", 0)
    jobs = [Job(spec, seed=100 + i) for i, spec in enumerate(JOBS)]
    # each call alone first: the reference bits, checked against the oracle
    refs = []
    for job in jobs:
        out = job.out0.clone()
        st = job.call(out, torch.cuda.current_stream(dev).cuda_stream)
        assert st == 0, lib.sgemm_f32_status_string(st)
        torch.cuda.synchronize()
        job.check_reference(oracle_lib, out.cpu().numpy())
        refs.append(out)
    say(f"references done for {len(jobs)} jobs; starting {len(jobs)} threads x {REPEATS} calls")

    start = threading.Barrier(len(jobs))
    errors = []

    def worker(i):
        try:
            job, ref = jobs[i], refs[i]
            s = torch.cuda.Stream(device=dev)
            outs = []
            start.wait()
            with torch.cuda.stream(s):
                for _ in range(REPEATS):
                    out = job.out0.clone()
                    st = job.call(out, s.cuda_stream)
                    if st != 0:
                        raise RuntimeError(f"{job.spec}: {lib.sgemm_f32_status_string(st)}")
                    outs.append(out)
            s.synchronize()
            for n, out in enumerate(outs):
                if not torch.equal(out.view(torch.int32), ref.view(torch.int32)):
                    raise AssertionError(f"{job.spec}: call {n} on its own stream differs from the call alone")
        except BaseException as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(jobs))]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    torch.cuda.synchronize()
    say(f"threads done, {len(errors)} errors")
    if errors:
        raise errors[0]
