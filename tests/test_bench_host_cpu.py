"""Host-side behaviour of bench.py that needs no GPU: the one-GPU guard, the
warm-up rule and the row shares it can time."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr


class _FakeCuda:
    @staticmethod
    def synchronize():
        pass


class _FakeTorch:
    cuda = _FakeCuda()


def _bench_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_warm_up_runs_the_count_and_the_minimum_time():
    import time
    bench = _bench_module()
    calls = []

    def slow(i):
        calls.append(i)
        time.sleep(0.002)

    t0 = time.perf_counter()
    n = bench.warm_up(_FakeTorch(), slow, 5)
    # an explicit count of 5 still warms for the minimum time, and reports what ran
    assert time.perf_counter() - t0 >= bench.WARMUP_MIN_SECONDS
    assert n == len(calls) > 5 and calls == list(range(n))
    calls.clear()
    n = bench.warm_up(_FakeTorch(), lambda i: calls.append(i), 300)
    assert n == len(calls) >= 300


def test_row_share_is_the_matching_rows_of_the_workload():
    import numpy as np
    import pytest

    from fp32_gemm_08_amd.inputs import make_config, make_row_share

    for name, parts in (("c5_512", 4), ("c3_ragged_bt", 8)):
        whole = make_config(name)
        for index in (0, parts - 1):
            s = make_row_share(name, parts, index)
            r0 = index * whole.M // parts
            assert s.M == whole.M // parts and (s.N, s.K, s.trans_b) == (whole.N, whole.K, whole.trans_b)
            assert np.array_equal(s.A, whole.A[r0:r0 + s.M]) and np.array_equal(s.B, whole.B)
            assert (s.C is None) == (whole.C is None)
            if s.C is not None:
                assert np.array_equal(s.C, whole.C[r0:r0 + s.M])
    with pytest.raises(ValueError):
        make_row_share("c3_ragged_bt", 3)       # 1000 rows do not split in 3
    with pytest.raises(ValueError):
        make_row_share("c5_512", 4, 4)
