"""Host-side behaviour of bench.py that needs no GPU: the one-GPU guard."""
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
