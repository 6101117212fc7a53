"""The device check every entry point makes before it enqueues work, without a
GPU: SGEMM_ERR_UNSUPPORTED_ARCH for any architecture but gfx950 (the "no
kernel image" case, "CUDA矩阵乘法性能优化实战：从朴素内核到寄存器分块与Nsight剖析"
section 6.2), and SGEMM_ERR_NO_DEVICE from every entry point, valid calls
included, in a process that sees no GPU.
"""
import os
import subprocess
import sys

import pytest

import fp32_gemm_08_amd as lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NO_DEVICE, UNSUPPORTED = 0, 3, 4


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(lib.LIB_PATH):
        pytest.skip("libsgemm_f32.so not built")


@pytest.mark.parametrize("arch", ["gfx950", "gfx950:sramecc+:xnack-", "gfx950:xnack+", "gfx950:sramecc-"])
def test_gfx950_accepted(arch):
    assert lib.sgemm_f32_arch_status(arch) == OK


@pytest.mark.parametrize("arch", ["gfx942", "gfx942:sramecc+:xnack-", "gfx90a", "gfx908", "gfx1100", "gfx9500",
                                  "gfx95", "gfx9", "GFX950", " gfx950", "gfx950 ", "", ":gfx950", "sm_90", None])
def test_other_architectures_rejected(arch):
    assert lib.sgemm_f32_arch_status(arch) == UNSUPPORTED


# Runs in a child process that is shown no GPU.  Every call below is valid,
# so it proceeds as far as the device check: the child makes them only after
# sgemm_f32_device_status() has reported that no device is there (a process
# that still sees a GPU reports SKIP and calls nothing).
CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
import fp32_gemm_08_amd as lib
st = lib.sgemm_f32_device_status()
if st != 3:
    print("SKIP", st)
    sys.exit(0)
PA, PB, PC, PW = 1 << 32, 1 << 40, 1 << 44, 1 << 48
M = N = K = 512
g = (M, N, K, 1.0, PA, K, PB, N, 0, 0.5, PC, N, 0)
w = g[:-1] + (PW, 1 << 30, 0)
calls = {"sgemm_f32": lib.sgemm_f32(*g), "scale_only": lib.sgemm_f32(M, N, 0, 1.0, PA, 1, PB, N, 0, 0.5, PC, N, 0)}
for name, algo in lib.ALGO.items():
    calls["algo_" + name] = lib.sgemm_f32_algo(algo, *g)
calls["ws"] = lib.sgemm_f32_ws(*w)
calls["splitk"] = lib.sgemm_f32_splitk(4, *w)
calls["streamk_256"] = lib.sgemm_f32_streamk(256, *w)
calls["streamk_128"] = lib.sgemm_f32_streamk(128, *w)
for p in (1, 2):
    calls[f"lowp_{p}"] = lib.sgemm_f32_lowp(p, *g)
    calls[f"lowp_ws_{p}"] = lib.sgemm_f32_lowp_ws(p, 2048, 2048, 2048, 1.0, PA, 2048, PB, 2048, 0, 0.0, PC, 2048,
                                                  PW, 1 << 30, 0)
    calls[f"lowp_2pass_{p}"] = lib.sgemm_f32_lowp_2pass(p, 0, *w)
for name, algo in lib.TRANSPOSE_ALGO.items():
    calls["transpose_" + name] = lib.sgemm_f32_transpose_algo(algo, 300, 200, PA, 200, PB, 300, 0)
calls["transpose"] = lib.sgemm_f32_transpose(300, 200, PA, 200, PB, 300, 0)
calls["probe"] = lib.sgemm_f32_mfma_probe(4, 4, PA, PB, 0)
for p in (1, 2):
    calls[f"probe_lp_{p}"] = lib.sgemm_f32_mfma_probe_lp(p, 0, 4, 4, PA, PB, 0)
calls["load_probe"] = lib.sgemm_f32_load_probe(8, 4, 256, PA, 1 << 30, 4 << 20, 1, 512, PB, 0)
bad = {k: v for k, v in calls.items() if v != 3}
print("BAD", bad if bad else "", len(calls))
"""


def test_no_device_from_every_entry_point():
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1")
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    out = r.stdout.strip().splitlines()[-1]
    if out.startswith("SKIP"):
        pytest.skip(f"the child process still sees a device (status {out.split()[1]})")
    assert out.startswith("BAD") and out.split()[1].isdigit(), out
    assert int(out.split()[1]) >= 20


def test_status_strings_name_the_device_errors():
    assert "device" in lib.sgemm_f32_status_string(NO_DEVICE).lower()
    assert "gfx950" in lib.sgemm_f32_status_string(UNSUPPORTED)
