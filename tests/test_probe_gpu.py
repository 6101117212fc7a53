"""GPU checks of the probes (sgemm_f32_mfma_probe, sgemm_f32_mfma_probe_lp, sgemm_f32_load_probe),
through the C ABI.

The probe is the measurement behind the FP32 roofline's unit rate: one
v_mfma_f32_32x32x2_f32 (4096 FLOP) per 64 shader cycles on each SIMD.  With
one wavefront per SIMD, a wavefront's chain of MFMAs must take 64 cycles per
MFMA (the chain is never stalled on a result: four independent accumulators),
and its clock readings must be a plausible shader clock.  The work-item sums
it writes have a closed form only in distribution, so they are checked for
being finite and written everywhere.

The 16-bit probe's unit rate is one v_mfma_f32_32x32x16 (32768 FLOP) per 32
cycles; its all-zero operands give sums of exactly zero.  The load probe has
no result but its timing: it must write one plausible pair per workgroup and
nothing else.
"""
import numpy as np
import pytest

import fp32_gemm_08_amd as lib

from gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch, torch.device("cuda", 0)


def run_probe(torch, dev, workgroups, trips):
    sink = torch.full((workgroups * 256 + 64,), float("nan"), dtype=torch.float32, device=dev)
    clocks = torch.zeros(workgroups * 2 + 8, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)
    say(f"mfma probe: {workgroups} workgroups x {trips} trips")
    st = lib.sgemm_f32_mfma_probe(workgroups, trips, sink.data_ptr(), clocks.data_ptr(), stream.cuda_stream)
    torch.cuda.synchronize()
    assert st == 0, lib.sgemm_f32_status_string(st)
    return sink.cpu().numpy(), clocks.cpu().numpy()


def test_one_wavefront_per_simd_issues_an_mfma_every_64_cycles(torch_dev):
    torch, dev = torch_dev
    wg, trips = 8, 4000                       # a few workgroups: one wavefront on each SIMD they land on
    run_probe(torch, dev, wg, trips)          # brings the clock up
    sink, clocks = run_probe(torch, dev, wg, trips)
    c = clocks[:2 * wg].reshape(wg, 2).astype(np.float64)
    assert np.all(c[:, 1] > 0) and np.all(c[:, 0] > 0)
    cyc = c[:, 0] / (trips * 8)
    mhz = 100.0 * c[:, 0] / c[:, 1]
    say(f"cycles per MFMA {np.median(cyc):.2f} (min {cyc.min():.2f}), clock {np.median(mhz):.0f} MHz")
    assert 62.0 <= np.median(cyc) <= 70.0
    assert 300.0 <= np.median(mhz) <= 3000.0
    assert np.all(np.isfinite(sink[:wg * 256])) and np.all(np.isnan(sink[wg * 256:]))
    assert np.all(clocks[2 * wg:] == 0)       # nothing written past the last workgroup's pair


def test_full_chip_rate_is_near_the_unit_count(torch_dev):
    torch, dev = torch_dev
    wg, trips = 512, 4000                     # two wavefronts per SIMD on every CU
    for _ in range(3):
        run_probe(torch, dev, wg, trips)
    stream = torch.cuda.current_stream(dev)
    sink = torch.empty(wg * 256, dtype=torch.float32, device=dev)
    clocks = torch.zeros(wg * 2, dtype=torch.int64, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        assert lib.sgemm_f32_mfma_probe(wg, trips, sink.data_ptr(), clocks.data_ptr(), stream.cuda_stream) == 0
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / 10
    c = clocks.cpu().numpy().reshape(wg, 2).astype(np.float64)
    mhz = float(np.mean(100.0 * c[:, 0] / c[:, 1]))
    tflops = wg * trips * 4 * 8 * 4096.0 / t / 1e12
    # 256 CUs x 4 SIMDs x 4096 FLOP / 64 cycles at the measured clock
    expect = 1024 * 64.0 * mhz * 1e6 / 1e12
    say(f"probe {tflops:.1f} TFLOP/s at {mhz:.0f} MHz (unit count at that clock: {expect:.1f})")
    assert 0.85 * expect <= tflops <= 1.02 * expect


def run_probe_lp(torch, dev, precision, zero, workgroups, trips):
    sink = torch.full((workgroups * 256 + 64,), float("nan"), dtype=torch.float32, device=dev)
    clocks = torch.zeros(workgroups * 2 + 8, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)
    say(f"16-bit mfma probe: precision {precision}, zero operands {zero}, {workgroups} workgroups x {trips} trips")
    st = lib.sgemm_f32_mfma_probe_lp(precision, zero, workgroups, trips, sink.data_ptr(), clocks.data_ptr(),
                                     stream.cuda_stream)
    torch.cuda.synchronize()
    assert st == 0, lib.sgemm_f32_status_string(st)
    return sink.cpu().numpy(), clocks.cpu().numpy()


@pytest.mark.parametrize("precision", [1, 2], ids=["fp16", "bf16"])
def test_16bit_chain_issues_an_mfma_every_32_cycles(torch_dev, precision):
    """v_mfma_f32_32x32x16_{f16,bf16}: 32768 FLOP per 32 cycles on a SIMD (the unit rate behind the
    published 2.5 PFLOP/s at 2.4 GHz).  All-zero operands must sum to exactly zero."""
    torch, dev = torch_dev
    wg, trips = 8, 4000
    run_probe_lp(torch, dev, precision, 0, wg, trips)
    sink, clocks = run_probe_lp(torch, dev, precision, 0, wg, trips)
    c = clocks[:2 * wg].reshape(wg, 2).astype(np.float64)
    assert np.all(c[:, 1] > 0) and np.all(c[:, 0] > 0)
    cyc = c[:, 0] / (trips * 8)
    mhz = 100.0 * c[:, 0] / c[:, 1]
    say(f"cycles per MFMA {np.median(cyc):.2f} (min {cyc.min():.2f}), clock {np.median(mhz):.0f} MHz")
    assert 31.0 <= np.median(cyc) <= 36.0
    assert 300.0 <= np.median(mhz) <= 3000.0
    assert np.all(np.isfinite(sink[:wg * 256])) and np.all(np.isnan(sink[wg * 256:]))
    assert np.all(clocks[2 * wg:] == 0)
    sink0, _ = run_probe_lp(torch, dev, precision, 1, wg, trips)
    assert np.all(sink0[:wg * 256] == 0.0) and np.all(np.isnan(sink0[wg * 256:]))


def test_load_probe_streams_into_lds(torch_dev):
    """Direct global->LDS loads, 8 wavefronts x 4 in flight on every CU, from an L2-resident
    region: each workgroup times its whole stream; the rate per CU must be a plausible share of an
    L1 that returns at most 128 bytes a cycle, and nothing past the last workgroup's pair is written."""
    torch, dev = torch_dev
    wg, waves, depth, region, share = 256, 8, 4, 256 << 10, 32
    loads = (1 << 20) // (waves * 1024)
    src_bytes = 8 * region
    src = torch.zeros(src_bytes // 4, dtype=torch.float32, device=dev)
    clocks = torch.zeros(wg * 2 + 8, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)
    say(f"load probe: {wg} workgroups x {waves} wavefronts, {depth} in flight, region {region}, share {share}")
    for _ in range(3):
        st = lib.sgemm_f32_load_probe(waves, depth, wg, src.data_ptr(), src_bytes, region, share, loads,
                                      clocks.data_ptr(), stream.cuda_stream)
        assert st == 0, lib.sgemm_f32_status_string(st)
    torch.cuda.synchronize()
    c = clocks.cpu().numpy()
    per = c[:2 * wg].reshape(wg, 2).astype(np.float64)
    assert np.all(per > 0)
    bpc = loads * waves * 1024.0 / per[:, 0]
    say(f"bytes per CU-cycle: median {np.median(bpc):.1f}, min {bpc.min():.1f}, max {bpc.max():.1f}")
    assert 4.0 <= np.median(bpc) <= 128.0
    assert np.all(c[2 * wg:] == 0)
    # a source one byte short of the regions read is refused before any launch
    assert lib.sgemm_f32_load_probe(waves, depth, wg, src.data_ptr(), src_bytes - 1, region, share, loads,
                                    clocks.data_ptr(), stream.cuda_stream) == 1
