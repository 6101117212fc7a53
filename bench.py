#!/usr/bin/env python3
"""FP32 GEMM throughput on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config c4_4096] [--algo auto]

A step is one call of the C ABI (``sgemm_f32``) over the whole workload, inputs
already resident in HBM.  The default workload is 4096x4096x4096, C = A*B,
alpha=1, beta=0, A and B uniform[-1,1) from seed 3.  W untimed warm-up calls
(default: at least 200 and at least 0.4 s of device time, so the engine clock
has reached its loaded state; the line reports the count run), then exactly K
timed calls (default 100) bracketed by device synchronisation; the JSON line
on stdout carries the throughput, the dominant kernel's roofline position
(its own average duration measured with events on the launch stream) and the
FP64 CPU oracle's rate on a bounded sample of the same workload.

Other modes:
  --copy-calibration   run a plain device copy of known size (for scaling the
                       FETCH_SIZE / WRITE_SIZE counters) and exit.
  --op transpose       the library's second operation, the out-of-place FP32
                       transpose (default workload 4096x4096, the size the
                       transpose page measures): one JSON line in GB/s against
                       the HBM roofline.  Each step transposes the next of
                       several source/destination pairs whose total exceeds the
                       256 MB Infinity Cache, so every step streams from HBM.
  --sweep              every algorithm on every workload of the chosen --op,
                       as a table.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP32_MFMA_PEAK_TFLOPS = 157.3   # matrix cores: 256 CU x 256 FLOP/clk x 2.4 GHz
FP32_VALU_PEAK_TFLOPS = 157.3   # vector ALU, same published figure (256 CU x 4 SIMD x 64 FLOP/clk x 2.4 GHz)
HALF_MFMA_PEAK_TFLOPS = 2500.0  # dense fp16 / bf16 matrix cores (published MI355X figure)
HBM_PEAK_GBS = 8000.0
METRIC = "FP32 GEMM TFLOP/s at 4096³ (and % of MI355X FP32 peak), 1 GPU"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_mfma_c4_4096.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "fp32_gemm_08_amd", "csrc", f) for f in ("k_mfma.hip", "sgemm_internal.h")]
TRANSPOSE_METRIC = "FP32 transpose effective bandwidth GB/s at 4096x4096 (and % of MI355X HBM peak), 1 GPU"
TRANSPOSE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_transpose_t_4096.txt")
TRANSPOSE_SOURCES = [os.path.join(ROOT, "fp32_gemm_08_amd", "csrc", f)
                     for f in ("k_transpose.hip", "transpose_internal.h", "sgemm_internal.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(sources=KERNEL_SOURCES):
    h = hashlib.sha256()
    for p in sources:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(path=TRAFFIC_FILE, sources=KERNEL_SOURCES):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source (else None)."""
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path, encoding="utf-8"):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash(sources):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(nbytes=1 << 30, reps=5):
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} copies of {nbytes} bytes ({nbytes // 1024} KiB read and written each)")


def cpu_baseline(case, D_gpu_host, target_s, precision=None):
    """Time the FP64 oracle on a bounded sample of the same workload (whole
    output rows), and check those rows of the GPU result against it.  With a
    precision, the mixed-precision oracle (operands rounded first)."""
    import numpy as np

    import oracle
    M, N, K = case.M, case.N, case.K
    if precision is not None:
        import dataclasses
        case = dataclasses.replace(case, A=oracle.round_to(precision, case.A), B=oracle.round_to(precision, case.B))
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    rng = np.random.default_rng(12345)
    # calibrate with one row per thread
    rows = np.sort(rng.choice(M, size=min(M, threads), replace=False))
    t0 = time.perf_counter()
    oracle.gemm_rows(M, N, K, case.alpha, case.A, case.B, case.trans_b, case.beta, case.C, rows=rows,
                     nthreads=threads)
    t_cal = time.perf_counter() - t0
    per_row = t_cal / len(rows) * threads  # single-row cost on one thread
    n_rows = int(max(threads, min(M, round(target_s * threads / max(per_row, 1e-9)))))
    n_rows = max(threads, (n_rows // threads) * threads)
    n_rows = min(n_rows, M)
    rows = np.sort(rng.choice(M, size=n_rows, replace=False))
    t0 = time.perf_counter()
    D, S, used = oracle.gemm_rows(M, N, K, case.alpha, case.A, case.B, case.trans_b, case.beta, case.C,
                                  rows=rows, nthreads=threads)
    t = time.perf_counter() - t0
    chk = oracle.check(D_gpu_host[rows, :N], D, S, K)
    flops = 2.0 * n_rows * N * K
    return {
        "value": flops / t / 1e12,
        "unit": "TFLOP/s",
        "cores": int(used),
        "kind": "oracle",
        "sample": f"{n_rows} of {M} output rows (all {N} columns, K={K}) of the same product, "
                  f"FP64 triple loop with the |a*b| sum, {t:.1f} s",
        "seconds": t,
        "sample_parity": {"ok": bool(chk["ok"]), "max_rho": chk["max_rho"], "rows": int(n_rows)},
    }


def sweep(algos=("naive", "naive_wg", "lds_tiled", "lds_tiled_nopad", "regblock", "mfma")):
    """Every algorithm on every workload: average kernel time over back-to-back
    calls (after a warm-up that brings the engine clock to its steady state)."""
    import torch

    import fp32_gemm_08_amd as lib
    from fp32_gemm_08_amd.inputs import CONFIGS, make_config
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    w = torch.rand(4096, 4096, device=dev)
    wc = torch.empty_like(w)
    for _ in range(300):
        lib.gemm(w, w, wc, algo="mfma")
    torch.cuda.synchronize()
    del w, wc
    rows = []
    print("| workload | algorithm | kernel | calls | avg ms | TFLOP/s | % of 157.3 |")
    print("|---|---|---|---|---|---|---|")
    for name in CONFIGS:
        case = make_config(name)
        M, N, K = case.M, case.N, case.K
        dA = torch.from_numpy(case.A).to(dev)
        dB = torch.from_numpy(case.B).to(dev)
        dC = torch.zeros((M, case.ldc), dtype=torch.float32, device=dev)
        if case.C is not None:
            dC.copy_(torch.from_numpy(case.C))
        flop = 2.0 * M * N * K
        for algo in algos:
            a = lib.ALGO[algo]
            st, kid, tm, tn, kname = lib.sgemm_f32_plan(a, M, N, K, case.alpha, dA.data_ptr(), case.lda,
                                                        dB.data_ptr(), case.ldb, int(case.trans_b), case.beta,
                                                        dC.data_ptr(), case.ldc)
            rate = 3e12 if algo in ("naive", "naive_wg", "lds_tiled", "lds_tiled_nopad") else 60e12
            reps = int(max(3, min(200, 0.2 / max(flop / rate, 1e-7))))

            def call():
                s = lib.sgemm_f32_algo(a, M, N, K, case.alpha, dA.data_ptr(), case.lda, dB.data_ptr(), case.ldb,
                                       int(case.trans_b), case.beta, dC.data_ptr(), case.ldc, stream.cuda_stream)
                if s != 0:
                    raise RuntimeError(lib.sgemm_f32_status_string(s))

            settle(torch, call, 0.2)
            for _ in range(max(2, reps // 4)):
                call()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(reps):
                call()
            e1.record(stream)
            torch.cuda.synchronize()
            avg = e0.elapsed_time(e1) * 1e-3 / reps
            tf = flop / avg / 1e12
            print(f"| {name} {M}x{N}x{K}{' B^T' if case.trans_b else ''} | {algo} | {kname.split()[0]} | {reps} | "
                  f"{avg * 1e3:.4f} | {tf:.2f} | {100 * tf / FP32_MFMA_PEAK_TFLOPS:.1f} |", flush=True)
            rows.append(dict(workload=name, algo=algo, kernel=kname, ms=avg * 1e3, tflops=tf))
        del dA, dB, dC
        torch.cuda.empty_cache()
    return rows


def oracle_table(target_s=8.0):
    """Time the FP64 oracle (reported only, not a target) on every GEMM workload
    with all the host's threads: whole products where they take a few seconds,
    otherwise a sample of whole output rows sized to about ``target_s``; plus
    single-thread times for the two smallest workloads."""
    import numpy as np

    import oracle
    from fp32_gemm_08_amd.inputs import CONFIGS, make_config
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    print(f"| workload | threads | rows timed | seconds | GFLOP/s |")
    print("|---|---|---|---|---|")
    for name in CONFIGS:
        case = make_config(name)
        M, N, K = case.M, case.N, case.K
        runs = [threads] + ([1] if name in ("c1_128", "c2_1024") else [])
        for th in runs:
            rng = np.random.default_rng(7)
            rows = np.sort(rng.choice(M, size=min(M, th), replace=False))
            t0 = time.perf_counter()
            oracle.gemm_rows(M, N, K, case.alpha, case.A, case.B, case.trans_b, case.beta, case.C, rows=rows,
                             nthreads=th)
            per_row = (time.perf_counter() - t0) / len(rows) * th
            n_rows = min(M, max(th, int(target_s * th / max(per_row, 1e-9)) // th * th))
            rows = np.arange(M) if n_rows >= M else np.sort(rng.choice(M, size=n_rows, replace=False))
            t0 = time.perf_counter()
            _, _, used = oracle.gemm_rows(M, N, K, case.alpha, case.A, case.B, case.trans_b, case.beta, case.C,
                                          rows=rows, nthreads=th)
            t = time.perf_counter() - t0
            print(f"| {name} {M}x{N}x{K} | {used} | {len(rows)} of {M} | {t:.2f} | "
                  f"{2.0 * len(rows) * N * K / t / 1e9:.2f} |", flush=True)


# Shapes for the MFMA tile-choice table: squares from 768 to 8192 and
# rectangles whose tile counts fall just above or below a multiple of 256.
TILE_SWEEP_SHAPES = [(n, n, n) for n in (768, 1024, 1280, 1536, 2048, 2560, 3072, 3584, 4096, 4608, 5120, 6144,
                                         7168, 8192)] + [
    (512, 4096, 4096), (1024, 8192, 2048), (3000, 3000, 3000), (16384, 4096, 1024), (8192, 1024, 4096),
    (2048, 8192, 1024), (6144, 6144, 2048), (1536, 1536, 4096), (4096, 4096, 1024), (2304, 2304, 8192)]


def sweep_tiles():
    """Each fixed MFMA tile, AUTO and the workspace schedules on uniform
    [-1, 1) operands, op(B) = B, alpha 1, beta 0: TFLOP/s from HIP events over
    back-to-back calls."""
    import torch

    import fp32_gemm_08_amd as lib
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    w = torch.rand(4096, 4096, device=dev)
    wc = torch.empty_like(w)
    for _ in range(300):
        lib.gemm(w, w, wc, algo="mfma")
    torch.cuda.synchronize()
    del w, wc
    g = torch.Generator(device=dev)
    g.manual_seed(11)

    def timeit(fn, reps):
        settle(torch, fn, 0.2)
        for _ in range(max(3, reps // 5)):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    algos = ("mfma_256", "mfma_128", "mfma_64", "auto")
    ws = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    print("| M×N×K | " + " | ".join(algos) + " | AUTO picks | stream-K 256 | stream-K 128 | with workspace "
          "| ws picks |")
    print("|---|" + "---|" * (len(algos) + 5))
    for (M, N, K) in TILE_SWEEP_SHAPES:
        A = torch.rand(M, K, device=dev, generator=g) * 2 - 1
        B = torch.rand(K, N, device=dev, generator=g) * 2 - 1
        C = torch.empty(M, N, device=dev)
        flop = 2.0 * M * N * K
        reps = max(10, min(400, int(0.08 / (flop / 120e12))))
        cells = []
        for algo in algos:
            t = timeit(lambda: lib.gemm(A, B, C, algo=algo), reps)
            cells.append(f"{flop / t / 1e12:.1f}")
        pick = lib.sgemm_f32_plan(0, M, N, K, 1.0, A.data_ptr(), K, B.data_ptr(), N, 0, 0.0, C.data_ptr(), N)[4]
        for tile in (256, 128):
            t = timeit(lambda: lib.gemm(A, B, C, workspace=ws, streamk=tile), reps)
            cells.append(f"{flop / t / 1e12:.1f}")
        t = timeit(lambda: lib.gemm(A, B, C, workspace=ws), reps)
        method = ("plain", "k-split", "stream-K")[lib.sgemm_f32_ws_plan(M, N, K, 0)[1]]
        cells.append(f"{flop / t / 1e12:.1f}")
        print(f"| {M}×{N}×{K} | " + " | ".join(cells[:4]) + f" | {pick.split()[0]} | " + " | ".join(cells[4:]) +
              f" | {method} |", flush=True)
        del A, B, C
        torch.cuda.empty_cache()


def transpose_cpu_baseline(src, rows, cols, D_gpu_host, target_s):
    """Time the transpose oracle on the same workload, repeated for about
    ``target_s`` seconds, and check its result against the GPU's bit for bit."""
    import numpy as np

    import oracle
    t0 = time.perf_counter()
    want = oracle.transpose(src, rows, cols)
    t1 = time.perf_counter() - t0
    reps = max(1, int(target_s / max(t1, 1e-6)))
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.transpose(src, rows, cols)
    t = time.perf_counter() - t0
    same = bool(np.array_equal(want.view(np.uint32), np.ascontiguousarray(D_gpu_host).view(np.uint32)))
    return {
        "value": 8.0 * rows * cols * reps / t / 1e9,
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"the whole {rows}x{cols} transpose, {reps} times in {t:.1f} s "
                  "(numpy row-by-row copy, one thread)",
        "seconds": t,
        "sample_parity": {"ok": same, "bit_exact": same},
    }


MFMA_PROBE_FLOP_PER_TRIP = 4 * 8 * 4096.0   # per workgroup: 4 wavefronts x 8 MFMAs x 4096 FLOP


WARMUP_MIN_CALLS = 200
WARMUP_MIN_SECONDS = 0.4


def warm_up(torch, call, warmup):
    """Untimed calls before the timed ones: at least `warmup` of them
    (WARMUP_MIN_CALLS when no count is given), and in any case at least
    WARMUP_MIN_SECONDS of device time.  The engine clock takes a few hundred
    milliseconds of load to reach its steady state: 5 warm-up calls of the
    4096^3 kernel left the next 20 timed ones 9% slow (1.048 against 0.957 ms
    per call), and 200 calls of a 23 us step leave it ~10% low.  Returns the
    count actually run, which is what the JSON line reports."""
    want = WARMUP_MIN_CALLS if warmup is None else warmup
    n, t0 = 0, time.perf_counter()
    while n < want or time.perf_counter() - t0 < WARMUP_MIN_SECONDS:
        for _ in range(max(1, min(50, want - n)) if n < want else 10):
            call(n)
            n += 1
        torch.cuda.synchronize()          # the wall clock then tracks the device
    return n


def settle(torch, call, seconds=0.3):
    """Run `call` back to back for about `seconds` of device time, so that the
    measurements that follow start at the engine clock of a loaded GPU (a pause
    on the host, e.g. generating the next workload, lets it drop)."""
    t0, batch = time.perf_counter(), 1
    while True:
        for _ in range(batch):
            call()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return
        batch = min(2 * batch, 64)        # one call first: some stages take a second per call


def per_call_times(torch, stream, call, n=20):
    """n calls, each between its own pair of events on the launch stream (the
    gap an event adds stays outside every span): sorted seconds per call."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for e0, e1 in evs:
        e0.record(stream)
        call()
        e1.record(stream)
    torch.cuda.synchronize()
    return sorted(e0.elapsed_time(e1) * 1e-3 for e0, e1 in evs)


def probe_clock(lib, torch, dev, stream, workgroups=512, trips=2000, launches=3):
    """Shader clock (MHz) right after the timed steps, read inside a kernel: the
    library's matrix-core probe counts shader cycles against the constant
    100 MHz counter on every workgroup.  (The driver's sysfs clock table lags
    by about half a second, so it misreports a ~0.1 s run.)"""
    sink = torch.empty(workgroups * 256, dtype=torch.float32, device=dev)
    clocks = torch.zeros(workgroups * 2, dtype=torch.int64, device=dev)
    for _ in range(launches):
        st = lib.sgemm_f32_mfma_probe(workgroups, trips, sink.data_ptr(), clocks.data_ptr(), stream.cuda_stream)
        if st != 0:
            return None
    torch.cuda.synchronize()
    c = clocks.cpu().view(workgroups, 2).double()
    mhz = 100.0 * c[:, 0] / c[:, 1]
    return {"mean": round(mhz.mean().item(), 1), "min": round(mhz.min().item(), 1),
            "max": round(mhz.max().item(), 1),
            "source": "shader cycles / 100 MHz ticks inside the library's MFMA probe, launched right after "
                      "the timed steps (each workgroup's wavefront 0)"}


def sustained_ceiling(lib, torch, dev, stream, precision="fp32"):
    """The matrix-core rate the device sustains with register operands only
    (the library's probe: FP32 chains, or 16-bit chains on random operands),
    measured after the timed steps: ~0.3 s of launches to let the clock settle
    under that load, then launches between two events.  The published peak
    assumes the full clock; under a 16-bit matrix-core load the part holds a
    lower one, so this is the rate a kernel of the same type can reach."""
    workgroups = 512
    sink = torch.empty(workgroups * 256, dtype=torch.float32, device=dev)
    clocks = torch.zeros(workgroups * 2, dtype=torch.int64, device=dev)
    if precision == "fp32":
        trips, flop = 10000, workgroups * 10000 * MFMA_PROBE_FLOP_PER_TRIP

        def launch():
            return lib.sgemm_f32_mfma_probe(workgroups, trips, sink.data_ptr(), clocks.data_ptr(), stream.cuda_stream)
    else:
        prec = lib.PRECISION[precision]
        trips, flop = 16000, workgroups * 16000 * LP_PROBE_FLOP_PER_TRIP

        def launch():
            return lib.sgemm_f32_mfma_probe_lp(prec, 0, workgroups, trips, sink.data_ptr(), clocks.data_ptr(),
                                               stream.cuda_stream)
    t_end = time.perf_counter() + 0.3
    while time.perf_counter() < t_end:
        for _ in range(4):
            if launch() != 0:
                return None
        torch.cuda.synchronize()
    n = 10
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        if launch() != 0:
            return None
    e1.record(stream)
    torch.cuda.synchronize()
    avg = e0.elapsed_time(e1) * 1e-3 / n
    c = clocks.cpu().view(workgroups, 2).double()
    return {"value": round(flop / avg / 1e12, 2), "unit": "TFLOP/s",
            "shader_clock_mhz": round((100.0 * c[:, 0] / c[:, 1]).mean().item(), 1),
            "source": f"the library's {'FP32' if precision == 'fp32' else precision} matrix-core probe "
                      "(register operands, 512 workgroups), right after the timed steps"}


def cu_scaling():
    """The 256 x 256 MFMA kernel with one tile per busy CU: M = 256 .. 4096
    (16 .. 256 tiles), N = K = 4096.  The same work per CU at every M, so a
    time that does not grow with the busy CUs means the kernel is bound inside
    each CU rather than by the memory system it shares."""
    import torch

    import fp32_gemm_08_amd as lib
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    print("| M | tiles = busy CUs | µs | TFLOP/s | per CU, % of 157.3/256 |")
    print("|---|---|---|---|---|")
    for M in (4096, 2048, 1024, 512, 256):
        N = K = 4096
        A = torch.rand(M, K, device=dev, generator=g) * 2 - 1
        B = torch.rand(K, N, device=dev, generator=g) * 2 - 1
        C = torch.empty(M, N, device=dev)

        def call():
            lib.gemm(A, B, C, algo="mfma_256")

        settle(torch, call, 0.3)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(60):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / 60
        per_cu = 2.0 * 256 * 256 * K / t / 1e12
        print(f"| {M} | {(M // 256) * (N // 256)} | {t * 1e6:.1f} | {2.0 * M * N * K / t / 1e12:.1f} | "
              f"{100 * per_cu / (FP32_MFMA_PEAK_TFLOPS / 256):.1f}% |", flush=True)
        del A, B, C


def bench_mfma_ceiling(args):
    """The FP32 matrix-core rate the device sustains with register operands
    only (no memory traffic), against the published 157.3 TFLOP/s."""
    import torch

    import fp32_gemm_08_amd as lib
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    workgroups, trips = 512, 20000      # 2 workgroups per CU: 2 wavefronts on every SIMD
    sink = torch.empty(workgroups * 256, dtype=torch.float32, device=dev)
    clocks = torch.zeros(workgroups * 2, dtype=torch.int64, device=dev)

    def launch():
        st = lib.sgemm_f32_mfma_probe(workgroups, trips, sink.data_ptr(), clocks.data_ptr(), stream.cuda_stream)
        if st != 0:
            raise RuntimeError(lib.sgemm_f32_status_string(st))

    for _ in range(max((args.warmup or 200) // 10, 5)):
        launch()
    torch.cuda.synchronize()
    steps = max(args.steps // 5, 5)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg = e0.elapsed_time(e1) * 1e-3 / steps
    flop = workgroups * trips * MFMA_PROBE_FLOP_PER_TRIP
    c = clocks.cpu().view(workgroups, 2).double()
    mhz = 100.0 * c[:, 0] / c[:, 1]
    out = {
        "metric": "FP32 matrix-core sustained TFLOP/s (register-only MFMA probe), 1 GPU",
        "value": round(steps * flop / wall / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "higher_is_better": True,
        "kernel_avg_ms": round(avg * 1e3, 4),
        "achieved": round(flop / avg / 1e12, 2), "peak": FP32_MFMA_PEAK_TFLOPS,
        "frac": round(flop / avg / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4),
        "config": {"workload": f"{workgroups} workgroups x 4 wavefronts x {trips * 8} v_mfma_f32_32x32x2_f32, "
                               "random register operands", "flop_per_launch": flop},
        "shader_clock_mhz": {"mean": round(mhz.mean().item(), 1), "min": round(mhz.min().item(), 1),
                             "max": round(mhz.max().item(), 1)},
        "device": device_record(torch, dev),
    }
    print(json.dumps(out), flush=True)


LP_PROBE_FLOP_PER_TRIP = 4 * 8 * 32768.0   # per workgroup: 4 wavefronts x 8 MFMAs x 32768 FLOP


def bench_mfma_ceiling_lp(args):
    """The 16-bit matrix-core rate the device sustains with register operands
    only, random and all-zero, against the published 2500 TFLOP/s: how far the
    clock falls under a full 16-bit matrix-core load sets the ceiling the
    mixed-precision GEMM is compared with."""
    import torch

    import fp32_gemm_08_amd as lib
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    prec = lib.PRECISION[args.precision]
    workgroups, trips = 512, 8000       # 2 workgroups per CU: 2 wavefronts on every SIMD; ~3-4 ms a launch
    sink = torch.empty(workgroups * 256, dtype=torch.float32, device=dev)
    clocks = torch.zeros(workgroups * 2, dtype=torch.int64, device=dev)
    flop = workgroups * trips * LP_PROBE_FLOP_PER_TRIP

    def measure(zero):
        def launch():
            st = lib.sgemm_f32_mfma_probe_lp(prec, zero, workgroups, trips, sink.data_ptr(), clocks.data_ptr(),
                                             stream.cuda_stream)
            if st != 0:
                raise RuntimeError(lib.sgemm_f32_status_string(st))

        t_end = time.perf_counter() + 0.5      # let the clock settle under this load
        while time.perf_counter() < t_end:
            for _ in range(10):
                launch()
            torch.cuda.synchronize()
        steps = max(args.steps // 5, 5)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
        avg = e0.elapsed_time(e1) * 1e-3 / steps
        c = clocks.cpu().view(workgroups, 2).double()
        mhz = 100.0 * c[:, 0] / c[:, 1]
        return steps, avg, {"mean": round(mhz.mean().item(), 1), "min": round(mhz.min().item(), 1),
                            "max": round(mhz.max().item(), 1)}

    steps, avg, clk = measure(0)
    _, avg0, clk0 = measure(1)
    out = {
        "metric": f"{args.precision.upper()} matrix-core sustained TFLOP/s (register-only MFMA probe), 1 GPU",
        "value": round(flop / avg / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
        "higher_is_better": True, "kernel_avg_ms": round(avg * 1e3, 4),
        "peak": HALF_MFMA_PEAK_TFLOPS, "frac": round(flop / avg / 1e12 / HALF_MFMA_PEAK_TFLOPS, 4),
        "config": {"workload": f"{workgroups} workgroups x 4 wavefronts x {trips * 8} "
                               f"v_mfma_f32_32x32x16_{args.precision}, random register operands in [-1, 1)",
                   "flop_per_launch": flop},
        "shader_clock_mhz": clk,
        "zero_operands": {"value": round(flop / avg0 / 1e12, 2), "kernel_avg_ms": round(avg0 * 1e3, 4),
                          "frac": round(flop / avg0 / 1e12 / HALF_MFMA_PEAK_TFLOPS, 4), "shader_clock_mhz": clk0},
        "device": device_record(torch, dev),
    }
    print(json.dumps(out), flush=True)


# Load-probe layouts: (name, region bytes, workgroups sharing a region).
LOAD_PROBE_MODES = (("L2-resident: 256 KiB per XCD, read by its 32 workgroups", 256 << 10, 32),
                    ("panels: 4 MiB read by 4 workgroups of one XCD (256 MiB in all)", 4 << 20, 4),
                    ("private: 4 MiB per workgroup (1 GiB in all, from HBM)", 4 << 20, 1))


def load_ceiling():
    """Bytes per shader cycle one CU stages into LDS with direct loads and
    nothing else running (one workgroup per CU, 4 MiB each), by wavefronts,
    loads in flight per wavefront and where the data come from: the feed
    ceiling of the MFMA kernels' staging."""
    import torch

    import fp32_gemm_08_amd as lib
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    workgroups = 256
    src_bytes = 1 << 30
    src = torch.zeros(src_bytes // 4, dtype=torch.float32, device=dev)
    clocks = torch.zeros(workgroups * 2, dtype=torch.int64, device=dev)
    print("| source | wavefronts | loads in flight per wavefront | KiB in flight per CU | B per CU-cycle | "
          "chip TB/s (events) | shader clock MHz |")
    print("|---|---|---|---|---|---|---|")
    for name, region, share in LOAD_PROBE_MODES:
        for waves in (4, 8):
            for depth in (1, 2, 4, 8):
                loads = (4 << 20) // (waves * 1024)

                def launch():
                    st = lib.sgemm_f32_load_probe(waves, depth, workgroups, src.data_ptr(), src_bytes, region, share,
                                                  loads, clocks.data_ptr(), stream.cuda_stream)
                    if st != 0:
                        raise RuntimeError(lib.sgemm_f32_status_string(st))

                for _ in range(3):
                    launch()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(5):
                    launch()
                e1.record(stream)
                torch.cuda.synchronize()
                t = e0.elapsed_time(e1) * 1e-3 / 5
                c = clocks.cpu().view(workgroups, 2).double()
                per_wg = loads * waves * 1024.0
                bpc = per_wg / c[:, 0].mean().item()
                mhz = (100.0 * c[:, 0] / c[:, 1]).mean().item()
                print(f"| {name} | {waves} | {depth} | {waves * depth} | {bpc:.1f} | "
                      f"{workgroups * per_wg / t / 1e12:.2f} | {mhz:.0f} |", flush=True)


def device_record(torch, dev, clock=None):
    """What the run ran on: device, compute units, memory, HIP/ROCm versions and
    the shader clock read right after the timed steps."""
    p = torch.cuda.get_device_properties(dev)
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    return {"arch": getattr(p, "gcnArchName", None), "name": p.name, "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2**30, 1), "hip": torch.version.hip, "rocm": rocm,
            "shader_clock_mhz": clock}


def _transpose_timed(lib, torch, algo_id, rows, cols, pairs, steps, warmup, stream):
    """Back-to-back transposes rotating over ``pairs``; returns (event span, wall,
    warm-up calls run)."""
    sp = stream.cuda_stream
    R = len(pairs)

    def step(k):
        src, dst = pairs[k % R]
        s = lib.sgemm_f32_transpose_algo(algo_id, rows, cols, src.data_ptr(), cols, dst.data_ptr(), rows, sp)
        if s != 0:
            raise RuntimeError(lib.sgemm_f32_status_string(s))

    warmed = warm_up(torch, step, warmup)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for k in range(steps):
        step(k)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3, time.perf_counter() - t0, warmed


def _rotation(torch, src_host, rows, cols, dev, min_bytes=1 << 30):
    """Source/destination pairs (each pair one copy of the workload) totalling at
    least ``min_bytes``, well above the 256 MB Infinity Cache."""
    per_pair = 8 * rows * cols
    R = max(1, -(-min_bytes // per_pair))
    base = torch.from_numpy(src_host).to(dev)
    return [(base if i == 0 else base.clone(), torch.empty((cols, rows), dtype=torch.float32, device=dev))
            for i in range(R)]


def bench_transpose(args):
    import torch

    import fp32_gemm_08_amd as lib
    from fp32_gemm_08_amd.inputs import TRANSPOSE_CONFIGS, make_transpose_config

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    name = args.config if args.config in TRANSPOSE_CONFIGS else "t_4096"
    algo_name = args.algo if args.algo in lib.TRANSPOSE_ALGO else "auto"
    algo = lib.TRANSPOSE_ALGO[algo_name]
    cfg = TRANSPOSE_CONFIGS[name]
    rows, cols = cfg["rows"], cfg["cols"]
    log(f"bench transpose: config={name} algo={algo_name} steps={args.steps} "
        f"warmup={args.warmup if args.warmup is not None else 'auto'}")
    src = make_transpose_config(name)
    pairs = _rotation(torch, src, rows, cols, dev)
    stream = torch.cuda.current_stream(dev)
    st, kid, blocks, kname = lib.sgemm_f32_transpose_plan(algo, rows, cols, pairs[0][0].data_ptr(), cols,
                                                          pairs[0][1].data_ptr(), rows)
    if st != 0:
        raise SystemExit(f"plan failed: {lib.sgemm_f32_status_string(st)}")
    span, wall, warmed = _transpose_timed(lib, torch, algo, rows, cols, pairs, args.steps, args.warmup, stream)
    clock = probe_clock(lib, torch, dev, stream)
    nbytes = 8.0 * rows * cols            # one read and one write of every element
    kern_avg = span / args.steps
    achieved = nbytes / kern_avg / 1e9
    value = args.steps * nbytes / wall / 1e9
    log(f"kernel {kname}: avg {kern_avg * 1e6:.2f} us over {args.steps} calls rotating {len(pairs)} pairs")
    same_pair = None
    if args.same_pair:
        # Context only: the same transpose repeated on one pair (source and
        # destination then stay in the Infinity Cache between calls).
        span1, _, _ = _transpose_timed(lib, torch, algo, rows, cols, pairs[:1], args.steps, 20, stream)
        same_pair = round(nbytes / (span1 / args.steps) / 1e9, 1)
        log(f"one pair repeated: {span1 / args.steps * 1e6:.2f} us")
    D_host = pairs[0][1].cpu().numpy()
    out = {
        "metric": TRANSPOSE_METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmed,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "strong",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "config": {
            "workload": f"transpose {rows}x{cols} float32 -> {cols}x{rows}, uniform inputs, seed {cfg['seed']}, "
                        f"{len(pairs)} source/destination pairs in rotation",
            "name": name, "rows": rows, "cols": cols, "algo": algo_name, "kernel": kname,
            "workgroups": blocks, "pairs": len(pairs), "same_pair_gbs": same_pair,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": read_traffic(TRANSPOSE_TRAFFIC_FILE, TRANSPOSE_SOURCES)
            if (name == "t_4096" and algo_name in ("auto", "lds")) else None,
            "kernel_avg_ms": round(kern_avg * 1e3, 5),
            "algorithmic_bytes_per_launch": nbytes,
        },
        "device": device_record(torch, dev, clock),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log(f"cpu baseline: transpose oracle for ~{args.cpu_seconds:.0f} s")
        out["cpu_baseline"] = transpose_cpu_baseline(src, rows, cols, D_host, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def sweep_transpose():
    import torch

    import fp32_gemm_08_amd as lib
    from fp32_gemm_08_amd.inputs import TRANSPOSE_CONFIGS, make_transpose_config
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    print("| workload | algorithm | kernel | pairs | avg us (rotating) | GB/s | % of 8000 | avg us (one pair) | GB/s |")
    print("|---|---|---|---|---|---|---|---|---|")
    for name, cfg in TRANSPOSE_CONFIGS.items():
        rows, cols = cfg["rows"], cfg["cols"]
        pairs = _rotation(torch, make_transpose_config(name), rows, cols, dev)
        nbytes = 8.0 * rows * cols
        for algo_name in ("naive", "narrow", "lds_nopad", "lds", "auto"):
            a = lib.TRANSPOSE_ALGO[algo_name]
            _, _, _, kname = lib.sgemm_f32_transpose_plan(a, rows, cols, pairs[0][0].data_ptr(), cols,
                                                          pairs[0][1].data_ptr(), rows)
            span, _, _ = _transpose_timed(lib, torch, a, rows, cols, pairs, 200, 100, stream)
            span1, _, _ = _transpose_timed(lib, torch, a, rows, cols, pairs[:1], 200, 20, stream)
            t, t1 = span / 200, span1 / 200
            print(f"| {name} {rows}x{cols} | {algo_name} | {kname} | {len(pairs)} | {t * 1e6:.2f} | "
                  f"{nbytes / t / 1e9:.0f} | {100 * nbytes / t / 1e9 / HBM_PEAK_GBS:.1f} | {t1 * 1e6:.2f} | "
                  f"{nbytes / t1 / 1e9:.0f} |", flush=True)
        # Reference point for what the memory system sustains: torch's own
        # contiguous device copy of the same bytes over the same rotation.
        R = len(pairs)
        flat = [(a.view(-1), b.view(-1)) for a, b in pairs]
        for k in range(100):
            flat[k % R][1].copy_(flat[k % R][0])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for k in range(200):
            flat[k % R][1].copy_(flat[k % R][0])
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / 200
        print(f"| {name} {rows}x{cols} | (device copy, same bytes) | torch copy_ | {R} | {t * 1e6:.2f} | "
              f"{nbytes / t / 1e9:.0f} | {100 * nbytes / t / 1e9 / HBM_PEAK_GBS:.1f} | | |", flush=True)
        del pairs, flat
        torch.cuda.empty_cache()


SPLITK_SHAPES = [("c1_128", None), ("c5_512", None), ("c2_1024", None), ("c3_ragged_bt", None),
                 ("768^3", (768, 768, 768)), ("1024x1024x4096", (1024, 1024, 4096)),
                 ("512x512x8192", (512, 512, 8192)), ("256x256x8192", (256, 256, 8192)),
                 ("256x256x32768", (256, 256, 32768)), ("512x256x16384", (512, 256, 16384)),
                 ("384x384x8192", (384, 384, 8192)), ("64x64x65536", (64, 64, 65536)), ("c5_2048", None)]


def sweep_splitk(splits_list=(1, 2, 3, 4, 6, 7, 8, 12, 14, 16, 24, 32, 48, 64, 0)):
    """Time the k-split path for several split counts on the small and long-k
    workloads (both kernels, average over back-to-back calls)."""
    import torch

    import fp32_gemm_08_amd as lib
    from fp32_gemm_08_amd.inputs import make_case, make_config
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    w = torch.rand(4096, 4096, device=dev)
    wc = torch.empty_like(w)
    for _ in range(300):
        lib.gemm(w, w, wc, algo="mfma")
    torch.cuda.synchronize()
    del w, wc
    print("| workload | splits asked | splits used | partial-pass kernel | workspace MiB | avg us | TFLOP/s |")
    print("|---|---|---|---|---|---|---|")
    for name, shape in SPLITK_SHAPES:
        case = make_config(name) if shape is None else make_case(*shape, seed=31)
        M, N, K = case.M, case.N, case.K
        dA = torch.from_numpy(case.A).to(dev)
        dB = torch.from_numpy(case.B).to(dev)
        dC = torch.zeros((M, case.ldc), dtype=torch.float32, device=dev)
        if case.C is not None:
            dC.copy_(torch.from_numpy(case.C))
        need = max(lib.sgemm_f32_splitk_plan(sp, M, N, K, int(case.trans_b))[3] for sp in splits_list)
        ws = torch.empty(max(need, 4) // 4, dtype=torch.float32, device=dev)
        flop = 2.0 * M * N * K
        for sp in splits_list:
            _, used, kid, nb = lib.sgemm_f32_splitk_plan(sp, M, N, K, int(case.trans_b))
            args = (M, N, K, case.alpha, dA.data_ptr(), case.lda, dB.data_ptr(), case.ldb, int(case.trans_b),
                    case.beta, dC.data_ptr(), case.ldc, ws.data_ptr(), need, stream.cuda_stream)

            def call():
                st = lib.sgemm_f32_splitk(sp, *args) if sp else lib.sgemm_f32_ws(*args)
                if st != 0:
                    raise RuntimeError(lib.sgemm_f32_status_string(st))

            reps = int(max(10, min(300, 0.1 / max(flop / 60e12, 2e-6))))
            settle(torch, call, 0.2)
            for _ in range(max(5, reps // 4)):
                call()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(reps):
                call()
            e1.record(stream)
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3 / reps
            kname = {40: "mfma 256x256", 41: "mfma 128x128 ks2", 42: "mfma 64x64", 45: "mfma 64x64 ks2"}.get(kid, str(kid))
            print(f"| {name} {M}x{N}x{K} | {sp if sp else 'auto'} | {used} | {kname} | {nb / 2**20:.1f} | "
                  f"{t * 1e6:.2f} | {flop / t / 1e12:.2f} |", flush=True)
        del dA, dB, dC, ws
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed calls first (default: at least 200 and at least 0.4 s of device time, "
                         "so the engine clock reaches its loaded state; the JSON line reports the count run)")
    ap.add_argument("--op", choices=("gemm", "transpose", "splitk"), default="gemm",
                    help="splitk: table of the k-split path over split counts (no JSON line)")
    ap.add_argument("--config", default="c4_4096",
                    help="workload name (GEMM: c1_128 ... c5_tall, k_* long-k, s_* stream-K; transpose: t_4096 ...)")
    ap.add_argument("--algo", default="auto")
    ap.add_argument("--row-share", type=int, default=1, metavar="P",
                    help="GEMM: run the first of P equal row shares of the workload (A and C rows, all of B): "
                         "one GPU's part when the output is split by rows over P GPUs")
    ap.add_argument("--precision", choices=("fp32", "fp16", "bf16"), default="fp32",
                    help="GEMM: fp16/bf16 run sgemm_f32_lowp (operands rounded to that format, FP32 sums), "
                         "reported against the dense fp16/bf16 matrix-core peak")
    ap.add_argument("--workspace", action="store_true",
                    help="GEMM: call sgemm_f32_ws with the workspace its plan asks for (k-split when the output tiles "
                         "are too few, stream-K when their last wave is partial; a step then includes the "
                         "reduction or fix-up kernel)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--same-pair", action="store_true",
                    help="transpose: also time one source/destination pair repeated (cache-resident context)")
    ap.add_argument("--sweep", action="store_true",
                    help="time every algorithm on every workload and print a table (no JSON line)")
    ap.add_argument("--oracle-table", action="store_true",
                    help="time the FP64 oracle on every GEMM workload (CPU only, reported, no JSON line)")
    ap.add_argument("--cu-scaling", action="store_true",
                    help="time the 256x256 MFMA kernel with 16..256 busy CUs, one tile each (table)")
    ap.add_argument("--load-ceiling", action="store_true",
                    help="table of the direct global->LDS load rate per CU (the library's load probe)")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="time the library's register-only MFMA probe: the FP32 matrix-core rate the device "
                         "sustains and its shader clock (one JSON line); with --precision fp16|bf16 the 16-bit "
                         "matrix cores, with random and with all-zero operands")
    ap.add_argument("--tile-sweep", action="store_true",
                    help="time each fixed MFMA tile, AUTO and the workspace schedules over a spread of shapes (no JSON line)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path (the GEMM would shard by "
              "rows of C with B replicated on every GPU). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.oracle_table:
        oracle_table()
        return

    import torch

    if args.copy_calibration:
        copy_calibration()
        return
    if args.mfma_ceiling and args.precision != "fp32":
        bench_mfma_ceiling_lp(args)
        return
    if args.load_ceiling:
        load_ceiling()
        return
    if args.mfma_ceiling:
        bench_mfma_ceiling(args)
        return
    if args.cu_scaling:
        cu_scaling()
        return
    if args.op == "splitk":
        sweep_splitk()
        return
    if args.op == "transpose":
        if args.sweep:
            sweep_transpose()
        else:
            bench_transpose(args)
        return
    if args.sweep:
        sweep()
        return
    if args.tile_sweep:
        sweep_tiles()
        return

    import fp32_gemm_08_amd as lib
    from fp32_gemm_08_amd.inputs import make_config, make_row_share

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    log(f"bench: config={args.config} algo={args.algo} steps={args.steps} "
        f"warmup={args.warmup if args.warmup is not None else 'auto'} row_share={args.row_share}")
    share = args.row_share > 1
    case = make_row_share(args.config, args.row_share, 0) if share else make_config(args.config)
    label = f"{args.config}, row share 1 of {args.row_share}" if share else args.config
    M, N, K = case.M, case.N, case.K
    dA = torch.from_numpy(case.A).to(dev)
    dB = torch.from_numpy(case.B).to(dev)
    dC = torch.from_numpy(case.C.copy()).to(dev) if case.C is not None else \
        torch.zeros((M, case.ldc), dtype=torch.float32, device=dev)
    C0 = dC.clone() if case.C is not None else None
    algo = lib.ALGO[args.algo]
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    pa, pb, pc = dA.data_ptr(), dB.data_ptr(), dC.data_ptr()
    st, kid, tm, tn, kname = lib.sgemm_f32_plan(algo, M, N, K, case.alpha, pa, case.lda, pb, case.ldb,
                                                int(case.trans_b), case.beta, pc, case.ldc)
    if st != 0:
        raise SystemExit(f"plan failed: {lib.sgemm_f32_status_string(st)}")
    splits, ws, ws_bytes = 1, None, 0
    lowp = args.precision != "fp32"
    if lowp:
        st, kid, tm, tn, kname = lib.sgemm_f32_lowp_plan(lib.PRECISION[args.precision], M, N, K, case.alpha, pa,
                                                         case.lda, pb, case.ldb, int(case.trans_b), case.beta, pc,
                                                         case.ldc)
        if st != 0:
            raise SystemExit(f"plan failed: {lib.sgemm_f32_status_string(st)}")
    if args.workspace and lowp:
        st, lkid, ltm, ltn, ws_bytes = lib.sgemm_f32_lowp_ws_plan(lib.PRECISION[args.precision], M, N, K,
                                                                   int(case.trans_b))
        if ws_bytes > 0:
            ws = torch.empty(ws_bytes // 4 + 1, dtype=torch.float32, device=dev)
            kid, tm, tn = lkid, ltm, ltn
            _, _, _, _, kname = lib.sgemm_f32_lowp_plan(lib.PRECISION[args.precision], M, N, K, case.alpha, pa,
                                                        case.lda, pb, case.ldb, int(case.trans_b), case.beta, pc,
                                                        case.ldc)
            tile = 256 if kid in (64, 65) else 128
            kname = f"two passes: rounding into the workspace + lp16 {args.precision} {tile}x{tile} GEMM"
    if args.workspace and not lowp:
        _, method, wkid, ws_bytes = lib.sgemm_f32_ws_plan(M, N, K, int(case.trans_b))
        if method == 1:
            _, splits, skid, ws_bytes = lib.sgemm_f32_splitk_plan(0, M, N, K, int(case.trans_b))
            ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device=dev)
            kid = skid
            kname = f"k-split x{splits}: mfma_64x64x32_w2x2 partial pass + splitk_reduce"
            tm, tn = -(-M // 64) * splits, -(-N // 64)
        elif method == 2:
            _, kid, dp, skt, wk, ws_bytes = lib.sgemm_f32_streamk_plan(0, M, N, K, int(case.trans_b))
            ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device=dev)
            tile = 256 if kid == 43 else 128
            kname = (f"stream-K {tile}x{tile}: {dp} data-parallel tiles + {skt} tiles over {wk} workgroups "
                     f"+ sk_fixup")
            tm, tn = dp + wk, 1

    def step():
        if lowp and ws is not None:
            s = lib.sgemm_f32_lowp_ws(lib.PRECISION[args.precision], M, N, K, case.alpha, pa, case.lda, pb,
                                      case.ldb, int(case.trans_b), case.beta, pc, case.ldc, ws.data_ptr(), ws_bytes,
                                      sp)
        elif lowp:
            s = lib.sgemm_f32_lowp(lib.PRECISION[args.precision], M, N, K, case.alpha, pa, case.lda, pb, case.ldb,
                                   int(case.trans_b), case.beta, pc, case.ldc, sp)
        elif ws is not None:
            s = lib.sgemm_f32_ws(M, N, K, case.alpha, pa, case.lda, pb, case.ldb, int(case.trans_b), case.beta,
                                 pc, case.ldc, ws.data_ptr(), ws_bytes, sp)
        else:
            s = lib.sgemm_f32_algo(algo, M, N, K, case.alpha, pa, case.lda, pb, case.ldb, int(case.trans_b),
                                   case.beta, pc, case.ldc, sp)
        if s != 0:
            raise RuntimeError(lib.sgemm_f32_status_string(s))

    warmed = warm_up(torch, lambda i: step(), args.warmup)

    # Timed region: exactly K back-to-back calls on one stream, events at its two
    # ends only (an event between launches inserts a gap of its own).  The
    # kernel's average duration is the event span over K; the throughput uses the
    # host wall clock between the two device synchronisations.
    K_steps = args.steps
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record(stream)
    for _ in range(K_steps):
        step()
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call = per_call_times(torch, stream, step)
    clock = probe_clock(lib, torch, dev, stream)
    span = e_start.elapsed_time(e_end) * 1e-3
    flop = 2.0 * M * N * K
    hbm_bytes = 4.0 * (M * K + K * N + M * N + (M * N if case.beta != 0.0 else 0))
    value = K_steps * flop / wall / 1e12
    kern_avg = span / K_steps
    achieved = flop / kern_avg / 1e12
    mfma = kid in (40, 41, 42, 43, 44, 45, 46, 47, 60, 61, 62, 63, 64, 65, 66, 67)  # every matrix-core kernel id
    peak = HALF_MFMA_PEAK_TFLOPS if lowp else FP32_MFMA_PEAK_TFLOPS if mfma else FP32_VALU_PEAK_TFLOPS
    log(f"{'step (both kernels)' if ws is not None else 'kernel'} {kname}: avg {kern_avg * 1e3:.4f} ms "
        f"over {K_steps} calls "
        f"(event span {span * 1e3:.3f} ms, wall {wall * 1e3:.3f} ms)")

    # output for the sample check (beta != 0 workloads accumulate across steps:
    # rerun once from the original C for the check)
    if C0 is not None:
        dC.copy_(C0)
        step()
        torch.cuda.synchronize()
    D_host = dC.cpu().numpy()

    out = {
        "metric": (METRIC if args.config == "c4_4096" and not share else f"FP32 GEMM TFLOP/s ({label}), 1 GPU")
        if not lowp else f"mixed-precision GEMM TFLOP/s ({args.precision} operands, FP32 sums; {label}), 1 GPU",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": warmed,
        "ms_per_step": round(wall / K_steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "strong",
        "vs_baseline": None,
        "dtype": "f32" if not lowp else f"{args.precision} operands, f32 accumulate",
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / (HALF_MFMA_PEAK_TFLOPS if lowp else FP32_MFMA_PEAK_TFLOPS), 2),
        "config": {
            "workload": f"sgemm {M}x{N}x{K} row-major, D=alpha*A*{'B^T' if case.trans_b else 'B'}+beta*C, "
                        f"alpha={case.alpha:g}, beta={case.beta:g}, {case.meta['dist']} inputs, "
                        f"seed {case.meta['seed']}"
                        + (f"; rows 0..{M - 1} of the {args.config} workload (one of {args.row_share} row shares, "
                           f"all of B)" if share else ""),
            "name": label, "M": M, "N": N, "K": K, "trans_b": case.trans_b,
            "lda": case.lda, "ldb": case.ldb, "ldc": case.ldc,
            "algo": args.algo, "kernel": kname, "workgroups": tm * tn,
            "k_splits": splits, "workspace_bytes": ws_bytes,
        },
        "roofline": {
            "bound": "mfma" if mfma else "alu",
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": None,
            "kernel_avg_ms": round(kern_avg * 1e3, 4),
            "algorithmic_flop_per_launch": flop,
            # the same launches against the HBM roofline: compulsory bytes (A and B
            # read once, C written once, and read once when beta != 0) over the
            # average launch; the bound on the small shapes, whose FLOP per byte
            # sits near the ridge (157.3 TFLOP/s / 8 TB/s = 19.7)
            "hbm": {"algorithmic_bytes_per_launch": hbm_bytes,
                    "flop_per_byte": round(flop / hbm_bytes, 2),
                    "achieved_gbs": round(hbm_bytes / kern_avg / 1e9, 1), "peak_gbs": HBM_PEAK_GBS,
                    "frac": round(hbm_bytes / kern_avg / 1e9 / HBM_PEAK_GBS, 4)},
            # after the timed steps: 20 more calls, each between its own events
            "per_call": {"calls": len(per_call), "median_ms": round(per_call[len(per_call) // 2] * 1e3, 4),
                         "best_ms": round(per_call[0] * 1e3, 4),
                         "median_tflops": round(flop / per_call[len(per_call) // 2] / 1e12, 3),
                         "best_tflops": round(flop / per_call[0] / 1e12, 3)},
        },
        "device": device_record(torch, dev, clock),
        "cpu_baseline": None,
    }
    traffic = read_traffic() if (args.config == "c4_4096" and not share and kid == 40) else None
    out["roofline"]["traffic"] = traffic
    if mfma:
        # context beside the published peak: the rate the chip sustains for this
        # type of matrix-core work, and this kernel's fraction of it
        ceil = sustained_ceiling(lib, torch, dev, stream, args.precision if lowp else "fp32")
        if ceil is not None:
            ceil["frac"] = round(achieved / ceil["value"], 4)
            out["roofline"]["sustained_ceiling"] = ceil
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on a sample of rows for ~{args.cpu_seconds:.0f} s")
        out["cpu_baseline"] = cpu_baseline(case, D_host, args.cpu_seconds,
                                           None if not lowp else args.precision)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
