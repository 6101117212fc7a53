"""C-ABI boundary tests that need no GPU.

The library loads without a device; argument validation, quick returns and the
planning query run on the host before any HIP call, so every status they
produce is checked here.  No compute call is made.
"""
import ctypes
import os
import re

import pytest

import fp32_gemm_08_amd as lib
from fp32_gemm_08_amd import sgemm as binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgemm_f32.h")

OK, INVALID, ALIAS = 0, 1, 2
KID_NONE, KID_SCALE, KID_NAIVE, KID_TILED, KID_TILED_NOPAD, KID_REG = 0, 1, 10, 20, 21, 30
KID_NAIVE_WG = 11
KID_L, KID_M, KID_S, KID_S2, KID_T, KID_R = 40, 41, 42, 45, 46, 47

# Fake, well-separated "device" addresses: planning only compares ranges.
PA, PB, PC = 1 << 32, 1 << 40, 1 << 44


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(lib.LIB_PATH):
        pytest.skip("libsgemm_f32.so not built")


def header_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sgemm_f32\w*)\s*\(", text)))


def test_exports_every_declared_symbol():
    declared = header_functions()
    assert declared == sorted(binding.EXPORTS)
    so = ctypes.CDLL(lib.LIB_PATH)
    for name in declared:
        assert hasattr(so, name), name


def test_version_and_status_strings():
    assert "gfx950" in lib.sgemm_f32_version()
    for code in range(7):
        assert lib.sgemm_f32_status_string(code).startswith("SGEMM_")
    assert "unknown" in lib.sgemm_f32_status_string(99)


def plan(algo=0, M=64, N=64, K=64, alpha=1.0, A=PA, lda=None, B=PB, ldb=None, transB=0, beta=0.0,
         C=PC, ldc=None):
    lda = K if lda is None else lda
    ldb = (K if transB else N) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return lib.sgemm_f32_plan(algo, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc)


def call(algo=0, M=64, N=64, K=64, alpha=1.0, A=PA, lda=None, B=PB, ldb=None, transB=0, beta=0.0,
         C=PC, ldc=None):
    lda = K if lda is None else lda
    ldb = (K if transB else N) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return lib.sgemm_f32_algo(algo, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, 0)


@pytest.mark.parametrize("kw", [
    dict(M=-1), dict(N=-1), dict(K=-1), dict(M=1 << 31), dict(K=1 << 31),
    dict(transB=2), dict(transB=-1),
    dict(lda=63), dict(ldb=63), dict(ldc=63), dict(transB=1, ldb=63),
    dict(A=0), dict(B=0), dict(C=0), dict(algo=12), dict(algo=-1),
    dict(M=(1 << 31) - 1024), dict(N=(1 << 31) - 1024), dict(K=(1 << 31) - 1024),
    dict(M=2, K=2, lda=1 << 61),
    # pointers off a float boundary
    dict(A=PA + 2), dict(B=PB + 1), dict(C=PC + 3), dict(C=PC + 2, K=0, beta=0.5), dict(A=PA + 6, algo=1),
])
def test_invalid_arguments(kw):
    assert plan(**kw)[0] == INVALID
    assert call(**kw) == INVALID


def test_ld_minimum_is_one_for_empty_rows():
    # K == 0: lda may be 1; N == 0: ldb/ldc may be 1
    assert plan(K=0, lda=1, beta=1.0)[0] == OK
    assert plan(N=0, ldb=1, ldc=1)[0] == OK
    assert plan(K=0, lda=0)[0] == INVALID


@pytest.mark.parametrize("transB", [0, 1])
def test_alias_detection(transB):
    M = N = K = 64
    a_bytes = ((M - 1) * K + K) * 4
    # C starts inside A
    assert plan(C=PA + a_bytes - 4, transB=transB)[0] == ALIAS
    # C ends inside A
    assert plan(A=PC + 64 * 64 * 4 - 4, transB=transB)[0] == ALIAS
    # C overlaps B
    assert plan(B=PC + 128, transB=transB)[0] == ALIAS
    # adjacent but not overlapping
    assert plan(C=PA + a_bytes, transB=transB)[0] == OK
    # A and B may alias each other (both are only read)
    assert plan(A=PB, transB=transB)[0] == OK
    assert call(C=PA + 4, transB=transB) == ALIAS


def test_quick_returns_touch_nothing():
    # M == 0 or N == 0: OK, nothing launches, NULL pointers allowed
    for kw in (dict(M=0, A=0, C=0), dict(N=0, B=0, C=0, ldb=1, ldc=1)):
        st, kid, tm, tn, _ = plan(**kw)
        assert (st, kid, tm, tn) == (OK, KID_NONE, 0, 0)
        assert call(**kw) == OK
    # alpha == 0 or K == 0 with beta == 1: C is already the result
    for kw in (dict(alpha=0.0, beta=1.0, A=0, B=0), dict(K=0, lda=1, beta=1.0, A=0, B=0)):
        st, kid, _, _, _ = plan(**kw)
        assert (st, kid) == (OK, KID_NONE)
        assert call(**kw) == OK


def test_product_free_cases_scale_c():
    # alpha == 0 or K == 0 with beta != 1: only C <- beta*C runs, A and B may be NULL
    for kw in (dict(alpha=0.0, beta=0.0, A=0, B=0), dict(K=0, lda=1, beta=-0.5, A=0, B=0),
               dict(alpha=0.0, beta=2.0, A=PC + 8)):
        st, kid, tm, tn, name = plan(**kw)
        assert (st, kid) == (OK, KID_SCALE), name
        assert (tm, tn) == (64, 1)


@pytest.mark.parametrize("algo,kid", [(1, KID_NAIVE), (2, KID_TILED), (3, KID_REG), (5, KID_TILED_NOPAD),
                                      (6, KID_NAIVE_WG), (7, KID_L), (8, KID_M), (9, KID_S), (10, KID_T),
                                      (11, KID_R)])
def test_explicit_algorithms(algo, kid):
    st, k, tm, tn, name = plan(algo=algo, M=1000, N=1017, K=999)
    assert (st, k) == (OK, kid)
    if kid == KID_NAIVE:
        assert (tm, tn) == (250, 16)
    elif kid == KID_NAIVE_WG:
        assert (tm, tn) == (1000, 1017) and name.startswith("naive_wave_per_output")
    elif kid in (KID_TILED, KID_TILED_NOPAD):
        assert (tm, tn) == (63, 64)
    elif kid == KID_L:
        assert (tm, tn) == (4, 4) and name.startswith("mfma_256x256")
    elif kid == KID_S:
        assert (tm, tn) == (16, 16) and name.startswith("mfma_64x64")
    elif kid == KID_T:
        assert (tm, tn) == (32, 32) and name.startswith("mfma_32x32x32_w1x1_ks4")
    elif kid == KID_R:
        assert (tm, tn) == (8, 16) and name.startswith("mfma_128x64x32_w4x1_ks2")
    else:
        assert (tm, tn) == (8, 8)


@pytest.mark.parametrize("shape,kid,tiles", [
    ((4096, 4096, 4096), KID_L, (16, 16)),
    ((8192, 8192, 8192), KID_L, (32, 32)),
    ((16384, 4096, 1024), KID_L, (64, 16)),
    ((2048, 2048, 2048), KID_M, (16, 16)),
    # the 64 x 64 tile: 8 wavefronts (k split in two); grids of 257..512 tiles: the 128 x 64 tile when it
    # gives at most 256 workgroups and pads at most 1/16 more rows, else (and with K < 256) 4 wavefronts
    ((1024, 1024, 1024), KID_S2, (16, 16)),
    ((1000, 1017, 999), KID_S2, (16, 16)),
    ((832, 832, 832), KID_S2, (13, 13)),       # 169 tiles
    ((768, 1024, 512), KID_S2, (12, 16)),      # 192 tiles
    # at most 144 tiles of 64 x 64: the 32 x 32 tile, k split four ways
    ((768, 768, 768), KID_T, (24, 24)),        # 144 tiles of 64 x 64
    ((512, 512, 512), KID_T, (16, 16)),
    ((128, 128, 128), KID_T, (4, 4)),
    ((1, 1, 1), KID_T, (1, 1)),
    ((128, 128, 256), KID_T, (4, 4)),
    ((512, 512, 8192), KID_T, (16, 16)),
    ((128, 4096, 1024), KID_T, (4, 128)),
    ((1280, 1280, 1280), KID_R, (10, 20)),     # 400 tiles of 64 x 64
    ((512, 4096, 4096), KID_R, (4, 64)),       # 512 tiles
    ((1088, 1024, 1024), KID_R, (9, 16)),      # 17 x 16 tiles; 9 x 128 rows pad 1/17 more
    ((576, 2048, 1024), KID_S, (9, 32)),       # 288 tiles; 5 x 128 rows would pad 1/9 more
    ((1280, 1280, 128), KID_S, (20, 20)),      # K below 256
    ((2176, 512, 1024), KID_R, (17, 8)),       # 272 tiles of 64 x 64
    ((576, 4096, 1024), KID_S2, (9, 64)),      # 576 tiles
    ((3584, 3584, 3584), KID_S2, (56, 56)),
    ((4608, 4608, 4608), KID_S2, (72, 72)),
])
def test_auto_tile_choice(shape, kid, tiles):
    M, N, K = shape
    for algo in (0, 4):
        st, k, tm, tn, name = plan(algo=algo, M=M, N=N, K=K)
        assert (st, k, (tm, tn)) == (OK, kid, tiles), name


def test_vector_path_needs_alignment():
    assert "vec=1" in plan(M=256, N=256, K=256)[4]
    assert "vec=0" in plan(M=256, N=256, K=255, lda=255)[4]          # lda % 4 != 0
    assert "vec=0" in plan(M=256, N=256, K=256, A=PA + 4)[4]         # A not 16-byte aligned
    assert "vec=0" in plan(M=256, N=256, K=256, transB=1, ldb=257)[4]
    assert "transB=1" in plan(transB=1)[4]


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        binding.sgemm_f32(1, 1, 1, 1.0, 0, 1, 0, 1, 0, 0.0, 0, 1, 0)


def test_gemm_wrapper_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    a = torch.zeros(4, 4)
    with pytest.raises(TypeError):
        lib.gemm(a, a, a.clone())


def test_launch_work_item_limit():
    # The naive kernel's 4 x 64 tiles at 2^17 x 2^17 would need 2^34 work-items;
    # the MFMA tiles of the same shape stay far below 2^32.
    n = 1 << 17
    assert plan(algo=1, M=n, N=n, K=1, lda=1, ldb=n, ldc=n, C=1 << 50)[0] == INVALID
    st, kid, tm, tn, _ = plan(algo=0, M=n, N=n, K=1, lda=1, ldb=n, ldc=n, C=1 << 50)
    assert (st, kid, tm, tn) == (OK, KID_L, n // 256, n // 256)
    # largest accepted dimension
    assert plan(M=(1 << 31) - 1025, N=1, K=1, lda=1, ldb=1, ldc=1, C=1 << 50)[0] == OK


def test_wave_per_output_has_no_grid_limit():
    # the kernel loops over outputs: 2^17 x 2^17 outputs are still accepted
    n = 1 << 17
    assert plan(algo=6, M=n, N=n, K=1, lda=1, ldb=n, ldc=n, C=1 << 50)[:2] == (OK, KID_NAIVE_WG)


@pytest.mark.parametrize("wg,trips,sink,clocks,status", [
    (0, 10, PA, PB, INVALID), (-1, 10, PA, PB, INVALID), ((1 << 20) + 1, 10, PA, PB, INVALID),
    (4, 0, PA, PB, INVALID), (4, (1 << 24) + 1, PA, PB, INVALID),
    (4, 10, 0, PB, INVALID), (4, 10, PA, 0, INVALID),
    (4, 10, PA, PA + 4 * 256 * 4 - 8, ALIAS),      # clocks inside the sink
    (4, 10, PB + 16, PB, ALIAS),                   # sink starts inside the clocks
])
def test_mfma_probe_rejects_bad_arguments(wg, trips, sink, clocks, status):
    # every case is refused on the host, before any HIP call
    assert lib.sgemm_f32_mfma_probe(wg, trips, sink, clocks, 0) == status


@pytest.mark.parametrize("prec,zero,wg,trips,sink,clocks,status", [
    (0, 0, 4, 10, PA, PB, INVALID), (3, 0, 4, 10, PA, PB, INVALID), (2, 2, 4, 10, PA, PB, INVALID),
    (2, -1, 4, 10, PA, PB, INVALID), (1, 0, 0, 10, PA, PB, INVALID), (2, 1, (1 << 20) + 1, 10, PA, PB, INVALID),
    (2, 0, 4, 0, PA, PB, INVALID), (1, 1, 4, (1 << 24) + 1, PA, PB, INVALID),
    (2, 0, 4, 10, 0, PB, INVALID), (2, 0, 4, 10, PA, 0, INVALID),
    (2, 0, 4, 10, PA, PA + 4 * 256 * 4 - 8, ALIAS),
])
def test_mfma_probe_lp_rejects_bad_arguments(prec, zero, wg, trips, sink, clocks, status):
    assert lib.sgemm_f32_mfma_probe_lp(prec, zero, wg, trips, sink, clocks, 0) == status


MiB = 1 << 20


@pytest.mark.parametrize("waves,depth,wg,src,src_bytes,region,share,loads,clocks,status", [
    (2, 4, 256, PA, 1 << 30, 4 * MiB, 1, 512, PB, INVALID),       # 4 or 8 wavefronts
    (8, 3, 256, PA, 1 << 30, 4 * MiB, 1, 512, PB, INVALID),       # 1, 2, 4 or 8 in flight
    (8, 16, 256, PA, 1 << 30, 4 * MiB, 1, 512, PB, INVALID),
    (8, 4, 0, PA, 1 << 30, 4 * MiB, 1, 512, PB, INVALID),
    (8, 4, (1 << 16) + 1, PA, 1 << 40, 1024, 1, 512, PB, INVALID),
    (8, 4, 256, PA, 1 << 30, 4 * MiB, 0, 512, PB, INVALID),
    (8, 4, 256, PA, 1 << 30, 4 * MiB, 1, 0, PB, INVALID),
    (8, 4, 256, PA, 1 << 30, 4 * MiB, 1, (1 << 24) + 1, PB, INVALID),
    (8, 4, 256, PA, 1 << 30, 1000, 1, 512, PB, INVALID),          # whole 1 KB chunks
    (8, 4, 256, PA, 1 << 40, 1 << 32, 1, 512, PB, INVALID),       # region above 2^31
    (8, 4, 256, PA + 4, 1 << 30, 4 * MiB, 1, 512, PB, INVALID),   # 16-byte aligned source
    (8, 4, 256, 0, 1 << 30, 4 * MiB, 1, 512, PB, INVALID),
    (8, 4, 256, PA, 1 << 30, 4 * MiB, 1, 512, 0, INVALID),
    (8, 4, 256, PA, (1 << 30) - 1, 4 * MiB, 1, 512, PB, INVALID),  # 256 regions of 4 MiB do not fit
    (8, 4, 256, PA, 256 * MiB, 4 * MiB, 4, 512, PB, OK),          # 64 regions: fits (host check only)
    (8, 4, 256, PA, 256 * MiB - 1, 4 * MiB, 4, 512, PB, INVALID),
    (8, 4, 9, PA, 16 * 1024, 1024, 1, 1, PB, OK),                 # workgroups 8 and 0 share region 8's row
    (8, 4, 9, PA, 15 * 1024, 1024, 1, 1, PB, INVALID),
    (8, 4, 256, PA, 1 << 30, 4 * MiB, 1, 512, PA + (1 << 29), ALIAS),   # clocks inside the regions read
])
def test_load_probe_rejects_bad_arguments(waves, depth, wg, src, src_bytes, region, share, loads, clocks, status):
    st = lib.sgemm_f32_load_probe(waves, depth, wg, src, src_bytes, region, share, loads, clocks, 0)
    if status == OK:
        # the arguments pass every host check; what follows is the device check
        assert st not in (INVALID, ALIAS)
    else:
        assert st == status


@pytest.mark.parametrize("wg,share", [(1, 1), (7, 1), (8, 1), (9, 1), (256, 1), (256, 4), (256, 32), (257, 3),
                                      (1000, 7), (65536, 1), (65536, 65536), (300, 300)])
def test_load_probe_regions_cover_every_read(wg, share):
    """Replay of the load probe's addressing: workgroup b reads region b % 8 + 8 * ((b / 8) / share),
    chunks 0 .. region/1024 - 1 of it.  The host check asks for (8 * (((wg - 1) / 8) / share) + 8)
    regions; every region a workgroup reads must lie inside them, that size must pass and one byte
    less must be refused."""
    region = 1024
    last = max(b % 8 + 8 * ((b // 8) // share) for b in range(wg))
    regions = 8 * (((wg - 1) // 8) // share) + 8
    assert last < regions                     # every region read lies inside what the host asks for
    ok = lib.sgemm_f32_load_probe(8, 4, wg, PA, regions * region, region, share, 1, PB, 0)
    assert ok not in (INVALID, ALIAS)         # exactly that much passes the host checks
    assert lib.sgemm_f32_load_probe(8, 4, wg, PA, regions * region - 1, region, share, 1, PB, 0) == INVALID


_OVERRIDE_CHILD = r"""
import json, sys
sys.path.insert(0, sys.argv[1])
import fp32_gemm_08_amd as lib
PA, PB, PC = 1 << 32, 1 << 40, 1 << 44
def plan(algo, M=1000, N=1017, K=999):
    return lib.sgemm_f32_plan(algo, M, N, K, 1.0, PA, K, PB, N, 0, 0.0, PC, N)[:2]
print(json.dumps([plan(0), plan(4), plan(1), lib.sgemm_f32_ws_plan(512, 512, 8192, 0)[:2], lib.sgemm_f32_lowp_plan(
    2, 4096, 4096, 4096, 1.0, PA, 4096, PB, 4096, 0, 0.0, PC, 4096)[:2]]))
"""


@pytest.mark.parametrize("value,auto", [("", (OK, KID_S2)), ("auto", (OK, KID_S2)), ("regblock", (OK, KID_REG)),
                                        ("mfma_256", (OK, KID_L)), ("9", (OK, KID_S)), ("mfma_32", (OK, KID_T)),
                                        ("naive_wg", (OK, KID_NAIVE_WG)), ("fastest", (INVALID, KID_NONE)),
                                        ("mfma_128x64", (OK, KID_R)), ("11", (OK, KID_R)),
                                        ("12", (INVALID, KID_NONE)), ("MFMA", (INVALID, KID_NONE))])
def test_algo_environment_override(value, auto):
    """SGEMM_F32_ALGO replaces AUTO's choice in sgemm_f32 / sgemm_f32_algo(AUTO) / the plan, fails loudly
    when it names no algorithm, and leaves explicit algorithms and the workspace and mixed-precision
    plans alone.  Host-only planning queries; each value in its own process (it is read once)."""
    import subprocess
    import sys
    env = dict(os.environ, SGEMM_F32_ALGO=value)
    r = subprocess.run([sys.executable, "-c", _OVERRIDE_CHILD, ROOT], env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    import json
    got = [tuple(x) for x in json.loads(r.stdout.strip().splitlines()[-1])]
    assert got[0] == auto
    assert got[1] == (OK, KID_S2)                   # SGEMM_ALGO_MFMA is explicit: never overridden
    assert got[2] == (OK, KID_NAIVE)
    assert got[3] == (OK, 1)                        # sgemm_f32_ws still splits 512 x 512 x 8192
    assert got[4] == (OK, 61)                       # the bf16 kernel of sgemm_f32_lowp
