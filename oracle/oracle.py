"""Python side of the FP64 CPU oracle (test infrastructure only).

The arithmetic lives in ``oracle_gemm.c`` (plain C, built by gcc without fast
math); this module builds it, marshals numpy arrays into it, and applies the
elementwise error bound that GPU results are held to:

    |D_gpu - D| <= 4 * K * 2^-24 * S + 1e-6,    S = sum_k |a(i,k) * b(k,j)|

The bound is the one the GEMM engine is specified against; D and S are the
oracle's FP64 values.  A result must also be finite to pass.

Matrices are passed as their storage: a 2-D float32 numpy array whose row
length is the leading dimension and whose first ``cols`` columns hold the
logical matrix (A: M x lda, B: K x ldb or N x ldb when transposed, C: M x ldc).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_SRC = os.path.join(_HERE, "oracle_gemm.c")
# SGEMM_ORACLE_LIBRARY names another build of the same source (the
# sanitizer build below); by default the gcc build next to this file is used.
ORACLE_GCC_SO = os.path.join(_HERE, "liboracle_gemm.so")
ORACLE_SO = os.environ.get("SGEMM_ORACLE_LIBRARY") or ORACLE_GCC_SO
ORACLE_SANITIZE_SO = os.path.join(_HERE, "liboracle_gemm_sanitize.so")

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast math, no FP contraction)."""
    if force or not os.path.exists(ORACLE_GCC_SO):
        tmp = ORACLE_GCC_SO + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", ORACLE_SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, ORACLE_GCC_SO)
    return ORACLE_GCC_SO


def build_sanitized(clang: str = "/opt/rocm/llvm/bin/clang") -> str:
    """The same source under AddressSanitizer and UndefinedBehaviorSanitizer,
    built by clang (whose shared sanitizer runtime the sanitized GEMM library
    uses too), with its OpenMP runtime found through an rpath."""
    libdir = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(clang))), "lib")
    tmp = ORACLE_SANITIZE_SO + ".tmp"
    cmd = [clang, "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           "-shared-libsan", ORACLE_SRC, "-o", tmp, "-lm", f"-Wl,-rpath,{libdir}"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, ORACLE_SANITIZE_SO)
    return ORACLE_SANITIZE_SO


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(ORACLE_SO):
                build()
            _lib = load_library(ORACLE_SO)
    return _lib


def _as_storage(x, name):
    if x is None:
        return None
    if not (isinstance(x, np.ndarray) and x.dtype == np.float32 and x.ndim == 2
            and x.flags.c_contiguous):
        raise TypeError(f"{name} must be a C-contiguous 2-D float32 numpy array")
    return x


def load_library(path):
    """Load an oracle build from ``path`` (used to check that the pins catch
    deliberately broken copies of the oracle)."""
    lib = ctypes.CDLL(path)
    i64, f32, vp = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
    lib.oracle_gemm_rows.restype = ctypes.c_int
    lib.oracle_gemm_rows.argtypes = [i64, i64, i64, f32, vp, i64, vp, i64, ctypes.c_int,
                                     f32, vp, i64, vp, i64, vp, vp, ctypes.c_int]
    return lib


def gemm_rows(M, N, K, alpha, A, B, trans_b, beta, C, rows=None, nthreads=0, lib=None):
    """FP64 rows of D and S.

    A, B, C are storage arrays (their row length is the leading dimension).
    ``rows`` selects output rows (default: all M).  Returns (D, S, threads),
    D and S float64 of shape (len(rows), N).  ``lib`` overrides the library.
    """
    A = _as_storage(A, "A")
    B = _as_storage(B, "B")
    C = _as_storage(C, "C")
    if rows is None:
        rows = np.arange(M, dtype=np.int64)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    nr = rows.shape[0]
    D = np.empty((nr, N), dtype=np.float64)
    S = np.empty((nr, N), dtype=np.float64)
    lda = A.shape[1] if A is not None else max(1, K)
    ldb = B.shape[1] if B is not None else 1
    ldc = C.shape[1] if C is not None else max(1, N)
    if A is not None and A.shape[0] < M:
        raise ValueError("A has fewer than M rows")
    if B is not None and B.shape[0] < (N if trans_b else K):
        raise ValueError("B has too few rows")
    lib = _load() if lib is None else lib
    ptr = lambda a: None if a is None else a.ctypes.data  # noqa: E731
    used = lib.oracle_gemm_rows(M, N, K, float(alpha), ptr(A), lda, ptr(B), ldb, int(bool(trans_b)),
                                float(beta), ptr(C), ldc, rows.ctypes.data, nr,
                                D.ctypes.data, S.ctypes.data, int(nthreads))
    if used < 0:
        raise ValueError("oracle rejected its arguments")
    return D, S, used


def gemm_full(M, N, K, alpha, A, B, trans_b, beta, C, nthreads=0, lib=None):
    """All rows: returns (D, S) of shape (M, N)."""
    D, S, _ = gemm_rows(M, N, K, alpha, A, B, trans_b, beta, C, None, nthreads, lib)
    return D, S


def tolerance(S, K):
    """Elementwise bound 4*K*2^-24*S + 1e-6 (float64 array like S)."""
    return 4.0 * float(K) * 2.0 ** -24 * np.asarray(S, dtype=np.float64) + 1e-6


def check(D_gpu, D, S, K):
    """Compare GPU rows (float32, same shape as D) with the oracle.

    Returns a dict: ok, n_fail, n_nonfinite, max_abs, max_rho (|delta| over the
    bound's rounding term K*2^-24*S + 1e-6/4, so a pass needs rho <= 4), worst
    (row, col) index into the given rows.
    """
    G = np.asarray(D_gpu, dtype=np.float64)
    if G.shape != D.shape:
        raise ValueError(f"shape mismatch {G.shape} vs {D.shape}")
    out = {"ok": True, "n_fail": 0, "n_nonfinite": 0, "max_abs": 0.0, "max_rho": 0.0,
           "worst": None, "count": int(G.size)}
    if G.size == 0:
        return out
    finite = np.isfinite(G)
    delta = np.abs(G - D)
    delta[~finite] = np.inf
    tol = tolerance(S, K)
    fail = ~(delta <= tol)
    rho = delta / (float(K) * 2.0 ** -24 * S + 0.25e-6)
    out["n_nonfinite"] = int((~finite).sum())
    out["n_fail"] = int(fail.sum())
    out["ok"] = out["n_fail"] == 0
    out["max_abs"] = float(np.max(delta))
    out["max_rho"] = float(np.max(rho))
    w = np.unravel_index(int(np.argmax(rho)), rho.shape)
    out["worst"] = (int(w[0]), int(w[1]))
    return out
