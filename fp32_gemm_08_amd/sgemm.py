"""ctypes binding for libsgemm_f32.so (argument marshalling only).

The entry points keep the C names and arguments of ``include/sgemm_f32.h``;
pointers are plain integers (device addresses) and ``stream`` is a hipStream_t
as an integer (0 = null stream).  ``gemm`` is a convenience wrapper over torch
tensors that derives the leading dimensions and the current stream; torch is
used for device memory and streams only, every FLOP runs in the HIP kernels.

There is no fallback: if the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

# SGEMM_F32_LIBRARY names another build of the same library (the LDS-poison
# debug build, a host-sanitizer build); by default the in-tree one is loaded.
LIB_PATH = os.environ.get("SGEMM_F32_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                               "libsgemm_f32.so")

SGEMM_OK = 0
SGEMM_ERR_INVALID_VALUE = 1
SGEMM_ERR_ALIAS = 2
SGEMM_ERR_NO_DEVICE = 3
SGEMM_ERR_UNSUPPORTED_ARCH = 4
SGEMM_ERR_LAUNCH = 5
SGEMM_ERR_SCRATCH_LIMIT = 6
SCRATCH_BYTES = 16 << 20

ALGO = {"auto": 0, "naive": 1, "lds_tiled": 2, "regblock": 3, "mfma": 4, "lds_tiled_nopad": 5, "naive_wg": 6,
        "mfma_256": 7, "mfma_128": 8, "mfma_64": 9, "mfma_32": 10, "mfma_128x64": 11}
TRANSPOSE_ALGO = {"auto": 0, "naive": 1, "lds": 2, "lds_nopad": 3, "narrow": 4}

# Symbols declared in include/sgemm_f32.h.
PRECISION = {"fp16": 1, "bf16": 2}

EXPORTS = ("sgemm_f32", "sgemm_f32_algo", "sgemm_f32_arch_status", "sgemm_f32_device_status", "sgemm_f32_lowp", "sgemm_f32_lowp_2pass", "sgemm_f32_lowp_2pass_plan",
           "sgemm_f32_lowp_plan", "sgemm_f32_lowp_ws",
           "sgemm_f32_lowp_ws_plan", "sgemm_f32_plan",
           "sgemm_f32_splitk", "sgemm_f32_splitk_noalloc", "sgemm_f32_splitk_plan",
           "sgemm_f32_load_probe", "sgemm_f32_mfma_probe", "sgemm_f32_mfma_probe_lp", "sgemm_f32_status_string", "sgemm_f32_streamk", "sgemm_f32_streamk_plan", "sgemm_f32_transpose",
           "sgemm_f32_transpose_algo", "sgemm_f32_transpose_plan", "sgemm_f32_version", "sgemm_f32_ws",
           "sgemm_f32_ws_plan")

_lock = threading.Lock()
_lib = None


class SgemmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def load():
    """Load the built library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m fp32_gemm_08_amd.build` "
                               "(or __graft_entry__.build()) first")
        lib = ctypes.CDLL(LIB_PATH)
        i64, f32, vp, ci = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_int
        gemm_args = [i64, i64, i64, f32, vp, i64, vp, i64, ci, f32, vp, i64, vp]
        lib.sgemm_f32.restype = ci
        lib.sgemm_f32.argtypes = gemm_args
        lib.sgemm_f32_algo.restype = ci
        lib.sgemm_f32_algo.argtypes = [ci] + gemm_args
        lib.sgemm_f32_plan.restype = ci
        lib.sgemm_f32_plan.argtypes = [ci, i64, i64, i64, f32, vp, i64, vp, i64, ci, f32, vp, i64,
                                       ctypes.POINTER(ci), ctypes.POINTER(i64), ctypes.POINTER(i64),
                                       ctypes.c_char_p, ci]
        lib.sgemm_f32_lowp.restype = ci
        lib.sgemm_f32_lowp.argtypes = [ci] + gemm_args
        lib.sgemm_f32_lowp_plan.restype = ci
        lib.sgemm_f32_lowp_plan.argtypes = [ci, i64, i64, i64, f32, vp, i64, vp, i64, ci, f32, vp, i64,
                                            ctypes.POINTER(ci), ctypes.POINTER(i64), ctypes.POINTER(i64),
                                            ctypes.c_char_p, ci]
        ws_args = gemm_args[:-1] + [vp, i64, vp]
        lib.sgemm_f32_ws.restype = ci
        lib.sgemm_f32_ws.argtypes = ws_args
        lib.sgemm_f32_splitk.restype = ci
        lib.sgemm_f32_splitk.argtypes = [i64] + ws_args
        lib.sgemm_f32_splitk_noalloc.restype = ci
        lib.sgemm_f32_splitk_noalloc.argtypes = [i64] + gemm_args
        lib.sgemm_f32_splitk_plan.restype = ci
        lib.sgemm_f32_splitk_plan.argtypes = [i64, i64, i64, i64, ci, ctypes.POINTER(i64), ctypes.POINTER(ci),
                                              ctypes.POINTER(i64)]
        lib.sgemm_f32_lowp_ws.restype = ci
        lib.sgemm_f32_lowp_ws.argtypes = [ci] + ws_args
        lib.sgemm_f32_lowp_2pass.restype = ci
        lib.sgemm_f32_lowp_2pass.argtypes = [ci, ci] + ws_args
        lib.sgemm_f32_lowp_2pass_plan.restype = ci
        lib.sgemm_f32_lowp_2pass_plan.argtypes = [ci, ci, i64, i64, i64, ci, ctypes.POINTER(ci),
                                                  ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(i64)]
        lib.sgemm_f32_lowp_ws_plan.restype = ci
        lib.sgemm_f32_lowp_ws_plan.argtypes = [ci, i64, i64, i64, ci, ctypes.POINTER(ci), ctypes.POINTER(i64),
                                               ctypes.POINTER(i64), ctypes.POINTER(i64)]
        lib.sgemm_f32_ws_plan.restype = ci
        lib.sgemm_f32_ws_plan.argtypes = [i64, i64, i64, ci, ctypes.POINTER(ci), ctypes.POINTER(ci),
                                          ctypes.POINTER(i64)]
        lib.sgemm_f32_streamk.restype = ci
        lib.sgemm_f32_streamk.argtypes = [ci] + ws_args
        lib.sgemm_f32_streamk_plan.restype = ci
        lib.sgemm_f32_streamk_plan.argtypes = [ci, i64, i64, i64, ci, ctypes.POINTER(ci), ctypes.POINTER(i64),
                                               ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(i64)]
        tr_args = [i64, i64, vp, i64, vp, i64, vp]
        lib.sgemm_f32_transpose.restype = ci
        lib.sgemm_f32_transpose.argtypes = tr_args
        lib.sgemm_f32_transpose_algo.restype = ci
        lib.sgemm_f32_transpose_algo.argtypes = [ci] + tr_args
        lib.sgemm_f32_transpose_plan.restype = ci
        lib.sgemm_f32_transpose_plan.argtypes = [ci, i64, i64, vp, i64, vp, i64, ctypes.POINTER(ci),
                                                 ctypes.POINTER(i64), ctypes.c_char_p, ci]
        lib.sgemm_f32_status_string.restype = ctypes.c_char_p
        lib.sgemm_f32_status_string.argtypes = [ci]
        lib.sgemm_f32_version.restype = ctypes.c_char_p
        lib.sgemm_f32_version.argtypes = []
        lib.sgemm_f32_mfma_probe.restype = ci
        lib.sgemm_f32_mfma_probe.argtypes = [i64, i64, vp, vp, vp]
        lib.sgemm_f32_mfma_probe_lp.restype = ci
        lib.sgemm_f32_mfma_probe_lp.argtypes = [ci, ci, i64, i64, vp, vp, vp]
        lib.sgemm_f32_load_probe.restype = ci
        lib.sgemm_f32_load_probe.argtypes = [ci, ci, i64, vp, i64, i64, i64, i64, vp, vp]
        lib.sgemm_f32_arch_status.restype = ci
        lib.sgemm_f32_arch_status.argtypes = [ctypes.c_char_p]
        lib.sgemm_f32_device_status.restype = ci
        lib.sgemm_f32_device_status.argtypes = []
        _lib = lib
        return lib


def sgemm_f32_arch_status(arch) -> int:
    """Host-only: SGEMM_OK when the architecture name (bytes or str, or None)
    is gfx950, else SGEMM_ERR_UNSUPPORTED_ARCH."""
    if isinstance(arch, str):
        arch = arch.encode()
    return load().sgemm_f32_arch_status(arch)


def sgemm_f32_device_status() -> int:
    """The device check every call makes: SGEMM_OK, SGEMM_ERR_NO_DEVICE or
    SGEMM_ERR_UNSUPPORTED_ARCH for the calling thread's current device."""
    return load().sgemm_f32_device_status()


def sgemm_f32(M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, stream=0) -> int:
    """C <- alpha*A*op(B) + beta*C (AUTO algorithm).  Returns the status code."""
    return load().sgemm_f32(M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, stream)


def sgemm_f32_algo(algo, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, stream=0) -> int:
    """Same operation with an explicit algorithm id.  Returns the status code."""
    return load().sgemm_f32_algo(algo, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, stream)


def sgemm_f32_plan(algo, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc):
    """Host-only planning query: (status, kernel_id, tiles_m, tiles_n, name)."""
    kid = ctypes.c_int(0)
    tm = ctypes.c_int64(0)
    tn = ctypes.c_int64(0)
    buf = ctypes.create_string_buffer(128)
    st = load().sgemm_f32_plan(algo, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc,
                               ctypes.byref(kid), ctypes.byref(tm), ctypes.byref(tn), buf, 128)
    return st, kid.value, tm.value, tn.value, buf.value.decode()


def sgemm_f32_lowp(precision, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, stream=0) -> int:
    """Mixed precision: operands rounded to fp16 (1) or bf16 (2), FP32 sums.  Returns the status."""
    return load().sgemm_f32_lowp(precision, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, stream)


def sgemm_f32_lowp_plan(precision, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc):
    """Host-only planning query: (status, kernel_id, tiles_m, tiles_n, name)."""
    kid = ctypes.c_int(0)
    tm = ctypes.c_int64(0)
    tn = ctypes.c_int64(0)
    buf = ctypes.create_string_buffer(128)
    st = load().sgemm_f32_lowp_plan(precision, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc,
                                    ctypes.byref(kid), ctypes.byref(tm), ctypes.byref(tn), buf, 128)
    return st, kid.value, tm.value, tn.value, buf.value.decode()


def sgemm_f32_ws(M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, workspace, workspace_bytes,
                 stream=0) -> int:
    """C <- alpha*A*op(B) + beta*C, splitting k when the workspace allows.  Returns the status."""
    return load().sgemm_f32_ws(M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, workspace,
                               workspace_bytes, stream)


def sgemm_f32_splitk(splits, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, workspace, workspace_bytes,
                     stream=0) -> int:
    """The same with an explicit split count.  Returns the status."""
    return load().sgemm_f32_splitk(splits, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, workspace,
                                   workspace_bytes, stream)


def sgemm_f32_splitk_noalloc(splits, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, stream=0) -> int:
    """The k-split with its partials in the library's static device scratch
    (no workspace argument, no allocation).  Returns the status."""
    return load().sgemm_f32_splitk_noalloc(splits, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, stream)


def sgemm_f32_splitk_plan(splits, M, N, K, transB=0):
    """Host-only query: (status, splits_used, kernel_id, workspace_bytes)."""
    su = ctypes.c_int64(0)
    kid = ctypes.c_int(0)
    nb = ctypes.c_int64(0)
    st = load().sgemm_f32_splitk_plan(splits, M, N, K, transB, ctypes.byref(su), ctypes.byref(kid), ctypes.byref(nb))
    return st, su.value, kid.value, nb.value


def sgemm_f32_lowp_ws(precision, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, workspace, workspace_bytes,
                      stream=0) -> int:
    """Mixed precision with a workspace: a rounding pass into it, then the
    16-bit GEMM (the one-pass call when the workspace is too small)."""
    return load().sgemm_f32_lowp_ws(precision, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, workspace,
                                    workspace_bytes, stream)


def sgemm_f32_lowp_ws_plan(precision, M, N, K, transB=0):
    """Host-only query: (status, kernel_id, tiles_m, tiles_n, workspace_bytes)."""
    kid = ctypes.c_int(0)
    tm, tn, nb = (ctypes.c_int64(0) for _ in range(3))
    st = load().sgemm_f32_lowp_ws_plan(precision, M, N, K, transB, ctypes.byref(kid), ctypes.byref(tm),
                                       ctypes.byref(tn), ctypes.byref(nb))
    return st, kid.value, tm.value, tn.value, nb.value


def sgemm_f32_lowp_2pass(precision, tile, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, workspace,
                         workspace_bytes, stream=0) -> int:
    """The two-pass mixed-precision call at any size (tile 0, 256 or 128)."""
    return load().sgemm_f32_lowp_2pass(precision, tile, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc,
                                       workspace, workspace_bytes, stream)


def sgemm_f32_lowp_2pass_plan(precision, tile, M, N, K, transB=0):
    """Host-only query: (status, kernel_id, tiles_m, tiles_n, workspace_bytes)."""
    kid = ctypes.c_int(0)
    tm, tn, nb = (ctypes.c_int64(0) for _ in range(3))
    st = load().sgemm_f32_lowp_2pass_plan(precision, tile, M, N, K, transB, ctypes.byref(kid), ctypes.byref(tm),
                                          ctypes.byref(tn), ctypes.byref(nb))
    return st, kid.value, tm.value, tn.value, nb.value


def sgemm_f32_ws_plan(M, N, K, transB=0):
    """Host-only query of what sgemm_f32_ws does: (status, method, kernel_id,
    workspace_bytes); method 0 = plain, 1 = k-split, 2 = stream-K."""
    method = ctypes.c_int(0)
    kid = ctypes.c_int(0)
    nb = ctypes.c_int64(0)
    st = load().sgemm_f32_ws_plan(M, N, K, transB, ctypes.byref(method), ctypes.byref(kid), ctypes.byref(nb))
    return st, method.value, kid.value, nb.value


def sgemm_f32_streamk(tile, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, workspace, workspace_bytes,
                      stream=0) -> int:
    """C <- alpha*A*op(B) + beta*C under a stream-K schedule (tile 0 = the
    library's choice, 256 or 128).  Returns the status code."""
    return load().sgemm_f32_streamk(tile, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, workspace,
                                    workspace_bytes, stream)


def sgemm_f32_streamk_plan(tile, M, N, K, transB=0):
    """Host-only query: (status, kernel_id, dp_tiles, sk_tiles, workers, workspace_bytes)."""
    kid = ctypes.c_int(0)
    dp, skt, wk, nb = (ctypes.c_int64(0) for _ in range(4))
    st = load().sgemm_f32_streamk_plan(tile, M, N, K, transB, ctypes.byref(kid), ctypes.byref(dp), ctypes.byref(skt),
                                       ctypes.byref(wk), ctypes.byref(nb))
    return st, kid.value, dp.value, skt.value, wk.value, nb.value


def sgemm_f32_transpose(rows, cols, src, ld_src, dst, ld_dst, stream=0) -> int:
    """dst <- src^T (AUTO algorithm).  Returns the status code."""
    return load().sgemm_f32_transpose(rows, cols, src, ld_src, dst, ld_dst, stream)


def sgemm_f32_transpose_algo(algo, rows, cols, src, ld_src, dst, ld_dst, stream=0) -> int:
    """dst <- src^T with an explicit algorithm id.  Returns the status code."""
    return load().sgemm_f32_transpose_algo(algo, rows, cols, src, ld_src, dst, ld_dst, stream)


def sgemm_f32_transpose_plan(algo, rows, cols, src, ld_src, dst, ld_dst):
    """Host-only planning query: (status, kernel_id, blocks, name)."""
    kid = ctypes.c_int(0)
    blocks = ctypes.c_int64(0)
    buf = ctypes.create_string_buffer(128)
    st = load().sgemm_f32_transpose_plan(algo, rows, cols, src, ld_src, dst, ld_dst, ctypes.byref(kid),
                                         ctypes.byref(blocks), buf, 128)
    return st, kid.value, blocks.value, buf.value.decode()


def sgemm_f32_status_string(status: int) -> str:
    return load().sgemm_f32_status_string(status).decode()


def sgemm_f32_version() -> str:
    return load().sgemm_f32_version().decode()


def sgemm_f32_mfma_probe(workgroups, trips, sink, clocks, stream=0) -> int:
    """Measurement aid: workgroups * 4 wavefronts each issue trips * 8 FP32
    MFMAs (4096 FLOP each) on register operands; clocks receives (shader
    cycles, 100 MHz ticks) per workgroup.  Returns the status code."""
    return load().sgemm_f32_mfma_probe(workgroups, trips, sink, clocks, stream)


def sgemm_f32_mfma_probe_lp(precision, zero_operands, workgroups, trips, sink, clocks, stream=0) -> int:
    """Measurement aid: as sgemm_f32_mfma_probe with 16-bit MFMAs (32768 FLOP
    each; precision 1 = fp16, 2 = bf16) on random or all-zero operands."""
    return load().sgemm_f32_mfma_probe_lp(precision, zero_operands, workgroups, trips, sink, clocks, stream)


def sgemm_f32_load_probe(waves, depth, workgroups, src, src_bytes, region_bytes, share, loads, clocks,
                         stream=0) -> int:
    """Measurement aid: each workgroup's `waves` wavefronts stream `loads` 1 KB
    direct global->LDS loads from its region of src, `depth` in flight;
    clocks receives (shader cycles, 100 MHz ticks) per workgroup."""
    return load().sgemm_f32_load_probe(waves, depth, workgroups, src, src_bytes, region_bytes, share, loads,
                                       clocks, stream)


def _check(status):
    if status != SGEMM_OK:
        raise SgemmError(status, sgemm_f32_status_string(status))


def _algo_id(algo, table=ALGO):
    if isinstance(algo, str):
        return table[algo]
    return int(algo)


def _check_matrix(name, t):
    import torch

    if t.dtype != torch.float32 or not t.is_cuda or t.dim() != 2:
        raise TypeError(f"{name} must be a 2-D float32 device tensor")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit stride along its last dimension")
    if t.shape[0] > 1 and t.stride(0) < t.shape[1]:
        raise ValueError(f"{name} rows overlap (row stride below the row length)")


def _ld(t):
    return max(t.stride(0) if t.shape[0] > 1 else t.shape[1], t.shape[1], 1)


def gemm(A, B, C, alpha=1.0, beta=0.0, trans_b=False, algo="auto", stream=None, workspace=None, splits=0,
         precision=None, streamk=None):
    """C <- alpha*A*op(B) + beta*C on torch float32 CUDA tensors, in place; returns C.

    A is (M, K), B is (K, N) or, with trans_b, (N, K); C is (M, N).  Each may be a
    row-strided view (last-dimension stride 1); its row stride is the leading
    dimension.  Runs on ``stream`` (a torch stream) or torch's current stream.
    With ``workspace`` (a contiguous device tensor) the product may split k over
    several workgroups per tile (``splits`` = 0: the library's choice, else that
    count; ``algo`` is then not used; ``streamk`` = 0, 256 or 128 runs the
    stream-K schedule with the library's tile or that one).  With ``precision`` ("fp16" or "bf16")
    the operands are rounded to that format and multiplied by the 16-bit matrix
    cores with FP32 sums (sgemm_f32_lowp; with ``workspace``, sgemm_f32_lowp_ws:
    a rounding pass into the workspace, then the GEMM on 16-bit operands).
    """
    import torch  # plumbing only: device memory and streams

    for name, t in (("A", A), ("B", B), ("C", C)):
        _check_matrix(name, t)
    M, K = A.shape
    N = B.shape[0] if trans_b else B.shape[1]
    if (B.shape[1] if trans_b else B.shape[0]) != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)} "
                         f"(trans_b={trans_b}), C {tuple(C.shape)}")
    ld = _ld
    s = (stream if stream is not None else torch.cuda.current_stream(C.device)).cuda_stream
    with torch.cuda.device(C.device):
        if precision is not None:
            args = (PRECISION[precision], M, N, K, float(alpha), A.data_ptr(), ld(A), B.data_ptr(), ld(B),
                    int(bool(trans_b)), float(beta), C.data_ptr(), ld(C))
            if workspace is None:
                st = sgemm_f32_lowp(*args, s)
            else:
                if not workspace.is_cuda or not workspace.is_contiguous():
                    raise ValueError("workspace must be a contiguous device tensor")
                st = sgemm_f32_lowp_ws(*args, workspace.data_ptr(), workspace.numel() * workspace.element_size(), s)
        elif workspace is None:
            st = sgemm_f32_algo(_algo_id(algo), M, N, K, float(alpha), A.data_ptr(), ld(A), B.data_ptr(), ld(B),
                                int(bool(trans_b)), float(beta), C.data_ptr(), ld(C), s)
        else:
            if not workspace.is_cuda or not workspace.is_contiguous():
                raise ValueError("workspace must be a contiguous device tensor")
            nbytes = workspace.numel() * workspace.element_size()
            args = (M, N, K, float(alpha), A.data_ptr(), ld(A), B.data_ptr(), ld(B), int(bool(trans_b)),
                    float(beta), C.data_ptr(), ld(C), workspace.data_ptr(), nbytes, s)
            if streamk is not None:
                st = sgemm_f32_streamk(int(streamk), *args)
            elif splits:
                st = sgemm_f32_splitk(int(splits), *args)
            else:
                st = sgemm_f32_ws(*args)
    _check(st)
    return C


def transpose(src, dst, algo="auto", stream=None):
    """dst <- src^T on torch float32 CUDA tensors; returns dst.

    src is (rows, cols) and dst is (cols, rows); either may be a row-strided view
    (last-dimension stride 1) whose row stride is its leading dimension.
    """
    import torch  # plumbing only: device memory and streams

    _check_matrix("src", src)
    _check_matrix("dst", dst)
    rows, cols = src.shape
    if tuple(dst.shape) != (cols, rows):
        raise ValueError(f"shape mismatch: src {tuple(src.shape)}, dst {tuple(dst.shape)}")
    s = (stream if stream is not None else torch.cuda.current_stream(dst.device)).cuda_stream
    with torch.cuda.device(dst.device):
        st = sgemm_f32_transpose_algo(_algo_id(algo, TRANSPOSE_ALGO), rows, cols, src.data_ptr(), _ld(src),
                                      dst.data_ptr(), _ld(dst), s)
    _check(st)
    return dst
