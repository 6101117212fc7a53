"""CPU oracle for the mixed-precision GEMM (test infrastructure only).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may use it; the library never does.

"GPU矩阵乘法优化：共享内存Tiling技术实战", section 7.1 (混合精度计算): the FP32 operands
are converted to half precision as they are staged into shared memory, and the
matrix cores multiply the half-precision values.  Read here as:

    D(i,j) = alpha * sum_k r(A(i,k)) * r(op(B)(k,j)) + beta * C(i,j)

with r the conversion to IEEE binary16 ("fp16") or to bfloat16 ("bf16"), both
rounding to nearest with ties to even, and the products summed in FP32 or
better.  Every product of two fp16 or bf16 values is exact in FP32 and in
FP64, so the exact result is the FP64 GEMM of the rounded operands: this
module rounds the operands and hands them to the FP64 oracle (``gemm_rows``),
which also returns S = sum_k |r(a) r(b)| for the elementwise bound.

The two rounding functions are written out here from the formats' definitions:
  fp16: 1 sign, 5 exponent (bias 15), 10 fraction bits; subnormals down to
        2^-24; finite maximum 65504; values at or beyond 65520 round to inf.
  bf16: the upper 16 bits of a binary32 (8 exponent, 7 fraction bits); rounding
        keeps the upper half and rounds the dropped 16 bits to nearest-even;
        finite values that round past the largest bf16 become inf.
NaN stays NaN (quiet) in both.
"""
from __future__ import annotations

import numpy as np

from .oracle import gemm_rows

PRECISIONS = ("fp16", "bf16")


def round_fp16(x: np.ndarray) -> np.ndarray:
    """float32 array -> float32 array of the nearest fp16 values (ties to even).

    Written from the format: for a normal result the spacing at |x| is
    2^(e-10) with e = floor(log2 |x|) (e >= -14); below 2^-14 the spacing is the
    subnormal step 2^-24.  x / spacing is rounded to the nearest integer, ties
    to even (numpy.rint), and scaled back; the scaling is exact.
    """
    x = np.asarray(x, dtype=np.float32)
    out = np.empty_like(x)
    xd = x.astype(np.float64)
    finite = np.isfinite(xd)
    a = np.abs(xd[finite])
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    # log2 of a value just below a power of two can round up to it in floating
    # point; correct the exponent with exact comparisons.
    e = np.where(np.exp2(e) > a, e - 1, e)
    e = np.where(np.exp2(e + 1) <= a, e + 1, e)
    e = np.maximum(e, -14.0)
    step = np.exp2(e - 10.0)
    q = np.rint(xd[finite] / step) * step
    q = np.where(np.abs(q) > 65504.0, np.copysign(np.inf, xd[finite]), q)
    res = np.empty_like(xd)
    res[finite] = q
    res[~finite] = xd[~finite]
    out[...] = res.astype(np.float32)
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array -> float32 array of the nearest bf16 values (ties to even).

    On the binary32 bit pattern u: add 0x7FFF plus the lowest kept bit (bit 16)
    and clear the low 16 bits.  This rounds the dropped half to nearest, ties to
    the even kept value; a carry out of the fraction steps the exponent, which
    is exactly the next binade (or inf past the largest finite value).  NaN
    keeps its sign and upper payload, with the quiet bit set.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    r = np.where(nan, (u.astype(np.uint32) | np.uint32(0x00400000)) & np.uint32(0xFFFF0000), r)
    return r.astype(np.uint32).view(np.float32).reshape(x.shape)


def round_to(precision: str, x: np.ndarray) -> np.ndarray:
    if precision == "fp16":
        return round_fp16(x)
    if precision == "bf16":
        return round_bf16(x)
    raise ValueError(f"unknown precision {precision!r}")


def gemm_lowp_rows(precision, M, N, K, alpha, A, B, trans_b, beta, C, rows=None, nthreads=0, lib=None):
    """(D, S, threads) of the mixed-precision GEMM for the requested rows: the
    FP64 GEMM of the rounded operands (A and B storage rounded elementwise;
    padding columns are never read).  C and the scalars stay FP32."""
    return gemm_rows(M, N, K, alpha, round_to(precision, A), round_to(precision, B), trans_b, beta, C,
                     rows=rows, nthreads=nthreads, lib=lib)
