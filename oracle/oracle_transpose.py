"""CPU oracle for the out-of-place FP32 matrix transpose (test infrastructure only).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may use it; the library never does.

"现代 CUDA 工具箱实战：从朴素代码到硬件极限的优化之路", section 代码实现 defines the
operation through its baseline kernel: the output element at (x, y) is the
input element at (y, x), for an N x N float32 matrix.  Here the matrix is
rows x cols and stored row-major with a leading dimension:

    dst(j, i) = src(i, j)        0 <= i < rows, 0 <= j < cols

The result is a copy of the input bits: no arithmetic touches them, so the
oracle's output is exact and the GPU result is compared with it bit for bit.

``src`` is passed as its storage: a 2-D numpy array whose row length is the
leading dimension and whose first ``cols`` columns hold the matrix (padding
columns beyond ``cols`` are never read).
"""
from __future__ import annotations

import numpy as np


def transpose(src: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Return the (cols x rows) transpose of the rows x cols matrix held in ``src``.

    One source row at a time: row i of the source becomes column i of the
    result.  The copy moves array elements, not values, so NaN payloads, signed
    zeros and subnormals come out unchanged.
    """
    if src.ndim != 2 or src.shape[0] < rows or src.shape[1] < cols:
        raise ValueError(f"storage {src.shape} cannot hold a {rows} x {cols} matrix")
    out = np.empty((cols, rows), dtype=src.dtype)
    for i in range(rows):
        out[:, i] = src[i, :cols]
    return out
