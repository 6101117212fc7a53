"""Seeded synthetic inputs for D = alpha*A*op(B) + beta*C.

This module only draws numbers; it holds none of the GEMM arithmetic.  The
oracle and the HIP path both consume the float32 arrays it returns.

Draw recipe (the pages give no RNG, so this is a stated choice):
  * ``numpy.random.default_rng(seed)`` (PCG64), one fresh generator per case;
  * draw A (M x K), then B in its stored shape (K x N, or N x K when op(B) = B^T),
    then C (M x N) only when the case carries a C input (beta != 0);
  * "uniform" is ``rng.uniform(-1, 1)``, "normal" is ``rng.standard_normal``,
    "int2" is integers in {-2..2} (every partial sum stays an exact small
    integer), all drawn as float64 and cast to float32.

Storage: a matrix is a C-contiguous float32 array of shape (rows, ld); the
logical matrix is its first ``cols`` columns and any padding columns hold
``pad_value`` (NaN by default, so a stray read of padding poisons a result).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# The benchmark workloads: sizes, op(B), alpha/beta, distribution, seed and
# leading dimensions.  Leading dimensions default to the tight row length.
CONFIGS = {
    "c1_128":      dict(M=128, N=128, K=128, trans_b=False, alpha=1.0, beta=0.0, dist="uniform", seed=0),
    "c2_1024":     dict(M=1024, N=1024, K=1024, trans_b=False, alpha=1.0, beta=0.0, dist="uniform", seed=1),
    "c3_ragged_bt": dict(M=1000, N=1017, K=999, trans_b=True, alpha=1.5, beta=-0.5, dist="uniform", seed=2),
    "c4_4096":     dict(M=4096, N=4096, K=4096, trans_b=False, alpha=1.0, beta=0.0, dist="uniform", seed=3),
    "c5_512":      dict(M=512, N=512, K=512, trans_b=False, alpha=1.0, beta=1.0, dist="normal", seed=4),
    "c5_2048":     dict(M=2048, N=2048, K=2048, trans_b=False, alpha=1.0, beta=1.0, dist="normal", seed=4),
    "c5_8192":     dict(M=8192, N=8192, K=8192, trans_b=False, alpha=1.0, beta=1.0, dist="normal", seed=4),
    "c5_tall":     dict(M=16384, N=4096, K=1024, trans_b=False, alpha=1.0, beta=1.0, dist="normal", seed=4),
}

# Products with few output tiles and a long k-range, where a caller workspace
# lets the k-range split over workgroups.
SPLITK_CONFIGS = {
    "k_256x256x8192": dict(M=256, N=256, K=8192, trans_b=False, alpha=1.0, beta=0.0, dist="uniform", seed=31),
    "k_512x512x8192": dict(M=512, N=512, K=8192, trans_b=False, alpha=1.0, beta=0.0, dist="uniform", seed=32),
    "k_64x64x65536": dict(M=64, N=64, K=65536, trans_b=False, alpha=1.0, beta=0.0, dist="uniform", seed=33),
}

# Products whose tile grid ends in a partial wave on 256 CUs (4608^3: 324
# tiles of 256 x 256), where a caller workspace lets the stream-K schedule
# share the last tiles' k-iterations over every CU.
STREAMK_CONFIGS = {
    "s_4608": dict(M=4608, N=4608, K=4608, trans_b=False, alpha=1.0, beta=0.0, dist="uniform", seed=51),
    "s_2304x2304x8192": dict(M=2304, N=2304, K=8192, trans_b=False, alpha=1.0, beta=0.0, dist="uniform", seed=52),
    "s_3584_bt": dict(M=3584, N=3584, K=3584, trans_b=True, alpha=1.0, beta=1.0, dist="normal", seed=53),
}


@dataclass
class Case:
    M: int
    N: int
    K: int
    trans_b: bool
    alpha: float
    beta: float
    A: np.ndarray                 # (M, lda) storage
    B: np.ndarray                 # (K, ldb) or (N, ldb) storage
    C: Optional[np.ndarray]       # (M, ldc) storage, or None when no C input is drawn
    ldc: int
    meta: dict = field(default_factory=dict)

    @property
    def lda(self):
        return self.A.shape[1]

    @property
    def ldb(self):
        return self.B.shape[1]

    def c_storage(self, fill=np.nan):
        """The C/D buffer handed to the GEMM: the drawn C, or a fresh fill."""
        if self.C is not None:
            return self.C.copy()
        return np.full((self.M, self.ldc), fill, dtype=np.float32)


def _draw(rng, dist, shape):
    if dist == "uniform":
        x = rng.uniform(-1.0, 1.0, size=shape)
    elif dist == "normal":
        x = rng.standard_normal(size=shape)
    elif dist == "int2":
        x = rng.integers(-2, 3, size=shape).astype(np.float64)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return x.astype(np.float32)


def _store(x, ld, pad_value):
    rows, cols = x.shape
    if ld < max(1, cols):
        raise ValueError("leading dimension below the row length")
    s = np.full((max(rows, 0), ld), pad_value, dtype=np.float32)
    s[:, :cols] = x
    return s


def make_case(M, N, K, trans_b=False, alpha=1.0, beta=0.0, dist="uniform", seed=0,
              lda=None, ldb=None, ldc=None, pad_value=np.nan, with_c=None) -> Case:
    """Draw one case in the documented order: A, then B (stored shape), then C."""
    rng = np.random.default_rng(seed)
    lda = max(1, K) if lda is None else lda
    ldb = (max(1, K) if trans_b else max(1, N)) if ldb is None else ldb
    ldc = max(1, N) if ldc is None else ldc
    A = _store(_draw(rng, dist, (M, K)), lda, pad_value)
    Bshape = (N, K) if trans_b else (K, N)
    B = _store(_draw(rng, dist, Bshape), ldb, pad_value)
    if with_c is None:
        with_c = beta != 0.0
    C = _store(_draw(rng, dist, (M, N)), ldc, pad_value) if with_c else None
    meta = dict(dist=dist, seed=seed)
    return Case(M, N, K, bool(trans_b), float(alpha), float(beta), A, B, C, ldc, meta)


def make_config(name: str, **overrides) -> Case:
    table = CONFIGS if name in CONFIGS else SPLITK_CONFIGS if name in SPLITK_CONFIGS else STREAMK_CONFIGS
    p = dict(table[name])
    p.update(overrides)
    c = make_case(**p)
    c.meta["config"] = name
    return c


def make_row_share(name: str, parts: int, index: int = 0) -> Case:
    """Rows [index*M/parts, (index+1)*M/parts) of workload `name` (A and C
    rows; all of B): what one of `parts` GPUs computes when the output is split
    by rows and B is replicated.  Output tiles are independent ("CUDA矩阵乘法
    性能优化实战", section 1.1), so no share needs another's rows."""
    base = make_config(name)
    if parts < 1 or base.M % parts != 0 or not 0 <= index < parts:
        raise ValueError(f"{name}: {base.M} rows do not split into {parts} equal shares (index {index})")
    r0, r1 = index * base.M // parts, (index + 1) * base.M // parts
    C = None if base.C is None else base.C[r0:r1].copy()
    meta = dict(base.meta, row_share=(parts, index))
    return Case(r1 - r0, base.N, base.K, base.trans_b, base.alpha, base.beta, base.A[r0:r1].copy(), base.B, C,
                base.ldc, meta)


def flops(M, N, K) -> float:
    """2*M*N*K, the FLOP convention every throughput figure uses."""
    return 2.0 * M * N * K


# Transpose workloads.  "现代 CUDA 工具箱实战" measures a 4096 x 4096 float32
# transpose (section 性能实测); the other shapes exercise ragged edges and
# strided storage.
TRANSPOSE_CONFIGS = {
    "t_4096": dict(rows=4096, cols=4096, seed=5),
    "t_8192": dict(rows=8192, cols=8192, seed=9),
    "t_ragged": dict(rows=1000, cols=1017, seed=6),
    "t_wide": dict(rows=3, cols=262147, seed=7),
    "t_tall": dict(rows=262147, cols=3, seed=8),
}

# Bit patterns that a transpose must carry through unchanged: quiet and
# signalling NaNs with payloads, both infinities, both zeros, subnormals and the
# largest finite values.
SPECIAL_BITS = np.array([0x7FC00001, 0xFFC12345, 0x7F800001, 0x7FA00000, 0x7F800000, 0xFF800000,
                         0x00000000, 0x80000000, 0x00000001, 0x807FFFFF, 0x7F7FFFFF, 0xFF7FFFFF],
                        dtype=np.uint32)


def make_transpose_input(rows, cols, seed=0, ld_src=None, dist="uniform", specials=False,
                         pad_value=np.nan) -> np.ndarray:
    """Source storage (rows x ld_src float32) for a transpose.

    Draws the rows x cols matrix from ``dist``; with ``specials`` about one
    element in 64 is then overwritten with a pattern from SPECIAL_BITS (chosen
    by the same generator).  Padding columns hold ``pad_value``.
    """
    rng = np.random.default_rng(seed)
    ld_src = max(1, cols) if ld_src is None else ld_src
    x = _draw(rng, dist, (rows, cols))
    if specials and x.size:
        mask = rng.random(size=x.shape) < 1.0 / 64
        pick = rng.integers(0, SPECIAL_BITS.size, size=x.shape)
        xb = x.view(np.uint32)
        xb[mask] = SPECIAL_BITS[pick[mask]]
    return _store(x, ld_src, pad_value)


def make_transpose_config(name: str, **overrides) -> np.ndarray:
    p = dict(TRANSPOSE_CONFIGS[name])
    p.update(overrides)
    return make_transpose_input(**p)
