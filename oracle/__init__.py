"""CPU oracles: FP64 D = alpha*A*op(B) + beta*C, and the exact matrix transpose.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may use it; the GEMM library never does.
"""
from .oracle import build, load_library, gemm_rows, gemm_full, tolerance, check, ORACLE_SO, ORACLE_SRC  # noqa: F401
from .oracle_transpose import transpose  # noqa: F401,E402
