"""CPU oracles: FP64 D = alpha*A*op(B) + beta*C, its mixed-precision variant
(operands rounded to fp16 or bf16), and the exact matrix transpose.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may use it; the GEMM library never does.
"""
from .oracle import (build, build_sanitized, load_library, gemm_rows, gemm_full, tolerance, check,  # noqa: F401
                     ORACLE_SANITIZE_SO, ORACLE_SO, ORACLE_SRC)
from .oracle_transpose import transpose  # noqa: F401,E402
from .oracle_lowp import PRECISIONS, gemm_lowp_rows, round_bf16, round_fp16, round_to  # noqa: F401,E402
