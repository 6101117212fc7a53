"""MI355X-native FP32 GEMM: C <- alpha*A*op(B) + beta*C, row-major, op(B) in {B, B^T},
and the out-of-place FP32 matrix transpose dst <- src^T.

The compute path is the HIP library ``libsgemm_f32.so`` (hand-written gfx950
kernels behind a C ABI, declared in include/sgemm_f32.h); this package is its
binding (``sgemm``), its build script (``build``) and the seeded input
generator (``inputs``).  Importing the package loads nothing; the first call
into ``sgemm`` loads the library and raises if it is missing.
"""
from .sgemm import (ALGO, EXPORTS, LIB_PATH, PRECISION, SCRATCH_BYTES, SGEMM_ERR_SCRATCH_LIMIT,  # noqa: F401
                    TRANSPOSE_ALGO, SgemmError, gemm, load,
                    sgemm_f32, sgemm_f32_algo, sgemm_f32_arch_status, sgemm_f32_device_status, sgemm_f32_lowp, sgemm_f32_lowp_2pass, sgemm_f32_lowp_2pass_plan,
                    sgemm_f32_lowp_plan, sgemm_f32_lowp_ws,
                    sgemm_f32_load_probe, sgemm_f32_lowp_ws_plan, sgemm_f32_mfma_probe, sgemm_f32_mfma_probe_lp,
                    sgemm_f32_plan,
                    sgemm_f32_splitk, sgemm_f32_splitk_noalloc, sgemm_f32_splitk_plan, sgemm_f32_status_string, sgemm_f32_streamk,
                    sgemm_f32_streamk_plan, sgemm_f32_ws, sgemm_f32_ws_plan,
                    sgemm_f32_transpose, sgemm_f32_transpose_algo, sgemm_f32_transpose_plan,
                    sgemm_f32_version, transpose)
