"""MI355X-native FP32 GEMM: D = alpha*A*op(B) + beta*C, row-major, op(B) in {B, B^T}."""
