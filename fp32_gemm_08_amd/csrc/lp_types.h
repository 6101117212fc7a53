// 16-bit operand types and the matrix-core step shared by the mixed-precision
// kernels: v_mfma_f32_32x32x16_{f16,bf16} adds to a 32x32 FP32 block the
// product of a 32x16 block of A and a 16x32 block of op(B); lane l supplies 8
// consecutive k values (16 bytes) of A row l%32 and of op(B) column l%32, the
// half l/32 choosing which 8 of the 16.  Accumulator register r of lane l holds
// row 8*(r/4) + 4*(l/32) + r%4, column l%32 of the block.
#pragma once
#include <hip/hip_runtime.h>

namespace sgemm {

typedef float lp_f32x4 __attribute__((ext_vector_type(4)));
typedef float lp_f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 lp_h8 __attribute__((ext_vector_type(8)));
typedef __bf16 lp_b8 __attribute__((ext_vector_type(8)));
typedef _Float16 lp_h4 __attribute__((ext_vector_type(4)));
typedef __bf16 lp_b4 __attribute__((ext_vector_type(4)));

template <bool BF16> struct Lp;
template <> struct Lp<false> {
    typedef _Float16 T;
    typedef lp_h8 V8;
    typedef lp_h4 V4;
    static __device__ __forceinline__ lp_f32x16 mma(V8 a, V8 b, lp_f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};
template <> struct Lp<true> {
    typedef __bf16 T;
    typedef lp_b8 V8;
    typedef lp_b4 V4;
    static __device__ __forceinline__ lp_f32x16 mma(V8 a, V8 b, lp_f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

}  // namespace sgemm
