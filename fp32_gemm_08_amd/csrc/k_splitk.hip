// Reduction of k-split partial products.
//
// With a caller workspace, a GEMM whose output tiles are too few to occupy the
// 256 CUs splits its k-range over several workgroups per tile (the split count
// is the grid's second dimension of the MFMA kernel); split s leaves its raw
// product sum_{k in its range} A(i,k) op(B)(k,j) in W + s*stride, rows of N
// floats.  This kernel adds the splits in a fixed order (s = 0, 1, ...) and
// applies the epilogue, so the result does not depend on scheduling:
//
//     C(i,j) <- alpha * sum_s W[s*stride + i*N + j] + beta * C(i,j)
//
// C is not read when beta == 0.  The output tiles are independent ("CUDA矩阵乘法
// 性能优化实战：从朴素内核到寄存器分块与Nsight剖析", section 1.1: every element is its
// own sum of K products), and a sum split into partial sums is the Tiling page's
// own device ("GPU矩阵乘法优化：共享内存Tiling技术实战", section 4.2, two partial
// accumulators).  The kernel is bound by memory bandwidth: (splits + 1) reads
// (splits without beta) and one write per element, mostly from the Infinity
// Cache, where the partials were just written.
#include "sgemm_internal.h"

namespace sgemm {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// One work-item per 4 consecutive elements of a row (VEC: N % 4 == 0, W, C and
// ldc 16-byte aligned, so whole float4s are read and written); 64 work-items
// per workgroup so that a small output still spreads over every CU.  The loads
// of up to SPLIT_BATCH splits are issued together and then added in split
// order, so the many small reads overlap while the sum keeps its fixed order.
constexpr int SPLIT_BATCH = 8;

template <bool VEC>
__global__ __launch_bounds__(64) void splitk_reduce_kernel(const float *__restrict__ W, int splits, int64_t stride,
                                                           int M, int N, float alpha, float beta,
                                                           float *__restrict__ C, int64_t ldc)
{
    const int quads = (N + 3) / 4;
    const int64_t total = (int64_t)M * quads;
    for (int64_t t = (int64_t)blockIdx.x * 64 + threadIdx.x; t < total; t += (int64_t)gridDim.x * 64) {
        const int i = (int)(t / quads), j = (int)(t % quads) * 4;
        const int n = VEC ? 4 : (N - j < 4 ? N - j : 4);
        const float *w = W + (int64_t)i * N + j;
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int s0 = 0; s0 < splits; s0 += SPLIT_BATCH) {
            f32x4 part[SPLIT_BATCH];
#pragma unroll
            for (int b = 0; b < SPLIT_BATCH; ++b) {
                const float *p = w + (int64_t)(s0 + b) * stride;
                if (s0 + b < splits) {
                    if (VEC) {
                        part[b] = *reinterpret_cast<const f32x4 *>(p);
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            part[b][q] = q < n ? p[q] : 0.0f;
                    }
                }
            }
#pragma unroll
            for (int b = 0; b < SPLIT_BATCH; ++b)
                if (s0 + b < splits)
                    acc = (s0 + b == 0) ? part[b] : acc + part[b];
        }
        float *c = C + (int64_t)i * ldc + j;
        if (VEC) {
            f32x4 out = alpha * acc;
            if (beta != 0.0f)
                out += beta * *reinterpret_cast<const f32x4 *>(c);
            *reinterpret_cast<f32x4 *>(c) = out;
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (q < n) {
                    float out = alpha * acc[q];
                    if (beta != 0.0f)
                        out += beta * c[q];
                    c[q] = out;
                }
            }
        }
    }
}

hipError_t launch_splitk_reduce(const float *W, int splits, int64_t stride, int M, int N, float alpha, float beta,
                                float *C, int64_t ldc, bool vec, hipStream_t stream)
{
    const int64_t total = (int64_t)M * ((N + 3) / 4);
    const int64_t blocks = ceil_div(total, 64) < (1 << 20) ? ceil_div(total, 64) : (1 << 20);
    if (vec)
        splitk_reduce_kernel<true><<<dim3((unsigned)blocks), dim3(64), 0, stream>>>(W, splits, stride, M, N, alpha,
                                                                                 beta, C, ldc);
    else
        splitk_reduce_kernel<false><<<dim3((unsigned)blocks), dim3(64), 0, stream>>>(W, splits, stride, M, N, alpha,
                                                                                  beta, C, ldc);
    return hipGetLastError();
}

}  // namespace sgemm
