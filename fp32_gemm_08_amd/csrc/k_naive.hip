// Stage 1: one work-item per output element, operands read straight from global
// memory ("CUDA矩阵乘法性能优化实战：从朴素内核到寄存器分块与Nsight剖析", section 2.1),
// plus the C <- beta*C kernel used when the product term vanishes.
//
// Workgroup shape for 64-wide wavefronts: 64 x 4 work-items, so one wavefront
// covers 64 consecutive columns of one output row.  Its B reads (transB == 0)
// are one contiguous 256-byte run and its A read is a single broadcast address;
// the page's 16x16 block split a 32-lane warp across two rows of A (section 2.2),
// which a 64-lane row avoids.
#include "sgemm_internal.h"

namespace sgemm {

template <bool TRANS_B>
__global__ __launch_bounds__(256) void sgemm_naive_kernel(GemmArgs a)
{
    const int tx = threadIdx.x & 63;
    const int ty = threadIdx.x >> 6;
    const int64_t nbn = ceil_div(a.N, 64);
    const int64_t bid = blockIdx.x;
    const int col = (int)(bid % nbn) * 64 + tx;
    const int row = (int)(bid / nbn) * 4 + ty;
    if (row >= a.M || col >= a.N)
        return;
    const float *__restrict__ arow = a.A + (int64_t)row * a.lda;
    float acc = 0.0f;
    if (TRANS_B) {
        const float *__restrict__ brow = a.B + (int64_t)col * a.ldb;
        for (int k = 0; k < a.K; ++k)
            acc = fmaf(arow[k], brow[k], acc);
    } else {
        const float *__restrict__ bcol = a.B + col;
        for (int k = 0; k < a.K; ++k)
            acc = fmaf(arow[k], bcol[(int64_t)k * a.ldb], acc);
    }
    float *cp = a.C + (int64_t)row * a.ldc + col;
    *cp = (a.beta == 0.0f) ? a.alpha * acc : fmaf(a.alpha, acc, a.beta * *cp);
}

// The second naive formulation (Baidu Cloud article comparing the naive and 2-D
// block-tiled CUDA matmul, paragraph on the naive implementation: one block per
// output element, its threads forming partial products that the block reduces):
// a group of work-items shares one output element; each forms a partial dot
// product and the group reduces them.  On MI355X the group is one
// 64-lane wavefront: lane l sums k = l, l+64, l+128, ... (the A row is read
// contiguously across the lanes; B's column is strided unless op(B) = B^T), and
// the 64 partials are added by a fixed butterfly of cross-lane exchanges
// (xor 32, 16, 8, 4, 2, 1), so every lane ends with the same, reproducible sum.
// Workgroups of one wavefront loop over the output elements.
template <bool TRANS_B>
__global__ __launch_bounds__(64) void sgemm_naive_wg_kernel(GemmArgs a)
{
    const int lane = threadIdx.x;
    const int64_t outputs = (int64_t)a.M * a.N;
    for (int64_t o = blockIdx.x; o < outputs; o += gridDim.x) {
        const int row = (int)(o / a.N), col = (int)(o % a.N);
        const float *__restrict__ arow = a.A + (int64_t)row * a.lda;
        float part = 0.0f;
        if (TRANS_B) {
            const float *__restrict__ brow = a.B + (int64_t)col * a.ldb;
            for (int k = lane; k < a.K; k += 64)
                part = fmaf(arow[k], brow[k], part);
        } else {
            const float *__restrict__ bcol = a.B + col;
            for (int k = lane; k < a.K; k += 64)
                part = fmaf(arow[k], bcol[(int64_t)k * a.ldb], part);
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            part += __shfl_xor(part, off, 64);
        if (lane == 0) {
            float *cp = a.C + (int64_t)row * a.ldc + col;
            *cp = (a.beta == 0.0f) ? a.alpha * part : fmaf(a.alpha, part, a.beta * *cp);
        }
    }
}

// C <- beta*C over the M x N window; beta == 0 writes zeros without reading C.
__global__ __launch_bounds__(256) void sgemm_scale_kernel(GemmArgs a)
{
    const int64_t nbn = ceil_div(a.N, 256);
    const int64_t row = blockIdx.x / nbn;
    const int64_t col = (blockIdx.x % nbn) * 256 + threadIdx.x;
    if (row >= a.M || col >= a.N)
        return;
    float *cp = a.C + row * a.ldc + col;
    *cp = (a.beta == 0.0f) ? 0.0f : a.beta * *cp;
}

hipError_t launch_naive(const GemmArgs &a, bool transB, hipStream_t stream)
{
    const int64_t blocks = ceil_div(a.N, 64) * ceil_div(a.M, 4);
    if (transB)
        sgemm_naive_kernel<true><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(a);
    else
        sgemm_naive_kernel<false><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_naive_wg(const GemmArgs &a, bool transB, hipStream_t stream)
{
    const int64_t outputs = (int64_t)a.M * a.N;
    const int64_t blocks = outputs < (1 << 20) ? outputs : (1 << 20);
    if (transB)
        sgemm_naive_wg_kernel<true><<<dim3((unsigned)blocks), dim3(64), 0, stream>>>(a);
    else
        sgemm_naive_wg_kernel<false><<<dim3((unsigned)blocks), dim3(64), 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_scale(const GemmArgs &a, hipStream_t stream)
{
    const int64_t blocks = ceil_div(a.N, 256) * (int64_t)a.M;
    sgemm_scale_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace sgemm
