// Stage 2: LDS-tiled kernel.  A 16x16 output tile per workgroup; each k-step
// stages a 16x16 tile of A and of op(B) in LDS, zero-filled outside the
// matrices, with one barrier after the stores and one before the next
// overwrite ("CUDA矩阵乘法性能优化实战：从朴素内核到寄存器分块与Nsight剖析",
// section 3.2).  Rows carry one padding float (section 3.3; "GPU矩阵乘法优化：
// 共享内存Tiling技术实战", section 4.1); PAD = 0 keeps the unpadded layout of
// that second page's section 3.1 for the bank-conflict comparison.
//
// With 64-wide wavefronts a 256-work-item workgroup is four wavefronts of
// 4 rows x 16 columns.  For op(B) = B^T the B tile is read along k (coalesced
// rows of B) and written transposed into LDS, the shared-memory transpose of
// "现代 CUDA 工具箱实战：从朴素代码到硬件极限的优化之路" (the padded version);
// that transposed store is where the padding column matters most.
#include "sgemm_internal.h"

namespace sgemm {

template <bool TRANS_B, int PAD>
__global__ __launch_bounds__(256) void sgemm_tiled_kernel(GemmArgs a)
{
    constexpr int T = 16;
    __shared__ float As[T][T + PAD];
    __shared__ float Bs[T][T + PAD];

    const int tx = threadIdx.x % T;
    const int ty = threadIdx.x / T;
    const int nbn = (a.N + T - 1) / T;
    const int bm = blockIdx.x / nbn;
    const int bn = blockIdx.x % nbn;
    const int row = bm * T + ty;
    const int col = bn * T + tx;

    float acc = 0.0f;
    for (int k0 = 0; k0 < a.K; k0 += T) {
        As[ty][tx] = (row < a.M && k0 + tx < a.K) ? a.A[(int64_t)row * a.lda + k0 + tx] : 0.0f;
        if (TRANS_B) {
            // op(B)(k, n) = B[n][k]: work-item (ty, tx) reads row n = bn*T+ty at
            // k = k0+tx and stores it at Bs[k - k0][n - bn*T].
            const int n = bn * T + ty;
            const int k = k0 + tx;
            Bs[tx][ty] = (n < a.N && k < a.K) ? a.B[(int64_t)n * a.ldb + k] : 0.0f;
        } else {
            Bs[ty][tx] = (k0 + ty < a.K && col < a.N) ? a.B[(int64_t)(k0 + ty) * a.ldb + col] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < T; ++k)
            acc = fmaf(As[ty][k], Bs[k][tx], acc);
        __syncthreads();
    }
    if (row < a.M && col < a.N) {
        float *cp = a.C + (int64_t)row * a.ldc + col;
        *cp = (a.beta == 0.0f) ? a.alpha * acc : fmaf(a.alpha, acc, a.beta * *cp);
    }
}

hipError_t launch_tiled(const GemmArgs &a, bool transB, bool pad, hipStream_t stream)
{
    const int64_t blocks = ceil_div(a.N, 16) * ceil_div(a.M, 16);
    const dim3 grid((unsigned)blocks), block(256);
    if (transB) {
        if (pad)
            sgemm_tiled_kernel<true, 1><<<grid, block, 0, stream>>>(a);
        else
            sgemm_tiled_kernel<true, 0><<<grid, block, 0, stream>>>(a);
    } else {
        if (pad)
            sgemm_tiled_kernel<false, 1><<<grid, block, 0, stream>>>(a);
        else
            sgemm_tiled_kernel<false, 0><<<grid, block, 0, stream>>>(a);
    }
    return hipGetLastError();
}

}  // namespace sgemm
