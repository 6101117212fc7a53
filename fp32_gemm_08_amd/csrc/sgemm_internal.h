// Internal declarations shared by the host dispatcher and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgemm {

// Problem description handed to every kernel by value (kernel arguments).
// Dimensions are validated to fit in int32; offsets are formed in int64.
struct GemmArgs {
    const float *A;
    const float *B;
    float *C;
    int64_t lda, ldb, ldc;
    int M, N, K;
    float alpha, beta;
    int flags;  // GEMM_FLAG_* bits
    // k-split partial pass (MFMA kernel, launched with gridDim.y = number of
    // splits): split s multiplies k in [s*k_split, min(K, (s+1)*k_split)) and
    // writes its raw product to C + s*c_split_stride.  Unused when gridDim.y == 1.
    int k_split;
    int64_t c_split_stride;
};

// Stream-K schedule of one MFMA launch over a T-tile grid whose tiles each
// take `iters` k-iterations (one LDS stage of k each).  The first `dp`
// workgroups take one whole tile each, as the plain kernel does; the next
// `workers` workgroups share the k-iterations of the remaining sk_tiles
// tiles, worker w taking iterations [w*S/workers, (w+1)*S/workers) of the
// S = sk_tiles*iters that follow the data-parallel tiles.  A worker writes a
// tile it covers whole straight into C; a piece of a tile goes into one of
// its two workspace slots (slot 0 for its first piece, 1 for its last), each
// BM x BN floats with row pitch BN, and the fix-up kernel adds a split tile's
// pieces in worker order and applies the epilogue.
struct SkArgs {
    float *ws;
    int dp;
    int workers;
    int sk_tiles;
    int iters;
};

// The MFMA kernel may stage interior tiles with direct global->LDS loads, whose
// per-lane source offsets are 32-bit: set when 256 rows of A (and of B) span
// fewer than 2^31 elements.
constexpr int GEMM_FLAG_DIRECT = 1;

// Kernel identifiers reported by the planning query.
enum KernelId : int {
    KID_NONE = 0,
    KID_SCALE = 1,          // C <- beta*C (alpha == 0 or K == 0)
    KID_NAIVE = 10,
    KID_NAIVE_WG = 11,      // one wavefront per output element, cross-lane reduction
    KID_TILED_PAD = 20,
    KID_TILED_NOPAD = 21,
    KID_REGBLOCK = 30,
    KID_MFMA_L = 40,        // 256 x 256 macro tile, 8 wavefronts
    KID_MFMA_M = 41,        // 128 x 128, 8 wavefronts: 2 x 2 over the tile x 2 over k
    KID_MFMA_S = 42,        // 64 x 64, 4 wavefronts
    KID_MFMA_L_SK = 43,     // KID_MFMA_L under a stream-K schedule (+ fix-up kernel)
    KID_MFMA_M_SK = 44,     // KID_MFMA_M under a stream-K schedule (+ fix-up kernel)
    KID_MFMA_S2 = 45,       // 64 x 64, 8 wavefronts: 2 x 2 over the tile x 2 over k
    KID_MFMA_T = 46,        // 32 x 32, 4 wavefronts: one per k-slice, k split 4 ways
    KID_MFMA_R = 47,        // 128 x 64, 8 wavefronts: 4 x 1 over the tile x 2 over k
    KID_MFMA_LP_F16 = 60,   // mixed precision, operands rounded to fp16, 256 x 256
    KID_MFMA_LP_BF16 = 61,  // the same with bf16
    KID_MFMA_LP_F16_S = 62, // mixed precision, fp16, 64 x 64 (few output tiles)
    KID_MFMA_LP_BF16_S = 63,
    KID_LP16_F16 = 64,      // two-pass mixed precision (rounding pass + 16-bit GEMM), fp16, 256 x 256
    KID_LP16_BF16 = 65,
    KID_LP16_F16_S = 66,    // the same with 128 x 128 tiles
    KID_LP16_BF16_S = 67,
};

// Tile geometry of each kernel (rows x cols of C per workgroup).
struct TileShape {
    int bm, bn;
};
TileShape tile_shape(int kid);

// Launchers: enqueue one kernel on `stream`, return hipGetLastError().
hipError_t launch_scale(const GemmArgs &a, hipStream_t stream);
hipError_t launch_naive(const GemmArgs &a, bool transB, hipStream_t stream);
hipError_t launch_naive_wg(const GemmArgs &a, bool transB, hipStream_t stream);
hipError_t launch_tiled(const GemmArgs &a, bool transB, bool pad, hipStream_t stream);
hipError_t launch_regblock(const GemmArgs &a, bool transB, bool vec, hipStream_t stream);
// The MFMA kernels load operands 16 bytes at a time from any 4-byte aligned
// address (the host requires float-aligned A and B).
hipError_t launch_mfma(const GemmArgs &a, int kid, bool transB, hipStream_t stream, int splits = 1);
// Stream-K launch of the 256 x 256 (KID_MFMA_L) or 128 x 128 (KID_MFMA_M)
// tile, then the fix-up of its split tiles (nothing when sk.sk_tiles == 0).
// `iters` must be ceil(K / mfma_stage_k(kid)).
hipError_t launch_mfma_sk(const GemmArgs &a, const SkArgs &sk, int kid, bool transB, hipStream_t stream);
int mfma_stage_k(int kid);
// Mixed precision: operands rounded to fp16 (bf16 = false) or bf16 while staged.
hipError_t launch_mfma_lp(const GemmArgs &a, bool large, bool bf16, bool transB, bool vec, hipStream_t stream);

// Two-pass mixed precision (rounding pass into the workspace, then the GEMM on
// 16-bit operands): 256 x 256 tiles when `large`, else 128 x 128.
struct Lp16Args {
    const void *A16;   // Kp/32 slabs of Mp rows x 32 values
    const void *B16;   // Kp/32 slabs of Np rows x 32 values
    float *C;
    int64_t slab_a, slab_b;  // values per slab: Mp*32, Np*32
    int64_t ldc;
    int M, N, Kp;
    float alpha, beta;
    int tiles_m, tiles_n;
};
TileShape lp16_tile_shape(bool large);
int64_t lp16_workspace_bytes(int64_t M, int64_t N, int64_t K, bool large);
hipError_t launch_lp16(const GemmArgs &a, bool large, bool bf16, bool transB, void *ws, hipStream_t stream);
TileShape lp_tile_shape(bool large);
// C <- alpha * sum_{s<splits} W[s*stride + i*N + j] + beta*C (C not read when beta == 0).
hipError_t launch_splitk_reduce(const float *W, int splits, int64_t stride, int M, int N, float alpha, float beta,
                                float *C, int64_t ldc, bool vec, hipStream_t stream);

// Debug build (-DSGEMM_DEBUG_POISON_LDS): before a workgroup stages data
// into an LDS region, the whole region is filled with a pattern that reads
// as NaN in FP32, FP16 and BF16 (0x7fc07fc0 per 32-bit word), every
// work-item a share, and the workgroup meets a barrier.  A read of a
// location the staging never writes, a read that runs ahead of the copy
// that fills it, or a staging write that lands while another wavefront
// still reads the previous contents (the missing second barrier of
// "CUDA矩阵乘法性能优化实战：从朴素内核到寄存器分块与Nsight剖析", section 3.2)
// then puts a NaN into the result, where the parity checks see it.  In the
// normal build the call is empty.  Call it from uniform control flow only.
#ifdef SGEMM_DEBUG_POISON_LDS
constexpr bool kPoisonLds = true;
#else
constexpr bool kPoisonLds = false;
#endif

__device__ __forceinline__ void poison_lds(void *p, int bytes)
{
    if constexpr (kPoisonLds) {
        uint32_t *w = static_cast<uint32_t *>(p);
        for (int i = (int)threadIdx.x; i < bytes / 4; i += (int)blockDim.x)
            w[i] = 0x7fc07fc0u;
        __syncthreads();
    }
}

// Number of workgroup tiles along one dimension.
__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace sgemm
