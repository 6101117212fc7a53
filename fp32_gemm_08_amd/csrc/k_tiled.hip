// Stage 2: LDS-tiled kernel, one output element per work-item.
//
// The operand tiles that a block of C needs go through LDS, so that each
// element read from global memory serves a whole row or column of outputs
// instead of one ("CUDA矩阵乘法性能优化实战：从朴素内核到寄存器分块与Nsight剖析",
// sections 3.1-3.2; "GPU矩阵乘法优化：共享内存Tiling技术实战", section 4.1).  Rows
// of the LDS tiles may carry one padding float (the first page, section 3.3):
// PAD = 0 keeps the unpadded pitch for the bank-conflict comparison.
//
// Layout for 64-wide wavefronts.  A workgroup is four wavefronts and owns a
// 16 x 16 block of C: lane q of wavefront w computes row 4w + q/16, column
// q%16, so each wavefront covers four whole rows of the block.  The k-range
// is walked in panels of KP = 64: a panel is the 16 x 64 slice of A and the
// 64 x 16 slice of op(B), 1024 floats each, four of each per work-item.
// Panels alternate between two LDS buffers: the loads of panel p+1 are
// issued into registers before panel p is multiplied and written to the
// other buffer after it, so there is one barrier per panel.  Elements outside
// the matrices are staged as zeros.
//
// Global reads: A and op(B) = B^T are read along k, 64 consecutive floats per
// wavefront; op(B) = B along n, four 16-float row pieces per wavefront.  For
// op(B) = B^T the panel is transposed on its way into LDS (the shared-memory
// transpose of "现代 CUDA 工具箱实战：从朴素代码到硬件极限的优化之路"): the 64
// lanes of a wavefront write one column of the k-major panel, a stride of
// 16 + PAD floats apart, which is where the padding column matters.
#include "sgemm_internal.h"

namespace sgemm {

namespace {

constexpr int kTile = 16;               // rows and columns of C per workgroup
constexpr int kPanel = 64;              // k values per panel
constexpr int kLanes = 256;             // work-items per workgroup
constexpr int kPer = kTile * kPanel / kLanes;  // panel elements staged per work-item

template <int PAD>
struct PanelBuf {
    float a[kTile][kPanel + PAD];   // a[i][k] = A(m0 + i, k0 + k)
    float b[kPanel][kTile + PAD];   // b[k][j] = op(B)(k0 + k, n0 + j)
};

// One work-item's share of a panel, held in registers between the global
// loads and the LDS stores.
template <bool TRANS_B, int PAD>
struct PanelStager {
    float va[kPer], vb[kPer];

    // Element s of this work-item: flat index e = tid + 256 s in the panel.
    // A: row e / 64, k e % 64.  op(B) = B: k e / 16, column e % 16.
    // op(B) = B^T: column e / 64, k e % 64 (a row of B, read along k).
    __device__ __forceinline__ void fetch(const GemmArgs &g, int m0, int n0, int k0, int tid)
    {
#pragma unroll
        for (int s = 0; s < kPer; ++s) {
            const int e = tid + kLanes * s;
            const int ar = m0 + e / kPanel, ak = k0 + e % kPanel;
            va[s] = (ar < g.M && ak < g.K) ? g.A[(int64_t)ar * g.lda + ak] : 0.0f;
            if constexpr (TRANS_B) {
                const int bn = n0 + e / kPanel, bk = k0 + e % kPanel;
                vb[s] = (bn < g.N && bk < g.K) ? g.B[(int64_t)bn * g.ldb + bk] : 0.0f;
            } else {
                const int bk = k0 + e / kTile, bn = n0 + e % kTile;
                vb[s] = (bk < g.K && bn < g.N) ? g.B[(int64_t)bk * g.ldb + bn] : 0.0f;
            }
        }
    }

    __device__ __forceinline__ void deposit(PanelBuf<PAD> &p, int tid) const
    {
#pragma unroll
        for (int s = 0; s < kPer; ++s) {
            const int e = tid + kLanes * s;
            p.a[e / kPanel][e % kPanel] = va[s];
            if constexpr (TRANS_B)
                p.b[e % kPanel][e / kPanel] = vb[s];
            else
                p.b[e / kTile][e % kTile] = vb[s];
        }
    }
};

template <bool TRANS_B, int PAD>
__global__ __launch_bounds__(kLanes) void sgemm_tiled_kernel(GemmArgs g)
{
    __shared__ PanelBuf<PAD> buf[2];

    const int tid = (int)threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int i = 4 * wave + (lane >> 4);   // row of C within the block
    const int j = lane & 15;                // column of C within the block
    const int blocks_n = (g.N + kTile - 1) / kTile;
    const int m0 = (int)(blockIdx.x / blocks_n) * kTile;
    const int n0 = (int)(blockIdx.x % blocks_n) * kTile;
    const int panels = (g.K + kPanel - 1) / kPanel;

    PanelStager<TRANS_B, PAD> st;
    st.fetch(g, m0, n0, 0, tid);
    poison_lds(&buf[0], sizeof(PanelBuf<PAD>));
    st.deposit(buf[0], tid);
    __syncthreads();

    float sum = 0.0f;
    for (int p = 0; p < panels; ++p) {
        const bool more = p + 1 < panels;
        if (more)
            st.fetch(g, m0, n0, (p + 1) * kPanel, tid);   // in flight during the products below
        const PanelBuf<PAD> &cur = buf[p & 1];
#pragma unroll 16
        for (int k = 0; k < kPanel; ++k)
            sum = fmaf(cur.a[i][k], cur.b[k][j], sum);
        if (more) {
            // buf[(p + 1) & 1] was last read in panel p - 1, before the barrier
            // that ended it
            poison_lds(&buf[(p + 1) & 1], sizeof(PanelBuf<PAD>));
            st.deposit(buf[(p + 1) & 1], tid);
            __syncthreads();
        }
    }

    const int r = m0 + i, c = n0 + j;
    if (r < g.M && c < g.N) {
        float *out = g.C + (int64_t)r * g.ldc + c;
        *out = (g.beta == 0.0f) ? g.alpha * sum : fmaf(g.alpha, sum, g.beta * *out);
    }
}

}  // namespace

hipError_t launch_tiled(const GemmArgs &a, bool transB, bool pad, hipStream_t stream)
{
    const int64_t blocks = ceil_div(a.N, kTile) * ceil_div(a.M, kTile);
    const dim3 grid((unsigned)blocks), block(kLanes);
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
