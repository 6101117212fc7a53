// Stage 3: register-blocked macro tile on the vector ALU.
//
// A 128x128 tile of C per 256-work-item workgroup, 8x8 outputs per work-item
// kept in registers ("CUDA矩阵乘法性能优化实战：从朴素内核到寄存器分块与Nsight剖析",
// section 5.2: with TMxTN outputs a thread issues (TM+TN) LDS reads per TM*TN
// FMAs, 0.25 here), 128-bit global loads when rows are 16-byte aligned
// (section 5.3), and double-buffered staging ("GPU矩阵乘法优化：共享内存Tiling技术实战",
// section 3.2, read as two LDS buffers in ping-pong: the global loads of tile t+1
// are in flight while tile t is consumed, one barrier per tile).
//
// The A tile is stored k-major (As[k][m]) so a work-item fetches its 8 rows of A
// for one k as two 128-bit LDS reads.  Rows and columns are split 4 + 4 (m, m+64
// and n, n+64), so within a wavefront the A reads touch 4 broadcast addresses and
// the 16 distinct B fragments form one contiguous 256-byte run.  The FMAs are
// plain v_fmac_f32 (packed FP32 is kept out of the build); the stage's ceiling is
// the vector FP32 rate.
#include "sgemm_internal.h"

namespace sgemm {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool TRANS_B, bool VEC>
__global__ __launch_bounds__(256) void sgemm_regblock_kernel(GemmArgs a)
{
    constexpr int BM = 128, BN = 128, BK = 8;
    constexpr int SA = BM + 4, SB = BN + 4;
    __shared__ __attribute__((aligned(16))) float As[2][BK * SA];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK * SB];

    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int nbn = (a.N + BN - 1) / BN;
    const int m0 = (blockIdx.x / nbn) * BM;
    const int n0 = (blockIdx.x % nbn) * BN;

    // Global staging assignment: one 4-float chunk of A and one of B per work-item.
    const int a_r = tid >> 1, a_c = (tid & 1) * 4;             // A: row, k offset
    const int b_r = TRANS_B ? (tid >> 1) : (tid >> 5);         // B^T: n row / B: k row
    const int b_c = TRANS_B ? (tid & 1) * 4 : (tid & 31) * 4;  // B^T: k offset / B: n offset

    auto load4 = [](const float *p, bool row_ok, int first, int limit, bool vec) {
        f32x4 v;
        if (vec && row_ok && first + 4 <= limit) {
            v = *reinterpret_cast<const f32x4 *>(p);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = (row_ok && first + e < limit) ? p[e] : 0.0f;
        }
        return v;
    };
    auto gload = [&](int k0, f32x4 &va, f32x4 &vb) {
        const int gm = m0 + a_r, gk = k0 + a_c;
        va = load4(a.A + (int64_t)gm * a.lda + gk, gm < a.M, gk, a.K, VEC);
        if (TRANS_B) {
            const int gn = n0 + b_r, gkb = k0 + b_c;
            vb = load4(a.B + (int64_t)gn * a.ldb + gkb, gn < a.N, gkb, a.K, VEC);
        } else {
            const int gkb = k0 + b_r, gn = n0 + b_c;
            vb = load4(a.B + (int64_t)gkb * a.ldb + gn, gkb < a.K, gn, a.N, VEC);
        }
    };
    auto sstore = [&](int buf, const f32x4 &va, const f32x4 &vb) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            As[buf][(a_c + e) * SA + a_r] = va[e];
        if (TRANS_B) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                Bs[buf][(b_c + e) * SB + b_r] = vb[e];
        } else {
            *reinterpret_cast<f32x4 *>(&Bs[buf][b_r * SB + b_c]) = vb;
        }
    };

    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[i][j] = 0.0f;

    const int nk = (a.K + BK - 1) / BK;
    f32x4 va, vb;
    gload(0, va, vb);
    poison_lds(As[0], sizeof(As[0]));
    poison_lds(Bs[0], sizeof(Bs[0]));
    sstore(0, va, vb);
    __syncthreads();
    for (int t = 0; t < nk; ++t) {
        const int cur = t & 1;
        if (t + 1 < nk)
            gload((t + 1) * BK, va, vb);
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            const f32x4 a0 = *reinterpret_cast<const f32x4 *>(&As[cur][k * SA + ty * 4]);
            const f32x4 a1 = *reinterpret_cast<const f32x4 *>(&As[cur][k * SA + 64 + ty * 4]);
            const f32x4 b0 = *reinterpret_cast<const f32x4 *>(&Bs[cur][k * SB + tx * 4]);
            const f32x4 b1 = *reinterpret_cast<const f32x4 *>(&Bs[cur][k * SB + 64 + tx * 4]);
            const float av[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            const float bv[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
        }
        if (t + 1 < nk) {
            poison_lds(As[cur ^ 1], sizeof(As[0]));
            poison_lds(Bs[cur ^ 1], sizeof(Bs[0]));
            sstore(cur ^ 1, va, vb);
        }
        __syncthreads();
    }

    // Epilogue: rows {ty*4+i, 64+ty*4+i}, columns {tx*4+j, 64+tx*4+j}.
    const bool cvec = ((reinterpret_cast<uintptr_t>(a.C) & 15) == 0) && ((a.ldc & 3) == 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = m0 + (i < 4 ? ty * 4 + i : 64 + ty * 4 + (i - 4));
        if (row >= a.M)
            continue;
        float *crow = a.C + (int64_t)row * a.ldc;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int col = n0 + h * 64 + tx * 4;
            if (cvec && col + 4 <= a.N) {
                f32x4 v;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    v[j] = a.alpha * acc[i][h * 4 + j];
                if (a.beta != 0.0f) {
                    const f32x4 old = *reinterpret_cast<const f32x4 *>(crow + col);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        v[j] = fmaf(a.alpha, acc[i][h * 4 + j], a.beta * old[j]);
                }
                *reinterpret_cast<f32x4 *>(crow + col) = v;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (col + j < a.N) {
                        float *cp = crow + col + j;
                        const float r = acc[i][h * 4 + j];
                        *cp = (a.beta == 0.0f) ? a.alpha * r : fmaf(a.alpha, r, a.beta * *cp);
                    }
                }
            }
        }
    }
}

hipError_t launch_regblock(const GemmArgs &a, bool transB, bool vec, hipStream_t stream)
{
    const int64_t blocks = ceil_div(a.N, 128) * ceil_div(a.M, 128);
    const dim3 grid((unsigned)blocks), block(256);
    if (transB) {
        if (vec)
            sgemm_regblock_kernel<true, true><<<grid, block, 0, stream>>>(a);
        else
            sgemm_regblock_kernel<true, false><<<grid, block, 0, stream>>>(a);
    } else {
        if (vec)
            sgemm_regblock_kernel<false, true><<<grid, block, 0, stream>>>(a);
        else
            sgemm_regblock_kernel<false, false><<<grid, block, 0, stream>>>(a);
    }
    return hipGetLastError();
}

}  // namespace sgemm
