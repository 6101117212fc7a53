// Stage 4: FP32 matrix-core (MFMA) path for gfx950.
//
// The contraction is dense, so it belongs on the CDNA matrix cores:
// v_mfma_f32_32x32x2_f32 multiplies a 32x2 FP32 block of A by a 2x32 FP32 block
// of B into a 32x32 FP32 accumulator (16 values per lane), at the chip's full
// FP32 matrix rate.  The tiling has the three levels of "GPU矩阵乘法优化：共享内存
// Tiling技术实战", section 7.3 (grid -> workgroup tile in LDS -> wavefront tile in
// registers), with the 2-D block tiling (b_m, b_n, b_k) of the Baidu Cloud article
// comparing naive and 2-D block-tiled matmul, and the LDS tiles double-buffered
// (the second page, section 3.2, read as a two-buffer ping-pong).
//
// Layout choices (MI355X-specific, not from the pages):
//   * k-permutation: an MFMA consumes two k values, one from each half of the
//     wavefront.  Over a group of 8 k values, half h of the wavefront supplies
//     k = 8g + 4h + s at step s (s = 0..3), so a lane's A operands for four MFMAs
//     are four consecutive floats of one A row: one 128-bit LDS read.  The sum
//     over k is unchanged; only its order differs, which the contract allows.
//   * column interleave (op(B) = B): a wavefront's IL column blocks are
//     interleaved so lane j owns columns IL*j .. IL*j+IL-1 of the group; the B
//     operands of IL blocks at one k are then one IL-wide LDS read, and the
//     epilogue writes IL consecutive columns per lane.
//   * op(B) = B^T is staged k-contiguous like A (rows of B are already k-major),
//     so it needs neither a transpose nor an interleave.
//   * LDS rows of A (and of B^T) are padded by 4 floats: the 16-byte rows read by
//     consecutive lanes then start on distinct banks (the +1 padding idea of
//     "CUDA矩阵乘法性能优化实战：从朴素内核到寄存器分块与Nsight剖析", section 3.3,
//     at 128-bit granularity).
//   * Workgroups are dispatched round-robin over the 8 XCDs; tiles are remapped
//     so each XCD gets a contiguous run, grouped 8 tile-rows at a time, so tiles
//     that share rows of A and columns of B run on the same L2.
#include "sgemm_internal.h"

namespace sgemm {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int W> struct vec_of;
template <> struct vec_of<1> { typedef float type; };
template <> struct vec_of<2> { typedef f32x2 type; };
template <> struct vec_of<4> { typedef f32x4 type; };

template <int W>
__device__ __forceinline__ float vget(const typename vec_of<W>::type &v, int i);
template <> __device__ __forceinline__ float vget<1>(const float &v, int) { return v; }
template <> __device__ __forceinline__ float vget<2>(const f32x2 &v, int i) { return v[i]; }
template <> __device__ __forceinline__ float vget<4>(const f32x4 &v, int i) { return v[i]; }

// Tile index for workgroup `bid` over an nbm x nbn tile grid (see header note).
__device__ __forceinline__ void map_tile(int bid, int nbm, int nbn, int &tm, int &tn)
{
    const int total = nbm * nbn;
    int t = bid;
    if ((total & 7) == 0)
        t = (bid & 7) * (total >> 3) + (bid >> 3);
    constexpr int G = 8;
    const int per_group = G * nbn;
    const int gi = t / per_group;
    const int first = gi * G;
    const int gsz = min(nbm - first, G);
    const int in = t - gi * per_group;
    tm = first + in % gsz;
    tn = in / gsz;
}

// Four consecutive floats starting at p[0]; elements at or beyond `limit`
// (or all of them when !ok) read as zero.  `vec` allows one 128-bit load.
__device__ __forceinline__ f32x4 load4(const float *p, bool ok, int first, int limit, bool vec)
{
    f32x4 v;
    if (vec && ok && first + 4 <= limit) {
        v = *reinterpret_cast<const f32x4 *>(p);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = (ok && first + e < limit) ? p[e] : 0.0f;
    }
    return v;
}

template <int BM, int BN, int BK, int WGM, int WGN, bool TRANS_B, bool VEC>
__global__ __launch_bounds__(256) void sgemm_mfma_kernel(GemmArgs a)
{
    static_assert(WGM * WGN == 4, "four wavefronts per workgroup");
    constexpr int NT = 256;
    constexpr int WM = BM / WGM, WN = BN / WGN;      // wavefront tile
    constexpr int FM = WM / 32, FN = WN / 32;        // 32x32 blocks per wavefront
    constexpr int IL = TRANS_B ? 1 : (FN >= 4 ? 4 : FN);
    constexpr int NG = FN / IL;                      // interleaved column groups
    constexpr int SA = BK + 4;                       // A row stride in LDS (floats)
    constexpr int SB = TRANS_B ? BK + 4 : BN;        // B^T row stride / B row stride
    constexpr int A_SZ = BM * SA;
    constexpr int B_SZ = TRANS_B ? BN * SB : BK * SB;
    constexpr int KC = BK / 4;                       // 4-float chunks per k-row
    constexpr int CA = BM * KC / NT;                 // A chunks per work-item
    constexpr int CB = (TRANS_B ? BN * KC : BK * (BN / 4)) / NT;
    static_assert(WM % 32 == 0 && WN % 32 == 0 && BK % 8 == 0, "tile shape");
    static_assert(BM * KC % NT == 0 && (TRANS_B ? BN * KC : BK * (BN / 4)) % NT == 0, "staging split");
    typedef typename vec_of<IL>::type bvec;

    __shared__ __attribute__((aligned(16))) float smem[2 * (A_SZ + B_SZ)];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int wm = wave / WGN, wn = wave % WGN;

    const int nbm = (a.M + BM - 1) / BM, nbn = (a.N + BN - 1) / BN;
    int tile_m, tile_n;
    map_tile(blockIdx.x, nbm, nbn, tile_m, tile_n);
    const int m0 = tile_m * BM, n0 = tile_n * BN;

    f32x4 ra[CA], rb[CB];

    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            const int q = tid + i * NT;
            const int r = q / KC, c = q % KC;
            const int gm = m0 + r, gk = k0 + 4 * c;
            ra[i] = load4(a.A + (int64_t)gm * a.lda + gk, gm < a.M, gk, a.K, VEC);
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int q = tid + i * NT;
            if (TRANS_B) {
                const int r = q / KC, c = q % KC;
                const int gn = n0 + r, gk = k0 + 4 * c;
                rb[i] = load4(a.B + (int64_t)gn * a.ldb + gk, gn < a.N, gk, a.K, VEC);
            } else {
                const int r = q / (BN / 4), c = q % (BN / 4);
                const int gk = k0 + r, gn = n0 + 4 * c;
                rb[i] = load4(a.B + (int64_t)gk * a.ldb + gn, gk < a.K, gn, a.N, VEC);
            }
        }
    };
    auto sstore = [&](int buf) {
        float *As = smem + buf * (A_SZ + B_SZ);
        float *Bs = As + A_SZ;
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            const int q = tid + i * NT;
            *reinterpret_cast<f32x4 *>(&As[(q / KC) * SA + 4 * (q % KC)]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int q = tid + i * NT;
            if (TRANS_B)
                *reinterpret_cast<f32x4 *>(&Bs[(q / KC) * SB + 4 * (q % KC)]) = rb[i];
            else
                *reinterpret_cast<f32x4 *>(&Bs[(q / (BN / 4)) * SB + 4 * (q % (BN / 4))]) = rb[i];
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = f32x16{0};

    auto compute = [&](int buf) {
        const float *As = smem + buf * (A_SZ + B_SZ);
        const float *Bs = As + A_SZ;
#pragma unroll
        for (int g = 0; g < BK / 8; ++g) {
            const int kq = 8 * g + 4 * hi;   // this half's first k in the group
            f32x4 af[FM];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                af[fm] = *reinterpret_cast<const f32x4 *>(&As[(wm * WM + 32 * fm + l32) * SA + kq]);
            if (TRANS_B) {
                f32x4 bt[FN];
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    bt[fn] = *reinterpret_cast<const f32x4 *>(&Bs[(wn * WN + 32 * fn + l32) * SB + kq]);
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                        for (int fn = 0; fn < FN; ++fn)
                            acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[fm][s], bt[fn][s],
                                                                               acc[fm][fn], 0, 0, 0);
            } else {
                bvec bf[4][NG];
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int gr = 0; gr < NG; ++gr)
                        bf[s][gr] = *reinterpret_cast<const bvec *>(
                            &Bs[(kq + s) * SB + wn * WN + gr * 32 * IL + IL * l32]);
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                        for (int gr = 0; gr < NG; ++gr)
#pragma unroll
                            for (int b = 0; b < IL; ++b)
                                acc[fm][gr * IL + b] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                                    af[fm][s], vget<IL>(bf[s][gr], b), acc[fm][gr * IL + b], 0, 0, 0);
            }
        }
    };

    const int nk = (a.K + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int t = 0; t < nk; ++t) {
        if (t + 1 < nk)
            gload((t + 1) * BK);
        compute(t & 1);
        if (t + 1 < nk)
            sstore((t + 1) & 1);
        __syncthreads();
    }

    // Epilogue.  Accumulator register r of a 32x32 block holds row
    // 8*(r/4) + 4*hi + (r%4) and column l32 of that block.
    const uintptr_t cbase = reinterpret_cast<uintptr_t>(a.C);
    const bool cvec = IL > 1 && (cbase % (4 * IL)) == 0 && (a.ldc % IL) == 0;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = m0 + wm * WM + 32 * fm + 8 * (r / 4) + 4 * hi + (r % 4);
            if (row >= a.M)
                continue;
            float *crow = a.C + (int64_t)row * a.ldc;
            if (TRANS_B) {
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    const int col = n0 + wn * WN + 32 * fn + l32;
                    if (col < a.N) {
                        const float v = acc[fm][fn][r];
                        crow[col] = (a.beta == 0.0f) ? a.alpha * v : fmaf(a.alpha, v, a.beta * crow[col]);
                    }
                }
            } else {
#pragma unroll
                for (int gr = 0; gr < NG; ++gr) {
                    const int col = n0 + wn * WN + gr * 32 * IL + IL * l32;
                    if (cvec && col + IL <= a.N) {
                        bvec v;
                        if constexpr (IL == 1) {
                            v = a.alpha * acc[fm][gr][r];
                        } else {
#pragma unroll
                            for (int b = 0; b < IL; ++b)
                                v[b] = a.alpha * acc[fm][gr * IL + b][r];
                        }
                        if (a.beta != 0.0f) {
                            const bvec old = *reinterpret_cast<const bvec *>(crow + col);
                            if constexpr (IL == 1) {
                                v = fmaf(a.alpha, acc[fm][gr][r], a.beta * old);
                            } else {
#pragma unroll
                                for (int b = 0; b < IL; ++b)
                                    v[b] = fmaf(a.alpha, acc[fm][gr * IL + b][r], a.beta * old[b]);
                            }
                        }
                        *reinterpret_cast<bvec *>(crow + col) = v;
                    } else {
#pragma unroll
                        for (int b = 0; b < IL; ++b) {
                            if (col + b < a.N) {
                                const float v = acc[fm][gr * IL + b][r];
                                float *cp = crow + col + b;
                                *cp = (a.beta == 0.0f) ? a.alpha * v : fmaf(a.alpha, v, a.beta * *cp);
                            }
                        }
                    }
                }
            }
        }
    }
}

TileShape tile_shape(int kid)
{
    switch (kid) {
    case KID_MFMA_L: return {128, 256};
    case KID_MFMA_M: return {128, 128};
    case KID_MFMA_S: return {64, 64};
    case KID_REGBLOCK: return {128, 128};
    case KID_TILED_PAD:
    case KID_TILED_NOPAD: return {16, 16};
    case KID_NAIVE: return {4, 64};
    default: return {0, 0};
    }
}

template <int BM, int BN, int BK, int WGM, int WGN>
static void launch_cfg(const GemmArgs &a, bool transB, bool vec, hipStream_t stream)
{
    const int64_t blocks = ceil_div(a.M, BM) * ceil_div(a.N, BN);
    const dim3 grid((unsigned)blocks), block(256);
    if (transB) {
        if (vec)
            sgemm_mfma_kernel<BM, BN, BK, WGM, WGN, true, true><<<grid, block, 0, stream>>>(a);
        else
            sgemm_mfma_kernel<BM, BN, BK, WGM, WGN, true, false><<<grid, block, 0, stream>>>(a);
    } else {
        if (vec)
            sgemm_mfma_kernel<BM, BN, BK, WGM, WGN, false, true><<<grid, block, 0, stream>>>(a);
        else
            sgemm_mfma_kernel<BM, BN, BK, WGM, WGN, false, false><<<grid, block, 0, stream>>>(a);
    }
}

hipError_t launch_mfma(const GemmArgs &a, int kid, bool transB, bool vec, hipStream_t stream)
{
    switch (kid) {
    case KID_MFMA_L: launch_cfg<128, 256, 16, 2, 2>(a, transB, vec, stream); break;
    case KID_MFMA_M: launch_cfg<128, 128, 16, 2, 2>(a, transB, vec, stream); break;
    case KID_MFMA_S: launch_cfg<64, 64, 32, 2, 2>(a, transB, vec, stream); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace sgemm
