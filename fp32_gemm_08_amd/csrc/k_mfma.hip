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
//
// Software pipeline (one barrier per k-tile).  The global loads of tile t+1 are
// in registers when iteration t starts; iteration t
//   1. stores them to the other LDS buffer (free: every wavefront finished
//      reading it before the previous barrier) and issues the global loads of
//      tile t+2, so global latency has a whole tile of MFMA work to hide under;
//   2. runs the MFMAs of k-groups 0..G-2, reading each next group's fragments
//      from LDS while the current group's MFMAs execute;
//   3. waits for its LDS traffic, passes the barrier, reads group 0 of tile t+1,
//      and only then issues the MFMAs of the last group, which cover the barrier
//      and the next tile's first LDS reads.
// Interior workgroups (the tile inside M x N, a full k-tile) load without masks;
// edge workgroups and the K tail load element-wise with zero fill.
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

// Four consecutive floats from p.  MASKED: elements at or beyond `limit` (or all
// of them when !ok) read as zero.  VEC: one 128-bit load when all four are in.
template <bool VEC, bool MASKED>
__device__ __forceinline__ f32x4 load4(const float *p, bool ok, int first, int limit)
{
    f32x4 v;
    if (!MASKED) {
        if (VEC) {
            v = *reinterpret_cast<const f32x4 *>(p);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = p[e];
        }
    } else if (VEC && ok && first + 4 <= limit) {
        v = *reinterpret_cast<const f32x4 *>(p);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = (ok && first + e < limit) ? p[e] : 0.0f;
    }
    return v;
}

// Compile-time geometry of one MFMA kernel configuration.
template <int BM_, int BN_, int BK_, int WGM_, int WGN_, int OCC_, bool TRANS_B>
struct Geo {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_, OCC = OCC_;
    static constexpr int NT = 64 * WGM * WGN;          // work-items per workgroup
    static constexpr int WM = BM / WGM, WN = BN / WGN; // wavefront tile
    static constexpr int FM = WM / 32, FN = WN / 32;   // 32x32 blocks per wavefront
    static constexpr int IL = TRANS_B ? 1 : (FN >= 4 ? 4 : FN);
    static constexpr int NG = FN / IL;                 // interleaved column groups
    static constexpr int G = BK / 8;                   // k-groups per tile
    static constexpr int SA = BK + 4;                  // A row stride in LDS (floats)
    static constexpr int SB = TRANS_B ? BK + 4 : BN;   // B^T row stride / B row stride
    static constexpr int A_SZ = BM * SA;
    static constexpr int B_SZ = TRANS_B ? BN * SB : BK * SB;
    static constexpr int STAGE = A_SZ + B_SZ;
    static constexpr int KC = BK / 4;                  // 4-float chunks per k-row
    static constexpr int CA = BM * KC / NT;            // A chunks per work-item
    static constexpr int CB = (TRANS_B ? BN * KC : BK * (BN / 4)) / NT;
    static_assert(WM % 32 == 0 && WN % 32 == 0 && BK % 8 == 0, "tile shape");
    static_assert(BM * KC % NT == 0 && (TRANS_B ? BN * KC : BK * (BN / 4)) % NT == 0, "staging split");
    static_assert(2 * STAGE * 4 <= 160 * 1024, "LDS budget");
    static_assert(G >= 2 && G % 2 == 0, "the fragment ping-pong needs an even number of k-groups");
};

// Fragments of one k-group: FM A operands (4 k-steps each) and the B operands.
template <class Gm, bool TRANS_B>
struct Frags {
    typedef typename vec_of<Gm::IL>::type bvec;
    f32x4 a[Gm::FM];
    bvec b[TRANS_B ? 1 : 4][TRANS_B ? 1 : Gm::NG];   // op(B) = B: [step][group]
    f32x4 bt[TRANS_B ? Gm::FN : 1];                  // op(B) = B^T: [block]
};

template <class Gm, bool TRANS_B>
__device__ __forceinline__ void read_frags(Frags<Gm, TRANS_B> &f, const float *As, const float *Bs, int g,
                                           int wm, int wn, int l32, int hi)
{
    const int kq = 8 * g + 4 * hi;  // this half-wavefront's first k of the group
#pragma unroll
    for (int fm = 0; fm < Gm::FM; ++fm)
        f.a[fm] = *reinterpret_cast<const f32x4 *>(&As[(wm * Gm::WM + 32 * fm + l32) * Gm::SA + kq]);
    if constexpr (TRANS_B) {
#pragma unroll
        for (int fn = 0; fn < Gm::FN; ++fn)
            f.bt[fn] = *reinterpret_cast<const f32x4 *>(&Bs[(wn * Gm::WN + 32 * fn + l32) * Gm::SB + kq]);
    } else {
        typedef typename vec_of<Gm::IL>::type bvec;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int gr = 0; gr < Gm::NG; ++gr)
                f.b[s][gr] = *reinterpret_cast<const bvec *>(
                    &Bs[(kq + s) * Gm::SB + wn * Gm::WN + gr * 32 * Gm::IL + Gm::IL * l32]);
    }
}

template <class Gm, bool TRANS_B>
__device__ __forceinline__ void mfma_group(f32x16 (&acc)[Gm::FM][Gm::FN], const Frags<Gm, TRANS_B> &f)
{
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int fm = 0; fm < Gm::FM; ++fm) {
            if constexpr (TRANS_B) {
#pragma unroll
                for (int fn = 0; fn < Gm::FN; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[fm][s], f.bt[fn][s], acc[fm][fn], 0, 0, 0);
            } else {
#pragma unroll
                for (int gr = 0; gr < Gm::NG; ++gr)
#pragma unroll
                    for (int b = 0; b < Gm::IL; ++b)
                        acc[fm][gr * Gm::IL + b] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                            f.a[fm][s], vget<Gm::IL>(f.b[s][gr], b), acc[fm][gr * Gm::IL + b], 0, 0, 0);
            }
        }
}

// The k-loop and epilogue for one workgroup tile.  FULL: the tile lies inside
// M x N, so only the K tail needs masks.
template <class Gm, bool TRANS_B, bool VEC, bool FULL>
__device__ __forceinline__ void gemm_tile(const GemmArgs &a, float *smem, int m0, int n0)
{
    constexpr int NT = Gm::NT, KC = Gm::KC, CA = Gm::CA, CB = Gm::CB, BK = Gm::BK, G = Gm::G;
    constexpr int BN4 = Gm::BN / 4;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int wm = wave / Gm::WGN, wn = wave % Gm::WGN;

    // Per work-item staging coordinates and global base pointers (k = 0).
    const float *pa[CA];
    const float *pb[CB];
    int ra_row[CA], ra_col[CA], rb_row[CB], rb_col[CB];
#pragma unroll
    for (int i = 0; i < CA; ++i) {
        const int q = tid + i * NT;
        ra_row[i] = q / KC;
        ra_col[i] = 4 * (q % KC);
        pa[i] = a.A + (int64_t)(m0 + ra_row[i]) * a.lda + ra_col[i];
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
        const int q = tid + i * NT;
        if constexpr (TRANS_B) {
            rb_row[i] = q / KC;           // n within the tile
            rb_col[i] = 4 * (q % KC);     // k within the tile
            pb[i] = a.B + (int64_t)(n0 + rb_row[i]) * a.ldb + rb_col[i];
        } else {
            rb_row[i] = q / BN4;          // k within the tile
            rb_col[i] = 4 * (q % BN4);    // n within the tile
            pb[i] = a.B + (int64_t)rb_row[i] * a.ldb + n0 + rb_col[i];
        }
    }
    const int64_t b_kstep = TRANS_B ? (int64_t)BK : (int64_t)BK * a.ldb;

    f32x4 ra[CA], rb[CB];
    auto gload = [&](int kt) {
        const int k0 = kt * BK;
        if (FULL && k0 + BK <= a.K) {
#pragma unroll
            for (int i = 0; i < CA; ++i)
                ra[i] = load4<VEC, false>(pa[i] + (int64_t)kt * BK, true, 0, 0);
#pragma unroll
            for (int i = 0; i < CB; ++i)
                rb[i] = load4<VEC, false>(pb[i] + (int64_t)kt * b_kstep, true, 0, 0);
        } else {
#pragma unroll
            for (int i = 0; i < CA; ++i)
                ra[i] = load4<VEC, true>(pa[i] + (int64_t)kt * BK, m0 + ra_row[i] < a.M, k0 + ra_col[i], a.K);
#pragma unroll
            for (int i = 0; i < CB; ++i) {
                if constexpr (TRANS_B)
                    rb[i] = load4<VEC, true>(pb[i] + (int64_t)kt * b_kstep, n0 + rb_row[i] < a.N,
                                             k0 + rb_col[i], a.K);
                else
                    rb[i] = load4<VEC, true>(pb[i] + (int64_t)kt * b_kstep, k0 + rb_row[i] < a.K,
                                             n0 + rb_col[i], a.N);
            }
        }
    };
    auto sstore = [&](int buf) {
        float *As = smem + buf * Gm::STAGE;
        float *Bs = As + Gm::A_SZ;
#pragma unroll
        for (int i = 0; i < CA; ++i)
            *reinterpret_cast<f32x4 *>(&As[ra_row[i] * Gm::SA + ra_col[i]]) = ra[i];
#pragma unroll
        for (int i = 0; i < CB; ++i)
            *reinterpret_cast<f32x4 *>(&Bs[rb_row[i] * Gm::SB + rb_col[i]]) = rb[i];
    };

    f32x16 acc[Gm::FM][Gm::FN];
#pragma unroll
    for (int i = 0; i < Gm::FM; ++i)
#pragma unroll
        for (int j = 0; j < Gm::FN; ++j)
            acc[i][j] = f32x16{0};

    const int nk = (a.K + BK - 1) / BK;
    Frags<Gm, TRANS_B> f[2];

    // Prologue: tile 0 into LDS buffer 0, tile 1 in flight, group 0 fragments.
    gload(0);
    sstore(0);
    if (nk > 1)
        gload(1);
    __syncthreads();
    read_frags<Gm, TRANS_B>(f[0], smem, smem + Gm::A_SZ, 0, wm, wn, l32, hi);

    for (int t = 0; t < nk; ++t) {
        const float *As = smem + (t & 1) * Gm::STAGE;
        const float *Bs = As + Gm::A_SZ;
        // 1. tile t+1 (in registers) to the free buffer; tile t+2 in flight
        if (t + 1 < nk) {
            sstore((t + 1) & 1);
            if (t + 2 < nk)
                gload(t + 2);
        }
        // 2. groups 0..G-2, next group's fragments read under the MFMAs
#pragma unroll
        for (int g = 0; g < G - 1; ++g) {
            read_frags<Gm, TRANS_B>(f[(g + 1) & 1], As, Bs, g + 1, wm, wn, l32, hi);
            mfma_group<Gm, TRANS_B>(acc, f[g & 1]);
        }
        // 3. barrier and the next tile's first fragments under the last group
        if (t + 1 < nk) {
            __syncthreads();
            const float *An = smem + ((t + 1) & 1) * Gm::STAGE;
            read_frags<Gm, TRANS_B>(f[G & 1], An, An + Gm::A_SZ, 0, wm, wn, l32, hi);
        }
        mfma_group<Gm, TRANS_B>(acc, f[(G - 1) & 1]);
    }

    // Epilogue.  Accumulator register r of a 32x32 block holds row
    // 8*(r/4) + 4*hi + (r%4) and column l32 of that block.
    typedef typename vec_of<Gm::IL>::type bvec;
    constexpr int IL = Gm::IL;
    const uintptr_t cbase = reinterpret_cast<uintptr_t>(a.C);
    const bool cvec = IL > 1 && (cbase % (4 * IL)) == 0 && (a.ldc % IL) == 0;
#pragma unroll
    for (int fm = 0; fm < Gm::FM; ++fm) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = m0 + wm * Gm::WM + 32 * fm + 8 * (r / 4) + 4 * hi + (r % 4);
            if (!FULL && row >= a.M)
                continue;
            float *crow = a.C + (int64_t)row * a.ldc;
            if constexpr (TRANS_B) {
#pragma unroll
                for (int fn = 0; fn < Gm::FN; ++fn) {
                    const int col = n0 + wn * Gm::WN + 32 * fn + l32;
                    if (FULL || col < a.N) {
                        const float v = acc[fm][fn][r];
                        crow[col] = (a.beta == 0.0f) ? a.alpha * v : fmaf(a.alpha, v, a.beta * crow[col]);
                    }
                }
            } else {
#pragma unroll
                for (int gr = 0; gr < Gm::NG; ++gr) {
                    const int col = n0 + wn * Gm::WN + gr * 32 * IL + IL * l32;
                    if (cvec && (FULL || col + IL <= a.N)) {
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

template <class Gm, bool TRANS_B, bool VEC>
__global__ __launch_bounds__(Gm::NT) __attribute__((amdgpu_waves_per_eu(Gm::OCC)))
void sgemm_mfma_kernel(GemmArgs a)
{
    __shared__ __attribute__((aligned(16))) float smem[2 * Gm::STAGE];
    const int nbm = (a.M + Gm::BM - 1) / Gm::BM, nbn = (a.N + Gm::BN - 1) / Gm::BN;
    int tile_m, tile_n;
    map_tile(blockIdx.x, nbm, nbn, tile_m, tile_n);
    const int m0 = tile_m * Gm::BM, n0 = tile_n * Gm::BN;
    if (m0 + Gm::BM <= a.M && n0 + Gm::BN <= a.N)
        gemm_tile<Gm, TRANS_B, VEC, true>(a, smem, m0, n0);
    else
        gemm_tile<Gm, TRANS_B, VEC, false>(a, smem, m0, n0);
}

TileShape tile_shape(int kid)
{
    switch (kid) {
    case KID_MFMA_L: return {256, 256};
    case KID_MFMA_M: return {128, 128};
    case KID_MFMA_S: return {64, 64};
    case KID_REGBLOCK: return {128, 128};
    case KID_TILED_PAD:
    case KID_TILED_NOPAD: return {16, 16};
    case KID_NAIVE: return {4, 64};
    default: return {0, 0};
    }
}

template <int BM, int BN, int BK, int WGM, int WGN, int OCC>
static void launch_cfg(const GemmArgs &a, bool transB, bool vec, hipStream_t stream)
{
    const int64_t blocks = ceil_div(a.M, BM) * ceil_div(a.N, BN);
    const dim3 grid((unsigned)blocks), block(64 * WGM * WGN);
    typedef Geo<BM, BN, BK, WGM, WGN, OCC, true> GT;
    typedef Geo<BM, BN, BK, WGM, WGN, OCC, false> GN;
    if (transB) {
        if (vec)
            sgemm_mfma_kernel<GT, true, true><<<grid, block, 0, stream>>>(a);
        else
            sgemm_mfma_kernel<GT, true, false><<<grid, block, 0, stream>>>(a);
    } else {
        if (vec)
            sgemm_mfma_kernel<GN, false, true><<<grid, block, 0, stream>>>(a);
        else
            sgemm_mfma_kernel<GN, false, false><<<grid, block, 0, stream>>>(a);
    }
}

hipError_t launch_mfma(const GemmArgs &a, int kid, bool transB, bool vec, hipStream_t stream)
{
    switch (kid) {
#ifndef SGEMM_MFMA_EXPERIMENT
    case KID_MFMA_L: launch_cfg<256, 256, 16, 4, 2, 2>(a, transB, vec, stream); break;
    case KID_MFMA_M: launch_cfg<128, 128, 32, 2, 2, 2>(a, transB, vec, stream); break;
    case KID_MFMA_S: launch_cfg<64, 64, 32, 2, 2, 4>(a, transB, vec, stream); break;
#else
    SGEMM_MFMA_EXPERIMENT
#endif
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace sgemm
