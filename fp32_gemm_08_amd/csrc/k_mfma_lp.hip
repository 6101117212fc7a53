// Mixed-precision GEMM: D = alpha * r(A) * r(op(B)) + beta * C with FP32
// operands in memory, r the conversion to fp16 or bf16 (round to nearest, ties
// to even) applied while tiles are staged into LDS, and the products summed by
// the matrix cores in FP32.
//
// "GPU矩阵乘法优化：共享内存Tiling技术实战", section 7.1 (混合精度计算): the tile is
// converted to half precision on its way into shared memory and the matrix
// cores multiply the half-precision values.
//
// MI355X version.  v_mfma_f32_32x32x16_{f16,bf16}: a 32x32 FP32 block += a
// 32x16 block of A times a 16x32 block of op(B); lane l supplies 8 consecutive
// k values (one 16-byte LDS read) of A row l%32 and of op(B) column l%32, the
// half l/32 choosing which 8 of the 16.  Accumulator register r of lane l holds
// row 8*(r/4) + 4*(l/32) + r%4, column l%32 of the block.
//
// Workgroup tile 256 x 256, 8 wavefronts as 4 (m) x 2 (n), each 64 x 128 =
// 2 x 4 blocks of 32 x 32 (128 FP32 accumulators per lane), or for products
// with fewer than 128 such tiles 64 x 64 with 2 wavefronts of 32 x 64.  k-tiles
// of 32.  LDS holds both operands k-contiguous as 16-bit values, A as
// As[BM][40] and op(B) as Bs[BN][40] (n-major): 32 values per row plus 8 of padding, an
// 80-byte pitch, so the 16-byte operand reads of 16 consecutive rows fall on
// 16 distinct 4-bank groups (bank unit 20*r mod 64).  Two stages, one barrier
// per k-tile; the next k-tile's FP32 loads are in flight while the current one
// is multiplied, then converted and written to the other stage.
//
// Staging per k-tile:
//   A (and op(B) = B^T, stored N x K): BM rows x 4 chunks of 8 k values; each
//     work-item loads its chunks as 2 x 128 bits each, converts, and writes
//     16 bytes per chunk.
//   op(B) = B (stored K x N): 8 quads of k x BN/4 quads of n; each work-item
//     loads 4 (k) x 4 (n) blocks (4 x 128 bits along n), converts, and writes
//     them transposed: 4 n-rows x 4 k values (8 bytes each).
// Edge tiles and the k tail load with masks and zero fill, element by element
// only for the chunks that leave the matrix; misaligned operands (base not
// 16-byte aligned or leading dimension not a multiple of 4) load element by
// element.
#include "sgemm_internal.h"
#include "lp_types.h"

namespace sgemm {
namespace {

constexpr int LBK = 32;
constexpr int LP_PITCH = LBK + 8;                      // 16-bit values per LDS row

// Workgroup tile BM x BN, WGM x WGN wavefronts each owning (BM/WGM) x (BN/WGN).
template <int BM_, int BN_, int WGM_, int WGN_>
struct LpGeo {
    static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_;
    static constexpr int NT = 64 * WGM * WGN;
    static constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
    static constexpr int STAGE = (BM + BN) * LP_PITCH;  // 16-bit values per stage
    static constexpr int UA = 4 * BM / NT;               // A units (8 k values) per work-item
    static constexpr int UBT = 4 * BN / NT;              // B^T units per work-item
    static constexpr int UB = 2 * BN / NT;               // B units (4 k x 4 n) per work-item
    static_assert(WM % 32 == 0 && WN % 32 == 0, "whole 32 x 32 blocks");
    static_assert(UA * NT == 4 * BM && UBT * NT == 4 * BN && UB * NT == 2 * BN && UB >= 1, "staging split");
    static_assert(2 * STAGE * 2 <= 160 * 1024, "two stages fit the LDS");
};

__device__ __forceinline__ int lp_wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Workgroup -> output tile: the dispatcher deals workgroups round-robin to the
// 8 XCDs, so consecutive ids are renumbered into one contiguous run per XCD
// (each XCD's L2 then sees neighbouring tiles), walked 8 tile-rows at a time.
__device__ __forceinline__ void lp_map_tile(int bid, int nbm, int nbn, int &tm, int &tn)
{
    const int nb = nbm * nbn;
    int id = bid;
    if (nb % 8 == 0)
        id = (bid % 8) * (nb / 8) + bid / 8;
    const int group = 8 * nbn;
    const int g = id / group, first_m = g * 8;
    const int gm = nbm - first_m < 8 ? nbm - first_m : 8;
    tm = first_m + (id % group) % gm;
    tn = (id % group) / gm;
}

template <class Gm, bool BF16, bool TRANS_B, bool VEC>
struct LpStage {
    typedef typename Lp<BF16>::T T;
    typedef typename Lp<BF16>::V8 V8;
    typedef typename Lp<BF16>::V4 V4;
    // A units (and B^T units): 8 k values each
    float a[Gm::UA][8];
    // B units: TRANS_B ? units of 8 k values : 4 (k) x 4 (n) blocks
    float b[TRANS_B ? Gm::UBT : Gm::UB][TRANS_B ? 8 : 16];

    // Load 8 consecutive floats of a k-contiguous row (zero past the matrix).
    template <bool MASKED>
    static __device__ __forceinline__ void load8(float (&dst)[8], const float *p, bool row_ok, int k, int K)
    {
        if (VEC && (!MASKED || (row_ok && k + 8 <= K))) {  // masks only where the chunk leaves the matrix
            const lp_f32x4 x0 = *reinterpret_cast<const lp_f32x4 *>(p);
            const lp_f32x4 x1 = *reinterpret_cast<const lp_f32x4 *>(p + 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                dst[q] = x0[q];
                dst[4 + q] = x1[q];
            }
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q)
                dst[q] = (!MASKED || (row_ok && k + q < K)) ? p[q] : 0.0f;
        }
    }

    template <bool MASKED>
    __device__ __forceinline__ void load(const GemmArgs &g, int m0, int n0, int k0)
    {
        const int t = threadIdx.x;
#pragma unroll
        for (int i = 0; i < Gm::UA; ++i) {
            const int u = t + Gm::NT * i, r = u >> 2, c = u & 3;
            const int k = k0 + 8 * c;
            load8<MASKED>(a[i], g.A + (int64_t)(m0 + r) * g.lda + k, m0 + r < g.M, k, g.K);
        }
        if constexpr (TRANS_B) {
#pragma unroll
            for (int i = 0; i < Gm::UBT; ++i) {
                const int u = t + Gm::NT * i, r = u >> 2, c = u & 3;
                const int k = k0 + 8 * c;
                load8<MASKED>(b[i], g.B + (int64_t)(n0 + r) * g.ldb + k, n0 + r < g.N, k, g.K);
            }
        } else {
#pragma unroll
            for (int i = 0; i < Gm::UB; ++i) {
                const int u = t + Gm::NT * i;
                const int kq = (u >> 3) & 7, nq = (u & 7) | ((u >> 6) << 3);
                const int n = n0 + 4 * nq;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int k = k0 + 4 * kq + j;
                    const float *p = g.B + (int64_t)k * g.ldb + n;
                    if (VEC && (!MASKED || (k < g.K && n + 4 <= g.N))) {
                        const lp_f32x4 x = *reinterpret_cast<const lp_f32x4 *>(p);
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            b[i][4 * j + q] = x[q];
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            b[i][4 * j + q] = (!MASKED || (k < g.K && n + q < g.N)) ? p[q] : 0.0f;
                    }
                }
            }
        }
    }

    static __device__ __forceinline__ V8 cvt8(const float (&x)[8])
    {
        V8 v;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            v[q] = (T)x[q];
        return v;
    }

    __device__ __forceinline__ void store(T *as, T *bs) const
    {
        const int t = threadIdx.x;
#pragma unroll
        for (int i = 0; i < Gm::UA; ++i) {
            const int u = t + Gm::NT * i, r = u >> 2, c = u & 3;
            *reinterpret_cast<V8 *>(as + r * LP_PITCH + 8 * c) = cvt8(a[i]);
        }
        if constexpr (TRANS_B) {
#pragma unroll
            for (int i = 0; i < Gm::UBT; ++i) {
                const int u = t + Gm::NT * i, r = u >> 2, c = u & 3;
                *reinterpret_cast<V8 *>(bs + r * LP_PITCH + 8 * c) = cvt8(b[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < Gm::UB; ++i) {
                const int u = t + Gm::NT * i;
                const int kq = (u >> 3) & 7, nq = (u & 7) | ((u >> 6) << 3);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    V4 v;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        v[q] = (T)b[i][4 * q + j];
                    *reinterpret_cast<V4 *>(bs + (4 * nq + j) * LP_PITCH + 4 * kq) = v;
                }
            }
        }
    }
};

template <class Gm, bool BF16, bool TRANS_B, bool VEC>
__global__ __launch_bounds__(Gm::NT) void sgemm_mfma_lp_kernel(GemmArgs g)
{
    typedef typename Lp<BF16>::T T;
    typedef typename Lp<BF16>::V8 V8;
    constexpr int LBM = Gm::BM, LBN = Gm::BN, LWM = Gm::WM, LWN = Gm::WN, LFM = Gm::FM, LFN = Gm::FN;
    constexpr int LP_STAGE = Gm::STAGE;
    __shared__ __attribute__((aligned(16))) T smem[2 * LP_STAGE];

    const int nbm = (g.M + LBM - 1) / LBM, nbn = (g.N + LBN - 1) / LBN;
    int tile_m, tile_n;
    lp_map_tile(blockIdx.x, nbm, nbn, tile_m, tile_n);
    const int m0 = tile_m * LBM, n0 = tile_n * LBN;
    const bool full = m0 + LBM <= g.M && n0 + LBN <= g.N;
    const int nk = (g.K + LBK - 1) / LBK;

    const int lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
    const int w = lp_wave_id(), wm = w / Gm::WGN, wn = w % Gm::WGN;

    lp_f32x16 acc[LFM][LFN];
#pragma unroll
    for (int fm = 0; fm < LFM; ++fm)
#pragma unroll
        for (int fn = 0; fn < LFN; ++fn)
            acc[fm][fn] = lp_f32x16{};

    LpStage<Gm, BF16, TRANS_B, VEC> st;
    auto load_tile = [&](int kt) {
        const int k0 = kt * LBK;
        if (full && k0 + LBK <= g.K)
            st.template load<false>(g, m0, n0, k0);
        else
            st.template load<true>(g, m0, n0, k0);
    };
    load_tile(0);
    poison_lds(smem, LP_STAGE * (int)sizeof(T));
    st.store(smem, smem + LBM * LP_PITCH);
    __syncthreads();

    // With 8 wavefronts, those with wave bit 2 set issue the next k-tile's
    // loads after the first 16-k step's MFMAs instead of at the top, so the
    // CU's address unit does not take all 8 wavefronts' loads at once
    // (measured on MI355X, bf16: 4096^3 790 -> 832 TFLOP/s, 8192^3 694 -> 707;
    // bits 0 and 1 were faster at 4096^3 but slower at 8192^3 and 6144^3).
    const bool late = Gm::NT == 512 && (w & 4) != 0;
    for (int kt = 0; kt < nk; ++kt) {
        T *as = smem + (kt & 1) * LP_STAGE;
        T *bs = as + LBM * LP_PITCH;
        if (!late && kt + 1 < nk)
            load_tile(kt + 1);
#pragma unroll
        for (int ks = 0; ks < LBK / 16; ++ks) {
            if (ks == 1 && late && kt + 1 < nk)
                load_tile(kt + 1);
            V8 af[LFM], bf[LFN];
#pragma unroll
            for (int fm = 0; fm < LFM; ++fm)
                af[fm] = *reinterpret_cast<const V8 *>(as + (wm * LWM + fm * 32 + l32) * LP_PITCH + 16 * ks + 8 * hi);
#pragma unroll
            for (int fn = 0; fn < LFN; ++fn)
                bf[fn] = *reinterpret_cast<const V8 *>(bs + (wn * LWN + fn * 32 + l32) * LP_PITCH + 16 * ks + 8 * hi);
#pragma unroll
            for (int fm = 0; fm < LFM; ++fm)
#pragma unroll
                for (int fn = 0; fn < LFN; ++fn)
                    acc[fm][fn] = Lp<BF16>::mma(af[fm], bf[fn], acc[fm][fn]);
        }
        if (kt + 1 < nk) {
            T *nas = smem + ((kt + 1) & 1) * LP_STAGE;
            poison_lds(nas, LP_STAGE * (int)sizeof(T));
            st.store(nas, nas + LBM * LP_PITCH);
        }
        __syncthreads();
    }

    // Epilogue: D = alpha * acc + beta * C (C not read when beta == 0).  With
    // beta != 0 rows go 8 at a time and all 8 rows' old values are loaded
    // before the first store: loads and stores share the pointer C, so a load
    // after a store could not be hoisted and would wait a full round trip.
    if (g.beta == 0.0f) {
#pragma unroll
        for (int fm = 0; fm < LFM; ++fm) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * LWM + fm * 32 + 8 * (r / 4) + 4 * hi + (r % 4);
                if (!full && row >= g.M)
                    continue;
                float *crow = g.C + (int64_t)row * g.ldc;
#pragma unroll
                for (int fn = 0; fn < LFN; ++fn) {
                    const int col = n0 + wn * LWN + fn * 32 + l32;
                    if (full || col < g.N)
                        crow[col] = g.alpha * acc[fm][fn][r];
                }
            }
        }
        return;
    }
#pragma unroll
    for (int fm = 0; fm < LFM; ++fm) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float old[8][LFN];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 8 * h + i;
                const int row = m0 + wm * LWM + fm * 32 + 8 * (r / 4) + 4 * hi + (r % 4);
                if (!full && row >= g.M)
                    continue;
                const float *crow = g.C + (int64_t)row * g.ldc;
#pragma unroll
                for (int fn = 0; fn < LFN; ++fn) {
                    const int col = n0 + wn * LWN + fn * 32 + l32;
                    old[i][fn] = (full || col < g.N) ? crow[col] : 0.0f;
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 8 * h + i;
                const int row = m0 + wm * LWM + fm * 32 + 8 * (r / 4) + 4 * hi + (r % 4);
                if (!full && row >= g.M)
                    continue;
                float *crow = g.C + (int64_t)row * g.ldc;
#pragma unroll
                for (int fn = 0; fn < LFN; ++fn) {
                    const int col = n0 + wn * LWN + fn * 32 + l32;
                    if (full || col < g.N)
                        crow[col] = fmaf(g.alpha, acc[fm][fn][r], g.beta * old[i][fn]);
                }
            }
        }
    }
}

}  // namespace

// Measured on MI355X (bf16, 8192^3 ... 512^3): the 256 x 256 tile is fastest
// once it keeps at least half the CUs busy (3584^3: 618 TFLOP/s against 309);
// below that the 64 x 64 tile (2 wavefronts, up to 8 workgroups per CU) is,
// by 2x at 2048^3 and 3x at 1024^3.  128 x 256 and 128 x 128 tiles never led
// by more than 15%.
typedef LpGeo<256, 256, 4, 2> LpL;   // 8 wavefronts of 64 x 128
typedef LpGeo<64, 64, 2, 1> LpS;     // 2 wavefronts of 32 x 64

TileShape lp_tile_shape(bool large) { return large ? TileShape{LpL::BM, LpL::BN} : TileShape{LpS::BM, LpS::BN}; }

template <class Gm>
static void launch_lp_cfg(const GemmArgs &a, bool bf16, bool transB, bool vec, hipStream_t stream)
{
    const int64_t blocks = ceil_div(a.M, Gm::BM) * ceil_div(a.N, Gm::BN);
    const dim3 grid((unsigned)blocks), block(Gm::NT);
#define LP_LAUNCH(BF, TB, V) sgemm_mfma_lp_kernel<Gm, BF, TB, V><<<grid, block, 0, stream>>>(a)
    if (bf16) {
        if (transB) { if (vec) LP_LAUNCH(true, true, true); else LP_LAUNCH(true, true, false); }
        else { if (vec) LP_LAUNCH(true, false, true); else LP_LAUNCH(true, false, false); }
    } else {
        if (transB) { if (vec) LP_LAUNCH(false, true, true); else LP_LAUNCH(false, true, false); }
        else { if (vec) LP_LAUNCH(false, false, true); else LP_LAUNCH(false, false, false); }
    }
#undef LP_LAUNCH
}

hipError_t launch_mfma_lp(const GemmArgs &a, bool large, bool bf16, bool transB, bool vec, hipStream_t stream)
{
    if (large)
        launch_lp_cfg<LpL>(a, bf16, transB, vec, stream);
    else
        launch_lp_cfg<LpS>(a, bf16, transB, vec, stream);
    return hipGetLastError();
}

}  // namespace sgemm
