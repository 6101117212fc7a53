// Mixed-precision GEMM in two passes, for callers that lend a workspace:
//
//   1. rounding pass: A -> A16 and op(B) -> B16, 16-bit (fp16 or bf16, round
//      to nearest, ties to even), zero-padded to whole tiles in m / n and to a
//      multiple of 32 in k, and stored k-tile major: slab s holds k values
//      [32s, 32s+32) of every row, 64 bytes per row, rows one after another
//      (op(B) = B is transposed on the way through an LDS tile);
//   2. GEMM on the 16-bit operands: D = alpha * A16 * B16^T + beta * C, FP32
//      sums on the matrix cores.
//
// The operation and its rounding are those of the one-pass kernel (each
// operand rounded once, products summed in FP32; "GPU矩阵乘法优化：共享内存Tiling
// 技术实战", section 7.1: convert to half precision, then multiply on the matrix
// cores).  Rounding once in its own pass halves the bytes the GEMM streams
// through L2 and LDS per k-step and lets it stage tiles with direct
// global->LDS loads (no registers, no conversion in the k-loop), which is what
// bounded the one-pass kernel.
//
// GEMM tile: BM x BN output, WGM x WGN wavefronts of (BM/WGM) x (BN/WGN), each
// a grid of 32 x 32 blocks (lp_types.h has the lane layout).  One stage holds
// 32 k of BM rows of A16 and BN rows of B16 -- in the slab layout, one
// contiguous 64 * BM (and 64 * BN) bytes of memory -- stored in LDS as 1 KB
// blocks of 16 rows whose four 16-byte chunks are XOR-permuted by
// ((r >> 1) ^ (r >> 2)) & 3, so that the 16-byte fragment reads of 8 (or 16)
// consecutive rows at one chunk touch distinct banks.  A wavefront fills a 1 KB
// block with one global_load_lds_dwordx4 (lane i -> row i/4, physical chunk
// i%4) from 1 KB of contiguous memory.  (Rows k-contiguous over the whole K,
// where each load used 64 bytes of sixteen 128-byte lines, measured 4-5%
// slower: 1059 against 1108 TFLOP/s at 4096^3.)  S stages rotate: stage kt+S-1 is requested while stage kt is
// multiplied, and each k-step waits only for the next stage (s_waitcnt on
// the count of loads still allowed in flight, then a barrier); the fragment
// reads of one 16-k step run under the MFMAs of the previous one.
#include "sgemm_internal.h"
#include "lp_types.h"

#include <algorithm>

namespace sgemm {
namespace {

typedef __attribute__((address_space(3))) void q_lds;

constexpr int QK = 32;    // k values per stage
constexpr int QROW = 64;  // bytes per row per stage

__device__ __forceinline__ int q_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

template <int BM_, int BN_, int WGM_, int WGN_, int S_>
struct QGeo {
    static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, S = S_;
    static constexpr int NW = WGM * WGN, NT = 64 * NW;
    static constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
    static constexpr int NA = BM / 16 / NW, NB = BN / 16 / NW;  // 1 KB blocks per wavefront per stage
    static constexpr int LOADS = NA + NB;                         // direct loads per wavefront per stage
    static constexpr int STAGE = (BM + BN) * QROW;                // bytes
    static_assert(WM % 32 == 0 && WN % 32 == 0, "whole 32 x 32 blocks");
    static_assert(NA * 16 * NW == BM && NB * 16 * NW == BN, "every wavefront loads whole blocks");
    static_assert(S >= 3 && S * STAGE <= 160 * 1024, "three buffers in use per step, all in the LDS");
    static_assert((S - 2) * LOADS <= 63, "vmcnt range");
};

// Workgroup -> output tile, as the other MFMA kernels: one contiguous run of
// tiles per XCD, walked 8 tile-rows at a time.
__device__ __forceinline__ void q_map_tile(int bid, int nbm, int nbn, int &tm, int &tn)
{
    const int nb = nbm * nbn;
    const int id = (nb % 8 == 0) ? (bid % 8) * (nb / 8) + bid / 8 : bid;
    const int group = 8 * nbn;
    const int g = id / group, first_m = g * 8;
    const int gm = min(nbm - first_m, 8);
    tm = first_m + (id % group) % gm;
    tn = (id % group) / gm;
}

// One direct global->LDS load: 16 bytes per lane from `src` into the 1 KB
// block at `lds` (lane i lands at byte 16*i).
__device__ __forceinline__ void q_load(const void *src, unsigned char *lds)
{
    __builtin_amdgcn_global_load_lds(src, (q_lds *)lds, 16, 0, 0);
}

// Wait until at most N of this wavefront's direct loads are outstanding and
// all its LDS reads are done, then meet the other wavefronts.  The wait is
// the s_waitcnt builtin (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt
// 6:4 left at 7, lgkmcnt 11:8 = 0), so the compiler knows which reads have
// completed and does not wait for them again; the barrier is an asm with a
// memory clobber, so no memory access moves across it.
template <int N>
__device__ __forceinline__ void q_wait_barrier()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | ((N >> 4) << 14));
    asm volatile("s_barrier" ::: "memory");
}

template <class Q, bool BF16>
__global__ __launch_bounds__(Q::NT) void lp16_gemm_kernel(Lp16Args g)
{
    typedef typename Lp<BF16>::T T;
    typedef typename Lp<BF16>::V8 V8;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[Q::S * Q::STAGE];

    int tm, tn;
    q_map_tile(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
    const int m0 = tm * Q::BM, n0 = tn * Q::BN;
    const int lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = w / Q::WGN, wn = w % Q::WGN;

    // This lane's source in each of its blocks: row 16*b + lane/4, logical
    // chunk (lane % 4) ^ swizzle of that row.
    const T *pa[Q::NA], *pb[Q::NB];
#pragma unroll
    for (int j = 0; j < Q::NA; ++j) {
        const int r = 16 * (w * Q::NA + j) + lane / 4;
        pa[j] = static_cast<const T *>(g.A16) + (int64_t)(m0 + r) * QK + 8 * ((lane & 3) ^ q_swz(r));
    }
#pragma unroll
    for (int j = 0; j < Q::NB; ++j) {
        const int r = 16 * (w * Q::NB + j) + lane / 4;
        pb[j] = static_cast<const T *>(g.B16) + (int64_t)(n0 + r) * QK + 8 * ((lane & 3) ^ q_swz(r));
    }
    // Request the k-tile `src` into the buffer of stage `slot`.
    auto issue = [&](int src, int slot) {
        unsigned char *st = smem + (slot % Q::S) * Q::STAGE;
        poison_lds(st, Q::STAGE);
#pragma unroll
        for (int j = 0; j < Q::NA; ++j)
            q_load(pa[j] + (int64_t)src * g.slab_a, st + (w * Q::NA + j) * 1024);
#pragma unroll
        for (int j = 0; j < Q::NB; ++j)
            q_load(pb[j] + (int64_t)src * g.slab_b, st + Q::BM * QROW + (w * Q::NB + j) * 1024);
    };

    lp_f32x16 acc[Q::FM][Q::FN];
#pragma unroll
    for (int fm = 0; fm < Q::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < Q::FN; ++fn)
            acc[fm][fn] = lp_f32x16{};

    // Fragments of one 16-k step: lane l32 of half hi reads 8 k values of
    // row l32 of each 32-row block (A) and of each 32-column block (B).
    auto read_frags = [&](int kt, int ks, V8 (&fa)[Q::FM], V8 (&fb)[Q::FN]) {
        const unsigned char *as = smem + (kt % Q::S) * Q::STAGE;
        const unsigned char *bs = as + Q::BM * QROW;
        const int c = 2 * ks + hi;
#pragma unroll
        for (int fm = 0; fm < Q::FM; ++fm) {
            const int r = wm * Q::WM + fm * 32 + l32;
            fa[fm] = *reinterpret_cast<const V8 *>(as + r * QROW + 16 * (c ^ q_swz(r)));
        }
#pragma unroll
        for (int fn = 0; fn < Q::FN; ++fn) {
            const int r = wn * Q::WN + fn * 32 + l32;
            fb[fn] = *reinterpret_cast<const V8 *>(bs + r * QROW + 16 * (c ^ q_swz(r)));
        }
    };
    // MFMAs of one 16-k step; `from` skips the first blocks (0 .. FM*FN).
    auto mma_step = [&](const V8 (&fa)[Q::FM], const V8 (&fb)[Q::FN], int from, int to) {
#pragma unroll
        for (int fm = 0; fm < Q::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < Q::FN; ++fn)
                if (fm * Q::FN + fn >= from && fm * Q::FN + fn < to)
                    acc[fm][fn] = Lp<BF16>::mma(fa[fm], fb[fn], acc[fm][fn]);
    };

    // Pipeline: stages 0 .. S-2 requested up front.  Step kt (the first 16-k
    // fragments of stage kt already in registers): one MFMA, then the reads of
    // the second fragments, then the other MFMAs of the first; wait for stage
    // kt+1 and meet the other wavefronts (everyone is then done with stage
    // kt-1, whose buffer takes stage kt+S-1); read the first fragments of
    // stage kt+1 and multiply the second of stage kt.  The LDS reads are in
    // flight under MFMAs of the other fragment set.
    //
    // Every step requests one stage, past the end a repeat of the last one
    // (into the free buffer of stage kt-1, never read again), so the number of
    // loads in flight is the same at every wait, and every step runs the same
    // branch-free code: the compiler then sees that the barrier's wait covered
    // all earlier LDS reads and waits only for the newer ones.
    const int nk = g.Kp / QK;
    constexpr int NF = Q::FM * Q::FN;
    // With 16 wavefronts, those with wave bit 3 set request their share of a
    // stage after the step's last MFMAs instead of right after the barrier,
    // so the CU's address unit does not take all the wavefronts' loads at
    // once (measured on MI355X, GEMM pass alone on the 16-wavefront layout:
    // 4096^3 123.1-124.1 -> 120.8-121.4 us against bits 0 or 2 or none; with
    // 8 wavefronts of 64 x 128, bit 1 had taken the two-pass step from 867.5
    // to 878.8 TFLOP/s).  The request still comes before the next wait, so
    // the count of loads in flight there is unchanged.  The LDS-poisoning
    // build poisons a stage with a barrier inside `issue`, which every
    // wavefront must reach at the same point: it keeps one issue point.
    const bool late = !kPoisonLds && Q::NT == 1024 && (w & 8) != 0;
#pragma unroll
    for (int st = 0; st < Q::S - 1; ++st)
        issue(min(st, nk - 1), st);
    V8 fa0[Q::FM], fb0[Q::FN], fa1[Q::FM], fb1[Q::FN];
    q_wait_barrier<(Q::S - 2) * Q::LOADS>();
    read_frags(0, 0, fa0, fb0);
    for (int kt = 0; kt < nk; ++kt) {
        mma_step(fa0, fb0, 0, 1);
        __builtin_amdgcn_sched_barrier(0);
        read_frags(kt, 1, fa1, fb1);
        __builtin_amdgcn_sched_barrier(0);
        mma_step(fa0, fb0, 1, NF);
        q_wait_barrier<(Q::S - 3) * Q::LOADS>();  // stage kt+1 has landed
        if (!late)
            issue(min(kt + Q::S - 1, nk - 1), kt + Q::S - 1);
        read_frags(kt + 1, 0, fa0, fb0);
        __builtin_amdgcn_sched_barrier(0);
        mma_step(fa1, fb1, 0, NF);
        __builtin_amdgcn_sched_barrier(0);
        if (late)
            issue(min(kt + Q::S - 1, nk - 1), kt + Q::S - 1);
    }

    // Epilogue: D = alpha * acc + beta * C, masked to M x N (C not read when
    // beta == 0; with beta != 0 the old values of 8 rows are loaded before any
    // of them is stored).
    const bool full = m0 + Q::BM <= g.M && n0 + Q::BN <= g.N;
#pragma unroll
    for (int fm = 0; fm < Q::FM; ++fm) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float old[8][Q::FN];
            if (g.beta != 0.0f) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int r = 8 * h + i;
                    const int row = m0 + wm * Q::WM + fm * 32 + 8 * (r / 4) + 4 * hi + (r % 4);
                    if (!full && row >= g.M)
                        continue;
                    const float *crow = g.C + (int64_t)row * g.ldc;
#pragma unroll
                    for (int fn = 0; fn < Q::FN; ++fn) {
                        const int col = n0 + wn * Q::WN + fn * 32 + l32;
                        old[i][fn] = (full || col < g.N) ? crow[col] : 0.0f;
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 8 * h + i;
                const int row = m0 + wm * Q::WM + fm * 32 + 8 * (r / 4) + 4 * hi + (r % 4);
                if (!full && row >= g.M)
                    continue;
                float *crow = g.C + (int64_t)row * g.ldc;
#pragma unroll
                for (int fn = 0; fn < Q::FN; ++fn) {
                    const int col = n0 + wn * Q::WN + fn * 32 + l32;
                    if (full || col < g.N) {
                        const float v = acc[fm][fn][8 * h + i];
                        crow[col] = g.beta != 0.0f ? fmaf(g.alpha, v, g.beta * old[i][fn]) : g.alpha * v;
                    }
                }
            }
        }
    }
}

// Four FP32 operand values, 16-byte aligned; NT: a streaming (non-temporal)
// load, which does not keep the line in the caches for a later reuse.
template <bool NT>
__device__ __forceinline__ lp_f32x4 lp16_load4(const float *p)
{
    if constexpr (NT)
        return __builtin_nontemporal_load(reinterpret_cast<const lp_f32x4 *>(p));
    else
        return *reinterpret_cast<const lp_f32x4 *>(p);
}

// Rounding pass, k-contiguous source (A, or op(B) = B^T stored N x K): item i
// rounds the 8 values at k = 32*slab + 8*c of row r, i = (slab*Rp + r)*4 + c,
// so consecutive items write consecutive 16-byte chunks of the slab layout;
// zero past R rows and K columns.
template <bool BF16, bool VEC, bool NTL>
__global__ __launch_bounds__(256) void lp16_round_rows(const float *src, int64_t ld, int R, int K, void *dst_,
                                                       int Rp, int Kp)
{
    typedef typename Lp<BF16>::T T;
    typedef typename Lp<BF16>::V8 V8;
    T *dst = static_cast<T *>(dst_);
    const int64_t total = (int64_t)Rp * (Kp / 8);
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int c = (int)(i & 3);
        const int64_t rs = i >> 2;
        const int r = (int)(rs % Rp), slab = (int)(rs / Rp);
        const int k = QK * slab + 8 * c;
        float x[8];
        const float *p = src + (int64_t)r * ld + k;
        if (VEC && r < R && k + 8 <= K) {
            const lp_f32x4 x0 = lp16_load4<NTL>(p);
            const lp_f32x4 x1 = lp16_load4<NTL>(p + 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                x[q] = x0[q];
                x[4 + q] = x1[q];
            }
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q)
                x[q] = (r < R && k + q < K) ? p[q] : 0.0f;
        }
        V8 v;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            v[q] = (T)x[q];
        *reinterpret_cast<V8 *>(dst + i * 8) = v;
    }
}

// Rounding pass for op(B) = B (stored K x N): element (n, k) of the slab layout
// <- r(B[k][n]) through a 64 x 64 LDS tile (rows read along n, written along
// k), zero past K and N.
template <bool BF16, bool VEC, bool NTL>
__global__ __launch_bounds__(256) void lp16_round_transpose(const float *B, int64_t ldb, int K, int N, void *dst_,
                                                            int Np, int Kp)
{
    typedef typename Lp<BF16>::T T;
    typedef typename Lp<BF16>::V8 V8;
    __shared__ T t[64][64 + 8];
    T *dst = static_cast<T *>(dst_);
    const int n0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
    poison_lds(t, (int)sizeof(t));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = threadIdx.x + 256 * i;
        const int kr = e / 16, nc = 4 * (e % 16);
        const int k = k0 + kr, n = n0 + nc;
        const float *p = B + (int64_t)k * ldb + n;
        float x[4];
        if (VEC && k < K && n + 4 <= N) {
            const lp_f32x4 v = lp16_load4<NTL>(p);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                x[q] = v[q];
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                x[q] = (k < K && n + q < N) ? p[q] : 0.0f;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            t[nc + q][kr] = (T)x[q];
    }
    __syncthreads();
    // two slabs of 64 rows x 4 chunks; consecutive work-items write
    // consecutive 16-byte chunks of a slab
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int e = threadIdx.x + 256 * i;
        const int sl = e / 256, nr = (e / 4) % 64, c = e % 4;
        const int n = n0 + nr, k = k0 + QK * sl + 8 * c;
        if (n < Np && k < Kp) {
            V8 v;
#pragma unroll
            for (int q = 0; q < 8; ++q)
                v[q] = t[nr][QK * sl + 8 * c + q];
            *reinterpret_cast<V8 *>(dst + ((int64_t)(k / QK) * Np + n) * QK + 8 * c) = v;
        }
    }
}

}  // namespace

// The 256 x 256 tile runs 16 wavefronts of 64 x 64 (four on each SIMD, 108
// VGPRs each), where 8 wavefronts of 64 x 128 (two per SIMD, 191 VGPRs) read
// a quarter fewer fragment bytes per FLOP from the LDS: the LDS has the
// bandwidth to spare (a CU reads over 300 bytes per cycle from it), and the
// second pair of wavefronts on each SIMD covers the fragment-read and barrier
// waits that held the matrix cores at half their rate.  Measured on MI355X
// (GEMM pass alone, bf16, same bits): 4096^3 120.1 -> 116.4 us, 6144^3 465.9 ->
// 453.5, 16384 x 4096 x 1024 166.9 -> 154.0, 4096 x 4096 x 1024 44.5 -> 38.9,
// 8192^3 level (884-905 us both).
//
// The 128 x 128 tile runs 8 wavefronts of 64 x 32 (with two workgroups on a
// CU, four wavefronts per SIMD) up to K = 3072 and 4 wavefronts of 64 x 64
// above: measured on
// MI355X (GEMM pass alone, bf16, same bits), 8 wavefronts took 2048 x 2048 x K
// from 15.9 to 12.7 us at K = 512, 20.2 -> 17.3 at 1024, 24.1 -> 21.9 at 1536,
// 28.2 -> 26.5 at 2048, 37.2 -> 35.3 at 3072, 1024^3 18.3 -> 15.2; level at
// K = 2560 and 4096; slower at 1024 x 1024 x 4096 (39.1 -> 40.3) and
// 2048 x 2048 x 8192 (73.9 -> 78.7).
typedef QGeo<256, 256, 4, 4, 4> QL;   // 16 wavefronts of 64 x 64, 4 stages (128 KB)
typedef QGeo<128, 128, 2, 4, 4> QS8;  // 8 wavefronts of 64 x 32, 4 stages (64 KB): K <= kQs8MaxK
typedef QGeo<128, 128, 2, 2, 4> QS;   // 4 wavefronts of 64 x 64, 4 stages (64 KB): longer K
static_assert(QL::NT <= 1024 && QS8::NT <= 1024 && QS::NT <= 1024, "the plan's launch-size check");
constexpr int64_t kQs8MaxK = 3072;    // padded K

template <class Q>
static void launch_q(const Lp16Args &g, bool bf16, hipStream_t s)
{
    const dim3 grid((unsigned)(g.tiles_m * g.tiles_n)), block(Q::NT);
    if (bf16)
        lp16_gemm_kernel<Q, true><<<grid, block, 0, s>>>(g);
    else
        lp16_gemm_kernel<Q, false><<<grid, block, 0, s>>>(g);
}

static int64_t up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// The rounding passes read the FP32 operands with streaming loads when A,
// op(B) and C together exceed kStreamBytes, a working set that the 256 MB
// Infinity Cache does not keep from one call to the next: the loads then pass
// by the caches instead of evicting the 16-bit operands that the GEMM pass
// reads right after.  Below it, ordinary loads keep the operands in the cache
// for a repeated call.  Measured on MI355X (bf16, full two-pass step, same
// bits): 16384 x 4096 x 1024 188.7 -> 176.6 us, 8192^3 1071 -> 1050, 6144^3
// 541 -> 535; with streaming loads at 4096^3 (192 MB) 152.1 -> 157.4 us.
constexpr int64_t kStreamBytes = int64_t{200} << 20;

template <bool BF16>
static void round_rows_t(const float *src, int64_t ld, int R, int K, void *dst, int64_t Rp, int64_t Kp, bool vec,
                         bool nt, hipStream_t s)
{
    const int64_t chunks = Rp * (Kp / 8);
    const unsigned grid = (unsigned)std::min<int64_t>((chunks + 255) / 256, 8192);
    if (!vec)
        lp16_round_rows<BF16, false, false><<<grid, 256, 0, s>>>(src, ld, R, K, dst, (int)Rp, (int)Kp);
    else if (nt)
        lp16_round_rows<BF16, true, true><<<grid, 256, 0, s>>>(src, ld, R, K, dst, (int)Rp, (int)Kp);
    else
        lp16_round_rows<BF16, true, false><<<grid, 256, 0, s>>>(src, ld, R, K, dst, (int)Rp, (int)Kp);
}

// R x K k-contiguous FP32 rows -> Rp x Kp 16-bit rows.
static void round_rows(const float *src, int64_t ld, int R, int K, void *dst, int64_t Rp, int64_t Kp, bool bf16,
                       bool vec, bool nt, hipStream_t s)
{
    if (bf16)
        round_rows_t<true>(src, ld, R, K, dst, Rp, Kp, vec, nt, s);
    else
        round_rows_t<false>(src, ld, R, K, dst, Rp, Kp, vec, nt, s);
}

// K x N FP32 op(B) = B -> Np x Kp 16-bit rows of B^T.
template <bool BF16>
static void round_transpose_t(const float *B, int64_t ldb, int K, int N, void *dst, int64_t Np, int64_t Kp, bool vec,
                              bool nt, hipStream_t s)
{
    const dim3 grid((unsigned)(Np / 64), (unsigned)((Kp + 63) / 64));
    if (!vec)
        lp16_round_transpose<BF16, false, false><<<grid, 256, 0, s>>>(B, ldb, K, N, dst, (int)Np, (int)Kp);
    else if (nt)
        lp16_round_transpose<BF16, true, true><<<grid, 256, 0, s>>>(B, ldb, K, N, dst, (int)Np, (int)Kp);
    else
        lp16_round_transpose<BF16, true, false><<<grid, 256, 0, s>>>(B, ldb, K, N, dst, (int)Np, (int)Kp);
}

TileShape lp16_tile_shape(bool large) { return large ? TileShape{QL::BM, QL::BN} : TileShape{QS::BM, QS::BN}; }

// Layout of the workspace: A16 (Kp/32 slabs of Mp x 32) at 0, B16 (Kp/32
// slabs of Np x 32) after it, each starting on a 256-byte boundary.
int64_t lp16_workspace_bytes(int64_t M, int64_t N, int64_t K, bool large)
{
    const TileShape t = lp16_tile_shape(large);
    const int64_t Kp = up(K, QK);
    return up(up(M, t.bm) * Kp * 2, 256) + up(N, t.bn) * Kp * 2;
}

hipError_t launch_lp16(const GemmArgs &a, bool large, bool bf16, bool transB, void *ws, hipStream_t s)
{
    const TileShape t = lp16_tile_shape(large);
    const int64_t Kp = up(a.K, QK), Mp = up(a.M, t.bm), Np = up(a.N, t.bn);
    unsigned char *base = static_cast<unsigned char *>(ws);
    void *A16 = base;
    void *B16 = base + up(Mp * Kp * 2, 256);

    const bool avec = (reinterpret_cast<uintptr_t>(a.A) & 15) == 0 && (a.lda & 3) == 0;
    const bool bvec = (reinterpret_cast<uintptr_t>(a.B) & 15) == 0 && (a.ldb & 3) == 0;
    const int64_t M = a.M, N = a.N, K = a.K;
    const bool nt = 4 * (M * K + K * N + M * N) > kStreamBytes;
    round_rows(a.A, a.lda, a.M, a.K, A16, Mp, Kp, bf16, avec, nt, s);
    if (transB)
        round_rows(a.B, a.ldb, a.N, a.K, B16, Np, Kp, bf16, bvec, nt, s);
    else if (bf16)
        round_transpose_t<true>(a.B, a.ldb, a.K, a.N, B16, Np, Kp, bvec, nt, s);
    else
        round_transpose_t<false>(a.B, a.ldb, a.K, a.N, B16, Np, Kp, bvec, nt, s);
    Lp16Args g;
    g.A16 = A16;
    g.B16 = B16;
    g.C = a.C;
    g.slab_a = Mp * QK;
    g.slab_b = Np * QK;
    g.ldc = a.ldc;
    g.M = a.M;
    g.N = a.N;
    g.Kp = (int)Kp;
    g.alpha = a.alpha;
    g.beta = a.beta;
    g.tiles_m = (int)(Mp / t.bm);
    g.tiles_n = (int)(Np / t.bn);
    if (large)
        launch_q<QL>(g, bf16, s);
    else if (Kp <= kQs8MaxK)
        launch_q<QS8>(g, bf16, s);
    else
        launch_q<QS>(g, bf16, s);
    return hipGetLastError();
}

}  // namespace sgemm
