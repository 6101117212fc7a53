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
//   * k-contiguous LDS tiles (A, B^T) are unpadded, with the 16-byte chunks of
//     each row permuted by an XOR of row bits: the 32 rows a half-wavefront reads
//     at one k then fall on distinct banks, and a whole 1 KB block of LDS can be
//     filled by one direct global->LDS load (the +1 padding of
//     "CUDA矩阵乘法性能优化实战：从朴素内核到寄存器分块与Nsight剖析", section 3.3,
//     cannot be expressed inside such a block; the permutation does its job).
//   * Workgroups are dispatched round-robin over the 8 XCDs; tiles are remapped
//     so each XCD gets a contiguous run, grouped 8 tile-rows at a time, so tiles
//     that share rows of A and columns of B run on the same L2.
//
// Two staging paths fill the same LDS layout:
//   * direct (interior tiles, and edge tiles whose clamped addresses stay
//     exact): global_load_lds_dwordx4 writes each 1 KB LDS block straight from
//     memory, no registers involved, 16 bytes per lane from any float-aligned
//     address (leading dimensions need not be multiples of 4).  Tile t+1 is
//     issued during iteration t into the free buffer (at its start, or by half
//     of the wavefronts of the 8-wavefront tiles one k-group later) and must
//     land before the iteration's barrier.  A partial last k-tile (K % BK != 0) is
//     staged through registers with zero fill and multiplied first.
//   * registers (edge tiles of op(B) = B with N % 4 != 0, and leading
//     dimensions too large for 32-bit offsets): masked loads into registers,
//     one tile ahead: iteration t stores tile t+1 to the free buffer and issues
//     the loads of tile t+2.
// In both, each k-group's fragments are read while the previous group's MFMAs
// run, and the one barrier per tile sits before the last group's MFMAs, which
// cover it and the next tile's first LDS reads.
#include "sgemm_internal.h"

namespace sgemm {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// Four floats in global memory at any 4-byte aligned address: 128-bit loads
// through this type need no 16-byte alignment (the device runs with unaligned
// access enabled for global memory).
typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

template <int W> struct vec_of;
template <> struct vec_of<1> { typedef float type; };
template <> struct vec_of<2> { typedef f32x2 type; };
template <> struct vec_of<4> { typedef f32x4 type; };

template <int W>
__device__ __forceinline__ float vget(const typename vec_of<W>::type &v, int i);
template <> __device__ __forceinline__ float vget<1>(const float &v, int) { return v; }
template <> __device__ __forceinline__ float vget<2>(const f32x2 &v, int i) { return v[i]; }
template <> __device__ __forceinline__ float vget<4>(const f32x4 &v, int i) { return v[i]; }

template <int W>
__device__ __forceinline__ void vset(typename vec_of<W>::type &v, int i, float x);
template <> __device__ __forceinline__ void vset<1>(float &v, int, float x) { v = x; }
template <> __device__ __forceinline__ void vset<2>(f32x2 &v, int i, float x) { v[i] = x; }
template <> __device__ __forceinline__ void vset<4>(f32x4 &v, int i, float x) { v[i] = x; }

// threadIdx.x; with OPQ, behind an empty asm, so that each tile's set-up
// derives its per-lane offsets afresh.  The stream-K kernel runs the tile code
// in a loop and would otherwise hoist them out of it and hold them (spilled)
// across the loop; the plain kernels keep the direct read (measured 0.6%
// faster at 4096^3).
template <bool OPQ>
__device__ __forceinline__ int work_item()
{
    int t = (int)threadIdx.x;
    if constexpr (OPQ)
        asm volatile("" : "+v"(t));
    return t;
}

// Wavefront index within the workgroup, as a wave-uniform (scalar) value: the
// LDS block addresses derived from it then stay in scalar registers, and M0 for
// the direct loads is set without a per-load vector-to-scalar move (measured ~1%).
template <bool OPQ>
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(work_item<OPQ>() >> 6); }

// Tile order: workgroups are dealt round-robin to the 8 XCDs, so ids are
// renumbered to give each XCD one contiguous run (xcd_remap), and the runs walk
// the tile grid 8 tile-rows at a time, column by column (group_order), so the
// tiles one XCD holds at once share rows of A and columns of B in its L2.
__device__ __forceinline__ int xcd_remap(int bid, int total)
{
    return (total & 7) == 0 ? (bid & 7) * (total >> 3) + (bid >> 3) : bid;
}

__device__ __forceinline__ void group_order(int t, int nbm, int nbn, int &tm, int &tn)
{
    constexpr int G = 8;
    const int per_group = G * nbn;
    const int gi = t / per_group;
    const int first = gi * G;
    const int gsz = min(nbm - first, G);
    const int in = t - gi * per_group;
    tm = first + in % gsz;
    tn = in / gsz;
}

// Tile index for workgroup `bid` over an nbm x nbn tile grid.
__device__ __forceinline__ void map_tile(int bid, int nbm, int nbn, int &tm, int &tn)
{
    group_order(xcd_remap(bid, nbm * nbn), nbm, nbn, tm, tn);
}

// Four consecutive floats from p, one 128-bit load when all four are in.
// MASKED: elements at or beyond `limit` (or all of them when !ok) read as zero.
template <bool MASKED>
__device__ __forceinline__ f32x4 load4(const float *p, bool ok, int first, int limit)
{
    f32x4 v;
    if (!MASKED || (ok && first + 4 <= limit)) {
        v = *reinterpret_cast<const f32x4u *>(p);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = (ok && first + e < limit) ? p[e] : 0.0f;
    }
    return v;
}

// Compile-time geometry of one MFMA kernel configuration.  KS > 1 splits the
// k-range of one output tile over KS groups of wavefronts ("k-slices"): an LDS
// stage then holds KS consecutive BK-deep k-tiles, slice s multiplies the s-th
// into its own accumulators, and the slices are added in LDS at the end.
template <int BM_, int BN_, int BK_, int WGM_, int WGN_, int OCC_, bool TRANS_B, int KS_ = 1, bool OPQ_ = false>
struct Geo {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_, OCC = OCC_, KS = KS_;
    static constexpr bool OPQ = OPQ_;                  // per-lane ids behind an asm (stream-K)
    static constexpr int NWO = WGM * WGN;              // wavefronts per k-slice (one output tile)
    static constexpr int NW = NWO * KS;                // wavefronts per workgroup
    static constexpr int NT = 64 * NW;                 // work-items per workgroup
    static constexpr int KT = KS * BK;                 // k values per LDS stage
    static constexpr int WM = BM / WGM, WN = BN / WGN; // wavefront tile
    static constexpr int FM = WM / 32, FN = WN / 32;   // 32x32 blocks per wavefront
    static constexpr int IL = TRANS_B ? 1 : (FN >= 4 ? 4 : FN);
    static constexpr int NG = FN / IL;                 // interleaved column groups
    static constexpr int G = BK / 8;                   // k-groups per slice tile
    static constexpr int CPR = BK / 4;                 // 16-byte chunks per k-row
    static constexpr int A_SZ = BM * BK;               // floats of A per slice tile
    static constexpr int B_SZ = BK * BN;               // floats of op(B) per slice tile
    static constexpr int SLICE = A_SZ + B_SZ;
    static constexpr int STAGE = KS * SLICE;           // floats per LDS stage
    static constexpr int CA = KS * BM * CPR / NT;      // register path: A chunks per work-item
    static constexpr int CB = KS * BK * BN / 4 / NT;   //                B chunks per work-item
    static constexpr int A_BLK = A_SZ / 256, B_BLK = B_SZ / 256;  // 1 KB blocks per slice tile
    static constexpr int A_BLK_W = KS * A_BLK / NW;    // direct path: blocks per wavefront
    static constexpr int B_BLK_W = KS * B_BLK / NW;
    static constexpr int ACC = FM * FN * 16;           // accumulators per lane
    static constexpr int UNITS = 2 * FM;               // output units per wavefront tile (8 accumulator rows)
    // k-slices that finish units: spread over up to four slices (measured on
    // MI355X: the 32 x 32 tile's four slices, 512^3 with beta = 1 47.5 -> 49.6
    // TFLOP/s); with two slices, slice 0 finishing the whole tile measured
    // faster (2048^3: 134.2 against 121.8 for the spread finish)
    static constexpr int FIN = KS >= 4 ? (KS < UNITS ? KS : UNITS) : 1;
    static constexpr int RED = KS == 1 ? 0 : (FIN == 1 ? KS - 1 : KS) * NWO * ACC * 64;  // floats for the k-slice sums
    static constexpr int SMEM = (2 * STAGE > RED) ? 2 * STAGE : RED;
    static_assert(WM % 32 == 0 && WN % 32 == 0, "tile shape");
    static_assert(BK == 16 || BK == 32, "the chunk permutation covers 4 or 8 chunks per row");
    static_assert((KS * BM * CPR) % NT == 0 && (KS * BK * BN / 4) % NT == 0, "register staging split");
    static_assert(A_SZ % 256 == 0 && B_SZ % 256 == 0, "whole 1 KB blocks");
    static_assert((KS * A_BLK) % NW == 0 && (KS * B_BLK) % NW == 0, "direct staging split");
    static_assert(TRANS_B || 256 % BN == 0, "op(B)=B rows must tile a 1 KB block");
    static_assert(SMEM * 4 <= 160 * 1024, "LDS budget");
    static_assert(G % 2 == 0, "the fragment ping-pong needs an even number of k-groups");
};

// What one wavefront does: its k-slice and its place in the output tile.
template <class Gm>
struct Role {
    int lane, l32, hi, slice, wo, wm, wn;
    __device__ __forceinline__ Role()
    {
        const int wave = wave_id<Gm::OPQ>();
        lane = work_item<Gm::OPQ>() & 63;
        l32 = lane & 31;
        hi = lane >> 5;
        slice = wave / Gm::NWO;
        wo = wave % Gm::NWO;
        wm = wo / Gm::WGN;
        wn = wo % Gm::WGN;
    }
};

// Physical 16-byte chunk of logical chunk c in row r of a k-contiguous tile.
// Rows r..r+7 get 8 distinct permutations (CPR=8), and any 16 rows split into
// pairs (r mod 2 or r mod 4) that differ too, so 8- and 16-lane read phases
// both touch every bank once.
template <int CPR>
__device__ __forceinline__ int swz(int r)
{
    if constexpr (CPR == 4)
        return ((r >> 1) ^ (r >> 2)) & 3;
    else
        return (r ^ (r >> 3)) & 7;
}

// Float offset of logical chunk c of row r in a k-contiguous tile.
template <int CPR>
__device__ __forceinline__ int koff(int r, int c)
{
    return r * (4 * CPR) + 4 * (c ^ swz<CPR>(r));
}

// Keeps the instruction scheduler from moving anything across this point.  The
// fragment reads of the next k-group are issued before the current group's
// MFMAs on purpose (their latency hides under ~32 MFMAs); left alone, the
// scheduler sinks them next to their first use to save registers.
__device__ __forceinline__ void pin_order() { __builtin_amdgcn_sched_barrier(0); }

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
    constexpr int CPR = Gm::CPR;
    const int c = 2 * g + hi;  // logical chunk: k = 8g + 4*hi .. +3
#pragma unroll
    for (int fm = 0; fm < Gm::FM; ++fm)
        f.a[fm] = *reinterpret_cast<const f32x4 *>(&As[koff<CPR>(wm * Gm::WM + 32 * fm + l32, c)]);
    if constexpr (TRANS_B) {
#pragma unroll
        for (int fn = 0; fn < Gm::FN; ++fn)
            f.bt[fn] = *reinterpret_cast<const f32x4 *>(&Bs[koff<CPR>(wn * Gm::WN + 32 * fn + l32, c)]);
    } else {
        typedef typename vec_of<Gm::IL>::type bvec;
        const int k = 8 * g + 4 * hi;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int gr = 0; gr < Gm::NG; ++gr)
                f.b[s][gr] = *reinterpret_cast<const bvec *>(
                    &Bs[(k + s) * Gm::BN + wn * Gm::WN + gr * 32 * Gm::IL + Gm::IL * l32]);
    }
}

// MFMA steps s0 .. s1-1 of one k-group (8 consecutive k values, 4 steps).
template <class Gm, bool TRANS_B>
__device__ __forceinline__ void mfma_steps(f32x16 (&acc)[Gm::FM][Gm::FN], const Frags<Gm, TRANS_B> &f, int s0,
                                           int s1)
{
#pragma unroll
    for (int s = s0; s < s1; ++s)
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

template <class Gm, bool TRANS_B>
__device__ __forceinline__ void mfma_group(f32x16 (&acc)[Gm::FM][Gm::FN], const Frags<Gm, TRANS_B> &f)
{
    mfma_steps<Gm, TRANS_B>(acc, f, 0, 4);
}

// Register staging of one LDS stage (KS k-tiles): masked (or, for interior
// tiles and full stages, plain) loads into registers, then stores in LDS layout.
template <class Gm, bool TRANS_B>
struct RegStage {
    static constexpr int CA = Gm::CA, CB = Gm::CB, CPR = Gm::CPR, BN4 = Gm::BN / 4;
    const float *pa[CA];
    const float *pb[CB];
    int ra_row[CA], ra_k[CA], ra_lds[CA];   // row in tile, k within the stage, LDS offset
    int rb_row[CB], rb_k[CB], rb_lds[CB];   // (B: n row / k row, k / n offset, LDS offset)
    f32x4 ra[CA], rb[CB];

    __device__ __forceinline__ void init(const GemmArgs &a, int m0, int n0)
    {
        const int tid = work_item<Gm::OPQ>();
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            const int q = tid + i * Gm::NT;
            const int sl = q / (Gm::BM * CPR), q2 = q % (Gm::BM * CPR);
            const int c = q2 % CPR;
            ra_row[i] = q2 / CPR;
            ra_k[i] = sl * Gm::BK + 4 * c;
            ra_lds[i] = sl * Gm::SLICE + koff<CPR>(ra_row[i], c);
            pa[i] = a.A + (int64_t)(m0 + ra_row[i]) * a.lda + ra_k[i];
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int q = tid + i * Gm::NT;
            if constexpr (TRANS_B) {
                const int sl = q / (Gm::BN * CPR), q2 = q % (Gm::BN * CPR);
                const int c = q2 % CPR;
                rb_row[i] = q2 / CPR;                        // n within the tile
                rb_k[i] = sl * Gm::BK + 4 * c;               // k within the stage
                rb_lds[i] = sl * Gm::SLICE + Gm::A_SZ + koff<CPR>(rb_row[i], c);
                pb[i] = a.B + (int64_t)(n0 + rb_row[i]) * a.ldb + rb_k[i];
            } else {
                const int sl = q / (Gm::BK * BN4), q2 = q % (Gm::BK * BN4);
                const int kr = q2 / BN4;
                rb_row[i] = sl * Gm::BK + kr;                // k within the stage
                rb_k[i] = 4 * (q2 % BN4);                    // n within the tile
                rb_lds[i] = sl * Gm::SLICE + Gm::A_SZ + kr * Gm::BN + rb_k[i];
                pb[i] = a.B + (int64_t)rb_row[i] * a.ldb + n0 + rb_k[i];
            }
        }
    }

    // MASKED=false: the tile lies inside M x N and stage kt is full.
    template <bool MASKED>
    __device__ __forceinline__ void load(const GemmArgs &a, int m0, int n0, int kt)
    {
        const int k0 = kt * Gm::KT;
#pragma unroll
        for (int i = 0; i < CA; ++i)
            ra[i] = load4<MASKED>(pa[i] + (int64_t)k0, m0 + ra_row[i] < a.M, k0 + ra_k[i], a.K);
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            if constexpr (TRANS_B)
                rb[i] = load4<MASKED>(pb[i] + (int64_t)k0, n0 + rb_row[i] < a.N, k0 + rb_k[i], a.K);
            else
                rb[i] = load4<MASKED>(pb[i] + (int64_t)k0 * a.ldb, k0 + rb_row[i] < a.K, n0 + rb_k[i], a.N);
        }
    }

    __device__ __forceinline__ void store(float *stage) const
    {
#pragma unroll
        for (int i = 0; i < CA; ++i)
            *reinterpret_cast<f32x4 *>(&stage[ra_lds[i]]) = ra[i];
#pragma unroll
        for (int i = 0; i < CB; ++i)
            *reinterpret_cast<f32x4 *>(&stage[rb_lds[i]]) = rb[i];
    }
};

// Direct staging of full stages with global->LDS loads.  A wavefront
// instruction (global_load_lds_dwordx4) fills one 1 KB LDS block, lane L
// writing floats e = 256*block + 4L .. 4L+3 of the stage's slice tile.  Each
// lane's source follows from where its LDS floats lie: in a k-contiguous tile
// (A, and op(B) = B^T) float e is row e / BK, physical k-position e % BK, whose
// 4-float chunk holds logical chunk (e % BK / 4) ^ swz(row); in the
// n-contiguous op(B) = B tile it is row e / BN, column e % BN.  A source needs
// 4-byte alignment only: with a leading dimension that is not a multiple of 4
// the 16 bytes of a chunk start anywhere on a float boundary, and the loads
// stay 16 bytes wide (4-byte loads would take four times the instructions).
// Sources are 32-bit float offsets from the tile's first element, valid
// because the host allows this path only when a tile's extent fits (rows x
// leading dimension < 2^31).
//
// EDGE: the tile reaches past M or N.  Rows of A (and of B^T) past the matrix
// load its last row instead, and for op(B) = B columns past N load its last
// whole 4-column chunk (the caller allows this only when N % 4 == 0): those
// values only reach outputs that the masked epilogue does not store, and every
// address stays inside the operands.
template <class Gm, bool TRANS_B>
struct DirectStage {
    static constexpr int W = 4, BW = 64 * W;
    static constexpr int A_N = Gm::KS * Gm::A_SZ / BW / Gm::NW;   // instructions per wavefront
    static constexpr int B_N = Gm::KS * Gm::B_SZ / BW / Gm::NW;
    static constexpr int A_BPS = Gm::A_SZ / BW, B_BPS = Gm::B_SZ / BW;  // blocks per slice tile
    static_assert(A_N * BW * Gm::NW == Gm::KS * Gm::A_SZ && B_N * BW * Gm::NW == Gm::KS * Gm::B_SZ,
                  "direct staging split");
    uint32_t a_off[A_N], b_off[B_N];
    int a_lds[A_N], b_lds[B_N];   // LDS float offsets within a stage (wave-uniform)
    const float *a_base;
    const float *b_base;
    int64_t b_kstep;

    // Source offset of LDS float e (first of W) of a k-contiguous tile row-major
    // in memory with leading dimension ld; rows clamped to `last` on edges.
    template <bool EDGE>
    static __device__ __forceinline__ uint32_t kcontig(int e, int sl, int ld, int last)
    {
        const int r = e / Gm::BK, q = e % Gm::BK;
        const int c = (q / 4) ^ swz<Gm::CPR>(r);
        const int rg = EDGE ? min(r, last) : r;
        return (uint32_t)(rg * ld + sl * Gm::BK + 4 * c + q % 4);
    }

    template <bool EDGE>
    __device__ __forceinline__ void init(const GemmArgs &a, int m0, int n0)
    {
        const int lane = work_item<Gm::OPQ>() & 63, wave = wave_id<Gm::OPQ>();
#pragma unroll
        for (int j = 0; j < A_N; ++j) {
            const int b = wave * A_N + j;
            const int sl = b / A_BPS, lb = b % A_BPS;
            a_off[j] = kcontig<EDGE>(lb * BW + W * lane, sl, (int)a.lda, a.M - 1 - m0);
            a_lds[j] = sl * Gm::SLICE + lb * BW;
        }
#pragma unroll
        for (int j = 0; j < B_N; ++j) {
            const int b = wave * B_N + j;
            const int sl = b / B_BPS, lb = b % B_BPS;
            const int e = lb * BW + W * lane;
            if constexpr (TRANS_B) {
                b_off[j] = kcontig<EDGE>(e, sl, (int)a.ldb, a.N - 1 - n0);
            } else {
                const int col = e % Gm::BN;
                const int cg = EDGE ? min(col, a.N - W - n0) : col;
                b_off[j] = (uint32_t)((sl * Gm::BK + e / Gm::BN) * (int)a.ldb + cg);
            }
            b_lds[j] = sl * Gm::SLICE + Gm::A_SZ + lb * BW;
        }
        a_base = a.A + (int64_t)m0 * a.lda;
        b_base = TRANS_B ? a.B + (int64_t)n0 * a.ldb : a.B + n0;
        b_kstep = TRANS_B ? (int64_t)Gm::KT : (int64_t)Gm::KT * a.ldb;
    }

    __device__ __forceinline__ void issue(int kt, float *stage) const
    {
        const float *ak = a_base + (int64_t)kt * Gm::KT;
        const float *bk = b_base + (int64_t)kt * b_kstep;
#pragma unroll
        for (int j = 0; j < A_N; ++j)
            __builtin_amdgcn_global_load_lds(ak + a_off[j], (lds_void *)(stage + a_lds[j]), 4 * W, 0, 0);
#pragma unroll
        for (int j = 0; j < B_N; ++j)
            __builtin_amdgcn_global_load_lds(bk + b_off[j], (lds_void *)(stage + b_lds[j]), 4 * W, 0, 0);
    }
};

// One finishing slice (FIN == 1) and KS > 1: k-slices 1..KS-1 leave their
// accumulators in LDS and slice 0 adds them in slice order (a fixed order, so
// results are reproducible).  Called by every wavefront; returns true for the
// wavefronts that write the output.
template <class Gm>
__device__ __forceinline__ bool reduce_slices(f32x16 (&acc)[Gm::FM][Gm::FN], float *smem, const Role<Gm> &ro)
{
    if constexpr (Gm::KS == 1) {
        return true;
    } else {
        __syncthreads();  // every wavefront is done with the stage buffers
        poison_lds(smem, Gm::RED * 4);
        if (ro.slice > 0) {
            float *dst = smem + ((ro.slice - 1) * Gm::NWO + ro.wo) * Gm::ACC * 64 + ro.lane;
#pragma unroll
            for (int fm = 0; fm < Gm::FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < Gm::FN; ++fn)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        dst[((fm * Gm::FN + fn) * 16 + r) * 64] = acc[fm][fn][r];
        }
        __syncthreads();
        if (ro.slice > 0)
            return false;
#pragma unroll
        for (int s = 1; s < Gm::KS; ++s) {
            const float *src = smem + ((s - 1) * Gm::NWO + ro.wo) * Gm::ACC * 64 + ro.lane;
#pragma unroll
            for (int fm = 0; fm < Gm::FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < Gm::FN; ++fn)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acc[fm][fn][r] += src[((fm * Gm::FN + fn) * 16 + r) * 64];
        }
        return true;
    }
}

template <class Gm, bool TRANS_B, bool FULL, bool RD>
__device__ __forceinline__ void epilogue_rows(const GemmArgs &a, const f32x16 (&acc)[Gm::FM][Gm::FN], int m0, int n0,
                                              const Role<Gm> &ro)
{
    // Accumulator register r of a 32x32 block holds row 8*(r/4) + 4*hi + (r%4)
    // and column l32 of that block.  Rows go 8 at a time; with beta != 0 the
    // old C values of all 8 are loaded before the first of them is stored:
    // loads and stores share the pointer C, so a load written after a store
    // cannot be hoisted above it and would wait out a whole memory round trip.
    // beta == 0 reads nothing and takes its own copy of the loop.
    typedef typename vec_of<Gm::IL>::type bvec;
    constexpr int IL = Gm::IL;
    const int l32 = ro.l32, hi = ro.hi, wm = ro.wm, wn = ro.wn;
    const uintptr_t cbase = reinterpret_cast<uintptr_t>(a.C);
    const bool cvec = IL > 1 && (cbase % (4 * IL)) == 0 && (a.ldc % IL) == 0;
    constexpr bool rd = RD;
#pragma unroll
    for (int fm = 0; fm < Gm::FM; ++fm) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float old[8][Gm::FN];
            if constexpr (rd) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int r = 8 * h + i;
                    const int row = m0 + wm * Gm::WM + 32 * fm + 8 * (r / 4) + 4 * hi + (r % 4);
                    if (!FULL && row >= a.M)
                        continue;
                    const float *crow = a.C + (int64_t)row * a.ldc;
#pragma unroll
                    for (int gr = 0; gr < Gm::NG; ++gr) {
                        const int col = n0 + wn * Gm::WN + gr * 32 * IL + IL * l32;
                        if (IL > 1 && cvec && (FULL || col + IL <= a.N)) {
                            const bvec o = *reinterpret_cast<const bvec *>(crow + col);
#pragma unroll
                            for (int b = 0; b < IL; ++b)
                                old[i][gr * IL + b] = vget<IL>(o, b);
                        } else {
#pragma unroll
                            for (int b = 0; b < IL; ++b)
                                old[i][gr * IL + b] = (FULL || col + b < a.N) ? crow[col + b] : 0.0f;
                        }
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 8 * h + i;
                const int row = m0 + wm * Gm::WM + 32 * fm + 8 * (r / 4) + 4 * hi + (r % 4);
                if (!FULL && row >= a.M)
                    continue;
                float *crow = a.C + (int64_t)row * a.ldc;
#pragma unroll
                for (int gr = 0; gr < Gm::NG; ++gr) {
                    const int col = n0 + wn * Gm::WN + gr * 32 * IL + IL * l32;
                    float v[IL];
#pragma unroll
                    for (int b = 0; b < IL; ++b) {
                        const float x = acc[fm][gr * IL + b][r];
                        v[b] = rd ? fmaf(a.alpha, x, a.beta * old[i][gr * IL + b]) : a.alpha * x;
                    }
                    if (IL > 1 && cvec && (FULL || col + IL <= a.N)) {
                        bvec o;
#pragma unroll
                        for (int b = 0; b < IL; ++b)
                            vset<IL>(o, b, v[b]);
                        *reinterpret_cast<bvec *>(crow + col) = o;
                    } else {
#pragma unroll
                        for (int b = 0; b < IL; ++b)
                            if (FULL || col + b < a.N)
                                crow[col + b] = v[b];
                    }
                }
            }
        }
    }
}

template <class Gm, bool TRANS_B, bool FULL>
__device__ __forceinline__ void epilogue(const GemmArgs &a, const f32x16 (&acc)[Gm::FM][Gm::FN], int m0, int n0,
                                         const Role<Gm> &ro)
{
    if (a.beta != 0.0f)
        epilogue_rows<Gm, TRANS_B, FULL, true>(a, acc, m0, n0, ro);
    else
        epilogue_rows<Gm, TRANS_B, FULL, false>(a, acc, m0, n0, ro);
}

// Old C of a wavefront that holds a single 32x32 block (the 64 x 64 tile): with
// beta != 0 its 16 values per lane are read before the k-loop, so their
// latency passes under the loop instead of following it at the end of the
// tile, where nothing else would overlap it.  Larger tiles would hold 64 or 128
// more registers for a tail that is a small share of their time, and keep the
// batched loads of epilogue_rows.  The arithmetic is epilogue_rows'.
template <class Gm>
struct OldC {
    static constexpr bool ON = Gm::FM * Gm::FN == 1;
    float v[ON ? 16 : 1];

    // One finishing slice: all 16 values of the block; more: the 8 of the unit
    // this wavefront's k-slice finishes (unit = slice, half h = slice; see Finish).
    template <bool FULL>
    __device__ __forceinline__ void load(const GemmArgs &a, int m0, int n0, const Role<Gm> &ro)
    {
        if constexpr (ON) {
            const int col = n0 + ro.wn * Gm::WN + ro.l32;
            constexpr int NV = Gm::FIN == 1 ? 16 : 8;
            const int r0 = Gm::FIN == 1 ? 0 : 8 * ro.slice;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int r = r0 + i;
                const int row = m0 + ro.wm * Gm::WM + 8 * (r / 4) + 4 * ro.hi + (r % 4);
                v[i] = (FULL || (row < a.M && col < a.N)) ? a.C[(int64_t)row * a.ldc + col] : 0.0f;
            }
        }
    }

    template <bool FULL>
    __device__ __forceinline__ void epilogue(const GemmArgs &a, const f32x16 (&acc)[Gm::FM][Gm::FN], int m0, int n0,
                                             const Role<Gm> &ro) const
    {
        if constexpr (ON) {
            const int col = n0 + ro.wn * Gm::WN + ro.l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + ro.wm * Gm::WM + 8 * (r / 4) + 4 * ro.hi + (r % 4);
                if (FULL || (row < a.M && col < a.N))
                    a.C[(int64_t)row * a.ldc + col] = fmaf(a.alpha, acc[0][0][r], a.beta * v[r]);
            }
        }
    }
};

// FIN > 1: the output of a wavefront tile is finished in units of 8
// accumulator rows (unit u = 2*fm + h: registers 8h .. 8h+7 of each of the FN
// blocks in block row fm), unit u by k-slice u % FIN, so that adding the
// slices' partial sums and storing the result are spread over up to FIN
// slices instead of falling to one.  Every slice leaves all its partial sums
// in LDS; a finishing slice reads back the KS partials of each of its units
// and adds them in slice order, as (p0 + p1) + p2 ..., so the result does not
// depend on which slice finishes a unit and repeats bit for bit.  The units
// and rows are picked with addresses, never with register indices, so the
// accumulators stay in fixed registers.
template <class Gm>
struct Finish {
    static constexpr int PER = Gm::UNITS / Gm::FIN;  // units per finishing slice
    f32x4 v[PER][Gm::FN][2];                        // unit k: registers 8h+4q .. 8h+4q+3 of block fn in v[k][fn][q]
};

// Returns true for the wavefronts that finish units.
template <class Gm>
__device__ __forceinline__ bool reduce_units(const f32x16 (&acc)[Gm::FM][Gm::FN], float *smem, const Role<Gm> &ro,
                                             Finish<Gm> &out)
{
    // Region of (slice, wavefront): the lane's ACC accumulators as ACC/4
    // float4s, float4 j of lane L at j*64 + L (128-bit LDS accesses).
    constexpr int Q = Gm::ACC / 4;
    f32x4 *red = reinterpret_cast<f32x4 *>(smem);
    __syncthreads();  // every wavefront is done with the stage buffers
    poison_lds(smem, Gm::RED * 4);
    f32x4 *mine = red + (ro.slice * Gm::NWO + ro.wo) * Q * 64 + ro.lane;
#pragma unroll
    for (int fm = 0; fm < Gm::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < Gm::FN; ++fn)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x16 &x = acc[fm][fn];
                mine[((fm * Gm::FN + fn) * 4 + q) * 64] = f32x4{x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]};
            }
    __syncthreads();
    if (ro.slice >= Gm::FIN)
        return false;
    const f32x4 *part = red + ro.wo * Q * 64 + ro.lane;
#pragma unroll
    for (int k = 0; k < Finish<Gm>::PER; ++k) {
        const int u = k * Gm::FIN + ro.slice, fm = u >> 1, h = u & 1;
#pragma unroll
        for (int fn = 0; fn < Gm::FN; ++fn)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int at = ((fm * Gm::FN + fn) * 4 + 2 * h + q) * 64;
                f32x4 v = part[at];
#pragma unroll
                for (int sl = 1; sl < Gm::KS; ++sl)
                    v += part[sl * Gm::NWO * Q * 64 + at];
                out.v[k][fn][q] = v;
            }
    }
    return true;
}

// The finished units to C.  MODE 0: beta == 0, C not read; 1: the 8 rows' old
// values of a unit are loaded before the first of them is stored (as in
// epilogue_rows); 2: old values loaded before the k-loop (OldC).
template <class Gm, bool TRANS_B, bool FULL, int MODE>
__device__ __forceinline__ void store_units(const GemmArgs &a, const Finish<Gm> &fin, const OldC<Gm> &oc, int m0,
                                            int n0, const Role<Gm> &ro)
{
    typedef typename vec_of<Gm::IL>::type bvec;
    constexpr int IL = Gm::IL;
    const int l32 = ro.l32, hi = ro.hi;
    const uintptr_t cbase = reinterpret_cast<uintptr_t>(a.C);
    const bool cvec = IL > 1 && (cbase % (4 * IL)) == 0 && (a.ldc % IL) == 0;
#pragma unroll
    for (int k = 0; k < Finish<Gm>::PER; ++k) {
        const int u = k * Gm::FIN + ro.slice, fm = u >> 1, h = u & 1;
        const int row0 = m0 + ro.wm * Gm::WM + 32 * fm + 16 * h + 4 * hi;  // rows row0 + 8*(i/4) + i%4
        float old[8][Gm::FN];
        if constexpr (MODE == 1) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int row = row0 + 8 * (i / 4) + (i % 4);
                if (!FULL && row >= a.M)
                    continue;
                const float *crow = a.C + (int64_t)row * a.ldc;
#pragma unroll
                for (int gr = 0; gr < Gm::NG; ++gr) {
                    const int col = n0 + ro.wn * Gm::WN + gr * 32 * IL + IL * l32;
                    if (IL > 1 && cvec && (FULL || col + IL <= a.N)) {
                        const bvec o = *reinterpret_cast<const bvec *>(crow + col);
#pragma unroll
                        for (int b = 0; b < IL; ++b)
                            old[i][gr * IL + b] = vget<IL>(o, b);
                    } else {
#pragma unroll
                        for (int b = 0; b < IL; ++b)
                            old[i][gr * IL + b] = (FULL || col + b < a.N) ? crow[col + b] : 0.0f;
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = row0 + 8 * (i / 4) + (i % 4);
            if (!FULL && row >= a.M)
                continue;
            float *crow = a.C + (int64_t)row * a.ldc;
#pragma unroll
            for (int gr = 0; gr < Gm::NG; ++gr) {
                const int col = n0 + ro.wn * Gm::WN + gr * 32 * IL + IL * l32;
                float v[IL];
#pragma unroll
                for (int b = 0; b < IL; ++b) {
                    const float x = fin.v[k][gr * IL + b][i / 4][i % 4];
                    if constexpr (MODE == 0)
                        v[b] = a.alpha * x;
                    else if constexpr (MODE == 1)
                        v[b] = fmaf(a.alpha, x, a.beta * old[i][gr * IL + b]);
                    else
                        v[b] = fmaf(a.alpha, x, a.beta * oc.v[i]);
                }
                if (IL > 1 && cvec && (FULL || col + IL <= a.N)) {
                    bvec o;
#pragma unroll
                    for (int b = 0; b < IL; ++b)
                        vset<IL>(o, b, v[b]);
                    *reinterpret_cast<bvec *>(crow + col) = o;
                } else {
#pragma unroll
                    for (int b = 0; b < IL; ++b)
                        if (FULL || col + b < a.N)
                            crow[col + b] = v[b];
                }
            }
        }
    }
}

// After the k-loop: add the k-slices (KS > 1) and write the tile's outputs.
// `pre`: this wavefront loaded its old C before the k-loop (OldC).
template <class Gm, bool TRANS_B, bool FULL>
__device__ __forceinline__ void finish_tile(const GemmArgs &a, f32x16 (&acc)[Gm::FM][Gm::FN], float *smem, int m0,
                                            int n0, const Role<Gm> &ro, bool pre, const OldC<Gm> &oc)
{
    if constexpr (Gm::FIN == 1) {
        if (reduce_slices<Gm>(acc, smem, ro)) {
            if (pre)
                oc.template epilogue<FULL>(a, acc, m0, n0, ro);
            else
                epilogue<Gm, TRANS_B, FULL>(a, acc, m0, n0, ro);
        }
    } else {
        Finish<Gm> fin;
        if (!reduce_units<Gm>(acc, smem, ro, fin))
            return;
        if (a.beta == 0.0f)
            store_units<Gm, TRANS_B, FULL, 0>(a, fin, oc, m0, n0, ro);
        else if constexpr (OldC<Gm>::ON)
            store_units<Gm, TRANS_B, FULL, 2>(a, fin, oc, m0, n0, ro);  // a finishing slice loaded its old C
        else
            store_units<Gm, TRANS_B, FULL, 1>(a, fin, oc, m0, n0, ro);
    }
}

// One k-group of one stage: the first MFMA step runs on fragments read a whole
// group earlier, before any new LDS traffic (so the wait in front of it never
// covers fresh reads); then `next()` issues the next fragments (or the barrier
// and the next stage's first fragments); then the other three steps.
template <class Gm, bool TRANS_B, class Next>
__device__ __forceinline__ void group_step(f32x16 (&acc)[Gm::FM][Gm::FN], const Frags<Gm, TRANS_B> &cur, Next next)
{
    mfma_steps<Gm, TRANS_B>(acc, cur, 0, 1);
    pin_order();
    next();
    pin_order();
    mfma_steps<Gm, TRANS_B>(acc, cur, 1, 4);
}

template <class Gm>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[Gm::FM][Gm::FN])
{
#pragma unroll
    for (int i = 0; i < Gm::FM; ++i)
#pragma unroll
        for (int j = 0; j < Gm::FN; ++j)
            acc[i][j] = f32x16{0};
}

// Register-staged k-loop.  FULL: the tile lies inside M x N (only the K tail
// needs masks).
template <class Gm, bool TRANS_B, bool FULL>
__device__ __forceinline__ void gemm_tile_regs(const GemmArgs &a, float *smem, int m0, int n0)
{
    constexpr int G = Gm::G;
    const Role<Gm> ro;
    const int sl_off = ro.slice * Gm::SLICE;
    OldC<Gm> oc;
    const bool pre = OldC<Gm>::ON && a.beta != 0.0f && ro.slice < Gm::FIN;
    if (pre)
        oc.template load<FULL>(a, m0, n0, ro);

    RegStage<Gm, TRANS_B> st;
    st.init(a, m0, n0);
    auto gload = [&](int kt) {
        if (FULL && (kt + 1) * Gm::KT <= a.K)
            st.template load<false>(a, m0, n0, kt);
        else
            st.template load<true>(a, m0, n0, kt);
    };

    f32x16 acc[Gm::FM][Gm::FN];
    zero_acc<Gm>(acc);

    const int nk = (a.K + Gm::KT - 1) / Gm::KT;
    Frags<Gm, TRANS_B> f[2];
    gload(0);
    poison_lds(smem, Gm::STAGE * 4);
    st.store(smem);
    if (nk > 1)
        gload(1);
    __syncthreads();
    read_frags<Gm, TRANS_B>(f[0], smem + sl_off, smem + sl_off + Gm::A_SZ, 0, ro.wm, ro.wn, ro.l32, ro.hi);

    for (int t = 0; t < nk; ++t) {
        const float *As = smem + (t & 1) * Gm::STAGE + sl_off;
        const float *Bs = As + Gm::A_SZ;
        float *Sn = smem + ((t + 1) & 1) * Gm::STAGE;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            group_step<Gm, TRANS_B>(acc, f[g & 1], [&] {
                if (g == 0 && t + 1 < nk) {
                    poison_lds(Sn, Gm::STAGE * 4);
                    st.store(Sn);   // stage t+1 into the free buffer
                    if (t + 2 < nk)
                        gload(t + 2);
                }
                if (g + 1 < G) {
                    read_frags<Gm, TRANS_B>(f[(g + 1) & 1], As, Bs, g + 1, ro.wm, ro.wn, ro.l32, ro.hi);
                } else if (t + 1 < nk) {
                    __syncthreads();
                    read_frags<Gm, TRANS_B>(f[G & 1], Sn + sl_off, Sn + sl_off + Gm::A_SZ, 0, ro.wm, ro.wn,
                                            ro.l32, ro.hi);
                }
            });
        }
    }
    finish_tile<Gm, TRANS_B, FULL>(a, acc, smem, m0, n0, ro, pre, oc);
}

// Where the wavefronts of an 8-wavefront workgroup issue the next stage's
// direct loads.  Issued by all eight at the top of the stage, they queue 64
// wavefront instructions at the CU's address unit at once, and each wavefront
// waits behind its own before its next MFMA.  So half the wavefronts (those
// with wave & MASK set) issue theirs after the first MFMA step of k-group
// GROUP instead, while the others multiply; the loads still land long before
// the stage's closing barrier.  The masks are the fastest measured on MI355X
// per kernel, among splits by wave bit 0, 1 or 2 at k-group 1 or 2 (4096^3
// 144.4 -> 146.5 TFLOP/s, 8192^3 145.5 -> 147.6; 128 x 128 tile at 6144^3
// 138.3 -> 140.3; 64 x 64 tile at 1024^3 105.8 -> 109.4; the stream-K
// 128 x 128 kernel at 2048^3 131.1 -> 133.1 with bit 2, where bit 0 gave
// 120.9); MASK 0: no split, as for the 4-wavefront tiles, where splitting
// by bit 0 or 1 measured up to 10% slower (k-split partial pass, 512 x 512
// x 8192 on the 32 x 32 tile).
template <class Gm>
struct IssueSplit {
    static constexpr int MASK = Gm::NW != 8 ? 0 : (Gm::BM == 64 || (Gm::OPQ && Gm::KS == 2)) ? 4 : 1;
    static constexpr int GROUP = 1;
    static_assert(MASK == 0 || GROUP < Gm::G - 1, "the late loads must come before the closing barrier's group");
};

// Direct-staged k-loop (interior tiles, and edge tiles whose clamped
// addresses are exact).
template <class Gm, bool TRANS_B, bool EDGE>
__device__ __forceinline__ void gemm_tile_direct(const GemmArgs &a, float *smem, int m0, int n0)
{
    constexpr int G = Gm::G;
    const Role<Gm> ro;
    const int sl_off = ro.slice * Gm::SLICE;
    float *buf0 = smem, *buf1 = smem + Gm::STAGE;
    OldC<Gm> oc;
    const bool pre = OldC<Gm>::ON && a.beta != 0.0f && ro.slice < Gm::FIN;
    if (pre)
        oc.template load<!EDGE>(a, m0, n0, ro);

    f32x16 acc[Gm::FM][Gm::FN];
    zero_acc<Gm>(acc);

    const int nf = a.K / Gm::KT;  // full stages
    Frags<Gm, TRANS_B> f[2];

    DirectStage<Gm, TRANS_B> ds;
    ds.template init<EDGE>(a, m0, n0);
    typedef IssueSplit<Gm> IS;
    const bool late = IS::MASK != 0 && (wave_id<Gm::OPQ>() & IS::MASK) != 0;  // wave-uniform
    if (nf > 0) {
        poison_lds(buf0, Gm::STAGE * 4);
        ds.issue(0, buf0);
    }

    // Partial last stage first (the order of the k sum is free): registers with
    // zero fill, through buffer 1, while stage 0 lands in buffer 0.
    if (nf * Gm::KT < a.K) {
        RegStage<Gm, TRANS_B> st;
        st.init(a, m0, n0);
        st.template load<true>(a, m0, n0, nf);
        poison_lds(buf1, Gm::STAGE * 4);
        st.store(buf1);
        __syncthreads();
#pragma unroll
        for (int g = 0; g < G; ++g) {
            read_frags<Gm, TRANS_B>(f[0], buf1 + sl_off, buf1 + sl_off + Gm::A_SZ, g, ro.wm, ro.wn, ro.l32, ro.hi);
            mfma_group<Gm, TRANS_B>(acc, f[0]);
        }
    }
    if (nf > 0) {
        __syncthreads();  // stage 0 has landed (and buffer 1 is free again)
        read_frags<Gm, TRANS_B>(f[0], buf0 + sl_off, buf0 + sl_off + Gm::A_SZ, 0, ro.wm, ro.wn, ro.l32, ro.hi);
        for (int t = 0; t < nf; ++t) {
            const float *As = ((t & 1) ? buf1 : buf0) + sl_off;
            const float *Bs = As + Gm::A_SZ;
            float *Sn = (t & 1) ? buf0 : buf1;
            // A wavefront's loads of stage t+1 go out together (measured against
            // spreading them over its MFMA steps, that is faster): at the top of
            // the stage, or for the late half at k-group IssueSplit::GROUP.
            if (t + 1 < nf) {
                poison_lds(Sn, Gm::STAGE * 4);
                if (!late)
                    ds.issue(t + 1, Sn);
                pin_order();
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                group_step<Gm, TRANS_B>(acc, f[g & 1], [&] {
                    if (late && g == IS::GROUP && t + 1 < nf)
                        ds.issue(t + 1, Sn);
                    if (g + 1 < G) {
                        read_frags<Gm, TRANS_B>(f[(g + 1) & 1], As, Bs, g + 1, ro.wm, ro.wn, ro.l32, ro.hi);
                    } else if (t + 1 < nf) {
                        __syncthreads();  // this wavefront's direct loads, then everyone's
                        read_frags<Gm, TRANS_B>(f[G & 1], Sn + sl_off, Sn + sl_off + Gm::A_SZ, 0, ro.wm, ro.wn,
                                                ro.l32, ro.hi);
                    }
                });
            }
        }
    }
    finish_tile<Gm, TRANS_B, !EDGE>(a, acc, smem, m0, n0, ro, pre, oc);
}

// One output tile at (m0, n0): direct staging for interior tiles (and edge
// tiles whose clamped addresses are exact: op(B) = B^T, or op(B) = B with N a
// multiple of 4, so that a 4-column chunk is wholly inside or outside),
// registers otherwise.  GD: geometry of the direct path; GR: geometry of the
// register path (same workgroup tile, wavefront layout and k-split, possibly a
// shorter k-tile so the register staging fits next to the accumulators).
template <class GD, class GR, bool TRANS_B>
__device__ __forceinline__ void mfma_tile(const GemmArgs &a, float *smem, int m0, int n0)
{
    const bool full = m0 + GD::BM <= a.M && n0 + GD::BN <= a.N;
    if (a.flags & GEMM_FLAG_DIRECT) {
        if (full || TRANS_B || (a.N & 3) == 0) {
            if (full)
                gemm_tile_direct<GD, TRANS_B, false>(a, smem, m0, n0);
            else
                gemm_tile_direct<GD, TRANS_B, true>(a, smem, m0, n0);
            return;
        }
    }
    if (full)
        gemm_tile_regs<GR, TRANS_B, true>(a, smem, m0, n0);
    else
        gemm_tile_regs<GR, TRANS_B, false>(a, smem, m0, n0);
}

template <class GD, class GR>
struct SharedGeo {
    static_assert(GD::BM == GR::BM && GD::BN == GR::BN && GD::NT == GR::NT && GD::WGN == GR::WGN &&
                      GD::KS == GR::KS,
                  "both paths share the workgroup tile");
    static constexpr int SMEM = GD::SMEM > GR::SMEM ? GD::SMEM : GR::SMEM;
};

template <class GD, class GR, bool TRANS_B>
__global__ __launch_bounds__(GD::NT) __attribute__((amdgpu_waves_per_eu(GD::OCC)))
void sgemm_mfma_kernel(GemmArgs a)
{
    __shared__ __attribute__((aligned(1024))) float smem[SharedGeo<GD, GR>::SMEM];
    if (gridDim.y > 1) {
        // k-split partial pass: this split's k-range and partial-product slice.
        const int s = blockIdx.y, k0 = s * a.k_split;
        a.A += k0;
        a.B += TRANS_B ? (int64_t)k0 : (int64_t)k0 * a.ldb;
        a.K = min(a.k_split, a.K - k0);
        a.C += (int64_t)s * a.c_split_stride;
    }
    const int nbm = (a.M + GD::BM - 1) / GD::BM, nbn = (a.N + GD::BN - 1) / GD::BN;
    int tile_m, tile_n;
    map_tile(blockIdx.x, nbm, nbn, tile_m, tile_n);
    mfma_tile<GD, GR, TRANS_B>(a, smem, tile_m * GD::BM, tile_n * GD::BN);
}

// A uniform value the compiler cannot see through (an empty asm that claims to
// rewrite the scalar register holding it).
__device__ __forceinline__ int64_t opaque(int64_t v)
{
    asm volatile("" : "+s"(v));
    return v;
}

// Stream-K: the k-iterations of all output tiles, one LDS stage of k each, in
// tile order (group_order) and k order within a tile.  Workgroups below sk.dp
// take whole tiles (XCD-remapped, as the plain kernel); the sk.workers after
// them split the iterations of the last sk.tiles tiles evenly, each a
// contiguous range, so every CU gets the same share of the work whatever the
// tile count (Osama et al., "Stream-K: Work-centric Parallel Decomposition for
// Dense Matrix-Matrix Multiplication on the GPU").  A range is cut into pieces
// at tile boundaries; each piece runs the ordinary tile code on its sub-range
// of k with the operand pointers moved to the tile's corner.  A piece that is
// a whole tile is finished in place; any other piece writes its raw partial
// product to the worker's slot and the fix-up kernel completes the tile.  No
// workgroup ever waits for another.
template <class GD, class GR, bool TRANS_B>
__global__ __launch_bounds__(GD::NT) __attribute__((amdgpu_waves_per_eu(GD::OCC)))
void sgemm_mfma_sk_kernel(GemmArgs a, SkArgs sk)
{
    __shared__ __attribute__((aligned(1024))) float smem[SharedGeo<GD, GR>::SMEM];
    const int nbm = (a.M + GD::BM - 1) / GD::BM, nbn = (a.N + GD::BN - 1) / GD::BN;
    const int iters = sk.iters;
    const int bid = blockIdx.x;
    int w = -1;
    int64_t it, end;
    if (bid < sk.dp) {
        it = (int64_t)xcd_remap(bid, sk.dp) * iters;
        end = it + iters;
    } else {
        const int P = sk.workers, raw = bid - sk.dp;
        w = (P & 7) == 0 ? (raw & 7) * (P >> 3) + (raw >> 3) : raw;
        const int64_t S = (int64_t)sk.sk_tiles * iters, base = (int64_t)sk.dp * iters;
        it = base + (int64_t)w * S / P;
        end = base + (int64_t)(w + 1) * S / P;
    }
    const int64_t first = it;
    while (it < end) {
        const int t = (int)(it / iters);
        const int kb = (int)(it - (int64_t)t * iters);
        const int ke = (int)min((int64_t)iters, kb + (end - it));
        int tm, tn;
        group_order(t, nbm, nbn, tm, tn);
        const int m0 = tm * GD::BM, n0 = tn * GD::BN;
        const int k0 = kb * GD::KT, k1 = min(a.K, ke * GD::KT);
        GemmArgs b = a;
        // The tile code's per-lane offsets depend only on the leading
        // dimensions and the lane; hidden from the compiler here, they are
        // recomputed per piece instead of being hoisted out of the loop and
        // held in registers across it (which spilled).
        b.lda = opaque(a.lda);
        b.ldb = opaque(a.ldb);
        b.ldc = opaque(a.ldc);
        b.A = a.A + (int64_t)m0 * a.lda + k0;
        b.B = TRANS_B ? a.B + (int64_t)n0 * a.ldb + k0 : a.B + (int64_t)k0 * a.ldb + n0;
        b.M = a.M - m0;
        b.N = a.N - n0;
        b.K = k1 - k0;
        if (kb == 0 && ke == iters) {
            b.C = a.C + (int64_t)m0 * a.ldc + n0;
        } else {
            b.C = sk.ws + (int64_t)(2 * w + (it == first ? 0 : 1)) * (GD::BM * GD::BN);
            b.ldc = GD::BN;
            b.alpha = 1.0f;
            b.beta = 0.0f;
        }
        if (it != first)
            __syncthreads();  // the previous piece's last LDS reads are done
        mfma_tile<GD, GR, TRANS_B>(b, smem, 0, 0);
        it += ke - kb;
    }
}

// Stream-K fix-up: workgroup (j, y) completes rows [16y, 16y + 16) of the j-th
// stream-K tile when more than one worker shared it, adding the pieces in
// worker (= k) order: C <- alpha * sum + beta * C (C not read when beta == 0).
// Worker w's range starts at floor(w*S/P), so the worker holding iteration x
// is floor(((x + 1)*P - 1) / S); its piece of tile j sits in slot 0 if the
// range starts inside or at the start of the tile, else in slot 1.
template <int BM, int BN, bool VEC>
__global__ __launch_bounds__(256) void sgemm_sk_fixup_kernel(GemmArgs a, SkArgs sk)
{
    constexpr int ROWS = 16, C4 = BN / 4, RPP = 256 / C4;
    const int j = blockIdx.x, iters = sk.iters, P = sk.workers;
    const int64_t S = (int64_t)sk.sk_tiles * iters;
    const int64_t lo = (int64_t)j * iters, hi = lo + iters - 1;
    const int w_lo = (int)(((lo + 1) * P - 1) / S), w_hi = (int)(((hi + 1) * P - 1) / S);
    if (w_lo == w_hi)
        return;  // one worker covered the tile and wrote C itself
    const int nbm = (a.M + BM - 1) / BM, nbn = (a.N + BN - 1) / BN;
    int tm, tn;
    group_order(sk.dp + j, nbm, nbn, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int c = 4 * (threadIdx.x % C4);
    const int col = n0 + c;
    if (col >= a.N)
        return;
    const bool vec = VEC && col + 4 <= a.N;
#pragma unroll
    for (int pass = 0; pass < ROWS / RPP; ++pass) {
        const int r = blockIdx.y * ROWS + pass * RPP + (int)threadIdx.x / C4;
        const int row = m0 + r;
        if (row >= a.M)
            continue;
        f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int w = w_lo; w <= w_hi; ++w) {
            const int slot = 2 * w + (lo <= (int64_t)w * S / P ? 0 : 1);
            const f32x4 v = *reinterpret_cast<const f32x4 *>(sk.ws + (int64_t)slot * (BM * BN) + r * BN + c);
            sum += v;
        }
        float *cp = a.C + (int64_t)row * a.ldc + col;
        if (vec) {
            f32x4 o = a.alpha * sum;
            if (a.beta != 0.0f) {
                const f32x4 old = *reinterpret_cast<const f32x4 *>(cp);
                for (int e = 0; e < 4; ++e)
                    o[e] = fmaf(a.alpha, sum[e], a.beta * old[e]);
            }
            *reinterpret_cast<f32x4 *>(cp) = o;
        } else {
            for (int e = 0; e < 4 && col + e < a.N; ++e)
                cp[e] = a.beta != 0.0f ? fmaf(a.alpha, sum[e], a.beta * cp[e]) : a.alpha * sum[e];
        }
    }
}

TileShape tile_shape(int kid)
{
    switch (kid) {
    case KID_MFMA_L: return {256, 256};
    case KID_MFMA_M: return {128, 128};
    case KID_MFMA_S:
    case KID_MFMA_S2: return {64, 64};
    case KID_MFMA_T: return {32, 32};
    case KID_MFMA_R: return {128, 64};
    case KID_REGBLOCK: return {128, 128};
    case KID_TILED_PAD:
    case KID_TILED_NOPAD: return {16, 16};
    case KID_NAIVE: return {4, 64};
    case KID_NAIVE_WG: return {1, 1};
    default: return {0, 0};
    }
}

template <int BM, int BN, int BKD, int BKR, int WGM, int WGN, int OCC, int KS>
static void launch_cfg(const GemmArgs &a, bool transB, hipStream_t stream, int splits)
{
    const int64_t blocks = ceil_div(a.M, BM) * ceil_div(a.N, BN);
    const dim3 grid((unsigned)blocks, (unsigned)splits), block(64 * WGM * WGN * KS);
    typedef Geo<BM, BN, BKD, WGM, WGN, OCC, true, KS> GDT;
    typedef Geo<BM, BN, BKR, WGM, WGN, OCC, true, KS> GRT;
    typedef Geo<BM, BN, BKD, WGM, WGN, OCC, false, KS> GDN;
    typedef Geo<BM, BN, BKR, WGM, WGN, OCC, false, KS> GRN;
    if (transB)
        sgemm_mfma_kernel<GDT, GRT, true><<<grid, block, 0, stream>>>(a);
    else
        sgemm_mfma_kernel<GDN, GRN, false><<<grid, block, 0, stream>>>(a);
}

template <int BM, int BN, int BKD, int BKR, int WGM, int WGN, int OCC, int KS>
static void launch_sk_cfg(const GemmArgs &a, const SkArgs &sk, bool transB, hipStream_t stream)
{
    const dim3 grid((unsigned)(sk.dp + sk.workers)), block(64 * WGM * WGN * KS);
    typedef Geo<BM, BN, BKD, WGM, WGN, OCC, true, KS, true> GDT;
    typedef Geo<BM, BN, BKR, WGM, WGN, OCC, true, KS, true> GRT;
    typedef Geo<BM, BN, BKD, WGM, WGN, OCC, false, KS, true> GDN;
    typedef Geo<BM, BN, BKR, WGM, WGN, OCC, false, KS, true> GRN;
    if (transB)
        sgemm_mfma_sk_kernel<GDT, GRT, true><<<grid, block, 0, stream>>>(a, sk);
    else
        sgemm_mfma_sk_kernel<GDN, GRN, false><<<grid, block, 0, stream>>>(a, sk);
    if (sk.sk_tiles > 0) {
        const dim3 fgrid((unsigned)sk.sk_tiles, BM / 16);
        const bool cvec = (reinterpret_cast<uintptr_t>(a.C) & 15) == 0 && (a.ldc & 3) == 0;
        if (cvec)
            sgemm_sk_fixup_kernel<BM, BN, true><<<fgrid, dim3(256), 0, stream>>>(a, sk);
        else
            sgemm_sk_fixup_kernel<BM, BN, false><<<fgrid, dim3(256), 0, stream>>>(a, sk);
    }
}

int mfma_stage_k(int kid)
{
    switch (kid) {
    case KID_MFMA_L: return 32;
    case KID_MFMA_M: return 64;
    default: return 0;
    }
}

hipError_t launch_mfma_sk(const GemmArgs &a, const SkArgs &sk, int kid, bool transB, hipStream_t stream)
{
    switch (kid) {
    case KID_MFMA_L: launch_sk_cfg<256, 256, 32, 16, 4, 2, 2, 1>(a, sk, transB, stream); break;
    case KID_MFMA_M: launch_sk_cfg<128, 128, 32, 32, 2, 2, 2, 2>(a, sk, transB, stream); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_mfma(const GemmArgs &a, int kid, bool transB, hipStream_t stream, int splits)
{
    switch (kid) {
    case KID_MFMA_L: launch_cfg<256, 256, 32, 16, 4, 2, 2, 1>(a, transB, stream, splits); break;
    case KID_MFMA_M: launch_cfg<128, 128, 32, 32, 2, 2, 2, 2>(a, transB, stream, splits); break;
    case KID_MFMA_S: launch_cfg<64, 64, 32, 32, 2, 2, 4, 1>(a, transB, stream, splits); break;
    case KID_MFMA_S2: launch_cfg<64, 64, 32, 32, 2, 2, 2, 2>(a, transB, stream, splits); break;
    case KID_MFMA_T: launch_cfg<32, 32, 32, 32, 1, 1, 2, 4>(a, transB, stream, splits); break;
    case KID_MFMA_R: launch_cfg<128, 64, 32, 32, 4, 1, 2, 2>(a, transB, stream, splits); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace sgemm
