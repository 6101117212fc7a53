// Out-of-place FP32 matrix transpose: dst (cols x rows) <- src (rows x cols)^T.
//
// "现代 CUDA 工具箱实战：从朴素代码到硬件极限的优化之路", section 代码实现: the naive
// baseline reads rows and writes columns (every store strided); the optimised
// version reads a tile along source rows into shared memory and writes it out
// along destination rows, so both global accesses are contiguous and the
// transposition happens in LDS, where one padding column per tile row keeps the
// column-wise LDS accesses spread over the banks (section 常见错误: without the
// padding every lane of a column access hits one bank).
//
// MI355X version.  A 128 x 128 tile (64.5 KB of LDS with the padding column,
// two workgroups per CU; 64 x 64 for small matrices).  One wavefront instruction moves 64 consecutive floats
// of one row (256 contiguous bytes) or, with 128-bit loads, 4 rows x 64 floats:
//   load:  lane l reads src(r, c0 + l) and writes LDS word r*P + l;
//   store: lane l reads LDS word l*P + j and writes dst(j, r0 + l).
// With the row pitch P = 129 (65) lane l of the column-wise read lands on bank
// (l + j) mod B for B = 32 or 64 banks, so no two lanes of a wavefront (or of a
// half-wavefront) share a bank; with P = 128 (64) all lanes hit one bank.
//
// Three launch shapes, chosen by the number of 128 x 128 tiles (measured on
// MI355X):
//   SMALL  (fewer tiles than the 256 CUs): 64 x 64 tiles instead, 256
//          work-items, one tile per workgroup, so the grid still spreads over
//          the chip;
//   PIPE   (up to 2048 tiles, e.g. 4096 x 4096): 256 work-items, a persistent
//          grid of two workgroups per CU; each workgroup issues the global loads
//          of its next tile before writing the current one out, so reads and
//          writes overlap instead of alternating chip-wide;
//   STREAM (larger): 512 work-items, one tile per workgroup, 128-bit loads
//          when the source is 16-byte aligned, tiles visited in groups of 8
//          tile-rows; loads and stores carry the non-temporal hint, since every
//          byte is touched once.
// Every element moves 8 bytes (one read, one write); the kernels are bound by
// memory bandwidth.
//
// Two element-per-work-item kernels serve narrow matrices, where a 128-wide tile
// would run mostly empty: the baseline (contiguous reads; with few source rows
// the few destination columns merge in L2) and a narrow kernel with one
// work-item per destination element (contiguous writes; with few source columns
// the reads of a wavefront share a few cache lines).
#include "transpose_internal.h"

namespace sgemm {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int TP_T = 128;                 // tile edge
constexpr int TP_T_SMALL = 64;            // tile edge of the SMALL shape
constexpr int TP_SMALL_MAX_TILES = 255;   // SMALL below one 128-tile per CU
constexpr int TP_PIPE_MAX_TILES = 2048;   // PIPE up to this many tiles, STREAM above
constexpr int64_t TP_MAX_BLOCKS = 1 << 20;
constexpr int TP_PIPE_BLOCKS = 512;       // two per CU

// Cache-policy hints.
template <bool NT> __device__ __forceinline__ float ld1(const float *p)
{
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT> __device__ __forceinline__ f32x4 ld4(const float *p)
{
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
    else return *reinterpret_cast<const f32x4 *>(p);
}
template <bool NT> __device__ __forceinline__ void st1(float *p, float v)
{
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// Tile (tr, tc) of tile number t: row-major over tiles, or (GROUP > 0) in groups
// of GROUP tile-rows walked column by column (the last group may be shorter).
template <int T, int GROUP>
__device__ __forceinline__ void tile_of(unsigned t, unsigned tiles_r, unsigned tiles_c, int &r0, int &c0)
{
    unsigned tr, tc;
    if constexpr (GROUP == 0) {
        tr = t / tiles_c;
        tc = t % tiles_c;
    } else {
        const unsigned per = GROUP * tiles_c, g = t / per, rem = t % per;
        const unsigned left = tiles_r - g * GROUP, gh = left < GROUP ? left : GROUP;
        tr = g * GROUP + rem % gh;
        tc = rem / gh;
    }
    r0 = (int)tr * T;
    c0 = (int)tc * T;
}

// One tile's registers and the moves between global memory, registers and LDS.
// TH work-items; V4: 128-bit loads (16 lanes per 64-float row segment).
template <int T, int TH, int PAD, bool V4, bool NTL, bool NTS>
struct TileMover {
    static_assert(T % 64 == 0 && (T / (V4 ? 4 : 1)) * (T / 64) % (TH / 64) == 0, "whole wavefront rows");
    static constexpr int P = T + PAD, NW = TH / 64;
    static constexpr int RPI = V4 ? 4 : 1;                  // rows per load instruction
    static constexpr int LOADS = (T / RPI) * (T / 64) / NW;
    static constexpr int STORES = T * (T / 64) / NW;
    static constexpr int REGS = LOADS * (V4 ? 4 : 1);
    float v[REGS];

    // Row and column (inside the tile) of load instruction i of wavefront w.
    static __device__ __forceinline__ void load_pos(int w, int lane, int i, int &r, int &c)
    {
        const int ch = w + NW * i;
        if constexpr (V4) {
            r = (ch / (T / 64)) * 4 + (lane >> 4);
            c = (ch % (T / 64)) * 64 + 4 * (lane & 15);
        } else {
            r = ch / (T / 64);
            c = (ch % (T / 64)) * 64 + lane;
        }
    }

    template <bool MASKED>
    __device__ __forceinline__ void load(const TransposeArgs &a, int r0, int c0, int w, int lane)
    {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            int r, c;
            load_pos(w, lane, i, r, c);
            const float *p = a.src + (int64_t)(r0 + r) * a.ld_src + (c0 + c);
            if constexpr (V4) {
                if (MASKED) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        v[4 * i + q] = (r0 + r < a.rows && c0 + c + q < a.cols) ? p[q] : 0.0f;
                } else {
                    const f32x4 x = ld4<NTL>(p);
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        v[4 * i + q] = x[q];
                }
            } else {
                v[i] = (!MASKED || (r0 + r < a.rows && c0 + c < a.cols)) ? ld1<NTL>(p) : 0.0f;
            }
        }
    }

    __device__ __forceinline__ void to_lds(float *tile, int w, int lane) const
    {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            int r, c;
            load_pos(w, lane, i, r, c);
#pragma unroll
            for (int q = 0; q < (V4 ? 4 : 1); ++q)
                tile[r * P + c + q] = v[(V4 ? 4 : 1) * i + q];
        }
    }

    template <bool MASKED>
    static __device__ __forceinline__ void store(const TransposeArgs &a, const float *tile, int r0, int c0, int w,
                                                 int lane)
    {
#pragma unroll
        for (int i = 0; i < STORES; ++i) {
            const int ch = w + NW * i;
            const int j = ch / (T / 64), r = (ch % (T / 64)) * 64 + lane;
            float *p = a.dst + (int64_t)(c0 + j) * a.ld_dst + (r0 + r);  // dst(c0 + j, r0 + r)
            if (!MASKED || (c0 + j < a.cols && r0 + r < a.rows))
                st1<NTS>(p, tile[r * P + j]);
        }
    }
};

template <int T>
__device__ __forceinline__ bool full_tile(const TransposeArgs &a, int r0, int c0)
{
    return r0 + T <= a.rows && c0 + T <= a.cols;
}

// PIPE: persistent workgroups; the next tile's loads are issued before the
// current tile is written out.
template <int PAD>
__global__ __launch_bounds__(256) void transpose_pipe_kernel(TransposeArgs a)
{
    using M = TileMover<TP_T, 256, PAD, false, true, false>;
    __shared__ float tile[TP_T * M::P];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // Dimensions stay below 2^31 - 1024 and the tile count below 2^32, so the
    // tile arithmetic fits in 32 bits.
    const unsigned tiles_c = ((unsigned)a.cols + TP_T - 1) / TP_T;
    const unsigned tiles_r = ((unsigned)a.rows + TP_T - 1) / TP_T;
    const unsigned tiles = tiles_c * tiles_r;
    M m;
    unsigned t = blockIdx.x;
    int r0 = 0, c0 = 0;
    if (t < tiles) {
        tile_of<TP_T, 0>(t, tiles_r, tiles_c, r0, c0);
        if (full_tile<TP_T>(a, r0, c0))
            m.template load<false>(a, r0, c0, w, lane);
        else
            m.template load<true>(a, r0, c0, w, lane);
    }
    for (; t < tiles; t += gridDim.x) {
        poison_lds(tile, (int)sizeof(tile));
        m.to_lds(tile, w, lane);
        __syncthreads();
        const int cr0 = r0, cc0 = c0;
        if (t + gridDim.x < tiles) {
            tile_of<TP_T, 0>(t + gridDim.x, tiles_r, tiles_c, r0, c0);
            if (full_tile<TP_T>(a, r0, c0))
                m.template load<false>(a, r0, c0, w, lane);
            else
                m.template load<true>(a, r0, c0, w, lane);
        }
        if (full_tile<TP_T>(a, cr0, cc0))
            M::template store<false>(a, tile, cr0, cc0, w, lane);
        else
            M::template store<true>(a, tile, cr0, cc0, w, lane);
        __syncthreads();  // the tile buffer is refilled by the next iteration
    }
}

// STREAM and SMALL: one tile per workgroup (the grid loops only past 2^20
// tiles); STREAM visits tiles in groups of 8 tile-rows with non-temporal loads
// and stores, SMALL keeps the default cache policy.
template <int T, int TH, int PAD, bool V4, bool NT>
__global__ __launch_bounds__(TH) void transpose_tile_kernel(TransposeArgs a)
{
    using M = TileMover<T, TH, PAD, V4, NT, NT>;
    __shared__ float tile[T * M::P];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const unsigned tiles_c = ((unsigned)a.cols + T - 1) / T;
    const unsigned tiles_r = ((unsigned)a.rows + T - 1) / T;
    const unsigned tiles = tiles_c * tiles_r;
    M m;
    for (unsigned t = blockIdx.x; t < tiles; t += gridDim.x) {
        int r0, c0;
        tile_of<T, NT ? 8 : 0>(t, tiles_r, tiles_c, r0, c0);
        const bool full = full_tile<T>(a, r0, c0);
        if (full)
            m.template load<false>(a, r0, c0, w, lane);
        else
            m.template load<true>(a, r0, c0, w, lane);
        poison_lds(tile, (int)sizeof(tile));
        m.to_lds(tile, w, lane);
        __syncthreads();
        if (full)
            M::template store<false>(a, tile, r0, c0, w, lane);
        else
            M::template store<true>(a, tile, r0, c0, w, lane);
        __syncthreads();
    }
}

// Baseline: one work-item per element, source read along rows (contiguous per
// wavefront), destination written along columns (a stride of ld_dst between the
// lanes of a wavefront).  A workgroup covers 64 columns x 16 rows per step.
__global__ __launch_bounds__(256) void transpose_naive_kernel(TransposeArgs a)
{
    const unsigned tiles_c = ((unsigned)a.cols + 63) / 64;
    const unsigned tiles = tiles_c * (((unsigned)a.rows + 15) / 16);
    for (unsigned t = blockIdx.x; t < tiles; t += gridDim.x) {
        const int r0 = (int)(t / tiles_c) * 16;
        const int c = (int)(t % tiles_c) * 64 + (threadIdx.x & 63);
        const int rq = threadIdx.x >> 6;
        if (c >= a.cols)
            continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = r0 + rq + 4 * i;
            if (r < a.rows)
                a.dst[(int64_t)c * a.ld_dst + r] = a.src[(int64_t)r * a.ld_src + c];
        }
    }
}

// Few source columns: one work-item per destination element, destination rows
// written contiguously (64 x 16 destination elements per workgroup step).
__global__ __launch_bounds__(256) void transpose_narrow_kernel(TransposeArgs a)
{
    const unsigned tiles_i = ((unsigned)a.rows + 63) / 64;  // along destination rows
    const unsigned tiles = tiles_i * (((unsigned)a.cols + 15) / 16);
    for (unsigned t = blockIdx.x; t < tiles; t += gridDim.x) {
        const int j0 = (int)(t / tiles_i) * 16;
        const int i = (int)(t % tiles_i) * 64 + (threadIdx.x & 63);
        const int jq = threadIdx.x >> 6;
        if (i >= a.rows)
            continue;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int j = j0 + jq + 4 * k;
            if (j < a.cols)
                a.dst[(int64_t)j * a.ld_dst + i] = a.src[(int64_t)i * a.ld_src + j];
        }
    }
}

int transpose_shape(int64_t rows, int64_t cols)
{
    const int64_t tiles = ceil_div(rows, TP_T) * ceil_div(cols, TP_T);
    return tiles <= TP_SMALL_MAX_TILES ? TSHAPE_SMALL : tiles <= TP_PIPE_MAX_TILES ? TSHAPE_PIPE : TSHAPE_STREAM;
}

int64_t transpose_tiles(int kid, int64_t rows, int64_t cols)
{
    switch (kid) {
    case KID_TRANSPOSE_NAIVE: return ceil_div(rows, 16) * ceil_div(cols, 64);
    case KID_TRANSPOSE_NARROW: return ceil_div(rows, 64) * ceil_div(cols, 16);
    default: {
        const int64_t t = transpose_shape(rows, cols) == TSHAPE_SMALL ? TP_T_SMALL : TP_T;
        return ceil_div(rows, t) * ceil_div(cols, t);
    }
    }
}

int64_t transpose_blocks(int kid, int64_t rows, int64_t cols)
{
    const int64_t t = transpose_tiles(kid, rows, cols);
    const bool pipe = (kid == KID_TRANSPOSE_LDS_PAD || kid == KID_TRANSPOSE_LDS_NOPAD) &&
                      transpose_shape(rows, cols) == TSHAPE_PIPE;
    const int64_t cap = pipe ? TP_PIPE_BLOCKS : TP_MAX_BLOCKS;
    return t < cap ? t : cap;
}

hipError_t launch_transpose(const TransposeArgs &a, int kid, bool vec, hipStream_t stream)
{
    const dim3 grid((unsigned)transpose_blocks(kid, a.rows, a.cols));
    const bool pad = kid == KID_TRANSPOSE_LDS_PAD;
    switch (kid) {
    case KID_TRANSPOSE_NAIVE: transpose_naive_kernel<<<grid, dim3(256), 0, stream>>>(a); break;
    case KID_TRANSPOSE_NARROW: transpose_narrow_kernel<<<grid, dim3(256), 0, stream>>>(a); break;
    case KID_TRANSPOSE_LDS_PAD:
    case KID_TRANSPOSE_LDS_NOPAD:
        switch (transpose_shape(a.rows, a.cols)) {
        case TSHAPE_SMALL:
            if (pad)
                transpose_tile_kernel<TP_T_SMALL, 256, 1, false, false><<<grid, dim3(256), 0, stream>>>(a);
            else
                transpose_tile_kernel<TP_T_SMALL, 256, 0, false, false><<<grid, dim3(256), 0, stream>>>(a);
            break;
        case TSHAPE_PIPE:
            if (pad)
                transpose_pipe_kernel<1><<<grid, dim3(256), 0, stream>>>(a);
            else
                transpose_pipe_kernel<0><<<grid, dim3(256), 0, stream>>>(a);
            break;
        default:
            if (pad && vec)
                transpose_tile_kernel<TP_T, 512, 1, true, true><<<grid, dim3(512), 0, stream>>>(a);
            else if (pad)
                transpose_tile_kernel<TP_T, 512, 1, false, true><<<grid, dim3(512), 0, stream>>>(a);
            else
                transpose_tile_kernel<TP_T, 512, 0, false, true><<<grid, dim3(512), 0, stream>>>(a);
            break;
        }
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace sgemm
